// Large-row full-sort solver ("Fast LapSum: Exact Differentiable Top-k at
// Million Scale", section 2.2, full-sort solver) as one cooperative launch:
//
//   for each 8-bit digit pass (least significant first):
//     H: per-tile digit histograms                       (grid sync)
//     S: per-digit exclusive scan over tiles            (grid sync)
//     X: stable scatter: wave-ballot ranking, LDS stage,
//        coalesced runs per digit                          (grid sync)
//   C: per-tile anchored aggregates of the sorted keys  (grid sync)
//   L: per row, scan of the tile aggregates (with the bracket's tail sums as
//      boundary seeds), threshold curve at tile ends, locate of the
//      balancing tile, per-knot curve inside it, closed-form root,
//      certification against the bracket.
//
// Modes: full rows (the full-sort path), the compacted band of the
// bracketing path (keys offset by the band's minimum key so that only the
// needed digit passes run), and the deterministic fallback, which sorts the
// whole row only for rows whose bracket missed (and returns at once when
// none did).  Tiles hold 4096 keys (256 threads x 16).
#include <hip/hip_cooperative_groups.h>

#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

namespace lapsum {

namespace cg = cooperative_groups;

struct TileAgg {
  float aP, aS;
  double sP, sS;
};
size_t tile_agg_bytes() { return sizeof(TileAgg); }
size_t pre_bytes() { return sizeof(Pre); }
size_t suf_bytes() { return sizeof(Suf); }

constexpr int kKpt = kTile / kSegThreads;  // 16 keys per thread
constexpr int kSegWaves = kSegThreads / kWave;

struct ScatterLds {
  uint32_t stage[kTile];
  uint32_t wcnt[kSegWaves][256];
  uint32_t tstart[256];
  uint32_t dglob[256];
  uint32_t wsum[kSegWaves];
};
union SegLds {
  ScatterLds sc;
  BlockTeamLds<kSegThreads, 1> tm;
};

LDEV bool seg_active(const SegArgs &a, int row) {
  const RowState &s = a.st[row];
  if (a.mode == kSegFull) return true;
  if (a.mode == kSegFallback) return (s.flags & LAPSUM_FLAG_FALLBACK) != 0;
  return s.band <= (unsigned long long)a.stride;
}
LDEV int64_t seg_len(const SegArgs &a, int row) {
  if (!seg_active(a, row)) return 0;
  if (a.mode == kSegBand) return (int64_t)a.st[row].band;
  return a.n;
}
LDEV uint32_t seg_kbase(const SegArgs &a, int row) {
  if (a.mode != kSegBand) return 0u;
  const RowState &s = a.st[row];
  return s.band > 0 ? s.kmin : 0u;
}

// exclusive scan of one uint32 per thread over the workgroup
LDEV uint32_t wg_excl_scan(uint32_t v, uint32_t *wsum) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  __syncthreads();
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < kSegWaves; ++i)
    if (i < w) before += wsum[i];
  return before + inc - v;
}

LDEV uint32_t load_key(const SegArgs &a, int pass, int row, int64_t i, uint32_t kbase) {
  if (pass == 0) {
    if (a.mode == kSegBand) return a.band[(int64_t)row * a.stride + i] - kbase;
    return key_of(a.r[(int64_t)row * a.n + i]);
  }
  const uint32_t *src = (pass & 1) ? a.A : a.B;
  return src[(int64_t)row * a.stride + i];
}

LDEV void phase_hist(const SegArgs &a, int pass, SegLds &L) {
  const int shift = 8 * pass;
  uint32_t *h = L.sc.wcnt[0];  // 256 counters
  const int64_t items = (int64_t)a.rows * a.max_tiles;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int row = (int)(it / a.max_tiles), tile = (int)(it % a.max_tiles);
    const int64_t len = seg_len(a, row);
    const int64_t nt = (len + kTile - 1) / kTile;
    if (tile >= nt) continue;
    const uint32_t kbase = seg_kbase(a, row);
    h[threadIdx.x] = 0u;
    __syncthreads();
    for (int q = 0; q < kKpt; ++q) {
      const int64_t gi = (int64_t)tile * kTile + q * kSegThreads + threadIdx.x;
      if (gi < len) atomicAdd(&h[(load_key(a, pass, row, gi, kbase) >> shift) & 255u], 1u);
    }
    __syncthreads();
    a.hist[((int64_t)row * 256 + threadIdx.x) * a.max_tiles + tile] = h[threadIdx.x];
    __syncthreads();
  }
}

LDEV void phase_scan_digits(const SegArgs &a) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t items = (int64_t)a.rows * 256;
  for (int64_t it = (int64_t)blockIdx.x * kSegWaves + w; it < items; it += (int64_t)gridDim.x * kSegWaves) {
    const int row = (int)(it >> 8), d = (int)(it & 255);
    const int64_t len = seg_len(a, row);
    const int nt = (int)((len + kTile - 1) / kTile);
    if (nt == 0) continue;
    uint32_t *h = a.hist + ((int64_t)row * 256 + d) * a.max_tiles;
    uint32_t carry = 0;
    for (int base = 0; base < nt; base += kWave) {
      const int i = base + lane;
      const uint32_t v = i < nt ? h[i] : 0u;
      uint32_t inc = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
      }
      if (i < nt) h[i] = carry + inc - v;
      carry += __shfl(inc, kWave - 1, kWave);
    }
    if (lane == 0) a.dtot[(int64_t)row * 256 + d] = carry;
  }
}

LDEV void phase_scatter(const SegArgs &a, int pass, SegLds &L) {
  const int shift = 8 * pass;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const unsigned long long ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t *dst = (pass & 1) ? a.B : a.A;
  const int64_t items = (int64_t)a.rows * a.max_tiles;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int row = (int)(it / a.max_tiles), tile = (int)(it % a.max_tiles);
    const int64_t len = seg_len(a, row);
    const int64_t nt = (len + kTile - 1) / kTile;
    if (tile >= nt) continue;
    const uint32_t kbase = seg_kbase(a, row);

    uint32_t key[kKpt], rnk[kKpt];
    int dig[kKpt];
#pragma unroll
    for (int q = 0; q < kKpt; ++q) {
      const int64_t gi = (int64_t)tile * kTile + w * (kWave * kKpt) + q * kWave + lane;
      const bool valid = gi < len;
      key[q] = valid ? load_key(a, pass, row, gi, kbase) : 0u;
      dig[q] = valid ? (int)((key[q] >> shift) & 255u) : 256;
    }
    // global start of each digit in this row, and this tile's offset within it
    const uint32_t dtot = a.dtot[(int64_t)row * 256 + threadIdx.x];
    const uint32_t dbase = wg_excl_scan(dtot, L.sc.wsum);
    const uint32_t tofs = a.hist[((int64_t)row * 256 + threadIdx.x) * a.max_tiles + tile];
    volatile uint32_t *wc = L.sc.wcnt[w];
#pragma unroll
    for (int i = 0; i < 256 / kWave; ++i) wc[lane + i * kWave] = 0u;
    __syncthreads();
    // stable rank within the wave's chunk, round by round
#pragma unroll
    for (int q = 0; q < kKpt; ++q) {
      const int d = dig[q];
      const bool valid = d < 256;
      unsigned long long peers = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool set = (d >> bit) & 1;
        const unsigned long long bb = __ballot(set);
        peers &= set ? bb : ~bb;
      }
      const uint32_t lt = (uint32_t)__popcll(peers & ltmask);
      uint32_t prev = 0u;
      if (valid) prev = wc[d];
      rnk[q] = prev + lt;
      if (valid && lt == 0u) wc[d] = prev + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    {
      const int d = threadIdx.x;
      uint32_t run = 0u;
#pragma unroll
      for (int ww = 0; ww < kSegWaves; ++ww) {
        const uint32_t c = L.sc.wcnt[ww][d];
        L.sc.wcnt[ww][d] = run;
        run += c;
      }
      const uint32_t ts = wg_excl_scan(run, L.sc.wsum);
      L.sc.tstart[d] = ts;
      L.sc.dglob[d] = dbase + tofs - ts;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kKpt; ++q) {
      const int d = dig[q];
      if (d < 256) L.sc.stage[L.sc.tstart[d] + L.sc.wcnt[w][d] + rnk[q]] = key[q];
    }
    __syncthreads();
    const int vc = (int)min((int64_t)kTile, len - (int64_t)tile * kTile);
    uint32_t *drow = dst + (int64_t)row * a.stride;
    for (int i = threadIdx.x; i < vc; i += kSegThreads) {
      const uint32_t kk = L.sc.stage[i];
      drow[L.sc.dglob[(kk >> shift) & 255u] + i] = kk;
    }
    __syncthreads();
  }
}

// sorted tile -> values (blocked, 16 per thread)
LDEV int load_sorted_tile(const SegArgs &a, const uint32_t *fin, int row, int tile, int64_t len, uint32_t kbase,
                          float (&s)[kKpt]) {
  const int64_t base = (int64_t)tile * kTile + (int64_t)threadIdx.x * kKpt;
  const int nv = (int)min(max(len - base, (int64_t)0), (int64_t)kKpt);
  const uint32_t *src = fin + (int64_t)row * a.stride + base;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) s[e] = (e < nv) ? value_of(src[e] + kbase) : 0.0f;
  return nv;
}

LDEV void phase_tiles(const SegArgs &a, const uint32_t *fin, SegLds &L) {
  BlockTeam<kSegThreads, 1> team(&L.tm);
  const int64_t items = (int64_t)a.rows * a.max_tiles;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int row = (int)(it / a.max_tiles), tile = (int)(it % a.max_tiles);
    const int64_t len = seg_len(a, row);
    const int64_t nt = (len + kTile - 1) / kTile;
    if (tile >= nt) continue;
    float s[kKpt];
    const int nv = load_sorted_tile(a, fin, row, tile, len, seg_kbase(a, row), s);
    float mul[kKpt];
    mul[0] = 0.0f;
#pragma unroll
    for (int e = 1; e < kKpt; ++e) mul[e] = (e < nv) ? wexpf(s[e - 1] - s[e], a.cf) : 0.0f;
    double pl = 0.0, sl = 0.0;
    float last = s[0];
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if (e < nv) {
        pl = pl * (double)mul[e] + 1.0;
        last = s[e];
      }
#pragma unroll
    for (int e = kKpt - 1; e >= 0; --e)
      if (e < nv) sl = (e + 1 < kKpt ? sl * (double)mul[e + 1] : 0.0) + 1.0;
    const Pre mp{last, nv > 0 ? pl : 0.0};
    const Suf ms{s[0], nv > 0 ? sl : 0.0};
    const Pre ep = team.excl_scan(mp, a.c);
    const Suf es = team.excl_scan(ms, a.c);
    TileAgg *ta = a.tagg + (int64_t)row * a.max_tiles + tile;
    if (threadIdx.x == kSegThreads - 1) {
      const Pre tp = join(ep, mp, a.c);
      ta->aP = tp.a;
      ta->sP = tp.s;
    }
    if (threadIdx.x == 0) {
      const Suf ts = join(ms, es, a.c);
      ta->aS = ts.a;
      ta->sS = ts.s;
    }
    __syncthreads();
  }
}

LDEV void phase_locate(const SegArgs &a, const uint32_t *fin, SegLds &L) {
  BlockTeam<kSegThreads, 1> team(&L.tm);
  for (int row = blockIdx.x; row < a.rows; row += gridDim.x) {
    RowState &S = a.st[row];
    if (a.mode == kSegBand && S.band > (unsigned long long)a.stride) {
      if (threadIdx.x == 0) S.flags |= LAPSUM_FLAG_OVERFLOW | LAPSUM_FLAG_FALLBACK;
      continue;
    }
    if (!seg_active(a, row)) continue;
    const int64_t len = seg_len(a, row);
    const int nt = (int)((len + kTile - 1) / kTile);
    const bool band = a.mode == kSegBand;
    const Pre seed_lo{(float)S.a_lo, (band && S.count_lo) ? S.tail_lo : 0.0};
    const Suf seed_hi{(float)S.a_hi, (band && S.count_hi) ? S.tail_hi : 0.0};
    const double cR = band ? (double)S.count_hi : 0.0;
    const TileAgg *ta = a.tagg + (int64_t)row * a.max_tiles;
    Pre *tp = a.tpre + (int64_t)row * a.max_tiles;
    Suf *ts = a.tsuf + (int64_t)row * a.max_tiles;

    Pre carry = seed_lo;
    for (int T0 = 0; T0 < nt; T0 += kSegThreads) {
      const int T = T0 + threadIdx.x;
      const Pre mine = T < nt ? Pre{ta[T].aP, ta[T].sP} : Pre{0.0f, 0.0};
      const Pre ex = team.excl_scan(mine, a.c);
      if (T < nt) tp[T] = join(carry, ex, a.c);
      const Pre tot = join(ex, mine, a.c);
      const Pre chunk{team.bcast(tot.a, kSegThreads - 1), team.bcast(tot.s, kSegThreads - 1)};
      carry = join(carry, chunk, a.c);
    }
    Suf carry_s = seed_hi;
    for (int T0 = ((nt - 1) / kSegThreads) * kSegThreads; nt > 0 && T0 >= 0; T0 -= kSegThreads) {
      const int T = T0 + threadIdx.x;
      const Suf mine = T < nt ? Suf{ta[T].aS, ta[T].sS} : Suf{0.0f, 0.0};
      const Suf ex = team.excl_scan(mine, a.c);
      if (T < nt) ts[T] = join(ex, carry_s, a.c);
      const Suf tot = join(mine, ex, a.c);
      const Suf chunk{team.bcast(tot.a, 0), team.bcast(tot.s, 0)};
      carry_s = join(chunk, carry_s, a.c);
    }
    __syncthreads();
    // threshold curve at the last knot of every tile
    int cnt = 0;
    for (int T = threadIdx.x; T < nt; T += kSegThreads) {
      const Pre pl = join(tp[T], Pre{ta[T].aP, ta[T].sP}, a.c);
      const Suf sa = ts[T];
      const double s_last = 1.0 + (sa.s == 0.0 ? 0.0 : sa.s * (double)wexp((double)pl.a - (double)sa.a, a.c));
      const int64_t nvT = min((int64_t)kTile, len - (int64_t)T * kTile);
      const int64_t j_last = (int64_t)T * kTile + nvT - 1;
      const double g = 0.5 * (pl.s - 1.0) + ((double)(len - j_last) + cR) - 0.5 * s_last;
      cnt += (g >= a.k) ? 1 : 0;
    }
    const int tstar = team.sum(cnt);
    const int tsel = nt == 0 ? 0 : min(tstar, nt - 1);
    float s[kKpt];
    int nv = 0;
    if (nt > 0) nv = load_sorted_tile(a, fin, row, tsel, len, seg_kbase(a, row), s);
    else {
#pragma unroll
      for (int e = 0; e < kKpt; ++e) s[e] = 0.0f;
    }
    PartInfo part;
    part.nvalid = nv;
    part.above = (double)(len - (int64_t)tsel * kTile) + cR;
    part.seed_lo = nt > 0 ? tp[tsel] : seed_lo;
    part.seed_hi = nt > 0 ? ts[tsel] : seed_hi;
    part.first = tsel == 0;
    part.last = tsel >= nt - 1;
    const double b = segment_solve<kKpt>(s, nv, part, a.k, a.t, a.c, a.cf, team);
    if (threadIdx.x == 0) {
      S.b = b;
      if (band) {
        const bool hit = (b >= S.a_lo) && (b < S.a_hi);
        S.flags |= hit ? LAPSUM_FLAG_HIT : LAPSUM_FLAG_FALLBACK;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSegThreads) void segment_kernel(SegArgs a) {
  __shared__ SegLds L;
  // uniform early exit (every workgroup reads the same state)
  int npasses = 4;
  if (a.mode == kSegFallback) {
    bool any = false;
    for (int row = 0; row < a.rows; ++row) any |= (a.st[row].flags & LAPSUM_FLAG_FALLBACK) != 0;
    if (!any) return;
  } else if (a.mode == kSegBand) {
    uint32_t span = 0u;
    for (int row = 0; row < a.rows; ++row) {
      const RowState &s = a.st[row];
      if (s.band > 1 && s.band <= (unsigned long long)a.stride && s.kmax > s.kmin) span = max(span, s.kmax - s.kmin);
    }
    const int bits = span == 0u ? 1 : 32 - __clz((int)span);
    npasses = (bits + 7) / 8;
  }
  cg::grid_group grid = cg::this_grid();
  for (int pass = 0; pass < npasses; ++pass) {
    phase_hist(a, pass, L);
    grid.sync();
    phase_scan_digits(a);
    grid.sync();
    phase_scatter(a, pass, L);
    grid.sync();
  }
  const uint32_t *fin = (npasses & 1) ? a.A : a.B;
  phase_tiles(a, fin, L);
  grid.sync();
  phase_locate(a, fin, L);
}

hipError_t launch_segment(const SegArgs &a, hipStream_t s) {
  static int cached_dev = -1, max_blocks = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (cached_dev != dev) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, segment_kernel, kSegThreads, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    max_blocks = cus * (per_cu < 4 ? per_cu : 4);
    cached_dev = dev;
  }
  int64_t need = (int64_t)a.rows * a.max_tiles;
  const int64_t scan_need = ((int64_t)a.rows * 256 + kSegWaves - 1) / kSegWaves;
  if (scan_need > need) need = scan_need;
  if ((int64_t)a.rows > need) need = a.rows;
  const int grid = (int)(need < max_blocks ? need : max_blocks);
  SegArgs copy = a;
  void *args[] = {(void *)&copy};
  return hipLaunchCooperativeKernel((const void *)segment_kernel, dim3(grid), dim3(kSegThreads), args, 0, s);
}

}  // namespace lapsum
