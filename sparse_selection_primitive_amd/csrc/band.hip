// Bucketed band solve for bands too large for one workgroup ("Fast LapSum:
// Exact Differentiable Top-k at Million Scale", section 2.2, probabilistic
// bracketing, step 3: the band is sorted and solved exactly, seeded with the
// tail sums; step 4: certification).
//
// The band keys lie in [kmin, kmax].  Bucket j holds the keys with
// (key - kmin) >> shift == j, shift the smallest value that leaves at most
// kBandBuckets buckets; every key of bucket j is below every key of bucket
// j + 1, so sorting each bucket on its own sorts the band (one
// most-significant-digit radix pass, then independent bucket sorts).
//
//   band_count_kernel    bucket counts of each workgroup's filter slots
//   band_scan_kernel     per bucket, offsets of the workgroups inside it
//   band_scatter_kernel  keys to their bucket (order inside a bucket free)
//   band_sort_kernel     one wave sorts each bucket of at most 1024 keys in
//                        registers; larger buckets are sorted by the whole
//                        workgroup; anchored aggregates of every bucket
//   band_locate_kernel   scan of the bucket aggregates between the tail
//                        seeds, threshold curve at the bucket ends, the
//                        balancing bucket, the root inside it,
//                        certification, and the full-sort fallback of a row
//                        whose bracket missed
//
// Every count is an integer and every floating-point sum runs over sorted
// keys in a fixed order, so the result does not depend on the order in which
// the scatter placed keys inside a bucket.
#include <limits.h>

#include "segment_dev.hpp"

namespace lapsum {

constexpr int kBT = 256;                   // threads per workgroup of every band kernel
constexpr int kBPT = kBandBuckets / kBT;   // buckets per thread in the per-row scans
constexpr int kWaveBucket = 16 * kWave;    // largest bucket one wave sorts
static_assert(kBPT * kBT == kBandBuckets, "bucket count must be a multiple of the workgroup size");

LDEV bool band_active(const RowState &S) { return !(S.flags & LAPSUM_FLAG_OVERFLOW); }

LDEV int band_shift(const RowState &S) {
  const uint32_t span = (S.band > 1 && S.kmax > S.kmin) ? S.kmax - S.kmin : 0u;
  const int bits = span == 0u ? 0 : 32 - __clz((int)span);
  return max(bits - kBandBucketBits, 0);
}

// Band keys of count/scatter workgroup `blk`: wave w walks the workgroup's
// slots w, w + 4, ...; its lanes stride through each slot.  The slot bounds
// of all the workgroup's slots are read first (one round trip), into `sb`.
constexpr int kMaxGroup = 64;  // filter slots per count/scatter workgroup, at most
LDEV void load_slot_bounds(const BandArgs &a, int64_t row, int blk, uint32_t *sb) {
  const uint32_t *ro = a.offs + row * (a.gx + 1);
  const int s0 = blk * a.group, ns = min(a.gx - s0, a.group);
  for (int i = threadIdx.x; i <= ns; i += kBT) sb[i] = ro[s0 + i];
}
template <class F>
LDEV void for_each_band_key(const BandArgs &a, int64_t row, int blk, const uint32_t *sb, F &&f) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int s0 = blk * a.group, ns = min(a.gx - s0, a.group);
  for (int i = w; i < ns; i += kBT / kWave) {
    const uint32_t cnt = sb[i + 1] - sb[i];
    const uint32_t *src = a.slots + (row * a.gx + s0 + i) * (int64_t)kBandSlot;
    for (uint32_t q = lane; q < cnt; q += kWave) f(src[q]);
  }
}

__global__ __launch_bounds__(kBT) void band_count_kernel(BandArgs a) {
  __shared__ uint32_t h[kBandBuckets];
  __shared__ uint32_t sb[kMaxGroup + 1];
  const int64_t row = blockIdx.y;
  const int blk = blockIdx.x;
  const RowState &S = a.st[row];
  load_slot_bounds(a, row, blk, sb);
  for (int j = threadIdx.x; j < kBandBuckets; j += kBT) h[j] = 0u;
  if (!band_active(S)) return;
  const uint32_t kmin = S.kmin;
  const int shift = band_shift(S);
  __syncthreads();
  for_each_band_key(a, row, blk, sb, [&](uint32_t key) { atomicAdd(&h[(key - kmin) >> shift], 1u); });
  __syncthreads();
  uint32_t *dst = a.hist + (row * a.nblk + blk) * (int64_t)kBandBuckets;
  for (int j = threadIdx.x; j < kBandBuckets; j += kBT) dst[j] = h[j];
}

// one thread per bucket: exclusive scan over the count workgroups, in
// place; every count is loaded before the first is used
__global__ __launch_bounds__(kBT) void band_scan_kernel(BandArgs a) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kBT + threadIdx.x;
  uint32_t *h = a.hist + row * a.nblk * (int64_t)kBandBuckets + j;
  uint32_t v[kBandCountBlocks];
#pragma unroll
  for (int b = 0; b < kBandCountBlocks; ++b) v[b] = b < a.nblk ? h[(int64_t)b * kBandBuckets] : 0u;
  if (!band_active(a.st[row])) return;
  uint32_t run = 0u;
#pragma unroll
  for (int b = 0; b < kBandCountBlocks; ++b) {
    if (b < a.nblk) h[(int64_t)b * kBandBuckets] = run;
    run += v[b];
  }
  a.btot[row * kBandBuckets + j] = run;
}

__global__ __launch_bounds__(kBT) void band_scatter_kernel(BandArgs a) {
  __shared__ uint32_t base[kBandBuckets];
  __shared__ uint32_t wsum[kBT / kWave];
  __shared__ uint32_t sb[kMaxGroup + 1];
  const int64_t row = blockIdx.y;
  const int blk = blockIdx.x;
  const RowState &S = a.st[row];
  // bucket sizes (thread i owns buckets i*kBPT ..), this workgroup's offset
  // inside each bucket and its slot bounds, all loaded before any is used
  const int64_t o = row * kBandBuckets;
  const uint32_t *hin = a.hist + (row * a.nblk + blk) * (int64_t)kBandBuckets;
  uint32_t v[kBPT], hv[kBPT];
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    v[u] = a.btot[o + threadIdx.x * kBPT + u];
    hv[u] = hin[threadIdx.x * kBPT + u];
  }
  load_slot_bounds(a, row, blk, sb);
  if (!band_active(S)) return;
  const uint32_t kmin = S.kmin;
  const int shift = band_shift(S);
  uint32_t sum = 0u;
#pragma unroll
  for (int u = 0; u < kBPT; ++u) sum += v[u];
  uint32_t run = wg_excl_scan<kBT>(sum, wsum);
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int j = threadIdx.x * kBPT + u;
    base[j] = run + hv[u];
    if (blk == 0) a.bstart[o + j] = run;
    run += v[u];
  }
  __syncthreads();
  uint32_t *dst = a.keys + row * a.cap;
  for_each_band_key(a, row, blk, sb, [&](uint32_t key) {
    const uint32_t pos = atomicAdd(&base[(key - kmin) >> shift], 1u);
    dst[pos] = key;
  });
}

// ------------------------------------------------------------ bucket sort
LDEV void write_agg(TileAgg *out, Pre p, Suf s) {
  out->aP = p.a;
  out->sP = p.s;
  out->aS = s.a;
  out->sS = s.s;
}

// One wave sorts a bucket of cnt <= 64*E keys in registers (blocked, E per
// lane), writes it back and stores its anchored aggregates.
template <int E>
LDEV void wave_bucket(uint32_t *kb, int cnt, double c, float cf, TileAgg *out) {
  WaveTeam<kWave> team;
  const int base = team.lane * E;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = (base + e < cnt) ? kb[base + e] : 0xFFFFFFFFu;
  bitonic_sort<E>(key, team);
  const int nv = min(max(cnt - base, 0), E);
  float s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s[e] = (e < nv) ? value_of(key[e]) : 0.0f;
    if (e < nv) kb[base + e] = key[e];
  }
  team_aggregate<E>(s, nv, c, cf, team, out);
}

union BandSortLds {
  RankLds<kBT> rk;
  BlockTeamLds<kBT, kKpt> sort;
  BlockTeamLds<kBT, 1> scan;
};

// The whole workgroup sorts one bucket of more than 1024 keys: a register
// bitonic sort up to 4096 keys, else a stable LSD radix sort (8-bit digits)
// of the keys relative to the bucket's lowest possible key `kb0` (they differ
// in their low `bits` bits only).  Then the bucket's aggregates, tile by tile.
LDEV void block_bucket(uint32_t *kb, uint32_t *tb, int cnt, uint32_t kb0, int bits, double c, float cf,
                       BandSortLds &L, TileAgg *lagg, TileAgg *out) {
  constexpr int TT = kBT * kKpt;
  if (cnt <= TT) {
    BlockTeam<kBT, kKpt> team(&L.sort);
    const int base = threadIdx.x * kKpt;
    uint32_t key[kKpt];
#pragma unroll
    for (int e = 0; e < kKpt; ++e) key[e] = (base + e < cnt) ? kb[base + e] : 0xFFFFFFFFu;
    bitonic_sort<kKpt>(key, team);
#pragma unroll
    for (int e = 0; e < kKpt; ++e)
      if (base + e < cnt) kb[base + e] = key[e];
    __syncthreads();
  } else {
    __shared__ uint32_t h[256];
    for (int i = threadIdx.x; i < cnt; i += kBT) kb[i] -= kb0;
    __syncthreads();
    uint32_t *src = kb, *dst = tb;
    const int npass = (bits + 7) / 8;
    const int ntiles = (cnt + TT - 1) / TT;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    for (int pass = 0; pass < npass; ++pass) {
      const int sh = 8 * pass;
      h[threadIdx.x] = 0u;
      __syncthreads();
      for (int i = threadIdx.x; i < cnt; i += kBT) atomicAdd(&h[(src[i] >> sh) & 255u], 1u);
      __syncthreads();
      uint32_t run = wg_excl_scan<kBT>(h[threadIdx.x], L.rk.wsum);
      for (int tile = 0; tile < ntiles; ++tile) {
        uint32_t key[kKpt];
        int dig[kKpt];
#pragma unroll
        for (int q = 0; q < kKpt; ++q) {
          const int gi = tile * TT + w * (kWave * kKpt) + q * kWave + lane;
          const bool valid = gi < cnt;
          key[q] = valid ? src[gi] : 0u;
          dig[q] = valid ? (int)((key[q] >> sh) & 255u) : 256;
        }
        const int vc = min(TT, cnt - tile * TT);
        run += scatter_tile<kBT>(key, dig, sh, vc, run, dst, L.rk);
      }
      uint32_t *x = src;
      src = dst;
      dst = x;
    }
    for (int i = threadIdx.x; i < cnt; i += kBT) kb[i] = src[i] + kb0;
    __syncthreads();
  }
  // aggregates of the sorted bucket, tile by tile, joined in order
  BlockTeam<kBT, 1> team(&L.scan);
  Pre ap{0.0f, 0.0};
  Suf as{0.0f, 0.0};
  for (int t0 = 0; t0 < cnt; t0 += TT) {
    float s[kKpt];
    const int nv = load_sorted_at<kBT>(kb, t0, cnt, 0u, s);
    team_aggregate<kKpt>(s, nv, c, cf, team, lagg);
    ap = join(ap, Pre{lagg->aP, lagg->sP}, c);
    as = join(as, Suf{lagg->aS, lagg->sS}, c);
    __syncthreads();
  }
  if (threadIdx.x == 0) write_agg(out, ap, as);
}

__global__ __launch_bounds__(kBT) void band_sort_kernel(BandArgs a) {
  __shared__ BandSortLds L;
  __shared__ TileAgg lagg;
  const int64_t row = blockIdx.y;
  const RowState &S = a.st[row];
  const int64_t o = row * kBandBuckets;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = blockIdx.x * (kBT / kWave) + (int)threadIdx.x / kWave;
  const int cnt = (int)a.btot[o + j];
  const uint32_t bst = a.bstart[o + j];
  if (!band_active(S)) return;
  const int shift = band_shift(S);
  uint32_t *kb = a.keys + row * a.cap + bst;
  TileAgg *out = a.bagg + o + j;
  if (cnt == 0) {
    if (lane == 0) write_agg(out, Pre{0.0f, 0.0}, Suf{0.0f, 0.0});
  } else if (shift == 0) {
    // every key of the bucket is the same value
    if (lane == 0) {
      const float x = value_of(kb[0]);
      write_agg(out, Pre{x, (double)cnt}, Suf{x, (double)cnt});
    }
  } else if (cnt <= 64) {
    wave_bucket<1>(kb, cnt, a.c, a.cf, out);
  } else if (cnt <= 128) {
    wave_bucket<2>(kb, cnt, a.c, a.cf, out);
  } else if (cnt <= 256) {
    wave_bucket<4>(kb, cnt, a.c, a.cf, out);
  } else if (cnt <= 512) {
    wave_bucket<8>(kb, cnt, a.c, a.cf, out);
  } else if (cnt <= kWaveBucket) {
    wave_bucket<16>(kb, cnt, a.c, a.cf, out);
  }
  if (shift == 0) return;
  // buckets beyond one wave: the whole workgroup, one after another
  for (int w = 0; w < kBT / kWave; ++w) {
    const int jj = blockIdx.x * (kBT / kWave) + w;
    const int cc = (int)a.btot[o + jj];
    if (cc <= kWaveBucket) continue;
    __syncthreads();
    const uint32_t st0 = a.bstart[o + jj];
    block_bucket(a.keys + row * a.cap + st0, a.tmp + row * a.cap + st0, cc, S.kmin + ((uint32_t)jj << shift), shift,
                 a.c, a.cf, L, &lagg, a.bagg + o + jj);
  }
}

// ---------------------------------------------------------------- locate
// One workgroup of kLocT threads per row, two buckets per thread: a
// workgroup scan of the bucket aggregates between the tail seeds, the
// threshold curve at the bucket ends, the balancing bucket, and the root
// inside it (by one wave when the bucket fits its registers, else by the
// whole workgroup).  A row whose root falls outside its bracket is then
// sorted and solved in full by the same workgroup (the deterministic
// fallback), so no separate launch is needed.
constexpr int kLocT = 1024;
constexpr int kLocPer = kBandBuckets / kLocT;
static_assert(kLocPer == 2, "two buckets per locate thread");

union BandLocLds {
  BlockTeamLds<kLocT, 1> team;
  SegLds<kLocT> fb;
};

__global__ __launch_bounds__(kLocT) void band_locate_kernel(BandArgs a, SegArgs fb) {
  __shared__ BandLocLds L;
  __shared__ int red[3][kLocT / kWave];
  __shared__ float sel_pa, sel_sa;
  __shared__ double sel_ps, sel_ss, sel_b;
  __shared__ uint32_t sel_c, sel_st;
  __shared__ int sel_fb;
  const int64_t row = blockIdx.x;
  RowState &S = a.st[row];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t o = row * kBandBuckets;
  const int j0 = threadIdx.x * kLocPer;
  // this thread's bucket records (issued before the row state is examined)
  TileAgg g[kLocPer];
  uint32_t cnt[kLocPer], st0[kLocPer];
#pragma unroll
  for (int u = 0; u < kLocPer; ++u) {
    g[u] = a.bagg[o + j0 + u];
    cnt[u] = a.btot[o + j0 + u];
    st0[u] = a.bstart[o + j0 + u];
  }
  const bool active = band_active(S);
  if (threadIdx.x == 0) sel_fb = active ? 0 : 1;  // overflow: the row is already flagged for the fallback
  if (active) {
    BlockTeam<kLocT, 1> team(&L.team);
    const double c = a.c;
    const int64_t M = (int64_t)S.band;
    const Pre seed_lo{(float)S.a_lo, S.count_lo ? S.tail_lo : 0.0};
    const Suf seed_hi{(float)S.a_hi, S.count_hi ? S.tail_hi : 0.0};
    const double cR = (double)S.count_hi;
    const Pre p0{g[0].aP, g[0].sP}, p1{g[1].aP, g[1].sP};
    const Suf q0{g[0].aS, g[0].sS}, q1{g[1].aS, g[1].sS};
    const Pre ex_p = join(seed_lo, team.excl_scan(join(p0, p1, c), c), c);
    const Suf ex_s = join(team.excl_scan(join(q0, q1, c), c), seed_hi, c);
    const Pre before[kLocPer] = {ex_p, join(ex_p, p0, c)};
    const Suf after[kLocPer] = {join(q1, ex_s, c), ex_s};
    // threshold curve at the last knot of every non-empty bucket
    int first_lt = INT_MAX, first_ne = INT_MAX, last_ne = -1;
#pragma unroll
    for (int u = 0; u < kLocPer; ++u) {
      if (cnt[u] > 0u) {
        const int j = j0 + u;
        const Pre pl = join(before[u], Pre{g[u].aP, g[u].sP}, c);
        const Suf sa = after[u];
        const double s_last = 1.0 + (sa.s == 0.0 ? 0.0 : sa.s * (double)wexp((double)pl.a - (double)sa.a, c));
        const int64_t j_last = (int64_t)st0[u] + cnt[u] - 1;
        const double gv = 0.5 * (pl.s - 1.0) + ((double)(M - j_last) + cR) - 0.5 * s_last;
        if (gv < a.k) first_lt = min(first_lt, j);
        first_ne = min(first_ne, j);
        last_ne = max(last_ne, j);
      }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      first_lt = min(first_lt, __shfl_xor(first_lt, m, kWave));
      first_ne = min(first_ne, __shfl_xor(first_ne, m, kWave));
      last_ne = max(last_ne, __shfl_xor(last_ne, m, kWave));
    }
    if (lane == 0) {
      red[0][w] = first_lt;
      red[1][w] = first_ne;
      red[2][w] = last_ne;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kLocT / kWave; ++i) {
      first_lt = min(first_lt, red[0][i]);
      first_ne = min(first_ne, red[1][i]);
      last_ne = max(last_ne, red[2][i]);
    }
    // the balancing bucket: the first whose last knot has g < k, else the last
    const int J = first_lt != INT_MAX ? first_lt : last_ne;  // -1: empty band
    if (J >= 0 && (int)threadIdx.x == J / kLocPer) {
      const int u = J % kLocPer;
      sel_pa = u == 0 ? before[0].a : before[1].a;
      sel_ps = u == 0 ? before[0].s : before[1].s;
      sel_sa = u == 0 ? after[0].a : after[1].a;
      sel_ss = u == 0 ? after[0].s : after[1].s;
      sel_c = u == 0 ? cnt[0] : cnt[1];
      sel_st = u == 0 ? st0[0] : st0[1];
    }
    __syncthreads();
    const int64_t cJ = J >= 0 ? (int64_t)sel_c : 0;
    const int64_t sJ = J >= 0 ? (int64_t)sel_st : 0;
    const Pre slo = J >= 0 ? Pre{sel_pa, sel_ps} : seed_lo;
    const Suf shi = J >= 0 ? Suf{sel_sa, sel_ss} : seed_hi;
    const double cR_eff = (double)(M - sJ - cJ) + cR;
    const bool first = J < 0 || J == first_ne;
    const bool last = J < 0 || J == last_ne;
    const uint32_t *src = a.keys + row * a.cap + sJ;
    if (cJ <= (int64_t)kWaveBucket) {
      if (w == 0) {
        WaveTeam<kWave> wteam;
        float s[16];
        const int base = wteam.lane * 16;
        const int nv = (int)min(max(cJ - base, (int64_t)0), (int64_t)16);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = e < nv ? value_of(src[base + e]) : 0.0f;
        PartInfo part;
        part.nvalid = nv;
        part.above = (double)cJ + cR_eff;
        part.seed_lo = slo;
        part.seed_hi = shi;
        part.first = first;
        part.last = last;
        const double bb = segment_solve<16>(s, nv, part, a.k, a.t, c, a.cf, wteam);
        if (lane == 0) sel_b = bb;
      }
    } else {
      // a bucket of several tiles: its tile aggregates, then locate over them
      constexpr int TT = kLocT * kKpt;
      TileAgg *ta = a.tagg + row * a.max_tiles;
      for (int64_t t0 = 0; t0 < cJ; t0 += TT) {
        float s[kKpt];
        const int nv = load_sorted_at<kLocT>(src, t0, cJ, 0u, s);
        tile_aggregate<kLocT>(s, nv, c, a.cf, team, ta + t0 / TT);
      }
      const double bb = locate_sorted<kLocT>(src, cJ, 0u, slo, shi, cR_eff, first, last, ta,
                                             a.tpre + row * a.max_tiles, a.tsuf + row * a.max_tiles, a.k, a.t, c,
                                             a.cf, team);
      if (threadIdx.x == 0) sel_b = bb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const double bb = sel_b;
      S.b = bb;
      const bool hit = (bb >= S.a_lo) && (bb < S.a_hi);
      S.flags |= hit ? LAPSUM_FLAG_HIT : LAPSUM_FLAG_FALLBACK;
      sel_fb = hit ? 0 : 1;
    }
  }
  __syncthreads();
  if (sel_fb) fallback_row<kLocT>(fb, (int)row, L.fb);
}

int band_count_blocks(int gx, int *group) {
  const int nblk = gx < kBandCountBlocks ? gx : kBandCountBlocks;
  *group = (gx + nblk - 1) / nblk;
  return (gx + *group - 1) / *group;
}

hipError_t launch_band_buckets(const BandArgs &a, const SegArgs &fb, hipStream_t s) {
  const dim3 blk((unsigned)a.nblk, (unsigned)a.rows);
  hipLaunchKernelGGL(band_count_kernel, blk, dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_scan_kernel, dim3(kBandBuckets / kBT, (unsigned)a.rows), dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_scatter_kernel, blk, dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_sort_kernel, dim3(kBandBuckets / (kBT / kWave), (unsigned)a.rows), dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_locate_kernel, dim3((unsigned)a.rows), dim3(kLocT), 0, s, a, fb);
  return hipGetLastError();
}

}  // namespace lapsum
