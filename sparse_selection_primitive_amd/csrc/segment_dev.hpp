// Device routines of the full-sort solver shared by the one-workgroup
// fallback, the on-chip band kernel (onchip.hip) and the bucketed band solve
// (band.hip): stable scatter of a tile, anchored aggregates of sorted runs,
// and locate + closed-form root over a sorted range.
// Method: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
// section 2.2, full-sort solver.
#pragma once

#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

namespace lapsum {

struct TileAgg {
  float aP, aS;
  double sP, sS;
};

constexpr int kKpt = 16;  // keys per thread in a tile

template <int NT>
struct RankLds {
  static constexpr int NW = NT / kWave;
  uint32_t stage[NT * kKpt];
  uint32_t wcnt[NW][256];
  uint32_t tstart[256];
  uint32_t dglob[256];
  uint32_t wsum[NW];
};

// Buckets of the one-workgroup fallback's key sets: counts, key extremes and
// fixed-point sums anchored at the extremes.
constexpr int kFallbackBucketBits = 11;
constexpr int kFallbackBuckets = 1 << kFallbackBucketBits;
struct BucketSelLds {
  uint32_t cnt[kFallbackBuckets], kmx[kFallbackBuckets], kmn[kFallbackBuckets];
  unsigned long long sp[kFallbackBuckets], ss[kFallbackBuckets];
  uint32_t ctr;  // gather cursor
};

// Widening of a missed bracket: radix-select histograms of the sample (two
// targets), and the per-wave partials of the row pass.
struct WidenLds {
  uint32_t hist[2][kFallbackBuckets];
  uint32_t pick[2][3];  // bin, rank inside the bin, count: per target
  double sum[2][16];
  unsigned long long cnt[2][16];
  uint32_t kext[2][16];
  uint32_t ctr;
};

template <int NT>
union SegLds {
  RankLds<NT> rk;
  BlockTeamLds<NT, 1> tm;
  BucketSelLds bs;
  WidenLds wd;
};

template <int NT>
LDEV uint32_t wg_excl_scan(uint32_t v, uint32_t *wsum) {
  constexpr int NW = NT / kWave;
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
  for (int i = 0; i < NW; ++i)
    if (i < w) before += wsum[i];
  return before + inc - v;
}

// ----------------------------------------------------------- tile routines
// Stable scatter of one tile.  Thread d < 256 passes in `digit_base`, the
// position in `dst` where this tile's keys of digit d start; it gets back the
// number of this tile's keys of digit d.
template <int NT>
LDEV uint32_t scatter_tile(const uint32_t (&key)[kKpt], const int (&dig)[kKpt], int shift, int vc,
                           uint32_t digit_base, uint32_t *dst, RankLds<NT> &L) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const unsigned long long ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  volatile uint32_t *wc = L.wcnt[w];
#pragma unroll
  for (int i = 0; i < 256 / kWave; ++i) wc[lane + i * kWave] = 0u;
  __syncthreads();
  // rank within the wave's chunk, round by round: peers with the same digit
  // by 8 ballots, one LDS read-modify-write per digit group
  uint32_t rnk[kKpt];
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
  const int d = threadIdx.x;
  uint32_t tcount = 0u;
  if (d < 256) {
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const uint32_t c = L.wcnt[ww][d];
      L.wcnt[ww][d] = tcount;
      tcount += c;
    }
  }
  const uint32_t ts = wg_excl_scan<NT>(d < 256 ? tcount : 0u, L.wsum);
  if (d < 256) {
    L.tstart[d] = ts;
    L.dglob[d] = digit_base - ts;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kKpt; ++q) {
    const int dq = dig[q];
    if (dq < 256) L.stage[L.tstart[dq] + L.wcnt[w][dq] + rnk[q]] = key[q];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < vc; i += NT) {
    const uint32_t kk = L.stage[i];
    dst[L.dglob[(kk >> shift) & 255u] + i] = kk;
  }
  __syncthreads();
  return tcount;
}

// Sorted keys t0 .. t0 + NT*16 of the sorted range `src` as values, blocked
// (16 per thread); kbase is added back to each stored key.
template <int NT>
LDEV int load_sorted_at(const uint32_t *src, int64_t t0, int64_t len, uint32_t kbase, float (&s)[kKpt]) {
  const int64_t base = t0 + (int64_t)threadIdx.x * kKpt;
  const int nv = (int)min(max(len - base, (int64_t)0), (int64_t)kKpt);
  const uint32_t *p = src + base;
#pragma unroll
  for (int e = 0; e < kKpt; ++e) s[e] = (e < nv) ? value_of(p[e] + kbase) : 0.0f;
  return nv;
}
// Anchored aggregates of a sorted run held blocked by a team (lane l holds
// its elements l*E .. l*E+E-1, nv of them valid): P-type relative to the
// run's last key (written by the team's last lane), S-type relative to its
// first key (written by lane 0).
template <int E, class Team>
LDEV void team_aggregate(const float (&s)[E], int nv, double c, float cf, const Team &team, TileAgg *out) {
  float mul[E];
  mul[0] = 0.0f;
#pragma unroll
  for (int e = 1; e < E; ++e) mul[e] = (e < nv) ? wexpf(s[e - 1] - s[e], cf) : 0.0f;
  double pl = 0.0, sl = 0.0;
  float last = s[0];
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e < nv) {
      pl = pl * (double)mul[e] + 1.0;
      last = s[e];
    }
#pragma unroll
  for (int e = E - 1; e >= 0; --e)
    if (e < nv) sl = (e + 1 < E ? sl * (double)mul[e + 1] : 0.0) + 1.0;
  const Pre mp{last, nv > 0 ? pl : 0.0};
  const Suf ms{s[0], nv > 0 ? sl : 0.0};
  const Pre ep = team.excl_scan(mp, c);
  const Suf es = team.excl_scan(ms, c);
  if (team.lane == Team::kLanes - 1) {
    const Pre tp = join(ep, mp, c);
    out->aP = tp.a;
    out->sP = tp.s;
  }
  if (team.lane == 0) {
    const Suf tsf = join(ms, es, c);
    out->aS = tsf.a;
    out->sS = tsf.s;
  }
  team.sync();
}
template <int NT>
LDEV void tile_aggregate(const float (&s)[kKpt], int nv, double c, float cf, const BlockTeam<NT, 1> &team,
                         TileAgg *out) {
  team_aggregate<kKpt>(s, nv, c, cf, team, out);
}

// Locate + closed-form root over one sorted range of `len` keys (stored
// minus kbase) split into tiles of NT*16 whose anchored aggregates `ta` are
// given: scan of the tile aggregates between the outer seeds, threshold
// curve at the tile ends, the balancing tile, and the root inside it.
// seed_lo / seed_hi hold everything below / above the range, cR counts the
// elements above it; first / last say whether the range starts / ends the
// sorted segment (no knots below / above it).  tp, ts: scratch [nt].
// Returns b on every thread.
template <int NT>
LDEV double locate_sorted(const uint32_t *src, int64_t len, uint32_t kbase, Pre seed_lo, Suf seed_hi, double cR,
                          bool first, bool last, const TileAgg *ta, Pre *tp, Suf *ts, double k, double t, double c,
                          float cf, const BlockTeam<NT, 1> &team) {
  constexpr int TT = NT * kKpt;
  const int nt = (int)((len + TT - 1) / TT);
  Pre carry = seed_lo;
  for (int T0 = 0; T0 < nt; T0 += NT) {
    const int T = T0 + threadIdx.x;
    const Pre mine = T < nt ? Pre{ta[T].aP, ta[T].sP} : Pre{0.0f, 0.0};
    const Pre ex = team.excl_scan(mine, c);
    if (T < nt) tp[T] = join(carry, ex, c);
    const Pre tot = join(ex, mine, c);
    const Pre chunk{team.bcast(tot.a, NT - 1), team.bcast(tot.s, NT - 1)};
    carry = join(carry, chunk, c);
  }
  Suf carry_s = seed_hi;
  for (int T0 = ((nt - 1) / NT) * NT; nt > 0 && T0 >= 0; T0 -= NT) {
    const int T = T0 + threadIdx.x;
    const Suf mine = T < nt ? Suf{ta[T].aS, ta[T].sS} : Suf{0.0f, 0.0};
    const Suf ex = team.excl_scan(mine, c);
    if (T < nt) ts[T] = join(ex, carry_s, c);
    const Suf tot = join(mine, ex, c);
    const Suf chunk{team.bcast(tot.a, 0), team.bcast(tot.s, 0)};
    carry_s = join(chunk, carry_s, c);
  }
  __syncthreads();
  // threshold curve at the last knot of every tile
  int cnt = 0;
  for (int T = threadIdx.x; T < nt; T += NT) {
    const Pre pl = join(tp[T], Pre{ta[T].aP, ta[T].sP}, c);
    const Suf sa = ts[T];
    const double s_last = 1.0 + (sa.s == 0.0 ? 0.0 : sa.s * (double)wexp((double)pl.a - (double)sa.a, c));
    const int64_t nvT = min((int64_t)TT, len - (int64_t)T * TT);
    const int64_t j_last = (int64_t)T * TT + nvT - 1;
    const double g = 0.5 * (pl.s - 1.0) + ((double)(len - j_last) + cR) - 0.5 * s_last;
    cnt += (g >= k) ? 1 : 0;
  }
  const int tstar = team.sum(cnt);
  const int tsel = nt == 0 ? 0 : min(tstar, nt - 1);
  float s[kKpt];
  int nv = 0;
  if (nt > 0) {
    nv = load_sorted_at<NT>(src, (int64_t)tsel * TT, len, kbase, s);
  } else {
#pragma unroll
    for (int e = 0; e < kKpt; ++e) s[e] = 0.0f;
  }
  PartInfo part;
  part.nvalid = nv;
  part.above = (double)(len - (int64_t)tsel * TT) + cR;
  part.seed_lo = nt > 0 ? tp[tsel] : seed_lo;
  part.seed_hi = nt > 0 ? ts[tsel] : seed_hi;
  part.first = first && tsel == 0;
  part.last = last && tsel >= nt - 1;
  return segment_solve<kKpt>(s, nv, part, k, t, c, cf, team);
}

}  // namespace lapsum
