// Per-row totals of the bracketing filter ("Fast LapSum: Exact
// Differentiable Top-k at Million Scale", section 2.2, probabilistic
// bracketing, step 2): the streaming filter leaves one partial per
// workgroup; the first kernel of the band solve adds them up inside each of
// its workgroups (in one fixed order, so every workgroup gets the same
// totals bit for bit), instead of a separate finalize launch.
#pragma once

#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

namespace lapsum {

// One streaming-filter workgroup's share of a row.
struct FilterPartial {
  double sl, sr;           // tail sums below a_L (anchored at a_L) and at or above a_R (anchored at a_R)
  unsigned long long cnl;  // scores at or above a_L
  uint32_t cnt;            // band keys this block found (may exceed kBandSlot)
  uint32_t kmn, kmx;       // key range of those band keys
  uint32_t pad;
};

struct FilterTotals {
  double tail_lo, tail_hi;
  unsigned long long count_lo, count_hi, band;
  uint32_t kmin, kmax;
  int overflow;  // a slot overflowed, or the band exceeds the capacity: the row takes the fallback
};

// A whole workgroup of NT threads adds the gx partials of one row (scores
// n, band capacity cap) and writes the exclusive slot offsets ro[0..gx]
// (ro[gx] = M; ro may point to LDS).  Returns the totals on every thread.
template <int NT>
LDEV FilterTotals filter_totals(const FilterPartial *__restrict__ vp, int gx, int64_t n, int64_t cap, uint32_t *ro) {
  constexpr int NW = NT / kWave;
  __shared__ double lds_d[2 * NW];
  __shared__ unsigned long long lds_c[NW];
  __shared__ uint32_t lds_k[3 * NW];
  __shared__ uint32_t wsum[NW];
  __shared__ FilterTotals tot;
  lds_poison(lds_d);
  lds_poison(lds_c);
  lds_poison(lds_k);
  lds_poison(wsum);
  lds_poison(tot);
  // a contiguous chunk of partials per thread, so the offsets come out in
  // order; loaded four at a time at clamped indices (no load waits for the
  // previous one), the counts kept for the offsets
  constexpr int PMAX = (kMaxFilterBlocks + NT - 1) / NT;  // partials per thread, at most
  static_assert(PMAX % 4 == 0, "partials are loaded four at a time");
  const int per = (gx + NT - 1) / NT;
  const int b0 = threadIdx.x * per;
  double a = 0.0, b = 0.0;
  unsigned long long c0 = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, csum = 0u, big = 0u;
  uint32_t cs[PMAX];
#pragma unroll
  for (int c = 0; c < PMAX; c += 4) {
    FilterPartial fp[4] = {};
    if (c < per) {  // uniform over the workgroup
#pragma unroll
      for (int q = 0; q < 4; ++q) fp[q] = vp[min(b0 + c + q, gx - 1)];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = c + q < per && b0 + c + q < gx;
      cs[c + q] = in ? fp[q].cnt : 0u;
      if (in) {
        a += fp[q].sl;
        b += fp[q].sr;
        c0 += fp[q].cnl;
        mn = min(mn, fp[q].kmn);
        mx = max(mx, fp[q].kmx);
        csum += fp[q].cnt;
        big |= fp[q].cnt > (uint32_t)kBandSlot ? 1u : 0u;
      }
    }
  }
  // exclusive scan of the chunk sums: inside each DPP row of 16 lanes, then
  // the row totals (v_readlane), then the wave totals through LDS
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const uint32_t inc = wave_incl_scan(csum);
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  uint32_t before = 0u, total = 0u;
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  uint32_t run = before + inc - csum;
#pragma unroll
  for (int i = 0; i < PMAX; ++i) {
    if (i < per && b0 + i < gx) {
      ro[b0 + i] = run;
      run += cs[i];
    }
  }
  if (threadIdx.x == NT - 1) ro[gx] = total;
  a = wave_reduce(a, [](double x, double y) { return x + y; });
  b = wave_reduce(b, [](double x, double y) { return x + y; });
  c0 = wave_reduce(c0, [](unsigned long long x, unsigned long long y) { return x + y; });
  mn = wave_reduce(mn, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  mx = wave_reduce(mx, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  big = wave_reduce(big, [](uint32_t x, uint32_t y) { return x | y; });
  if (lane == 0) {
    lds_d[2 * w] = a;
    lds_d[2 * w + 1] = b;
    lds_c[w] = c0;
    lds_k[3 * w] = mn;
    lds_k[3 * w + 1] = mx;
    lds_k[3 * w + 2] = big;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ta = 0.0, tb = 0.0;
    unsigned long long tc0 = 0;
    uint32_t tmn = 0xFFFFFFFFu, tmx = 0u, tbig = 0u;
    for (int i = 0; i < NW; ++i) {
      ta += lds_d[2 * i];
      tb += lds_d[2 * i + 1];
      tc0 += lds_c[i];
      tmn = min(tmn, lds_k[3 * i]);
      tmx = max(tmx, lds_k[3 * i + 1]);
      tbig |= lds_k[3 * i + 2];
    }
    tot.tail_lo = ta;
    tot.tail_hi = tb;
    // every score is below a_L, inside the band or at or above a_R
    tot.count_lo = (unsigned long long)n - tc0;
    tot.count_hi = tc0 - total;
    tot.band = total;
    tot.kmin = tmn;
    tot.kmax = tmx;
    tot.overflow = (tbig || (int64_t)total > cap) ? 1 : 0;
  }
  __syncthreads();
  return tot;
}

// The row state fields the filter totals fix (written once per row).
LDEV void store_filter_totals(RowState &S, const FilterTotals &T) {
  S.tail_lo = T.tail_lo;
  S.tail_hi = T.tail_hi;
  S.count_lo = T.count_lo;
  S.count_hi = T.count_hi;
  S.band = T.band;
  S.kmin = T.kmin;
  S.kmax = T.kmax;
  if (T.overflow) S.flags |= LAPSUM_FLAG_OVERFLOW | LAPSUM_FLAG_FALLBACK;
}

}  // namespace lapsum
