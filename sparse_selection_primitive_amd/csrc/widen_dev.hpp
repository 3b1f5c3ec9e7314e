// Iterative widening of a bracket that failed its certification ("Fast
// LapSum: Exact Differentiable Top-k at Million Scale", section 2.2,
// probabilistic bracketing, step 4: a failed check widens the bracket and
// tries again).  Run by the one workgroup of the band kernel that found the
// miss, before the exact whole-row fallback:
//   1. the wider bracket: order statistics of the row's noised sample at
//      ranks set for a smaller miss probability (radix selection in LDS);
//   2. one pass over the row: counts and tail sums outside the bracket, the
//      keys inside it appended to the row's key buffer;
//   3. the exact root over those keys, seeded with the tails (the nested
//      bucket selection of the fallback, on the band only);
//   4. certification: the root must lie inside the wider bracket.
// Every sum is taken in one fixed order and the band solve is order-free,
// so a widened row is as reproducible as one whose first bracket held.
#pragma once

#include "bucket_dev.hpp"

namespace lapsum {

// Keys of ranks R[tg] (0-based, want[tg]) among key_of(X[0 .. m)), by three
// histogram passes of 11, 11 and 10 bits over the keys that share the
// prefix found so far.  Every thread gets both keys.
template <int NT>
LDEV void wg_select2(const float *__restrict__ X, int64_t m, const int64_t (&R0)[2], const bool (&want)[2],
                     uint32_t (&out)[2], WidenLds &W) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  uint32_t prefix[2] = {0u, 0u};
  uint32_t R[2] = {(uint32_t)(want[0] ? R0[0] : 0), (uint32_t)(want[1] ? R0[1] : 0)};
  int done = 0;  // leading bits fixed so far
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = widths[pass];
    const int nb = 1 << bits, sh = 32 - done - bits;
    for (int j = threadIdx.x; j < 2 * kFallbackBuckets; j += NT) (&W.hist[0][0])[j] = 0u;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < m; i += NT) {
      const uint32_t key = key_of(X[i]);
      const uint32_t bin = (key >> sh) & (uint32_t)(nb - 1);
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
        if (want[tg] && (done == 0 || (key >> (32 - done)) == prefix[tg])) atomicAdd(&W.hist[tg][bin], 1u);
    }
    __syncthreads();
    // wave tg finds the bin of rank R[tg]: lane l sums bins l*per .. l*per+per-1
    if (w < 2 && want[w]) {
      const int per = nb / kWave;
      const uint32_t *h = W.hist[w];
      uint32_t local = 0u;
      for (int q = 0; q < per; ++q) local += h[lane * per + q];
      const uint32_t inc = wave_incl_scan(local);
      const uint32_t before = inc - local;
      if (R[w] >= before && R[w] < inc) {
        uint32_t acc = before;
        for (int q = 0; q < per; ++q) {
          const uint32_t cq = h[lane * per + q];
          if (R[w] >= acc && R[w] < acc + cq) {
            W.pick[w][0] = (uint32_t)(lane * per + q);
            W.pick[w][1] = R[w] - acc;
          }
          acc += cq;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      if (!want[tg]) continue;
      prefix[tg] = (prefix[tg] << bits) | W.pick[tg][0];
      R[tg] = W.pick[tg][1];
    }
    done += bits;
    __syncthreads();
  }
  out[0] = prefix[0];
  out[1] = prefix[1];
}

// Totals of the row pass against a bracket [aL, aR).
struct WidenTotals {
  double sl, sr;                    // tail sums anchored at aL and aR
  unsigned long long cl, cr;        // counts below aL and at or above aR
  uint32_t M, kmin, kmax;           // band size and key range
};

// One pass over the row's scores: tails outside [aL, aR) (fp32 terms, fp64
// sums per thread, then reduced in a fixed order) and the band keys appended
// to dst (one LDS cursor, reserved per wave).
template <int NT>
LDEV WidenTotals widen_filter(const SegArgs &a, int row, float aL, float aR, uint32_t *dst, WidenLds &W) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const unsigned long long ltmask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const float cf = a.cf;
  if (threadIdx.x == 0) W.ctr = 0u;
  __syncthreads();
  double sl = 0.0, sr = 0.0;
  unsigned long long cl = 0, cr = 0;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
  fallback_each_key(a, row, nullptr, a.n, NT, [&](uint32_t key) {
    const float x = value_of(key);
    const bool lo = x < aL, hi = x >= aR;
    if (lo) {
      ++cl;
      sl += (double)__builtin_amdgcn_exp2f((x - aL) * cf);
    }
    if (hi) {
      ++cr;
      sr += (double)__builtin_amdgcn_exp2f((aR - x) * cf);
    }
    const bool in = !lo && !hi;
    const unsigned long long mk = __ballot(in);
    if (mk != 0ull) {
      const int leader = __ffsll((long long)mk) - 1;
      uint32_t base = 0u;
      if (lane == leader) base = atomicAdd(&W.ctr, (uint32_t)__popcll(mk));
      base = (uint32_t)__shfl((int)base, leader, kWave);
      if (in) {
        dst[base + (uint32_t)__popcll(mk & ltmask)] = key;
        kmn = min(kmn, key);
        kmx = max(kmx, key);
      }
    }
  });
  sl = wave_reduce(sl, [](double x, double y) { return x + y; });
  sr = wave_reduce(sr, [](double x, double y) { return x + y; });
  cl = wave_reduce(cl, [](unsigned long long x, unsigned long long y) { return x + y; });
  cr = wave_reduce(cr, [](unsigned long long x, unsigned long long y) { return x + y; });
  kmn = wave_reduce(kmn, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  kmx = wave_reduce(kmx, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  if (lane == 0) {
    W.sum[0][w] = sl;
    W.sum[1][w] = sr;
    W.cnt[0][w] = cl;
    W.cnt[1][w] = cr;
    W.kext[0][w] = kmn;
    W.kext[1][w] = kmx;
  }
  __syncthreads();
  WidenTotals T{0.0, 0.0, 0, 0, W.ctr, 0xFFFFFFFFu, 0u};
  for (int i = 0; i < NW; ++i) {
    T.sl += W.sum[0][i];
    T.sr += W.sum[1][i];
    T.cl += W.cnt[0][i];
    T.cr += W.cnt[1][i];
    T.kmin = min(T.kmin, W.kext[0][i]);
    T.kmax = max(T.kmax, W.kext[1][i]);
  }
  if (T.M == 0u) T.kmin = T.kmax = 0u;
  __syncthreads();
  return T;
}

// Up to a.nwiden widened brackets for a row whose first bracket failed.  On
// success the row state holds the certified bracket, its tails and b, and the
// row's flags say WIDENED instead of FALLBACK; returns false (state unchanged
// but for the key buffers) when every widened bracket fails too, or when the
// row has no sample (a bracket given by the caller).
template <int NT>
LDEV bool widen_row(const SegArgs &a, int row, SegLds<NT> &L) {
  if (a.samples == nullptr || a.nwiden <= 0) return false;
  const float *X = a.samples + (int64_t)row * a.m;
  uint32_t *band = a.A + (int64_t)row * a.stride;
  for (int i = 0; i < a.nwiden && i < kMaxWiden; ++i) {
    const int64_t lo = a.wlo[i], hi = a.whi[i];
    const bool want[2] = {lo >= 1, hi <= a.m};
    const int64_t R[2] = {lo - 1, hi - 1};
    uint32_t key2[2];
    wg_select2<NT>(X, a.m, R, want, key2, L.wd);
    const float aL = want[0] ? value_of(key2[0]) : -INFINITY;
    const float aR = want[1] ? value_of(key2[1]) : INFINITY;
    const WidenTotals T = widen_filter<NT>(a, row, aL, aR, band, L.wd);
    const Pre slo{aL, T.cl ? T.sl : 0.0};
    const Suf shi{aR, T.cr ? T.sr : 0.0};
    const double b = bucket_set_solve<NT>(a, row, band, (int64_t)T.M, 1, T.kmin, T.kmax, slo, shi, (double)T.cr, L);
    if (b >= (double)aL && b < (double)aR) {
      if (threadIdx.x == 0) {
        RowState &S = a.st[row];
        S.a_lo = aL;
        S.a_hi = aR;
        S.tail_lo = T.sl;
        S.tail_hi = T.sr;
        S.count_lo = T.cl;
        S.count_hi = T.cr;
        S.band = T.M;
        S.kmin = T.kmin;
        S.kmax = T.kmax;
        S.b = b;
        S.flags = (S.flags & ~LAPSUM_FLAG_FALLBACK) | LAPSUM_FLAG_WIDENED;
      }
      __syncthreads();
      return true;
    }
  }
  return false;
}

// A row whose bracket missed or whose band overflowed: widened brackets
// first, then the exact whole-row fallback.  (Inlined: a call would make
// every launch of the band kernels set up a stack, which costs more than
// the spills this path adds outside the hit path.)
// With per-row budgets the row's own k, t (as the per-row bracket kernel
// stored them) replace the call's, there are no widened brackets (their
// indices depend on k), and a row whose k or t was out of range gets NaN.
// (With the spread fallback the band kernels do not call it.)
template <int NT>
LDEV void missed_row(const SegArgs &a, int row, SegLds<NT> &L) {
  if (a.per_row) {
    const RowState &S = a.st[row];
    if (S.flags & LAPSUM_FLAG_INVALID) {
      if (threadIdx.x == 0) a.st[row].b = __builtin_nan("");
      __syncthreads();
      return;
    }
    SegArgs r = a;
    r.k = S.k;
    r.t = S.t;
    r.c = S.c;
    r.cf = S.cf;
    r.nwiden = 0;
    fallback_row<NT>(r, row, L);
    return;
  }
  if (!widen_row<NT>(a, row, L)) fallback_row<NT>(a, row, L);
}

}  // namespace lapsum
