// Per-query bisection baseline ("Fast LapSum: Exact Differentiable Top-k at
// Million Scale", section 2.2: the full-sort solver replaces the iterative
// bisection of earlier LapSum implementations; section 4.1 compares the
// two).  The threshold b of eq. (2) is found by halving a bracket of the
// monotone budget f(b) = sum_i F((r_i - b)/t), with no sort:
//
//   start   with q = F^-1(k/n), every score >= min r gives
//           f(min r - t q) >= k and every score <= max r gives
//           f(max r - t q) <= k, so [min r - t q, max r - t q] holds b;
//   step    the residual f(mid) - k = (#{r > mid} - k)
//                                     + sum_{r <= mid} e^{(r-mid)/t}/2
//                                     - sum_{r > mid} e^{-(r-mid)/t}/2
//           (an exact count and two sums of terms in [0, 1/2], fp32 terms,
//           fp64 sums); its sign says which half holds b;
//   stop    when the midpoint no longer lies strictly inside the bracket
//           (fp64 resolution), or after the step budget.
//
// Rows of up to 16384 scores: one workgroup per row holds the row in
// registers and runs every step itself (bisect_onchip_kernel; 512 threads
// above 4096 scores, for the registers), then writes p.
// Longer rows: one streaming pass over the row per step
// (bisect_step_kernel), each workgroup leaving its partial residual; every
// workgroup of the next step adds the previous step's partials in one fixed
// order, so all of them take the same decision, with no extra launch.  The
// streaming apply of stream.hip then writes p.
#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

namespace lapsum {

constexpr int kBisNT = 1024;          // threads of the on-chip bisection (rows of up to 4096 scores)
constexpr int kBisNTWide = 512;       // ... of longer rows (twice the registers per thread)
constexpr int kBisMaxIter = 2000;     // on-chip step budget (fp64 halving stops far earlier)
constexpr int kBisStreamSteps = 64;   // streaming steps (64 halvings: below fp64 resolution)
constexpr int kBisStreamNT = 256;

LDEV double laplace_quantile(double u) { return u <= 0.5 ? log(2.0 * u) : -log(2.0 * (1.0 - u)); }

// The starting bracket from the row's extremes, widened by a few ulps.
LDEV void bisect_start(float mn, float mx, double k, double n, double t, double &lo, double &hi) {
  const double q = laplace_quantile(k / n);
  lo = (double)mn - t * q;
  hi = (double)mx - t * q;
  lo -= fabs(lo) * 1e-15 + 1e-300;
  hi += fabs(hi) * 1e-15 + 1e-300;
}

// The point b split for fp32 arithmetic: b = bh + bl with bh = fp32(b);
// z = (x - b) log2(e)/t is then fma(x - bh, cf, -bl cf), where x - bh is
// exact or rounds relative to itself (the same form as the on-chip apply).
struct SplitB {
  float bh, blcf, cf;
};
LDEV SplitB split_b(double b, double c) {
  const float bh = (float)b, cf = (float)c;
  return SplitB{bh, (float)(b - (double)bh) * cf, cf};
}
// One score's share of the residual at b: its side and e^{-|r - b|/t}/2.  A
// score within rounding of b may land on either side; its two shares then
// differ by 1 - 2h ~ 0, so the residual stays continuous.
LDEV void residual_term(float x, const SplitB &sb, double &below, double &above, uint32_t &cnt) {
  const float z = __builtin_fmaf(x - sb.bh, sb.cf, -sb.blcf);
  const float h = 0.5f * __builtin_amdgcn_exp2f(-fabsf(z));
  if (z > 0.0f) {
    above += (double)h;
    ++cnt;
  } else {
    below += (double)h;
  }
}

template <int NT>
struct BisLds {
  double s[2 * NT / kWave];
  unsigned long long c[NT / kWave];
  float m[2 * NT / kWave];
};

// Sum over the workgroup, in one fixed order, identical on every thread.
template <int NT>
LDEV double block_residual(double below, double above, unsigned long long cnt, double k, BisLds<NT> &L) {
  below = wave_reduce(below, [](double x, double y) { return x + y; });
  above = wave_reduce(above, [](double x, double y) { return x + y; });
  cnt = wave_reduce(cnt, [](unsigned long long x, unsigned long long y) { return x + y; });
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    L.s[2 * w] = below;
    L.s[2 * w + 1] = above;
    L.c[w] = cnt;
  }
  __syncthreads();
  double sb = 0.0, sa = 0.0;
  unsigned long long sc = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    sb += L.s[2 * i];
    sa += L.s[2 * i + 1];
    sc += L.c[i];
  }
  return ((double)sc - k) + (sb - sa);
}

template <int NT, int E>
__global__ __launch_bounds__(NT) void bisect_onchip_kernel(const float *__restrict__ r, int64_t rows, int n,
                                                           double k, double t, RowParams rp, float *__restrict__ p,
                                                           double *__restrict__ bout) {
  __shared__ BisLds<NT> L;
  const int64_t row = grid_row();
  if (row >= rows) return;
  const bool good = row_params(rp.k, rp.t, row, n, k, t);
  const double c = kLog2e / t;
  const float *rr = r + row * n;
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * NT + threadIdx.x;
    v[e] = rr[i < n ? i : 0];
  }
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e * NT + (int)threadIdx.x < n) {
      mn = fminf(mn, v[e]);
      mx = fmaxf(mx, v[e]);
    }
  }
  mn = __uint_as_float(wave_reduce(__float_as_uint(mn), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
  }));
  mx = __uint_as_float(wave_reduce(__float_as_uint(mx), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    L.m[2 * w] = mn;
    L.m[2 * w + 1] = mx;
  }
  __syncthreads();
  for (int i = 0; i < NT / kWave; ++i) {
    mn = fminf(mn, L.m[2 * i]);
    mx = fmaxf(mx, L.m[2 * i + 1]);
  }
  double lo, hi;
  bisect_start(mn, mx, k, (double)n, t, lo, hi);
  auto residual = [&](double b) {
    const SplitB sb = split_b(b, c);
    double below = 0.0, above = 0.0;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e * NT + (int)threadIdx.x < n) residual_term(v[e], sb, below, above, cnt);
    return block_residual(below, above, (unsigned long long)cnt, k, L);
  };
  bool exact = false;
  for (int it = 0; it < kBisMaxIter; ++it) {
    const double mid = lo + 0.5 * (hi - lo);
    if (!(mid > lo && mid < hi)) break;
    const double res = residual(mid);
    if (res > 0.0) {
      lo = mid;  // f(mid) > k: the root lies above mid
    } else if (res < 0.0) {
      hi = mid;
    } else {
      lo = hi = mid;
      exact = true;
      break;
    }
  }
  double b = lo;
  if (!exact) {
    const double rlo = residual(lo), rhi = residual(hi);
    b = fabs(rlo) <= fabs(rhi) ? lo : hi;
  }
  if (!good) b = __builtin_nan("");
  float *pp = p + row * n;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * NT + threadIdx.x;
    if (i < n) {
      const float z2 = (float)(((double)v[e] - b) * c);
      pp[i] = z2 < 0.0f ? 0.5f * __builtin_amdgcn_exp2f(z2) : 1.0f - 0.5f * __builtin_amdgcn_exp2f(-z2);
    }
  }
  if (threadIdx.x == 0) bout[row] = b;
}

// ------------------------------------------------------------- streaming
struct BisState {
  double lo, hi, mid;
  int32_t done, pad;
};
struct BisPartial {
  double below, above;
  unsigned long long cnt;
  float mn, mx;  // step 0 only: the chunk's extremes
};

template <class T>
LDEV void bis_block_sum(T &v, T *lds) {
  v = wave_reduce(v, [](T x, T y) { return x + y; });
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  v = T(0);
  for (int i = 0; i < kBisStreamNT / kWave; ++i) v += lds[i];
}

// Step `it` of the streaming bisection for one row.  Reads the bracket left
// by the previous step (state[it & 1]) and that step's partials
// (part[it & 1]), takes the decision, writes the new bracket
// (state[(it+1) & 1], first workgroup) and this workgroup's partial at the
// new midpoint (part[(it+1) & 1]).  Step 0 reduces the extremes instead.
// final = true: take the last decision and write b to the row state.
template <bool FINAL>
__global__ __launch_bounds__(kBisStreamNT) void bisect_step_kernel(const float *__restrict__ r, int64_t rows,
                                                                   int64_t n, double k, double t, RowParams rp,
                                                                   BisState *__restrict__ state,
                                                                   BisPartial *__restrict__ part, int gx, int it,
                                                                   RowState *__restrict__ st) {
  __shared__ double lds_d[kBisStreamNT / kWave];
  __shared__ unsigned long long lds_c[kBisStreamNT / kWave];
  __shared__ float lds_f[kBisStreamNT / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const bool good = row_params(rp.k, rp.t, row, n, k, t);
  const double c = kLog2e / t;
  const BisPartial *pin = part + ((int64_t)(it & 1) * rows + row) * gx;
  BisPartial *pout = part + ((int64_t)((it + 1) & 1) * rows + row) * gx;
  BisState S;
  if (it == 0) {
    float mn = INFINITY, mx = -INFINITY;
    for (int i = threadIdx.x; i < gx; i += kBisStreamNT) {
      mn = fminf(mn, pin[i].mn);
      mx = fmaxf(mx, pin[i].mx);
    }
    mn = __uint_as_float(wave_reduce(__float_as_uint(mn), [](uint32_t x, uint32_t y) {
      return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
    }));
    mx = __uint_as_float(wave_reduce(__float_as_uint(mx), [](uint32_t x, uint32_t y) {
      return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) lds_f[w] = mn;
    __syncthreads();
    for (int i = 0; i < kBisStreamNT / kWave; ++i) mn = fminf(mn, lds_f[i]);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) lds_f[w] = mx;
    __syncthreads();
    for (int i = 0; i < kBisStreamNT / kWave; ++i) mx = fmaxf(mx, lds_f[i]);
    bisect_start(mn, mx, k, (double)n, t, S.lo, S.hi);
    S.done = 0;
  } else {
    S = state[(int64_t)(it & 1) * rows + row];
    if (!S.done) {
      double below = 0.0, above = 0.0;
      unsigned long long cnt = 0;
      for (int i = threadIdx.x; i < gx; i += kBisStreamNT) {
        below += pin[i].below;
        above += pin[i].above;
        cnt += pin[i].cnt;
      }
      bis_block_sum(below, lds_d);
      bis_block_sum(above, lds_d);
      bis_block_sum(cnt, lds_c);
      const double res = ((double)cnt - k) + (below - above);
      if (res > 0.0) S.lo = S.mid;
      else if (res < 0.0) S.hi = S.mid;
      else S.lo = S.hi = S.mid;
    }
  }
  S.mid = S.lo + 0.5 * (S.hi - S.lo);
  if (!(S.mid > S.lo && S.mid < S.hi)) S.done = 1;
  if (FINAL) {
    if (blockIdx.x == 0 && threadIdx.x == 0) st[row].b = good ? S.mid : __builtin_nan("");
    return;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) state[(int64_t)((it + 1) & 1) * rows + row] = S;
  if (S.done) return;
  // this workgroup's share of the residual at the new midpoint
  double below = 0.0, above = 0.0;
  uint32_t cnt32 = 0;
  const SplitB sb = split_b(S.mid, c);
  const float *rr = r + row * n;
  if ((n & 3) == 0 && ((uintptr_t)rr & 15u) == 0) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 *r4 = reinterpret_cast<const f4 *>(rr);
    const int64_t n4 = n >> 2;
    for (int64_t i = (int64_t)blockIdx.x * kBisStreamNT + threadIdx.x; i < n4; i += (int64_t)gx * kBisStreamNT) {
      const f4 x = __builtin_nontemporal_load(r4 + i);
      residual_term(x.x, sb, below, above, cnt32);
      residual_term(x.y, sb, below, above, cnt32);
      residual_term(x.z, sb, below, above, cnt32);
      residual_term(x.w, sb, below, above, cnt32);
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kBisStreamNT + threadIdx.x; i < n; i += (int64_t)gx * kBisStreamNT)
      residual_term(rr[i], sb, below, above, cnt32);
  }
  unsigned long long cnt = cnt32;
  bis_block_sum(below, lds_d);
  bis_block_sum(above, lds_d);
  bis_block_sum(cnt, lds_c);
  if (threadIdx.x == 0) pout[blockIdx.x] = BisPartial{below, above, cnt, 0.0f, 0.0f};
}

// The row's extremes per workgroup (into part[0], read by step 0).
__global__ __launch_bounds__(kBisStreamNT) void bisect_minmax_kernel(const float *__restrict__ r, int64_t rows,
                                                                     int64_t n, BisPartial *__restrict__ part,
                                                                     int gx) {
  __shared__ float lds_f[2 * kBisStreamNT / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const float *rr = r + row * n;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t i = (int64_t)blockIdx.x * kBisStreamNT + threadIdx.x; i < n; i += (int64_t)gx * kBisStreamNT) {
    mn = fminf(mn, rr[i]);
    mx = fmaxf(mx, rr[i]);
  }
  mn = __uint_as_float(wave_reduce(__float_as_uint(mn), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
  }));
  mx = __uint_as_float(wave_reduce(__float_as_uint(mx), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds_f[2 * w] = mn;
    lds_f[2 * w + 1] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < kBisStreamNT / kWave; ++i) {
      mn = fminf(mn, lds_f[2 * i]);
      mx = fmaxf(mx, lds_f[2 * i + 1]);
    }
    part[row * gx + blockIdx.x] = BisPartial{0.0, 0.0, 0ull, mn, mx};
  }
}

bool bisect_onchip(int64_t n) { return n <= 32 * kBisNTWide; }

int bisect_grid_x(int64_t rows, int64_t n) {
  int64_t gx = (n + kBisStreamNT * 16 - 1) / (kBisStreamNT * 16);
  int64_t most = 4096 / (rows > 0 ? rows : 1);
  if (most < 1) most = 1;
  if (gx > most) gx = most;
  return (int)(gx < 1 ? 1 : gx);
}
size_t bisect_state_bytes(int64_t rows) { return sizeof(BisState) * 2 * (size_t)rows; }
size_t bisect_partial_bytes(int64_t rows, int gx) { return sizeof(BisPartial) * 2 * (size_t)rows * (size_t)gx; }

template <int NT, int E>
static hipError_t launch_bis_onchip(const float *r, int64_t rows, int n, double k, double t, RowParams rp, float *p,
                                    double *b, hipStream_t s) {
  hipLaunchKernelGGL((bisect_onchip_kernel<NT, E>), rows_grid(1u, rows), dim3(NT), 0, s, r, rows, n, k, t, rp, p, b);
  return hipGetLastError();
}

hipError_t launch_bisect_onchip(const float *r, int64_t rows, int64_t n, double k, double t, RowParams rp, float *p,
                                double *b, hipStream_t s) {
  if (n <= kBisNT) return launch_bis_onchip<kBisNT, 1>(r, rows, (int)n, k, t, rp, p, b, s);
  if (n <= 4 * kBisNT) return launch_bis_onchip<kBisNT, 4>(r, rows, (int)n, k, t, rp, p, b, s);
  if (n <= 16 * kBisNTWide) return launch_bis_onchip<kBisNTWide, 16>(r, rows, (int)n, k, t, rp, p, b, s);
  return launch_bis_onchip<kBisNTWide, 32>(r, rows, (int)n, k, t, rp, p, b, s);
}

hipError_t launch_bisect_stream(const float *r, int64_t rows, int64_t n, double k, double t, RowParams rp,
                                void *state, void *partials, int gx, RowState *st, hipStream_t s) {
  BisState *S = reinterpret_cast<BisState *>(state);
  BisPartial *P = reinterpret_cast<BisPartial *>(partials);
  const dim3 grid = rows_grid((unsigned)gx, rows);
  hipLaunchKernelGGL(bisect_minmax_kernel, grid, dim3(kBisStreamNT), 0, s, r, rows, n, P, gx);
  for (int it = 0; it < kBisStreamSteps; ++it)
    hipLaunchKernelGGL(bisect_step_kernel<false>, grid, dim3(kBisStreamNT), 0, s, r, rows, n, k, t, rp, S, P, gx,
                       it, st);
  hipLaunchKernelGGL(bisect_step_kernel<true>, rows_grid(1u, rows), dim3(kBisStreamNT), 0, s, r, rows, n, k, t, rp,
                     S, P, gx, kBisStreamSteps, st);
  return hipGetLastError();
}

}  // namespace lapsum
