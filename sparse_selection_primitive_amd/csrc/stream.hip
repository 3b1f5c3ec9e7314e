// Streaming (HBM-bound) kernels for large rows.
//
//  * apply: p_i = F((r_i - b)/t) ("Fast LapSum: Exact Differentiable Top-k at
//    Million Scale", section 2.1, eq. (1)), 4 B read + 4 B written per score;
//  * backward, section 2.1 (analytic VJP): pass 1 reads g and p (8 B/score)
//    and leaves one fp64 partial (sum d, sum g d) per workgroup; pass 2
//    reads g and p again, and every one of its workgroups first adds the
//    row's partials in one fixed order (so all hold the same dk = G/D bit
//    for bit, with no finalize launch), then writes dr = d (g - dk)
//    (12 B/score), d = min(p, 1 - p)/t.
//
// Loads and stores are 16 B per lane and non-temporal: every byte is used
// once, so nothing is worth keeping in the caches.  Grids are workgroups
// per row in x and rows folded over y and z (rows_grid), with grid-stride
// loops inside a row.
#include <atomic>
#include <mutex>

#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

// Fixed device scratch of lapsum_backward_noalloc (for callers that cannot
// allocate): the streaming backward's per-workgroup partials, written in
// full by the reduce pass before the apply pass reads them, so nothing in
// it needs clearing.  Each device holds its own copy for the life of the
// process; calls that overlap on one device share it and race.  Host code
// never passes this name to a kernel: it passes the device address that
// noalloc_scratch() looks up per device.
static __device__ __align__(256) unsigned char scratch[LAPSUM_NOALLOC_SCRATCH_BYTES];

namespace lapsum {

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *q = addr[dev].load(std::memory_order_acquire);
  if (q == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    q = addr[dev].load(std::memory_order_relaxed);
    if (q == nullptr) {
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (q == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(q, std::memory_order_release);
    }
  }
  *ptr = q;
  return hipSuccess;
}

typedef float f4 __attribute__((ext_vector_type(4)));

LDEV bool aligned16(const void *q) { return ((uintptr_t)q & 15u) == 0; }

LDEV float cdf_at(float x, double b, double c) {
  const float z2 = (float)(((double)x - b) * c);
  return z2 < 0.0f ? 0.5f * __builtin_amdgcn_exp2f(z2) : 1.0f - 0.5f * __builtin_amdgcn_exp2f(-z2);
}

// ----------------------------------------------------------- row state
// Per-call reset of every row's state, with the row's budget, temperature
// and c = log2(e)/t (its own values if given: an out-of-range one is
// replaced and the row flagged invalid).
__global__ void init_rows_kernel(RowState *st, int64_t rows, int32_t flags, int has_override, double o_lo,
                                 double o_hi, int64_t n, double k, double t, RowParams rp) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const bool good = row_params(rp.k, rp.t, row, n, k, t);
  reset_row_state(st, row, flags | (good ? 0 : LAPSUM_FLAG_INVALID), has_override, o_lo, o_hi);
  RowState &S = st[row];
  S.k = k;
  S.t = t;
  S.c = kLog2e / t;
  S.cf = (float)S.c;
}

hipError_t launch_init_rows(RowState *st, int64_t rows, int32_t flags, const double *override2, int64_t n,
                            double k, double t, RowParams rp, hipStream_t s) {
  const int64_t grid = (rows + 255) / 256;
  hipLaunchKernelGGL(init_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, st, rows, flags, override2 ? 1 : 0,
                     override2 ? override2[0] : 0.0, override2 ? override2[1] : 0.0, n, k, t, rp);
  return hipGetLastError();
}

__global__ void copy_stats_kernel(const RowState *st, int64_t rows, lapsum_row_stats *out) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  const RowState &s = st[row];
  lapsum_row_stats o;
  o.a_lo = s.a_lo;
  o.a_hi = s.a_hi;
  o.tail_lo = s.tail_lo;
  o.tail_hi = s.tail_hi;
  o.count_lo = (int64_t)s.count_lo;
  o.count_hi = (int64_t)s.count_hi;
  o.band = (int64_t)s.band;
  o.flags = s.flags;
  o.reserved = 0;
  out[row] = o;
}

hipError_t launch_copy_stats(const RowState *st, int64_t rows, lapsum_row_stats *stats, hipStream_t s) {
  const int64_t grid = (rows + 255) / 256;
  hipLaunchKernelGGL(copy_stats_kernel, dim3((unsigned)grid), dim3(256), 0, s, st, rows, stats);
  return hipGetLastError();
}

size_t row_state_bytes() { return sizeof(RowState); }

// ---------------------------------------------------------------- apply
__global__ __launch_bounds__(kStreamThreads) void apply_kernel(const float *__restrict__ r, int64_t rows,
                                                               int64_t n, const RowState *__restrict__ st,
                                                               double t, RowParams rp, float *__restrict__ p,
                                                               double *__restrict__ bout) {
  const int64_t row = grid_row();
  if (row >= rows) return;
  const double b = st[row].b;  // NaN for a row with invalid per-row k or t
  double kr = 0.5 * (double)n;
  if (rp.t) row_params(nullptr, rp.t, row, n, kr, t);
  const double c = kLog2e / t;
  if (blockIdx.x == 0 && threadIdx.x == 0) bout[row] = b;
  const float *rr = r + row * n;
  float *pp = p + row * n;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  if ((n & 3) == 0 && aligned16(r) && aligned16(p)) {
    const int64_t n4 = n >> 2;
    const f4 *r4 = reinterpret_cast<const f4 *>(rr);
    f4 *p4 = reinterpret_cast<f4 *>(pp);
    for (int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x; i0 < n4;
         i0 += stride * kUnroll) {
      f4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + u * kStreamThreads;
        x[u] = i < n4 ? __builtin_nontemporal_load(r4 + i) : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + u * kStreamThreads;
        if (i < n4) {
          f4 y;
          y.x = cdf_at(x[u].x, b, c);
          y.y = cdf_at(x[u].y, b, c);
          y.z = cdf_at(x[u].z, b, c);
          y.w = cdf_at(x[u].w, b, c);
          __builtin_nontemporal_store(y, p4 + i);
        }
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride)
      pp[i] = cdf_at(rr[i], b, c);
  }
}

// Workgroups per row of the apply and backward passes: one per
// kStreamThreads * kUnroll float4s, at most 4096 over all rows (16 per CU;
// on the 1e8 row 4096 measured ~2 µs faster per pass than 2048, 1024 slower).
static int stream_grid_x(int64_t rows, int64_t n) {
  const int64_t per_row_need = (n / 4 + kStreamThreads * kUnroll - 1) / (kStreamThreads * kUnroll);
  int64_t target = 4096 / (rows > 0 ? rows : 1);
  if (target < 1) target = 1;
  int64_t gx = per_row_need < target ? per_row_need : target;
  if (gx < 1) gx = 1;
  return (int)gx;
}

hipError_t launch_apply(const float *r, int64_t rows, int64_t n, const RowState *st, double t, RowParams rp,
                        float *p, double *b, hipStream_t s) {
  const int gx = stream_grid_x(rows, n);
  hipLaunchKernelGGL(apply_kernel, rows_grid((unsigned)gx, rows), dim3(kStreamThreads), 0, s, r, rows, n, st, t, rp,
                     p, b);
  return hipGetLastError();
}

// ------------------------------------------------------------ backward
struct BwdPartial {
  double D, G;
};

template <int NT>
LDEV void block_sum2(double &a, double &b, double *lds) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    a += __shfl_xor(a, m, kWave);
    b += __shfl_xor(b, m, kWave);
  }
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds[2 * w] = a;
    lds[2 * w + 1] = b;
  }
  __syncthreads();
  a = 0.0;
  b = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    a += lds[2 * i];
    b += lds[2 * i + 1];
  }
}

__global__ __launch_bounds__(kStreamThreads) void bwd_reduce_kernel(const float *__restrict__ g,
                                                                    const float *__restrict__ p, int64_t rows,
                                                                    int64_t n, BwdPartial *__restrict__ part,
                                                                    int gx) {
  __shared__ double lds[2 * kStreamThreads / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const float *gg = g + row * n;
  const float *pp = p + row * n;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  // Every product g q and every sum in fp64 (g and q are fp32, so g q is
  // exact): when one score holds nearly all of the d-weight, dk is within a
  // few 1e-4 of that score's g, and dr = d (g - dk) keeps the relative
  // accuracy of dk only if dk itself is accurate far below fp32 rounding.
  double D = 0.0, G = 0.0;
  if ((n & 3) == 0 && aligned16(g) && aligned16(p)) {
    const int64_t n4 = n >> 2;
    const f4 *g4 = reinterpret_cast<const f4 *>(gg);
    const f4 *p4 = reinterpret_cast<const f4 *>(pp);
    double Du[kUnroll], Gu[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Du[u] = Gu[u] = 0.0;
    for (int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x; i0 < n4;
         i0 += stride * kUnroll) {
      f4 pv[kUnroll], gv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + u * kStreamThreads;
        const bool ok = i < n4;
        pv[u] = ok ? __builtin_nontemporal_load(p4 + i) : f4{0.f, 0.f, 0.f, 0.f};
        gv[u] = ok ? __builtin_nontemporal_load(g4 + i) : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const double q0 = fminf(pv[u].x, 1.0f - pv[u].x), q1 = fminf(pv[u].y, 1.0f - pv[u].y);
        const double q2 = fminf(pv[u].z, 1.0f - pv[u].z), q3 = fminf(pv[u].w, 1.0f - pv[u].w);
        Du[u] += (q0 + q1) + (q2 + q3);
        Gu[u] += ((double)gv[u].x * q0 + (double)gv[u].y * q1) + ((double)gv[u].z * q2 + (double)gv[u].w * q3);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      D += Du[u];
      G += Gu[u];
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride) {
      const float q = fminf(pp[i], 1.0f - pp[i]);
      D += (double)q;
      G += (double)gg[i] * (double)q;
    }
  }
  block_sum2<kStreamThreads>(D, G, lds);
  if (threadIdx.x == 0) part[row * gx + blockIdx.x] = BwdPartial{D, G};
}

// dr = d (g - dk).  Every workgroup adds the reduce pass's partials of its
// row in the same fixed order, so all of them hold the same dk (bitwise) and
// no finalize launch is needed; the first one writes dk.  The first batch of
// scores is already in flight while the partials are added.
// The row's temperature into t (per-row value if given); false if that
// value is out of range (then t = 1 and the row's outputs become NaN).
LDEV bool bwd_row_t(const RowParams &rp, int64_t row, int64_t n, double &t) {
  if (!rp.t) return true;
  double kr = 0.5 * (double)n;
  return row_params(nullptr, rp.t, row, n, kr, t);
}

LDEV void bwd_row_total(const BwdPartial *__restrict__ vp, int gx, double *lds, double &dkd, bool &degenerate) {
  double Ds = 0.0, Gs = 0.0;
  for (int i = threadIdx.x; i < gx; i += kStreamThreads) {
    Ds += vp[i].D;
    Gs += vp[i].G;
  }
  block_sum2<kStreamThreads>(Ds, Gs, lds);
  degenerate = !(Ds > 0.0);
  dkd = degenerate ? 0.0 : Gs / Ds;
}

__global__ __launch_bounds__(kStreamThreads) void bwd_apply_kernel(const float *__restrict__ g,
                                                                   const float *__restrict__ p, int64_t rows,
                                                                   int64_t n, const BwdPartial *__restrict__ part,
                                                                   int gx, double t, RowParams rp,
                                                                   float *__restrict__ dr, float *__restrict__ dk,
                                                                   lapsum_row_stats *stats) {
  __shared__ double lds[2 * kStreamThreads / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const BwdPartial *vp = part + row * gx;
  const float *gg = g + row * n;
  const float *pp = p + row * n;
  float *dd = dr + row * n;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  double dkd;
  bool degenerate, good;
  if ((n & 3) == 0 && aligned16(g) && aligned16(p) && aligned16(dr)) {
    const int64_t n4 = n >> 2;
    const f4 *g4 = reinterpret_cast<const f4 *>(gg);
    const f4 *p4 = reinterpret_cast<const f4 *>(pp);
    f4 *d4 = reinterpret_cast<f4 *>(dd);
    f4 pv[kUnroll], gv[kUnroll];
    int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x;
    auto load = [&](int64_t j0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = j0 + u * kStreamThreads;
        const bool ok = i < n4;
        pv[u] = ok ? __builtin_nontemporal_load(p4 + i) : f4{0.f, 0.f, 0.f, 0.f};
        gv[u] = ok ? __builtin_nontemporal_load(g4 + i) : f4{0.f, 0.f, 0.f, 0.f};
      }
    };
    load(i0);
    good = bwd_row_t(rp, row, n, t);
    bwd_row_total(vp, gx, lds, dkd, degenerate);
    if (!good) dkd = __builtin_nan("");  // NaN through every dr of the row
    const float inv_t = degenerate ? 0.0f : (float)(1.0 / t);
    while (i0 < n4) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + u * kStreamThreads;
        if (i < n4) {
          f4 o;
          o.x = fminf(pv[u].x, 1.0f - pv[u].x) * inv_t * (float)((double)gv[u].x - dkd);
          o.y = fminf(pv[u].y, 1.0f - pv[u].y) * inv_t * (float)((double)gv[u].y - dkd);
          o.z = fminf(pv[u].z, 1.0f - pv[u].z) * inv_t * (float)((double)gv[u].z - dkd);
          o.w = fminf(pv[u].w, 1.0f - pv[u].w) * inv_t * (float)((double)gv[u].w - dkd);
          __builtin_nontemporal_store(o, d4 + i);
        }
      }
      i0 += stride * kUnroll;
      if (i0 < n4) load(i0);
    }
  } else {
    good = bwd_row_t(rp, row, n, t);
    bwd_row_total(vp, gx, lds, dkd, degenerate);
    if (!good) dkd = __builtin_nan("");
    const float inv_t = degenerate ? 0.0f : (float)(1.0 / t);
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride)
      dd[i] = fminf(pp[i], 1.0f - pp[i]) * inv_t * (float)((double)gg[i] - dkd);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    dk[row] = (float)dkd;
    if (stats && !good) atomicOr(&stats[row].flags, LAPSUM_FLAG_INVALID);
    else if (stats && degenerate) atomicOr(&stats[row].flags, LAPSUM_FLAG_DEGENERATE);
  }
}

int bwd_grid_x(int64_t rows, int64_t n) { return stream_grid_x(rows, n); }
size_t bwd_partial_bytes(int64_t rows, int grid_x) { return sizeof(BwdPartial) * (size_t)rows * (size_t)grid_x; }

hipError_t launch_bwd_reduce(const float *g, const float *p, int64_t rows, int64_t n, void *partials, int grid_x,
                             hipStream_t s) {
  hipLaunchKernelGGL(bwd_reduce_kernel, rows_grid((unsigned)grid_x, rows), dim3(kStreamThreads), 0, s, g, p, rows,
                     n, reinterpret_cast<BwdPartial *>(partials), grid_x);
  return hipGetLastError();
}

hipError_t launch_bwd_apply(const float *g, const float *p, int64_t rows, int64_t n, const void *partials,
                            int npart, double t, RowParams rp, float *dr, float *dk, lapsum_row_stats *stats,
                            hipStream_t s) {
  const int gx = stream_grid_x(rows, n);
  hipLaunchKernelGGL(bwd_apply_kernel, rows_grid((unsigned)gx, rows), dim3(kStreamThreads), 0, s, g, p, rows, n,
                     reinterpret_cast<const BwdPartial *>(partials), npart, t, rp, dr, dk, stats);
  return hipGetLastError();
}

}  // namespace lapsum
