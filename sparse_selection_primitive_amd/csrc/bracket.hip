// Probabilistic bracketing ("Fast LapSum: Exact Differentiable Top-k at
// Million Scale", section 2.2, "Probabilistic Bracketing"):
//
//  step 1, localisation -- sample_kernel draws m kernel-noised scores
//    X_j = r_I + t L (I uniform with replacement, L ~ Laplace(0, 1)), whose
//    CDF is 1 - f(x)/n, so #{X_j <= b} ~ Bin(m, 1 - k/n); select_kernel takes
//    the binomial order statistics X_(lo), X_(hi) as the bracket [a_L, a_R);
//  step 2, stream and filter -- filter_kernel reads every score once: below
//    a_L it adds e^{(r - a_L)/t} to S_L, at or above a_R it adds
//    e^{-(r - a_R)/t} to S_R, and in between it appends the key to the band
//    (wave ballot, one atomic per wave).  Tail sums are fp64 and finalized in
//    a fixed order by the last block.
//
// Random numbers: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with
// key (seed low, seed high) and counter (j, row, 0, 0): words x0, x1 give
// I = floor((x1 2^32 + x0) n / 2^64), word x2 gives u = (x2 + 1/2)/2^32 and
// L = F^-1(u) in fp64; X is rounded to fp32.
#include "lapsum_device.hpp"
#include "lapsum_internal.hpp"

namespace lapsum {

LDEV void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

__global__ __launch_bounds__(256) void sample_kernel(const float *__restrict__ r, int64_t n, double t, int64_t m,
                                                     uint32_t k0, uint32_t k1, float *__restrict__ samples,
                                                     RowState *__restrict__ st, int32_t flags) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = blockIdx.y;
  if (j == 0) reset_row_state(st, row, flags, 0, 0.0, 0.0);  // this call's state of the row
  if (j >= m) return;
  uint32_t c[4] = {(uint32_t)j, (uint32_t)row, 0u, 0u};
  philox4x32_10(c, k0, k1);
  const uint64_t nn = (uint64_t)n;
  const uint64_t idx = ((uint64_t)c[1] * nn + (((uint64_t)c[0] * nn) >> 32)) >> 32;
  const double u = ((double)c[2] + 0.5) * 0x1p-32;
  const double lap = u < 0.5 ? log(2.0 * u) : -log(2.0 * (1.0 - u));
  const double x = __dadd_rn((double)r[row * n + (int64_t)idx], __dmul_rn(t, lap));
  samples[row * m + j] = (float)x;
}

hipError_t launch_sample(const float *r, int64_t rows, int64_t n, double t, int64_t m, uint64_t seed,
                         float *samples, RowState *st, int32_t flags, hipStream_t s) {
  const int64_t gx = (m + 255) / 256;
  hipLaunchKernelGGL(sample_kernel, dim3((unsigned)gx, (unsigned)rows), dim3(256), 0, s, r, n, t, m,
                     (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), samples, st, flags);
  return hipGetLastError();
}

// ------------------------------------------------------- order statistics
// One workgroup of 1024 threads per row selects the ranks lo-1 and hi-1
// (0-based) of the m samples, by key.  A histogram of the key's top 15 bits
// in LDS gives each rank's bin and its rank inside the bin; the bin's keys
// are then gathered and ranked directly when few (<= kSelectCap), while a
// crowded bin is refined by histograms of the next 9 bits, then the last 8.
// Every pass over the samples is latency-bound, so each thread issues all
// of its loads (16 x 16 B per 65536 samples) before using any of them.
constexpr int kSelThreads = 1024;
constexpr int kSelBins = 1 << 15;
constexpr int kSelChunk = kSelThreads * 64;

struct SelectLds {
  uint32_t hist[kSelBins];
  uint32_t cand[2][kSelectCap];
  uint32_t ccount[2];
  uint32_t wsum[kSelThreads / kWave];
  uint32_t found_bin[2];
  uint32_t found_rank[2];
  uint32_t found_cnt[2];
  uint32_t result[2];
};

// f(key) for every sample; thread t handles 64 consecutive samples per chunk
template <class F>
LDEV void for_each_sample(const float *X, int64_t m, F &&f) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  for (int64_t c0 = 0; c0 < m; c0 += kSelChunk) {
    const int64_t base = c0 + (int64_t)threadIdx.x * 64;
    f4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
      v[q] = (base + 4 * q < m) ? *reinterpret_cast<const f4 *>(X + base + 4 * q) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (base + 4 * q < m) {
        f(key_of(v[q].x));
        f(key_of(v[q].y));
        f(key_of(v[q].z));
        f(key_of(v[q].w));
      }
    }
  }
}

LDEV uint32_t block_excl_scan_u32(uint32_t v, uint32_t *wsum) {
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
  for (int i = 0; i < kSelThreads / kWave; ++i)
    if (i < w) before += wsum[i];
  return before + inc - v;
}

// Bins holding ranks R[0] and R[1] (where want[t]) of the LDS histogram of
// `nbins` counts, one scan for both: each thread owns `per` consecutive bins
// (read 16 B at a time when per is a multiple of 4); writes
// found_bin/rank/cnt[t].
LDEV void locate_ranks(int nbins, const uint32_t (&R)[2], const bool (&want)[2], SelectLds &L) {
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const int per = (nbins + kSelThreads - 1) / kSelThreads;
  const int b0 = threadIdx.x * per;
  uint32_t c[32];
  uint32_t local = 0;
  if (per == 32) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u4 v = *reinterpret_cast<const u4 *>(&L.hist[b0 + 4 * q]);
      c[4 * q] = v.x;
      c[4 * q + 1] = v.y;
      c[4 * q + 2] = v.z;
      c[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = (i < per && b0 + i < nbins) ? L.hist[b0 + i] : 0u;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) local += c[i];
  const uint32_t before = block_excl_scan_u32(local, L.wsum);
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg] || local == 0 || R[tg] < before || R[tg] >= before + local) continue;
    uint32_t acc = before;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (R[tg] >= acc && R[tg] < acc + c[i]) {
        L.found_bin[tg] = (uint32_t)(b0 + i);
        L.found_rank[tg] = R[tg] - acc;
        L.found_cnt[tg] = c[i];
      }
      acc += c[i];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float *__restrict__ samples, int64_t m,
                                                             int64_t lo, int64_t hi, RowState *__restrict__ st) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SelectLds &L = *reinterpret_cast<SelectLds *>(lds_raw);
  const int64_t row = blockIdx.x;
  const float *X = samples + row * m;
  const bool want[2] = {lo >= 1, hi <= m};
  uint32_t R[2] = {(uint32_t)(lo - 1), (uint32_t)(hi - 1)};
  uint32_t prefix[2] = {0u, 0u}, cnt[2] = {0u, 0u};
  int pshift[2] = {17, 17};

  {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 z4 = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < kSelBins / 4; i += kSelThreads) reinterpret_cast<u4 *>(L.hist)[i] = z4;
  }
  __syncthreads();
  for_each_sample(X, m, [&](uint32_t kk) { atomicAdd(&L.hist[kk >> 17], 1u); });
  __syncthreads();
  locate_ranks(kSelBins, R, want, L);
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg]) continue;
    prefix[tg] = L.found_bin[tg];
    R[tg] = L.found_rank[tg];
    cnt[tg] = L.found_cnt[tg];
  }
  // refinement of a crowded bin: 9 more bits, then the last 8
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg]) continue;
    while (cnt[tg] > (uint32_t)kSelectCap && pshift[tg] > 0) {
      const int sh = pshift[tg] > 8 ? 8 : 0;
      const int nb = pshift[tg] - sh;
      const uint32_t pf = prefix[tg];
      const int ps = pshift[tg];
      __syncthreads();
      for (int i = threadIdx.x; i < (1 << nb); i += kSelThreads) L.hist[i] = 0u;
      __syncthreads();
      for_each_sample(X, m, [&](uint32_t kk) {
        if ((kk >> ps) == pf) atomicAdd(&L.hist[(kk >> sh) & ((1u << nb) - 1u)], 1u);
      });
      __syncthreads();
      const uint32_t Rt[2] = {R[tg], R[tg]};
      const bool wt[2] = {tg == 0, tg == 1};
      locate_ranks(1 << nb, Rt, wt, L);
      prefix[tg] = (pf << nb) | L.found_bin[tg];
      R[tg] = L.found_rank[tg];
      cnt[tg] = L.found_cnt[tg];
      pshift[tg] = sh;
    }
  }
  // gather the candidates of each target's final bin
  if (threadIdx.x < 2) {
    L.ccount[threadIdx.x] = 0u;
    L.result[threadIdx.x] = 0u;
  }
  __syncthreads();
  const bool gather0 = want[0] && pshift[0] > 0, gather1 = want[1] && pshift[1] > 0;
  if (gather0 || gather1) {
    const int ps0 = pshift[0], ps1 = pshift[1];
    const uint32_t pf0 = prefix[0], pf1 = prefix[1];
    for_each_sample(X, m, [&](uint32_t kk) {
      if (gather0 && (kk >> ps0) == pf0) {
        const uint32_t slot = atomicAdd(&L.ccount[0], 1u);
        if (slot < (uint32_t)kSelectCap) L.cand[0][slot] = kk;
      }
      if (gather1 && (kk >> ps1) == pf1) {
        const uint32_t slot = atomicAdd(&L.ccount[1], 1u);
        if (slot < (uint32_t)kSelectCap) L.cand[1][slot] = kk;
      }
    });
  }
  __syncthreads();
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg]) continue;
    if (pshift[tg] == 0) {
      if (threadIdx.x == 0) L.result[tg] = prefix[tg];
      continue;
    }
    const uint32_t nc = min(L.ccount[tg], (uint32_t)kSelectCap);
    for (uint32_t i = threadIdx.x; i < nc; i += kSelThreads) {
      const uint32_t ci = L.cand[tg][i];
      uint32_t less = 0, leq = 0;
      for (uint32_t q = 0; q < nc; ++q) {
        const uint32_t cq = L.cand[tg][q];
        less += cq < ci ? 1u : 0u;
        leq += cq <= ci ? 1u : 0u;
      }
      if (less <= R[tg] && R[tg] < leq) L.result[tg] = ci;  // equal keys write the same value
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    st[row].a_lo = want[0] ? (double)value_of(L.result[0]) : -INFINITY;
    st[row].a_hi = want[1] ? (double)value_of(L.result[1]) : INFINITY;
  }
}

hipError_t launch_select(const float *samples, int64_t rows, int64_t m, int64_t lo, int64_t hi, RowState *st,
                         hipStream_t s) {
  static bool attr_set = false;
  const size_t lds = sizeof(SelectLds);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(kSelThreads), lds, s, samples, m, lo, hi, st);
  return hipGetLastError();
}

// --------------------------------------------------------- stream & filter
struct FilterPartial {
  double sl, sr;
  unsigned long long cl, cr;
  uint32_t cnt;       // band keys this block found (may exceed kBandSlot)
  uint32_t kmn, kmx;  // key range of those band keys
  uint32_t pad;
};

LDEV void filter_one(float x, float aL, float aR, float cf, float &fl, float &fr, uint32_t &cl, uint32_t &cr,
                     bool &mid) {
  const bool lo = x < aL;
  const bool hi = x >= aR;
  const float z = lo ? (x - aL) : (aR - x);  // <= 0 whenever it is used
  const float w = __builtin_amdgcn_exp2f(z * cf);
  fl += lo ? w : 0.0f;
  fr += hi ? w : 0.0f;
  cl += lo ? 1u : 0u;
  cr += hi ? 1u : 0u;
  mid = !lo && !hi;
}

LDEV uint32_t mbcnt64(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// One coalesced pass over the row.  Band keys go to this block's own slot
// (positions reserved by an LDS counter, one LDS atomic per wave); the tail
// sums, counts and the band key range go to the block's partial.  No global
// atomics: the per-row finalize adds the partials in a fixed order and turns
// the slot counts into offsets.
__global__ __launch_bounds__(kStreamThreads) void filter_kernel(const float *__restrict__ r, int64_t n,
                                                                const RowState *__restrict__ st,
                                                                uint32_t *__restrict__ slots,
                                                                FilterPartial *__restrict__ part, int gx, double t) {
  __shared__ double lds_d[2 * kStreamThreads / kWave];
  __shared__ unsigned long long lds_c[2 * kStreamThreads / kWave];
  __shared__ uint32_t lds_k[2 * kStreamThreads / kWave];
  __shared__ uint32_t lcount;
  const int64_t row = blockIdx.y;
  const RowState &S = st[row];
  if (threadIdx.x == 0) lcount = 0u;
  __syncthreads();
  const float aL = (float)S.a_lo, aR = (float)S.a_hi;
  const float cf = (float)(kLog2e / t);
  const float *rr = r + row * n;
  uint32_t *slot = slots + ((int64_t)row * gx + blockIdx.x) * kBandSlot;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  double sl = 0.0, sr = 0.0;
  uint32_t cl = 0, cr = 0;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;

  typedef float f4 __attribute__((ext_vector_type(4)));
  const bool vec = (n & 3) == 0 && (((uintptr_t)r & 15u) == 0);
  const int64_t nitems = vec ? (n >> 2) : n;
  // kUnroll items (16 B each on the vector path) per thread and iteration,
  // all loads issued before any is used
  for (int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x; i0 < nitems;
       i0 += stride * kUnroll) {
    float x[4 * kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kStreamThreads;
      f4 v = {0.f, 0.f, 0.f, 0.f};
      if (i < nitems) {
        if (vec) v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(rr) + i);
        else v.x = rr[i];
      }
      x[4 * u] = v.x;
      x[4 * u + 1] = v.y;
      x[4 * u + 2] = v.z;
      x[4 * u + 3] = v.w;
    }
    float fl = 0.0f, fr = 0.0f;
    bool mid[4 * kUnroll];
    bool any = false;
#pragma unroll
    for (int q = 0; q < 4 * kUnroll; ++q) {
      const int64_t i = i0 + (q / 4) * kStreamThreads;
      const bool ok = i < nitems && (vec || (q & 3) == 0);
      mid[q] = false;
      if (ok) filter_one(x[q], aL, aR, cf, fl, fr, cl, cr, mid[q]);
      any |= mid[q];
    }
    sl += (double)fl;
    sr += (double)fr;
    const unsigned long long wany = __ballot(any);
    if (wany) {
      const unsigned long long active = __ballot(1);
      const int leader = __ffsll((long long)active) - 1;
      unsigned long long mq[4 * kUnroll];
      uint32_t tot = 0;
#pragma unroll
      for (int q = 0; q < 4 * kUnroll; ++q) {
        mq[q] = __ballot(mid[q]);
        tot += (uint32_t)__popcll(mq[q]);
      }
      uint32_t base = 0u;
      if (lane_id() == leader) base = atomicAdd(&lcount, tot);
      base = __shfl(base, leader, kWave);
      uint32_t off = base;
#pragma unroll
      for (int q = 0; q < 4 * kUnroll; ++q) {
        if (mid[q]) {
          const uint32_t pos = off + mbcnt64(mq[q]);
          const uint32_t kk = key_of(x[q]);
          if (pos < (uint32_t)kBandSlot) slot[pos] = kk;  // beyond the slot: counted, row falls back
          kmn = min(kmn, kk);
          kmx = max(kmx, kk);
        }
        off += (uint32_t)__popcll(mq[q]);
      }
    }
  }

  // block reduction (fixed order)
  unsigned long long ccl = cl, ccr = cr;
#pragma unroll
  for (int msk = 1; msk < kWave; msk <<= 1) {
    sl += __shfl_xor(sl, msk, kWave);
    sr += __shfl_xor(sr, msk, kWave);
    ccl += __shfl_xor(ccl, msk, kWave);
    ccr += __shfl_xor(ccr, msk, kWave);
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, msk, kWave));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, msk, kWave));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds_d[2 * w] = sl;
    lds_d[2 * w + 1] = sr;
    lds_c[2 * w] = ccl;
    lds_c[2 * w + 1] = ccr;
    lds_k[2 * w] = kmn;
    lds_k[2 * w + 1] = kmx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    FilterPartial fp;
    fp.sl = 0.0;
    fp.sr = 0.0;
    fp.cl = 0;
    fp.cr = 0;
    fp.kmn = 0xFFFFFFFFu;
    fp.kmx = 0u;
    for (int i = 0; i < kStreamThreads / kWave; ++i) {
      fp.sl += lds_d[2 * i];
      fp.sr += lds_d[2 * i + 1];
      fp.cl += lds_c[2 * i];
      fp.cr += lds_c[2 * i + 1];
      fp.kmn = min(fp.kmn, lds_k[2 * i]);
      fp.kmx = max(fp.kmx, lds_k[2 * i + 1]);
    }
    fp.cnt = lcount;
    fp.pad = 0u;
    part[row * gx + blockIdx.x] = fp;
  }
}

// Per row, in a fixed order: tail sums and counts, band size M, band key
// range, and the exclusive offsets of the block slots (offs[gx] = M).  A
// slot that overflowed, or M beyond the band capacity, sends the row to the
// full-sort fallback.
__global__ __launch_bounds__(kStreamThreads) void filter_finalize_kernel(const FilterPartial *__restrict__ part,
                                                                         int gx, int64_t cap,
                                                                         RowState *__restrict__ st,
                                                                         uint32_t *__restrict__ offs) {
  __shared__ double lds_d[2 * kStreamThreads / kWave];
  __shared__ unsigned long long lds_c[2 * kStreamThreads / kWave];
  __shared__ uint32_t lds_k[3 * kStreamThreads / kWave];
  __shared__ uint32_t wsum[kStreamThreads / kWave];
  const int64_t row = blockIdx.x;
  const FilterPartial *vp = part + row * gx;
  uint32_t *ro = offs + row * (int64_t)(gx + 1);
  // contiguous chunk of blocks per thread, so the offsets come out in order
  const int per = (gx + kStreamThreads - 1) / kStreamThreads;
  const int b0 = threadIdx.x * per;
  double a = 0.0, b = 0.0;
  unsigned long long c0 = 0, c1 = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, csum = 0u, big = 0u;
  for (int i = 0; i < per; ++i) {
    const int j = b0 + i;
    if (j < gx) {
      const FilterPartial fp = vp[j];
      a += fp.sl;
      b += fp.sr;
      c0 += fp.cl;
      c1 += fp.cr;
      mn = min(mn, fp.kmn);
      mx = max(mx, fp.kmx);
      csum += fp.cnt;
      big |= fp.cnt > (uint32_t)kBandSlot ? 1u : 0u;
    }
  }
  // exclusive scan of the chunk sums
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  uint32_t inc = csum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  uint32_t before = 0u, total = 0u;
  for (int i = 0; i < kStreamThreads / kWave; ++i) {
    if (i < w) before += wsum[i];
    total += wsum[i];
  }
  uint32_t run = before + inc - csum;
  for (int i = 0; i < per; ++i) {
    const int j = b0 + i;
    if (j < gx) {
      ro[j] = run;
      run += vp[j].cnt;
    }
  }
  if (threadIdx.x == kStreamThreads - 1) ro[gx] = total;
#pragma unroll
  for (int msk = 1; msk < kWave; msk <<= 1) {
    a += __shfl_xor(a, msk, kWave);
    b += __shfl_xor(b, msk, kWave);
    c0 += __shfl_xor(c0, msk, kWave);
    c1 += __shfl_xor(c1, msk, kWave);
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, msk, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, msk, kWave));
    big |= (uint32_t)__shfl_xor((int)big, msk, kWave);
  }
  if (lane == 0) {
    lds_d[2 * w] = a;
    lds_d[2 * w + 1] = b;
    lds_c[2 * w] = c0;
    lds_c[2 * w + 1] = c1;
    lds_k[3 * w] = mn;
    lds_k[3 * w + 1] = mx;
    lds_k[3 * w + 2] = big;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ta = 0.0, tb = 0.0;
    unsigned long long tc0 = 0, tc1 = 0;
    uint32_t tmn = 0xFFFFFFFFu, tmx = 0u, tbig = 0u;
    for (int i = 0; i < kStreamThreads / kWave; ++i) {
      ta += lds_d[2 * i];
      tb += lds_d[2 * i + 1];
      tc0 += lds_c[2 * i];
      tc1 += lds_c[2 * i + 1];
      tmn = min(tmn, lds_k[3 * i]);
      tmx = max(tmx, lds_k[3 * i + 1]);
      tbig |= lds_k[3 * i + 2];
    }
    RowState &S = st[row];
    S.tail_lo = ta;
    S.tail_hi = tb;
    S.count_lo = tc0;
    S.count_hi = tc1;
    S.band = total;
    S.kmin = tmn;
    S.kmax = tmx;
    if (tbig || (int64_t)total > cap) S.flags |= LAPSUM_FLAG_OVERFLOW | LAPSUM_FLAG_FALLBACK;
  }
}

int filter_grid_x(int64_t rows, int64_t n) {
  const int64_t per_row_need = (n / 4 + kStreamThreads * kUnroll - 1) / (kStreamThreads * kUnroll);
  int64_t target = 1024 / (rows > 0 ? rows : 1);
  if (target < 1) target = 1;
  int64_t gx = per_row_need < target ? per_row_need : target;
  return (int)(gx < 1 ? 1 : gx);
}

size_t filter_partial_bytes(int64_t rows, int grid_x) {
  return sizeof(FilterPartial) * (size_t)rows * (size_t)grid_x;
}
size_t band_slot_bytes(int64_t rows, int grid_x) {
  return sizeof(uint32_t) * (size_t)rows * (size_t)grid_x * (size_t)kBandSlot;
}
size_t band_offs_bytes(int64_t rows, int grid_x) { return sizeof(uint32_t) * (size_t)rows * (size_t)(grid_x + 1); }

hipError_t launch_filter(const float *r, int64_t rows, int64_t n, double t, RowState *st, uint32_t *slots,
                         uint32_t *offs, int64_t cap, void *partials, int grid_x, hipStream_t s) {
  hipLaunchKernelGGL(filter_kernel, dim3(grid_x, (unsigned)rows), dim3(kStreamThreads), 0, s, r, n, st, slots,
                     reinterpret_cast<FilterPartial *>(partials), grid_x, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(filter_finalize_kernel, dim3((unsigned)rows), dim3(kStreamThreads), 0, s,
                     reinterpret_cast<const FilterPartial *>(partials), grid_x, cap, st, offs);
  return hipGetLastError();
}

}  // namespace lapsum
