// Probabilistic bracketing ("Fast LapSum: Exact Differentiable Top-k at
// Million Scale", section 2.2, "Probabilistic Bracketing"):
//
//  step 1, localisation -- sample_kernel draws m kernel-noised scores
//    X_j = r_I + t L (I uniform with replacement, L ~ Laplace(0, 1)), whose
//    CDF is 1 - f(x)/n, so #{X_j <= b} ~ Bin(m, 1 - k/n); select_kernel takes
//    the binomial order statistics X_(lo), X_(hi) as the bracket [a_L, a_R);
//  step 2, stream and filter -- filter_kernel reads every score once: below
//    a_L it adds e^{(r - a_L)/t} to S_L, at or above a_R it adds
//    e^{-(r - a_R)/t} to S_R, and in between it appends the key to its
//    workgroup's band slot and leaves its partial sums and counts; the band
//    solve's first kernel adds them per row in a fixed order (fp64).
//
// Random numbers: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with
// key (seed low, seed high) and counter (j, row, 0, 0): words x0, x1 give
// I = floor((x1 2^32 + x0) n / 2^64), word x2 gives u = (x2 + 1/2)/2^32 and
// L = F^-1(u) in fp64; X is rounded to fp32.
#include <algorithm>
#include <atomic>

#include "filter_dev.hpp"
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

// Each workgroup draws kSampleWg consecutive samples of one row (counters
// j = group * kSampleWg + q * kSampleThreads + thread), sorts them inside the
// workgroup by the top kCoarseBits bits of their keys, and writes them in
// that order to its slice of `samples`, with the 16-bit start of every
// coarse bin inside the slice to `starts`.  (The sample is a multiset: its order statistics
// do not depend on the order it is stored in.)
constexpr int kSampleThreads = 1024;
constexpr int kSamplePerThread = 2;
constexpr int kSampleWg = kSampleThreads * kSamplePerThread;
constexpr int kCoarseBits = 10;
constexpr int kCoarseBins = 1 << kCoarseBits;
static_assert(kCoarseBins == kSampleThreads, "one coarse bin per sample thread");

// Top-side selection ("tail mode"): when both bracket ranks lie within the
// Q largest samples, each sample workgroup also writes its own Q largest
// keys, sorted descending; the R-th largest of the whole sample (R <= Q) is
// then the R-th largest of those lists (no group contributes more than R of
// its own keys to the top R), so the selection reads groups x Q keys instead
// of the whole sample.
constexpr int kTailWaveSort = 16 * kWave;  // largest candidate set one wave sorts
template <int E>
LDEV void wave_sort_pick(const uint32_t *f, int nf, uint32_t R, uint32_t *out);
constexpr int kTailMaxKeys = 4096;        // groups x Q the selection holds in LDS

// One wave sorts the nc candidate scores src[0..nc) (with nc, Q <= 64*E) and
// writes the Q largest keys, descending, to out (key 0, below every key, pads).
template <int E>
LDEV void wave_top_sorted(const float *src, int nc, int Q, uint32_t *out) {
  WaveTeam<kWave> team;
  const int base = team.lane * E;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = base + e < nc ? key_of(src[base + e]) : 0u;
  bitonic_sort<E>(key, team);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = kWave * E - 1 - (base + e);  // rank from the top
    if (i < Q) out[i] = key[e];
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
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i)
    if (i < w) before += wsum[i];
  return before + inc - v;
}

template <bool TAIL>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(const float *__restrict__ r, int64_t rows,
                                                                int64_t n, double t, int64_t m, uint32_t k0,
                                                                uint32_t k1, float *__restrict__ samples,
                                                                uint16_t *__restrict__ starts,
                                                                RowState *__restrict__ st, int32_t flags,
                                                                uint32_t *__restrict__ tail, int Q,
                                                                const double *__restrict__ t_rows) {
  __shared__ uint32_t cnt[kCoarseBins];
  __shared__ uint32_t wsum[kSampleThreads / kWave];
  __shared__ float stage[kSampleWg];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const int64_t g0 = (int64_t)blockIdx.x * kSampleWg;
  if (blockIdx.x == 0 && threadIdx.x == 0) reset_row_state(st, row, flags, 0, 0.0, 0.0);  // this call's state
  if (t_rows != nullptr) {  // the row's own temperature (an out-of-range one: 1, the row is flagged later)
    const double tr = t_rows[row];
    t = tr > 0.0 && tr < INFINITY ? tr : 1.0;
  }
  cnt[threadIdx.x] = 0u;
  // indices of this thread's samples first and all the gathers issued, then
  // the noise, whose logarithms overlap the gathers' latency
  const uint64_t nn = (uint64_t)n;
  int64_t idx[kSamplePerThread];
  uint32_t ubits[kSamplePerThread];
#pragma unroll
  for (int q = 0; q < kSamplePerThread; ++q) {
    const int64_t j = g0 + q * kSampleThreads + threadIdx.x;
    uint32_t c[4] = {(uint32_t)j, (uint32_t)row, 0u, 0u};
    philox4x32_10(c, k0, k1);
    idx[q] = (int64_t)(((uint64_t)c[1] * nn + (((uint64_t)c[0] * nn) >> 32)) >> 32);
    ubits[q] = c[2];
  }
  // unconditional loads (score 0 stands in past the sample's end), so no
  // branch makes each gather wait before the next is issued
  float rv[kSamplePerThread];
#pragma unroll
  for (int q = 0; q < kSamplePerThread; ++q)
    rv[q] = r[row * n + ((g0 + q * kSampleThreads + threadIdx.x < m) ? idx[q] : 0)];
  // L = F^-1(u): ln(2u) below 1/2, -ln(2(1 - u)) above (one logarithm)
  double lap[kSamplePerThread];
#pragma unroll
  for (int q = 0; q < kSamplePerThread; ++q) {
    const double u = ((double)ubits[q] + 0.5) * 0x1p-32;
    const bool low = u < 0.5;
    const double l = log(2.0 * (low ? u : 1.0 - u));
    lap[q] = low ? l : -l;
  }
  float x[kSamplePerThread];
  uint32_t bin[kSamplePerThread], slot[kSamplePerThread];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSamplePerThread; ++q) {
    x[q] = (float)__dadd_rn((double)rv[q], __dmul_rn(t, lap[q]));
    bin[q] = key_of(x[q]) >> (32 - kCoarseBits);
    slot[q] = 0u;
    if (g0 + q * kSampleThreads + threadIdx.x < m) slot[q] = atomicAdd(&cnt[bin[q]], 1u);
  }
  __syncthreads();
  const uint32_t c = cnt[threadIdx.x];
  const uint32_t start = block_excl_scan_u32(c, wsum);
  starts[(row * gridDim.x + blockIdx.x) * (int64_t)kCoarseBins + threadIdx.x] = (uint16_t)start;
  cnt[threadIdx.x] = start;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kSamplePerThread; ++q)
    if (g0 + q * kSampleThreads + threadIdx.x < m) stage[cnt[bin[q]] + slot[q]] = x[q];
  __syncthreads();
  const int nvalid = (int)min(m - g0, (int64_t)kSampleWg);
  for (int i = threadIdx.x; i < nvalid; i += kSampleThreads) samples[row * m + g0 + i] = stage[i];
  if constexpr (TAIL) {
    // this group's Q largest keys, descending: the candidates are the staged
    // scores from the start of the coarse bin that holds the Q-th largest on
    // (stage is in ascending bin order; cnt holds the bin starts)
    __shared__ uint32_t cbeg;
    __shared__ BlockTeamLds<kSampleThreads, 2> blds;
    const int j0 = nvalid > Q ? nvalid - Q : 0;
    {
      const uint32_t s0 = cnt[threadIdx.x];
      const uint32_t s1 = threadIdx.x + 1 < (unsigned)kCoarseBins ? cnt[threadIdx.x + 1] : (uint32_t)nvalid;
      if (s0 <= (uint32_t)j0 && (uint32_t)j0 < s1) cbeg = s0;  // exactly one bin holds j0
    }
    __syncthreads();
    const int nc = nvalid - (int)cbeg;
    uint32_t *out = tail + (row * gridDim.x + blockIdx.x) * (int64_t)Q;
    const int need = nc > Q ? nc : Q;
    if (need <= kTailWaveSort) {
      if (threadIdx.x < kWave) {
        const float *src = stage + cbeg;
        if (need <= 64) wave_top_sorted<1>(src, nc, Q, out);
        else if (need <= 128) wave_top_sorted<2>(src, nc, Q, out);
        else if (need <= 256) wave_top_sorted<4>(src, nc, Q, out);
        else if (need <= 512) wave_top_sorted<8>(src, nc, Q, out);
        else wave_top_sorted<16>(src, nc, Q, out);
      }
    } else {
      // a crowded coarse bin: the whole workgroup sorts all its samples
      BlockTeam<kSampleThreads, 2> team(&blds);
      uint32_t key[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * (int)threadIdx.x + e;
        key[e] = i < nvalid ? key_of(stage[i]) : 0u;
      }
      bitonic_sort<2>(key, team);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = kSampleWg - 1 - (2 * (int)threadIdx.x + e);
        if (i < Q) out[i] = key[e];
      }
    }
  }
}

int sample_groups(int64_t m) { return (int)((m + kSampleWg - 1) / kSampleWg); }
size_t sample_start_bytes(int64_t rows, int64_t m) {
  return sizeof(uint16_t) * (size_t)rows * (size_t)sample_groups(m) * kCoarseBins;
}

hipError_t launch_sample(const float *r, int64_t rows, int64_t n, double t, int64_t m, uint64_t seed,
                         float *samples, uint16_t *starts, RowState *st, int32_t flags, uint32_t *tail, int Q,
                         const double *t_rows, hipStream_t s) {
  const dim3 grid = rows_grid((unsigned)sample_groups(m), rows);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  if (tail != nullptr)
    hipLaunchKernelGGL(sample_kernel<true>, grid, dim3(kSampleThreads), 0, s, r, rows, n, t, m, k0, k1, samples,
                       starts, st, flags, tail, Q, t_rows);
  else
    hipLaunchKernelGGL(sample_kernel<false>, grid, dim3(kSampleThreads), 0, s, r, rows, n, t, m, k0, k1, samples,
                       starts, st, flags, tail, Q, t_rows);
  return hipGetLastError();
}

// ------------------------------------------- per-row bracket indices
// With a budget per row, step 1's order-statistic indices depend on the row:
// one workgroup per row computes them on the device from the same
// definition the host applies to a single budget.  With N ~ Bin(m, q),
// q = 1 - k/n (the share of the row below b),
//   lo = max{l in [0, m]   : P(N <= l - 1) <= delta/2},
//   hi = min{h in [1, m+1] : P(N >= h)     <= delta/2}.
// The pmf is summed over mean +- 40 sd (the rest of its mass is far below
// fp64 resolution): each thread walks its stretch of j with the ratio
// recurrence from a start value taken from lgamma, and the tail sums come
// from block prefix / suffix sums of the stretches.  The row's k and t (an
// out-of-range value replaced and the row flagged invalid) and c go to its
// state for the later stages.
constexpr int kBrThreads = 1024;

__global__ __launch_bounds__(kBrThreads) void bracket_rows_kernel(const double *__restrict__ k_rows,
                                                                  const double *__restrict__ t_rows, double k,
                                                                  double t, int64_t rows, int64_t n, int64_t m,
                                                                  double delta, RowState *__restrict__ st) {
  __shared__ double wsum[2][kBrThreads / kWave];
  __shared__ int wext[2][kBrThreads / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const bool good = row_params(k_rows, t_rows, row, n, k, t);
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  constexpr int NW = kBrThreads / kWave;
  const double pk = k / (double)n;  // 1 - q
  const double qd = 1.0 - pk;
  const double lq = log1p(-pk), l1q = log(pk), ratio = qd / pk;
  const double mean = (double)m * qd, sd = sqrt((double)m * qd * pk);
  const double wdt = 40.0 * sd + 40.0;
  const int64_t j0 = (int64_t)fmax(0.0, floor(mean - wdt)), j1 = (int64_t)fmin((double)m, ceil(mean + wdt));
  const int64_t len = j1 - j0 + 1, per = (len + kBrThreads - 1) / kBrThreads;
  const int64_t js = j0 + (int64_t)threadIdx.x * per, je = min(js + per - 1, j1);
  // log pmf relative to its value at the mode (the bulk stays near 1)
  const double lgm = lgamma((double)m + 1.0);
  auto lpmf = [&](int64_t j) {
    return lgm - lgamma((double)j + 1.0) - lgamma((double)(m - j) + 1.0) + (double)j * lq + (double)(m - j) * l1q;
  };
  const int64_t mode = min(max((int64_t)floor((double)(m + 1) * qd), (int64_t)0), m);
  const double lref = lpmf(mode);
  const double p0 = js <= je ? exp(lpmf(js) - lref) : 0.0;
  double part = 0.0;
  {
    double p = p0;
    for (int64_t j = js; j <= je; ++j) {
      part += p;
      p *= (double)(m - j) / (double)(j + 1) * ratio;
    }
  }
  // exclusive prefix and suffix of the stretch sums (each a sum over the
  // other stretches only, never a difference), and the total
  double inc = part, sinc = part;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(inc, off, kWave), z = __shfl_down(sinc, off, kWave);
    if (lane >= off) inc += y;
    if (lane + off < kWave) sinc += z;
  }
  if (lane == kWave - 1) wsum[0][w] = inc;
  if (lane == 0) wsum[1][w] = sinc;
  const double exc = __shfl_up(inc, 1, kWave), sexc = __shfl_down(sinc, 1, kWave);
  __syncthreads();
  double before = lane == 0 ? 0.0 : exc, after = lane == kWave - 1 ? 0.0 : sexc, tot = 0.0;
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += wsum[0][i];
    if (i > w) after += wsum[1][i];
    tot += wsum[0][i];
  }
  const double half = 0.5 * delta * tot;
  // walks: the last j with P(N <= j) <= half, the first h with P(N >= h) <= half
  int cand_lo = -1, cand_hi = (int)m + 2;  // m <= 2^20
  {
    double p = p0, acc = before;
    for (int64_t j = js; j <= je; ++j) {
      acc += p;
      if (acc <= half) cand_lo = (int)j;
      p *= (double)(m - j) / (double)(j + 1) * ratio;
    }
  }
  if (js <= je) {
    // backwards from je: the stretch's pmf values again, from its end
    double pe = exp(lpmf(je) - lref), acc = after;
    for (int64_t j = je; j >= js; --j) {
      acc += pe;
      if (acc <= half) cand_hi = (int)j;
      pe *= (double)j / (double)(m - j + 1) / ratio;
    }
  }
  cand_lo = wave_reduce(cand_lo, [](int x, int y) { return x > y ? x : y; });
  cand_hi = wave_reduce(cand_hi, [](int x, int y) { return x < y ? x : y; });
  if (lane == 0) {
    wext[0][w] = cand_lo;
    wext[1][w] = cand_hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t cl = -1, ch = m + 2;
    for (int i = 0; i < NW; ++i) {
      cl = max(cl, wext[0][i]);
      ch = min(ch, wext[1][i]);
    }
    RowState &S = st[row];
    S.blo = cl >= 0 ? cl + 1 : j0;
    S.bhi = ch <= m ? ch : j1 + 1;
    S.k = k;
    S.t = t;
    S.c = kLog2e / t;
    S.cf = (float)S.c;
    if (!good) S.flags |= LAPSUM_FLAG_INVALID;
  }
}

hipError_t launch_bracket_rows(const double *k_rows, const double *t_rows, double k, double t, int64_t rows,
                               int64_t n, int64_t m, double delta, RowState *st, hipStream_t s) {
  hipLaunchKernelGGL(bracket_rows_kernel, rows_grid(1u, rows), dim3(kBrThreads), 0, s, k_rows, t_rows, k, t, rows, n,
                     m, delta, st);
  return hipGetLastError();
}

// Top-side depth of the bracket ranks: the lo-th and hi-th smallest of m
// samples are the (m - lo + 1)-th and (m - hi + 1)-th largest.  Returns the
// depth Q the tail lists must hold, or 0 when tail mode does not apply.
int tail_depth(int64_t m, int64_t lo, int64_t hi) {
  int64_t q = 1;
  if (lo >= 1) q = std::max(q, m - lo + 1);
  if (hi <= m) q = std::max(q, m - hi + 1);
  const int64_t groups = sample_groups(m);
  if (q > kTailWaveSort || groups * q > kTailMaxKeys) return 0;
  return (int)q;
}
size_t tail_bytes(int64_t rows, int64_t m, int Q) {
  return sizeof(uint32_t) * (size_t)rows * (size_t)sample_groups(m) * (size_t)Q;
}

// One workgroup per row: the bracket ends from the groups' top-Q lists.
// For each target, the ascending rank groups*Q - R among the groups*Q keys
// (held 16 per thread) is found by bucketing relative to the keys' own
// range: 2048 LDS buckets over the top 11 bits of (key - kmin), the bucket
// that holds the rank, and, while that bucket holds more than one wave can
// sort, the same again inside it on the next bits; the last bucket's keys
// are gathered and sorted by one wave.  (Digit passes over the raw key bits
// would pile every candidate of a narrow range onto one LDS counter.)
constexpr int kTailThreads = 256;
constexpr int kTailPerThread = kTailMaxKeys / kTailThreads;
constexpr int kTailBinBits = 11;
constexpr int kTailBins = 1 << kTailBinBits;
constexpr int kTailBinsPer = kTailBins / kTailThreads;

struct TailLds {
  uint32_t hist[kTailBins];
  uint32_t cand[kTailWaveSort];
  uint32_t wsum[kTailThreads / kWave];
  uint32_t red[2 * kTailThreads / kWave];
  uint32_t bin, rank, count, ncand, result;
};

// Key of ascending rank `rank` among the N valid keys, all of which lie in
// [lo, lo + 2^wbits).  Each pass splits the current range into at most
// kTailBins buckets of 2^shift keys and keeps the one that holds the rank.
LDEV uint32_t tail_select_rank(const uint32_t (&key)[kTailPerThread], int N, uint32_t rank, uint32_t lo,
                               int wbits, TailLds &L) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  uint32_t cnt = (uint32_t)N;
  for (;;) {
    const int shift = wbits > kTailBinBits ? wbits - kTailBinBits : 0;
    const uint64_t width = (uint64_t)1 << wbits;
    for (int j = threadIdx.x; j < kTailBins; j += kTailThreads) L.hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTailPerThread; ++j) {
      const uint32_t kk = key[j];
      if (j * kTailThreads + (int)threadIdx.x < N && kk >= lo && (uint64_t)(kk - lo) < width)
        atomicAdd(&L.hist[(kk - lo) >> shift], 1u);
    }
    __syncthreads();
    // exclusive scan over the buckets (kTailBinsPer consecutive ones per thread)
    uint32_t c[kTailBinsPer], local = 0u;
#pragma unroll
    for (int q = 0; q < kTailBinsPer; ++q) {
      c[q] = L.hist[threadIdx.x * kTailBinsPer + q];
      local += c[q];
    }
    const uint32_t inc = wave_incl_scan(local);
    if (lane == kWave - 1) L.wsum[w] = inc;
    __syncthreads();
    uint32_t acc = inc - local;
    for (int i = 0; i < w; ++i) acc += L.wsum[i];
    if (rank >= acc && rank < acc + local) {  // exactly one thread
#pragma unroll
      for (int q = 0; q < kTailBinsPer; ++q) {
        if (rank >= acc && rank < acc + c[q]) {
          L.bin = threadIdx.x * kTailBinsPer + q;
          L.rank = rank - acc;
          L.count = c[q];
        }
        acc += c[q];
      }
    }
    __syncthreads();
    lo += L.bin << shift;
    rank = L.rank;
    cnt = L.count;
    wbits = shift;
    __syncthreads();
    if (wbits == 0) return lo;  // the bucket holds a single key value
    if (cnt <= (uint32_t)kTailWaveSort) break;
  }
  // gather the keys of the last bucket and let one wave sort them
  if (threadIdx.x == 0) L.ncand = 0u;
  __syncthreads();
  const uint64_t width = (uint64_t)1 << wbits;
#pragma unroll
  for (int j = 0; j < kTailPerThread; ++j) {
    const uint32_t kk = key[j];
    if (j * kTailThreads + (int)threadIdx.x < N && kk >= lo && (uint64_t)(kk - lo) < width)
      L.cand[atomicAdd(&L.ncand, 1u)] = kk;  // cnt <= kTailWaveSort of them
  }
  __syncthreads();
  if (w == 0) {
    const int nf = (int)L.ncand;
    if (nf <= 64) wave_sort_pick<1>(L.cand, nf, rank, &L.result);
    else if (nf <= 128) wave_sort_pick<2>(L.cand, nf, rank, &L.result);
    else if (nf <= 256) wave_sort_pick<4>(L.cand, nf, rank, &L.result);
    else if (nf <= 512) wave_sort_pick<8>(L.cand, nf, rank, &L.result);
    else wave_sort_pick<16>(L.cand, nf, rank, &L.result);
  }
  __syncthreads();
  const uint32_t res = L.result;
  __syncthreads();
  return res;
}

__global__ __launch_bounds__(kTailThreads) void select_tail_kernel(const uint32_t *__restrict__ tail, int64_t rows,
                                                                   int groups, int Q, int64_t m, int64_t lo,
                                                                   int64_t hi, RowState *__restrict__ st) {
  __shared__ TailLds L;
  const int64_t row = grid_row();
  if (row >= rows) return;
  const int N = groups * Q;
  const uint32_t *src = tail + row * (int64_t)N;
  uint32_t key[kTailPerThread];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < kTailPerThread; ++j) {
    const int i = j * kTailThreads + (int)threadIdx.x;
    key[j] = src[i < N ? i : 0];
  }
#pragma unroll
  for (int j = 0; j < kTailPerThread; ++j) {
    if (j * kTailThreads + (int)threadIdx.x < N) {
      mn = min(mn, key[j]);
      mx = max(mx, key[j]);
    }
  }
  // the keys' range over the workgroup (padding keys 0 included)
  mn = wave_reduce(mn, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  mx = wave_reduce(mx, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  if (lane == 0) {
    L.red[2 * w] = mn;
    L.red[2 * w + 1] = mx;
  }
  __syncthreads();
  for (int i = 0; i < kTailThreads / kWave; ++i) {
    mn = min(mn, L.red[2 * i]);
    mx = max(mx, L.red[2 * i + 1]);
  }
  const uint32_t span = mx - mn;
  const int bits = span == 0u ? 0 : 32 - __clz((int)span);
  const int wbits = bits > kTailBinBits ? bits : kTailBinBits;
  const bool want[2] = {lo >= 1, hi <= m};
  uint32_t res[2] = {0u, 0u};
#pragma unroll
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg]) continue;  // uniform over the workgroup
    const uint32_t R = (uint32_t)(tg == 0 ? m - lo + 1 : m - hi + 1);
    res[tg] = span == 0u ? mn : tail_select_rank(key, N, (uint32_t)N - R, mn, wbits, L);
  }
  if (threadIdx.x == 0) {
    st[row].a_lo = want[0] ? (double)value_of(res[0]) : -INFINITY;
    st[row].a_hi = want[1] ? (double)value_of(res[1]) : INFINITY;
  }
}

hipError_t launch_select_tail(const uint32_t *tail, int64_t rows, int64_t m, int Q, int64_t lo, int64_t hi,
                              RowState *st, hipStream_t s) {
  hipLaunchKernelGGL(select_tail_kernel, rows_grid(1u, rows), dim3(kTailThreads), 0, s, tail, rows,
                     sample_groups(m), Q, m, lo, hi, st);
  return hipGetLastError();
}

// ------------------------------------------------------- order statistics
// One workgroup of 1024 threads per row selects the ranks lo-1 and hi-1
// (0-based) of the m samples, by key.  General path (any m):  A histogram of the key's top 15 bits
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float *__restrict__ samples, int64_t rows,
                                                             int64_t m, int64_t lo, int64_t hi,
                                                             RowState *__restrict__ st) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  SelectLds &L = *reinterpret_cast<SelectLds *>(lds_raw);
  const int64_t row = grid_row();
  if (row >= rows) return;
  if (lo < 0) {  // per-row indices
    lo = st[row].blo;
    hi = st[row].bhi;
  }
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

// Fast path, m <= kSelMaxGroups * kSampleWg: the sample arrives bucketed by
// coarse bin inside each sample workgroup, with the bins' starts, so this
// workgroup reads the starts (64 KB) and then only the keys of the two
// target bins.  A crowded bin is refined by histograms of the next (up to)
// 11 bits until at most kSortCand keys share the prefix; one wave sorts
// those in registers and reads the rank off.  Scans over bins are done by
// one wave (no workgroup barriers inside).
constexpr int kSelMaxGroups = 32;
constexpr int kCandCap = 8192;
constexpr int kFineBins = 2048;
constexpr int kSortCand = 16 * kWave;  // largest key set one wave sorts in registers

struct SelectBucketLds {
  uint16_t start[kSelMaxGroups][kCoarseBins];  // bin starts inside each group's slice
  uint32_t hist[kFineBins];
  uint32_t cand[kCandCap];
  uint32_t fin[2][kSortCand];
  uint32_t goff[2][kSelMaxGroups + 1];  // candidate index where each group's part of the bin starts
  uint32_t bin[2], rank[2], count[2];
  uint32_t nfin[2], result[2];
};

// One wave sorts the nf <= 64*E keys f[] in registers (blocked, E per lane)
// and writes the key of rank R to *out.
template <int E>
LDEV void wave_sort_pick(const uint32_t *f, int nf, uint32_t R, uint32_t *out) {
  WaveTeam<kWave> team;
  const int base = team.lane * E;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = base + e < nf ? f[base + e] : 0xFFFFFFFFu;
  bitonic_sort<E>(key, team);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((uint32_t)(base + e) == R) *out = key[e];
}

// One wave: for each wanted target tg, the bin of rank R[tg] in the LDS
// histogram h of NB (a multiple of 64) counts, its rank inside the bin and
// its count, to bin/rank/count[tg].  Lane l owns bins l*PER .. l*PER+PER-1
// (summed in a rotated order: no bank conflicts).
template <int NB>
LDEV void wave_locate(const uint32_t *h, const uint32_t (&R)[2], const bool (&want)[2], SelectBucketLds &L) {
  constexpr int PER = NB / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int b0 = lane * PER;
  uint32_t c[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) c[q] = h[b0 + ((q + lane) & (PER - 1))];
  uint32_t local = 0u;
#pragma unroll
  for (int q = 0; q < PER; ++q) local += c[q];
  uint32_t inc = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  const uint32_t before = inc - local;
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg] || R[tg] < before || R[tg] >= before + local) continue;
    uint32_t acc = before;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const uint32_t cq = h[b0 + q];
      if (R[tg] >= acc && R[tg] < acc + cq) {
        L.bin[tg] = (uint32_t)(b0 + q);
        L.rank[tg] = R[tg] - acc;
        L.count[tg] = cq;
      }
      acc += cq;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void select_bucket_kernel(const float *__restrict__ samples,
                                                                    const uint16_t *__restrict__ starts,
                                                                    int64_t rows, int groups, int64_t m, int64_t lo,
                                                                    int64_t hi, RowState *__restrict__ st) {
  __shared__ SelectBucketLds L;
  const int64_t row = grid_row();
  if (row >= rows) return;
  if (lo < 0) {  // per-row indices
    lo = st[row].blo;
    hi = st[row].bhi;
  }
  const float *X = samples + row * m;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  {
    // bin starts of every group (16-bit, read as pairs): thread t reads
    // pair t & 511 of groups (t >> 9), (t >> 9) + 2, ...
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(starts + row * (int64_t)groups * kCoarseBins);
    const int col = threadIdx.x & (kCoarseBins / 2 - 1), g0 = threadIdx.x / (kCoarseBins / 2);
    constexpr int kStep = kSelThreads / (kCoarseBins / 2);
    uint32_t v[kSelMaxGroups / kStep];
#pragma unroll
    for (int j = 0; j < kSelMaxGroups / kStep; ++j) {
      const int g = g0 + kStep * j;
      v[j] = g < groups ? s32[g * (kCoarseBins / 2) + col] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kSelMaxGroups / kStep; ++j) {
      const int g = g0 + kStep * j;
      if (g < groups) reinterpret_cast<uint32_t *>(L.start[g])[col] = v[j];
    }
  }
  __syncthreads();
  // count of bin b in group g: the next start (or the group's size) minus this one
  auto gcount = [&](int g, uint32_t b) -> uint32_t {
    const uint32_t end = b + 1 < (uint32_t)kCoarseBins
                             ? (uint32_t)L.start[g][b + 1]
                             : (uint32_t)min((int64_t)kSampleWg, m - (int64_t)g * kSampleWg);
    return end - (uint32_t)L.start[g][b];
  };
  // bin totals as differences of the starts summed over the groups
  {
    uint32_t S = 0u;
    for (int g = 0; g < groups; ++g) S += L.start[g][threadIdx.x];
    L.hist[threadIdx.x] = S;  // kCoarseBins == kSelThreads
  }
  __syncthreads();
  {
    const uint32_t nxt = threadIdx.x + 1 < (unsigned)kCoarseBins ? L.hist[threadIdx.x + 1] : (uint32_t)m;
    const uint32_t tot = nxt - L.hist[threadIdx.x];
    __syncthreads();
    L.hist[threadIdx.x] = tot;
  }
  __syncthreads();
  const bool want[2] = {lo >= 1, hi <= m};
  uint32_t R[2] = {(uint32_t)(lo - 1), (uint32_t)(hi - 1)};
  if (w == 0) {
    // target bins, then the groups' offsets into each target's candidate list
    wave_locate<kCoarseBins>(L.hist, R, want, L);
    __builtin_amdgcn_wave_barrier();
    for (int tg = 0; tg < 2; ++tg) {
      if (!want[tg]) continue;
      const uint32_t c = lane < groups ? gcount(lane, L.bin[tg]) : 0u;
      uint32_t inc = c;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
      }
      if (lane <= groups) L.goff[tg][lane] = inc - c;
    }
  }
  __syncthreads();
  uint32_t B[2], nc[2];
  for (int tg = 0; tg < 2; ++tg) {
    B[tg] = want[tg] ? L.bin[tg] : 0u;
    R[tg] = want[tg] ? L.rank[tg] : 0u;
    nc[tg] = want[tg] ? L.count[tg] : 0u;
  }
  // candidates of both targets into LDS (once when they share a bin)
  const bool same = want[0] && want[1] && B[0] == B[1];
  const bool fit[2] = {nc[0] <= (uint32_t)kCandCap,
                       same ? nc[0] <= (uint32_t)kCandCap
                            : nc[1] <= (uint32_t)kCandCap - (nc[0] <= (uint32_t)kCandCap ? nc[0] : 0u)};
  const uint32_t cbase[2] = {0u, same ? 0u : (fit[0] ? nc[0] : 0u)};
  auto cand_global = [&](int tg, uint32_t i) -> uint32_t {
    int lo_g = 0, hi_g = groups - 1;  // last group with goff <= i
    while (lo_g < hi_g) {
      const int mid = (lo_g + hi_g + 1) >> 1;
      if (L.goff[tg][mid] <= i) lo_g = mid;
      else hi_g = mid - 1;
    }
    return key_of(X[(int64_t)lo_g * kSampleWg + L.start[lo_g][B[tg]] + (i - L.goff[tg][lo_g])]);
  };
  {
    const uint32_t n0 = (want[0] && fit[0]) ? nc[0] : 0u;
    const uint32_t n1 = (want[1] && fit[1] && !same) ? nc[1] : 0u;
    for (uint32_t i = threadIdx.x; i < n0 + n1; i += kSelThreads) {
      const int tg = i < n0 ? 0 : 1;
      const uint32_t j = i < n0 ? i : i - n0;
      L.cand[cbase[tg] + j] = cand_global(tg, j);
    }
  }
  __syncthreads();
  auto cand_at = [&](int tg, uint32_t i) -> uint32_t { return fit[tg] ? L.cand[cbase[tg] + i] : cand_global(tg, i); };
  // refine a crowded bin by histograms of the next (up to) 11 bits
  uint32_t prefix[2] = {B[0], B[1]};
  int shift[2] = {32 - kCoarseBits, 32 - kCoarseBits};
  for (int tg = 0; tg < 2; ++tg) {
    if (!want[tg]) continue;
    uint32_t nct = nc[tg];
    while (nct > (uint32_t)kSortCand && shift[tg] > 0) {
      const int nb = shift[tg] < 11 ? shift[tg] : 11;
      const int sh = shift[tg] - nb;
      for (int i = threadIdx.x; i < kFineBins; i += kSelThreads) L.hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < nc[tg]; i += kSelThreads) {
        const uint32_t kk = cand_at(tg, i);
        if ((kk >> shift[tg]) == prefix[tg]) atomicAdd(&L.hist[(kk >> sh) & ((1u << nb) - 1u)], 1u);
      }
      __syncthreads();
      const uint32_t Rq[2] = {R[tg], 0u};
      const bool wq[2] = {true, false};
      if (w == 0) wave_locate<kFineBins>(L.hist, Rq, wq, L);
      __syncthreads();
      prefix[tg] = (prefix[tg] << nb) | L.bin[0];
      R[tg] = L.rank[0];
      nct = L.count[0];
      shift[tg] = sh;
      __syncthreads();
    }
  }
  // the keys sharing each target's final prefix (at most kSortCand), sorted
  // by one wave; both targets share the sort when their prefixes agree
  const bool live[2] = {want[0] && shift[0] > 0, want[1] && shift[1] > 0};
  const bool share = live[0] && live[1] && shift[0] == shift[1] && prefix[0] == prefix[1];
  if (threadIdx.x < 2) L.nfin[threadIdx.x] = 0u;
  __syncthreads();
  for (int tg = 0; tg < 2; ++tg) {
    if (!live[tg] || (tg == 1 && share)) continue;
    for (uint32_t i = threadIdx.x; i < nc[tg]; i += kSelThreads) {
      const uint32_t kk = cand_at(tg, i);
      if ((kk >> shift[tg]) == prefix[tg]) L.fin[tg][atomicAdd(&L.nfin[tg], 1u)] = kk;  // <= kSortCand
    }
  }
  __syncthreads();
  if (w < 2 && live[w]) {
    const int src = (w == 1 && share) ? 0 : w;
    const int nf = (int)L.nfin[src];
    const uint32_t *f = L.fin[src];
    if (nf <= 64) wave_sort_pick<1>(f, nf, R[w], &L.result[w]);
    else if (nf <= 128) wave_sort_pick<2>(f, nf, R[w], &L.result[w]);
    else if (nf <= 256) wave_sort_pick<4>(f, nf, R[w], &L.result[w]);
    else if (nf <= 512) wave_sort_pick<8>(f, nf, R[w], &L.result[w]);
    else wave_sort_pick<16>(f, nf, R[w], &L.result[w]);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t r0 = live[0] ? L.result[0] : prefix[0];
    const uint32_t r1 = live[1] ? L.result[1] : prefix[1];
    st[row].a_lo = want[0] ? (double)value_of(r0) : -INFINITY;
    st[row].a_hi = want[1] ? (double)value_of(r1) : INFINITY;
  }
}

hipError_t launch_select(const float *samples, const uint16_t *starts, int64_t rows, int64_t m, int64_t lo,
                         int64_t hi, RowState *st, hipStream_t s) {
  if (sample_groups(m) <= kSelMaxGroups) {
    hipLaunchKernelGGL(select_bucket_kernel, rows_grid(1u, rows), dim3(kSelThreads), 0, s, samples, starts, rows,
                       sample_groups(m), m, lo, hi, st);
    return hipGetLastError();
  }
  // the kernel's dynamic LDS exceeds the default limit: raise it once per
  // device (the attribute is set on the current device)
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> attr_set[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const size_t lds = sizeof(SelectLds);
  if (dev < 0 || dev >= kMaxDevices || !attr_set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute((const void *)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(select_kernel, rows_grid(1u, rows), dim3(kSelThreads), lds, s, samples, rows, m, lo, hi, st);
  return hipGetLastError();
}

// --------------------------------------------------------- stream & filter
LDEV uint32_t mbcnt64(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// One coalesced pass over the row.  A score below a_L (the bulk of the row
// when k is small) costs one compare, its lower-tail term and a masked add.
// Scores at or above a_L are rare: a wave takes a uniform branch only for a
// group of elements that holds one, counts them from the ballot, adds the
// upper-tail terms of those at or above a_R and appends the band keys to
// this block's own slot (positions reserved by an LDS counter, one LDS atomic
// per wave and group).  The tail sums, the count at or above a_L and the band
// key range go to the block's partial.  No global atomics: the band solve
// adds the partials in a fixed order, derives the counts below a_L and above
// a_R and turns the slot counts into offsets (filter_totals).
template <bool CHECK>
LDEV void filter_items(const float (&x)[4 * kUnroll], const bool (&ok)[4 * kUnroll], float aL, float aR, float cf,
                       double &sl, double &sr, unsigned long long &cnl, uint32_t &kmn, uint32_t &kmx,
                       uint32_t *slot, uint32_t &lcount) {
  float fl = 0.0f, fr = 0.0f;
#pragma unroll
  for (int q = 0; q < 4 * kUnroll; ++q) {
    const bool valid = !CHECK || ok[q];
    const bool lo = valid && x[q] < aL;
    const float w = __builtin_amdgcn_exp2f((x[q] - aL) * cf);  // used only below a_L, where it is <= 1
    fl += lo ? w : 0.0f;
    const unsigned long long nl = __ballot(valid && !lo);
    if (nl) {  // wave-uniform: some lane holds a score at or above a_L at position q
      cnl += (unsigned long long)__popcll(nl);
      const bool hi = valid && x[q] >= aR;
      if (hi) fr += __builtin_amdgcn_exp2f((aR - x[q]) * cf);
      const unsigned long long mq = nl & ~__ballot(hi);
      if (mq) {  // band keys
        uint32_t base = 0u;
        if (lane_id() == __ffsll((long long)mq) - 1) base = atomicAdd(&lcount, (uint32_t)__popcll(mq));
        base = __shfl(base, __ffsll((long long)mq) - 1, kWave);
        if ((mq >> lane_id()) & 1ull) {
          const uint32_t pos = base + mbcnt64(mq);
          const uint32_t kk = key_of(x[q]);
          if (pos < (uint32_t)kBandSlot) slot[pos] = kk;  // beyond the slot: counted, row falls back
          kmn = min(kmn, kk);
          kmx = max(kmx, kk);
        }
      }
    }
  }
  sl += (double)fl;
  sr += (double)fr;
}

__global__ __launch_bounds__(kStreamThreads) void filter_kernel(const float *__restrict__ r, int64_t n,
                                                                const RowState *__restrict__ st,
                                                                uint32_t *__restrict__ slots,
                                                                FilterPartial *__restrict__ part, int gx, double t,
                                                                int64_t rows, int per_row) {
  __shared__ double lds_d[2 * kStreamThreads / kWave];
  __shared__ unsigned long long lds_c[kStreamThreads / kWave];
  __shared__ uint32_t lds_k[2 * kStreamThreads / kWave];
  __shared__ uint32_t lcount;
  lds_poison(lds_d);
  lds_poison(lds_c);
  lds_poison(lds_k);
  lds_poison(lcount);
  const int64_t row = grid_row();
  if (row >= rows) return;
  const RowState &S = st[row];
  if (threadIdx.x == 0) lcount = 0u;
  __syncthreads();
  const float aL = (float)S.a_lo, aR = (float)S.a_hi;
  const float cf = per_row ? S.cf : (float)(kLog2e / t);
  const float *rr = r + row * n;
  uint32_t *slot = slots + ((int64_t)row * gx + blockIdx.x) * kBandSlot;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  double sl = 0.0, sr = 0.0;
  unsigned long long cnl = 0;  // wave-uniform
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;

  typedef float f4 __attribute__((ext_vector_type(4)));
  const bool vec = (n & 3) == 0 && (((uintptr_t)r & 15u) == 0);
  const int64_t nitems = vec ? (n >> 2) : n;
  bool ok[4 * kUnroll];
  float x[4 * kUnroll];
  // kUnroll items (16 B each on the vector path) per thread and iteration,
  // all loads issued before any is used; whole waves of full iterations
  // skip the bounds checks
  const int lane = threadIdx.x & (kWave - 1);
  int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kUnroll + threadIdx.x;
  if (vec) {
    // the wave's last item of this iteration is i0 - lane + 63 + (kUnroll-1)*kStreamThreads
    for (; i0 - lane + (kWave - 1) + (kUnroll - 1) * kStreamThreads < nitems; i0 += stride * kUnroll) {
      f4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(rr) + i0 + u * kStreamThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        x[4 * u] = v[u].x;
        x[4 * u + 1] = v[u].y;
        x[4 * u + 2] = v[u].z;
        x[4 * u + 3] = v[u].w;
      }
      filter_items<false>(x, ok, aL, aR, cf, sl, sr, cnl, kmn, kmx, slot, lcount);
    }
  }
  // the rest (and every item of the scalar path), with bounds checks
  for (; i0 - lane < nitems; i0 += stride * kUnroll) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kStreamThreads;
      f4 v = {0.f, 0.f, 0.f, 0.f};
      const bool in = i < nitems;
      if (in) {
        if (vec) v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(rr) + i);
        else v.x = rr[i];
      }
      x[4 * u] = v.x;
      x[4 * u + 1] = v.y;
      x[4 * u + 2] = v.z;
      x[4 * u + 3] = v.w;
      ok[4 * u] = in;
      ok[4 * u + 1] = in && vec;
      ok[4 * u + 2] = in && vec;
      ok[4 * u + 3] = in && vec;
    }
    filter_items<true>(x, ok, aL, aR, cf, sl, sr, cnl, kmn, kmx, slot, lcount);
  }

  // block reduction (fixed order); cnl is already per wave
#pragma unroll
  for (int msk = 1; msk < kWave; msk <<= 1) {
    sl += __shfl_xor(sl, msk, kWave);
    sr += __shfl_xor(sr, msk, kWave);
    kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, msk, kWave));
    kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, msk, kWave));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds_d[2 * w] = sl;
    lds_d[2 * w + 1] = sr;
    lds_c[w] = cnl;
    lds_k[2 * w] = kmn;
    lds_k[2 * w + 1] = kmx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    FilterPartial fp;
    fp.sl = 0.0;
    fp.sr = 0.0;
    fp.cnl = 0;
    fp.kmn = 0xFFFFFFFFu;
    fp.kmx = 0u;
    for (int i = 0; i < kStreamThreads / kWave; ++i) {
      fp.sl += lds_d[2 * i];
      fp.sr += lds_d[2 * i + 1];
      fp.cnl += lds_c[i];
      fp.kmn = min(fp.kmn, lds_k[2 * i]);
      fp.kmx = max(fp.kmx, lds_k[2 * i + 1]);
    }
    fp.cnt = lcount;
    fp.pad = 0u;
    part[row * gx + blockIdx.x] = fp;
  }
}

// Filter workgroups per row: about 1024 over all rows, but never fewer than
// 2 cap / kBandSlot per row (when the row has that many vector groups), so
// the workgroups' slots hold twice the band capacity (six times the expected
// band) and a band that fits its capacity does not overflow a slot unless
// its keys crowd into a few workgroups' chunks of the row.
int filter_grid_x(int64_t rows, int64_t n, int64_t cap) {
  const int64_t per_row_need = (n / 4 + kStreamThreads * kUnroll - 1) / (kStreamThreads * kUnroll);
  int64_t target = 1024 / (rows > 0 ? rows : 1);
  const int64_t slots_need = (2 * cap + kBandSlot - 1) / kBandSlot;
  if (target < slots_need) target = slots_need;
  if (target > kMaxFilterBlocks) target = kMaxFilterBlocks;
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
                         void *partials, int grid_x, bool per_row, hipStream_t s) {
  hipLaunchKernelGGL(filter_kernel, rows_grid((unsigned)grid_x, rows), dim3(kStreamThreads), 0, s, r, n, st, slots,
                     reinterpret_cast<FilterPartial *>(partials), grid_x, t, rows, per_row ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lapsum
