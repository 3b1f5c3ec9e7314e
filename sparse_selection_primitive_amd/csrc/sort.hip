// Whole-row sort solver ("Fast LapSum: Exact Differentiable Top-k at Million
// Scale", section 2.2, Full-Sort Solver, taken literally): every score of the
// row is sorted, one stable prefix/suffix scan over the sorted row gives the
// threshold curve, an index lookup finds the interval where the budget
// balances and the root is taken there in closed form.  (The bucket path
// sorts only the balancing bucket; this path sorts everything, as the pages'
// solver does, and is the comparator the bracketing path is measured
// against.)
//
// Sort: least-significant-digit radix sort of the order-preserving uint32
// keys, four passes of 8-bit digits, each pass reduce-then-scan with no
// inter-workgroup waiting:
//   rsort_count_kernel    per tile of 4096 keys, the histogram of the pass's
//                         digit, stored digit-major [row][digit][tile]
//   rsort_scan_kernel     per (digit, row), the exclusive scan over the
//                         tiles in place, and the digit's total
//   rsort_scatter_kernel  per tile, its keys to their place: the start of
//                         the digit (scan of the 256 totals) plus the tile's
//                         offset inside the digit plus the key's stable rank
//                         inside the tile (ballot ranking, staged in LDS so
//                         that each digit's run is written contiguously)
// Solve over the sorted row (tiles of 16384 keys):
//   rsort_agg_kernel      anchored aggregates of each tile
//   rsort_locate_kernel   one workgroup per row: scan of the tile
//                         aggregates, the threshold curve at the tile ends,
//                         the balancing tile and the closed-form root in it
// The streaming apply of stream.hip then writes p.
//
// DFTopK midpoint (section 2.3): on the same sorted keys, the k-th and
// (k+1)-th largest scores are read off directly and the mass the Laplace
// kernel assigns at their midpoint is reduced over the row:
//   midpoint_pick_kernel, midpoint_mass_kernel, midpoint_total_kernel.
#include "segment_dev.hpp"

namespace lapsum {

constexpr int kSortNT = 256;
constexpr int kSortTile = kSortNT * kKpt;    // keys per sort tile (4096)
constexpr int kSolveNT = 1024;
constexpr int kSolveTile = kSolveNT * kKpt;  // keys per solve tile (16384)
constexpr int kSortPasses = 4;

// Key of tile position gi of a row on pass `pass`: pass 0 reads the scores
// themselves, later passes the previous pass's output.
LDEV uint32_t sort_key_at(const SortArgs &a, int pass, int64_t row, int64_t gi) {
  return pass == 0 ? key_of(a.r[row * a.n + gi]) : (pass & 1 ? a.A : a.B)[row * a.stride + gi];
}

// This thread's keys of tile `tile`: position tile*4096 + w*1024 + q*64 + lane
// for round q (the order the stable ranking of scatter_tile assumes); every
// load issued before any is used.
LDEV void load_sort_tile(const SortArgs &a, int pass, int64_t row, int64_t tile, uint32_t (&key)[kKpt],
                         int (&dig)[kKpt]) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int sh = 8 * pass;
  const int64_t base = tile * kSortTile + w * (kWave * kKpt) + lane;
#pragma unroll
  for (int q = 0; q < kKpt; ++q) {
    const int64_t gi = base + q * kWave;
    key[q] = sort_key_at(a, pass, row, gi < a.n ? gi : 0);
  }
#pragma unroll
  for (int q = 0; q < kKpt; ++q) {
    const bool valid = base + q * kWave < a.n;
    dig[q] = valid ? (int)((key[q] >> sh) & 255u) : 256;
  }
}

__global__ __launch_bounds__(kSortNT) void rsort_count_kernel(SortArgs a, int pass) {
  __shared__ uint32_t h[256];
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const int64_t tile = blockIdx.x;
  h[threadIdx.x] = 0u;  // kSortNT == 256
  uint32_t key[kKpt];
  int dig[kKpt];
  load_sort_tile(a, pass, row, tile, key, dig);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kKpt; ++q)
    if (dig[q] < 256) atomicAdd(&h[dig[q]], 1u);
  __syncthreads();
  a.cnt[(row * 256 + threadIdx.x) * (int64_t)a.ntiles + tile] = h[threadIdx.x];
}

// One workgroup per (digit, row): exclusive scan of the digit's counts over
// the row's tiles, 16 consecutive counts per thread and round.
__global__ __launch_bounds__(kSortNT) void rsort_scan_kernel(SortArgs a) {
  __shared__ uint32_t wsum[kSortNT / kWave];
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const int d = blockIdx.x;
  uint32_t *c = a.cnt + (row * 256 + d) * (int64_t)a.ntiles;
  uint32_t carry = 0u;
  for (int t0 = 0; t0 < a.ntiles; t0 += kSortNT * kKpt) {
    const int b0 = t0 + threadIdx.x * kKpt;
    uint32_t v[kKpt];
    uint32_t sum = 0u;
#pragma unroll
    for (int q = 0; q < kKpt; ++q) {
      v[q] = b0 + q < a.ntiles ? c[b0 + q] : 0u;
      sum += v[q];
    }
    uint32_t run = carry + wg_excl_scan<kSortNT>(sum, wsum);
#pragma unroll
    for (int q = 0; q < kKpt; ++q) {
      if (b0 + q < a.ntiles) c[b0 + q] = run;
      run += v[q];
    }
    // the round's total: the last thread's running sum, shared through LDS
    __syncthreads();
    if (threadIdx.x == kSortNT - 1) wsum[0] = run;
    __syncthreads();
    carry = wsum[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dtot[row * 256 + d] = carry;
}

__global__ __launch_bounds__(kSortNT) void rsort_scatter_kernel(SortArgs a, int pass) {
  __shared__ RankLds<kSortNT> L;
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const int64_t tile = blockIdx.x;
  uint32_t key[kKpt];
  int dig[kKpt];
  load_sort_tile(a, pass, row, tile, key, dig);
  // thread d: where this tile's keys of digit d start in the output row
  const int d = threadIdx.x;
  const uint32_t tot = a.dtot[row * 256 + d];
  const uint32_t inside = a.cnt[(row * 256 + d) * (int64_t)a.ntiles + tile];
  const uint32_t dstart = wg_excl_scan<kSortNT>(tot, L.wsum);
  uint32_t *dst = (pass & 1 ? a.B : a.A) + row * a.stride;
  const int vc = (int)min((int64_t)kSortTile, a.n - tile * kSortTile);
  scatter_tile<kSortNT>(key, dig, 8 * pass, vc, dstart + inside, dst, L);
}

// Anchored aggregates of every solve tile of the sorted row (in B).
__global__ __launch_bounds__(kSolveNT) void rsort_agg_kernel(SortArgs a) {
  __shared__ BlockTeamLds<kSolveNT, 1> lds;
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  double k = a.k, t = a.t;
  row_params(a.rp.k, a.rp.t, row, a.n, k, t);
  const double c = kLog2e / t;
  BlockTeam<kSolveNT, 1> team(&lds);
  float s[kKpt];
  const int nv = load_sorted_at<kSolveNT>(a.B + row * a.stride, (int64_t)blockIdx.x * kSolveTile, a.n, 0u, s);
  tile_aggregate<kSolveNT>(s, nv, c, (float)c, team, a.ta + row * a.nst + blockIdx.x);
}

// One workgroup per row: locate over the tile aggregates and the root.
__global__ __launch_bounds__(kSolveNT) void rsort_locate_kernel(SortArgs a) {
  __shared__ BlockTeamLds<kSolveNT, 1> lds;
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  double k = a.k, t = a.t;
  const bool good = row_params(a.rp.k, a.rp.t, row, a.n, k, t);
  const double c = kLog2e / t;
  BlockTeam<kSolveNT, 1> team(&lds);
  const double b = locate_sorted<kSolveNT>(a.B + row * a.stride, a.n, 0u, Pre{0.0f, 0.0}, Suf{0.0f, 0.0}, 0.0,
                                           true, true, a.ta + row * a.nst, a.tp + row * a.nst,
                                           a.ts + row * a.nst, k, t, c, (float)c, team);
  if (threadIdx.x == 0) a.st[row].b = good ? b : __builtin_nan("");
}

hipError_t launch_row_sort(const SortArgs &a, hipStream_t s) {
  const dim3 tiles = rows_grid((unsigned)a.ntiles, a.rows);
  for (int pass = 0; pass < kSortPasses; ++pass) {
    hipLaunchKernelGGL(rsort_count_kernel, tiles, dim3(kSortNT), 0, s, a, pass);
    hipLaunchKernelGGL(rsort_scan_kernel, rows_grid(256u, a.rows), dim3(kSortNT), 0, s, a);
    hipLaunchKernelGGL(rsort_scatter_kernel, tiles, dim3(kSortNT), 0, s, a, pass);
  }
  return hipGetLastError();
}

hipError_t launch_row_sort_solve(const SortArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(rsort_agg_kernel, rows_grid((unsigned)a.nst, a.rows), dim3(kSolveNT), 0, s, a);
  hipLaunchKernelGGL(rsort_locate_kernel, rows_grid(1u, a.rows), dim3(kSolveNT), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------- DFTopK midpoint
// (after launch_row_sort: the row's keys ascending in B)
__global__ void midpoint_pick_kernel(SortArgs a, int64_t kk, double *b_mid) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= a.rows) return;
  const uint32_t *s = a.B + row * a.stride;
  // k-th largest = ascending position n - k, (k+1)-th = n - k - 1
  const double hi = (double)value_of(s[a.n - kk]), lo = (double)value_of(s[a.n - kk - 1]);
  b_mid[row] = 0.5 * (hi + lo);
}

struct MassPartial {
  double below, above;     // sums of e^{-|r - b|/t}/2 on either side
  unsigned long long cnt;  // scores above b
  unsigned long long pad;
};

// mass = #{r > b} + sum_{r <= b} e^{(r-b)/t}/2 - sum_{r > b} e^{-(r-b)/t}/2:
// an exact count plus two sums of small terms (each in [0, 1/2]).
__global__ __launch_bounds__(kSortNT) void midpoint_mass_kernel(const float *__restrict__ r, int64_t rows, int64_t n,
                                                               double t, const double *__restrict__ b_mid,
                                                               MassPartial *__restrict__ part) {
  __shared__ double lsum[2 * kSortNT / kWave];
  __shared__ unsigned long long lcnt[kSortNT / kWave];
  const int64_t row = grid_row();
  if (row >= rows) return;
  const double b = b_mid[row], c = kLog2e / t;
  const float *rr = r + row * n;
  double below = 0.0, above = 0.0;
  unsigned long long cnt = 0;
  for (int64_t i = (int64_t)blockIdx.x * kSortNT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kSortNT) {
    const double d = (double)rr[i] - b;
    const float h = 0.5f * __builtin_amdgcn_exp2f((float)(-fabs(d) * c));
    if (d > 0.0) {
      above += (double)h;
      ++cnt;
    } else {
      below += (double)h;
    }
  }
  below = wave_reduce(below, [](double x, double y) { return x + y; });
  above = wave_reduce(above, [](double x, double y) { return x + y; });
  cnt = wave_reduce(cnt, [](unsigned long long x, unsigned long long y) { return x + y; });
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lsum[2 * w] = below;
    lsum[2 * w + 1] = above;
    lcnt[w] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    MassPartial mp{0.0, 0.0, 0ull, 0ull};
    for (int i = 0; i < kSortNT / kWave; ++i) {
      mp.below += lsum[2 * i];
      mp.above += lsum[2 * i + 1];
      mp.cnt += lcnt[i];
    }
    part[row * gridDim.x + blockIdx.x] = mp;
  }
}

// One thread per row adds the row's partials in order.
__global__ void midpoint_total_kernel(const MassPartial *__restrict__ part, int64_t rows, int gx,
                                      double *__restrict__ mass) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  double below = 0.0, above = 0.0;
  unsigned long long cnt = 0;
  for (int i = 0; i < gx; ++i) {
    const MassPartial &mp = part[row * gx + i];
    below += mp.below;
    above += mp.above;
    cnt += mp.cnt;
  }
  mass[row] = ((double)cnt + below) - above;
}

int midpoint_grid_x(int64_t rows, int64_t n) {
  int64_t gx = (n + kSortNT * 16 - 1) / (kSortNT * 16);
  int64_t most = 2048 / (rows > 0 ? rows : 1);
  if (most < 1) most = 1;
  if (gx > most) gx = most;
  return (int)(gx < 1 ? 1 : gx);
}
size_t midpoint_partial_bytes(int64_t rows, int gx) { return sizeof(MassPartial) * (size_t)rows * (size_t)gx; }

hipError_t launch_midpoint(const SortArgs &a, int64_t kk, double *b_mid, double *mass, void *partials, int gx,
                           hipStream_t s) {
  const unsigned rg = (unsigned)((a.rows + 255) / 256);
  hipLaunchKernelGGL(midpoint_pick_kernel, dim3(rg), dim3(256), 0, s, a, kk, b_mid);
  MassPartial *part = reinterpret_cast<MassPartial *>(partials);
  hipLaunchKernelGGL(midpoint_mass_kernel, rows_grid((unsigned)gx, a.rows), dim3(kSortNT), 0, s, a.r, a.rows, a.n,
                     a.t, b_mid, part);
  hipLaunchKernelGGL(midpoint_total_kernel, dim3(rg), dim3(256), 0, s, part, a.rows, gx, mass);
  return hipGetLastError();
}

int sort_tiles(int64_t n) { return (int)((n + kSortTile - 1) / kSortTile); }
int solve_tiles(int64_t n) { return (int)((n + kSolveTile - 1) / kSolveTile); }
int64_t sort_stride(int64_t n) { return (n + kSolveTile - 1) / kSolveTile * kSolveTile; }

}  // namespace lapsum
