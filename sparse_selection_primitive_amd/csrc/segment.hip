// Large-row full-sort solver ("Fast LapSum: Exact Differentiable Top-k at
// Million Scale", section 2.2, full-sort solver) for rows that do not fit one
// workgroup's registers: the full-sort path and the bracketing fallback.
//
//   sort:  least-significant-digit radix sort of the order-preserving keys,
//          8-bit digits; per pass a tile histogram, a per-digit scan over
//          tiles, and a stable scatter (wave-ballot ranking inside the tile,
//          LDS staging, coalesced runs per digit);
//   curve: per-tile anchored aggregates of the sorted keys, then per row a
//          scan of the tile aggregates (seeded with the bracket's tail sums),
//          the threshold curve at tile ends, the balancing tile, the curve at
//          every knot inside it, and the closed-form root.
//
// Full-sort rows run one regular launch per phase (a kernel boundary is the
// cheapest grid-wide synchronisation on this GPU, far below a cooperative
// launch or an in-kernel grid barrier).  The bracketing fallback
// (fallback_row) instead sorts and solves a whole row inside one workgroup,
// at the end of the band kernel of that row: when every bracket held it costs
// nothing; on a miss it is slower but exact and deterministic.
#include "segment_dev.hpp"

namespace lapsum {

size_t tile_agg_bytes() { return sizeof(TileAgg); }
size_t pre_bytes() { return sizeof(Pre); }
size_t suf_bytes() { return sizeof(Suf); }

// --------------------------------------------- multi-launch kernels (256)
constexpr int kNT = kSegThreads;

__global__ __launch_bounds__(kNT) void seg_hist_kernel(SegArgs a, int pass) {
  __shared__ uint32_t h[256];
  const int row = blockIdx.y, tile = blockIdx.x;
  const int64_t len = seg_len(a, row);
  if ((int64_t)tile * kTile >= len) return;
  const int shift = 8 * pass;
  h[threadIdx.x] = 0u;
  __syncthreads();
  for (int q = 0; q < kKpt; ++q) {
    const int64_t gi = (int64_t)tile * kTile + q * kNT + threadIdx.x;
    if (gi < len) atomicAdd(&h[(load_key(a, pass, row, gi) >> shift) & 255u], 1u);
  }
  __syncthreads();
  a.hist[((int64_t)row * 256 + threadIdx.x) * a.max_tiles + tile] = h[threadIdx.x];
}

// one wave per (row, digit): exclusive scan over the row's tiles, in place
__global__ __launch_bounds__(kNT) void seg_scan_kernel(SegArgs a, int pass) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int row = blockIdx.y, d = blockIdx.x * (kNT / kWave) + w;
  const int64_t len = seg_len(a, row);
  const int nt = (int)((len + kTile - 1) / kTile);
  if (nt == 0) return;
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

__global__ __launch_bounds__(kNT) void seg_scatter_kernel(SegArgs a, int pass) {
  __shared__ RankLds<kNT> L;
  const int row = blockIdx.y, tile = blockIdx.x;
  const int64_t len = seg_len(a, row);
  if ((int64_t)tile * kTile >= len) return;
  const int shift = 8 * pass;
  uint32_t key[kKpt];
  int dig[kKpt];
  load_tile<kNT>(a, pass, row, (int64_t)tile * kTile, len, shift, key, dig);
  // global start of each digit in this row, plus this tile's offset within it
  const uint32_t dtot = a.dtot[(int64_t)row * 256 + threadIdx.x];
  const uint32_t dbase = wg_excl_scan<kNT>(dtot, L.wsum);
  const uint32_t tofs = a.hist[((int64_t)row * 256 + threadIdx.x) * a.max_tiles + tile];
  const int vc = (int)min((int64_t)kTile, len - (int64_t)tile * kTile);
  scatter_tile<kNT>(key, dig, shift, vc, dbase + tofs, pass_dst(a, pass) + (int64_t)row * a.stride, L);
}

__global__ __launch_bounds__(kNT) void seg_tiles_kernel(SegArgs a) {
  __shared__ BlockTeamLds<kNT, 1> lds;
  BlockTeam<kNT, 1> team(&lds);
  const int row = blockIdx.y, tile = blockIdx.x;
  const int64_t len = seg_len(a, row);
  if ((int64_t)tile * kTile >= len) return;
  float s[kKpt];
  const int nv = load_sorted<kNT>(a, row, (int64_t)tile * kTile, len, s);
  tile_aggregate<kNT>(s, nv, a.c, a.cf, team, a.tagg + (int64_t)row * a.max_tiles + tile);
}

__global__ __launch_bounds__(kNT) void seg_locate_kernel(SegArgs a) {
  __shared__ BlockTeamLds<kNT, 1> lds;
  BlockTeam<kNT, 1> team(&lds);
  const int row = blockIdx.x;
  if (!seg_active(a, row)) return;
  locate_row<kNT>(a, row, team);
}

hipError_t launch_segment(const SegArgs &a, hipStream_t s) {
  const dim3 tiles((unsigned)a.max_tiles, (unsigned)a.rows);
  for (int pass = 0; pass < 4; ++pass) {
    hipLaunchKernelGGL(seg_hist_kernel, tiles, dim3(kNT), 0, s, a, pass);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(256 / (kNT / kWave), (unsigned)a.rows), dim3(kNT), 0, s, a, pass);
    hipLaunchKernelGGL(seg_scatter_kernel, tiles, dim3(kNT), 0, s, a, pass);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(seg_tiles_kernel, tiles, dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(seg_locate_kernel, dim3((unsigned)a.rows), dim3(kNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace lapsum
