// Bucketed sort + solve ("Fast LapSum: Exact Differentiable Top-k at Million
// Scale", section 2.2) for key sets too large for one workgroup: the band of
// the probabilistic bracketing (step 3: the band is sorted and solved
// exactly, seeded with the tail sums; step 4: certification), and whole rows
// of the full-sort solver (full-row mode: the keys are read from the scores,
// a min/max pass first gives their range, and there is no bracket).
//
// The band keys lie in [kmin, kmax].  Bucket j holds the keys with
// (key - kmin) >> shift == j, shift the smallest value that leaves at most
// 2^bbits buckets (bbits chosen for about 32 keys per bucket, at most
// kBandBuckets buckets); every key of bucket j is below every key of bucket
// j + 1 (one most-significant-digit radix pass).  The anchored sums of a
// bucket need only its smallest and largest key, so no bucket is sorted but
// the one that holds the root.
//
//   band_minmax_kernel   (full-row mode) key range of each workgroup's chunk
//   band_count_kernel    bucket counts and key extremes of each workgroup's
//                        filter slots or chunk
//   band_scan_kernel     per bucket, offsets of the workgroups inside it
//                        and its size (band mode; band_scan_full_kernel for
//                        whole rows, with many more workgroups, also the
//                        bucket's key extremes)
//   band_scatter_kernel  keys to their bucket (order inside a bucket free)
//   band_agg_*_kernel    anchored sums of every bucket, order-free: by
//                        buckets (band mode) or by key ranges (full-row
//                        mode, where crowded buckets must be shared)
//   band_locate_kernel   scan of the bucket aggregates between the tail
//                        seeds, threshold curve at the bucket ends, the
//                        balancing bucket, its sort (or nested bucket
//                        selection when crowded) and the root inside it,
//                        certification, and the widening or exact fallback
//                        of a row whose bracket missed
//
// Whole rows of at least kNestedMinN scores bucket a crowded balancing
// bucket (the key bits of a row spread over binades can put millions of
// scores in one) a second time with the same kernels, every workgroup
// taking part: the first locate records the bucket and everything around
// it in the row state, and the second level reads that bucket's keys.
//
// Every count is an integer, the bucket sums are fixed-point integer sums,
// and the balancing bucket is sorted before anything is summed over it in
// order, so the result does not depend on the order in which the scatter
// placed keys inside a bucket.
#include <limits.h>

#include "bucket_dev.hpp"
#include "filter_dev.hpp"
#include "widen_dev.hpp"

namespace lapsum {

constexpr int kBT = 256;                   // threads per workgroup of every band kernel
constexpr int kBPT = kBandBuckets / kBT;   // buckets per thread in the per-row scans
constexpr int kWaveBucket = 16 * kWave;    // largest balancing bucket one wave sorts
static_assert(kBPT * kBT == kBandBuckets, "bucket count must be a multiple of the workgroup size");

// A row takes part in a launch unless its band overflowed (it then takes
// the fallback), and only if its flags hold the launch's `need` bits (the
// second level of whole rows: a crowded balancing bucket; the whole-row
// solve after the band kernels: a missed bracket).
LDEV bool band_active(const BandArgs &a, const RowState &S) {
  return (a.need == 0 || (S.flags & a.need) != 0) && !(S.flags & LAPSUM_FLAG_OVERFLOW);
}
// Launches restricted to flagged rows check the row first, before any load.
LDEV bool band_skip(const BandArgs &a, const RowState &S) { return a.need != 0 && !band_active(a, S); }

// Count/scatter workgroups that take part for a row: all of them, or on the
// second level one per kSetChunk keys of the crowded bucket (the others
// return at once; the scan reads only the records of those that took part).
constexpr int64_t kSetChunk = 8192;
LDEV int row_blocks(const BandArgs &a, const RowState &S) {
  if (a.src2 == nullptr) return a.nblk;
  const int64_t want = ((int64_t)S.band + kSetChunk - 1) / kSetChunk;
  return (int)min(max(want, (int64_t)1), (int64_t)a.nblk);
}

// Budget, temperature and c = log2(e)/t of one row: the call's, or (with
// per-row values, full-row mode) the row's own as the per-call reset stored
// them (both uniform over the workgroup, so they stay in scalar registers).
LDEV void band_row_params(const BandArgs &a, const RowState &S, double &k, double &t, double &c, float &cf) {
  const bool pr = a.rp.any();
  k = pr ? S.k : a.k;
  t = pr ? S.t : a.t;
  c = pr ? S.c : a.c;
  cf = pr ? S.cf : a.cf;
}

LDEV int band_shift(const RowState &S, int bbits) {
  const uint32_t span = (S.band > 1 && S.kmax > S.kmin) ? S.kmax - S.kmin : 0u;
  const int bits = span == 0u ? 0 : 32 - __clz((int)span);
  return max(bits - bbits, 0);
}

// Workgroups go to the eight XCDs in turn (linear id mod 8), each XCD with
// an L2 of its own.  Renumbered so that consecutive (row, chunk) pairs share
// an XCD, the partial-line key writes of one row (and their later reads)
// stay inside one L2 instead of being merged from eight.
// (Rows are folded over grid.y and grid.z; a renumbered row past the last
// one belongs to no row and its workgroup returns.)
constexpr int kXcds = 8;
LDEV int64_t xcd_linear() {
  const int64_t T = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t L = blockIdx.x + (int64_t)gridDim.x * grid_row();
  const int64_t x = L % kXcds, per = T / kXcds, rem = T % kXcds;
  return x * per + min(x, rem) + L / kXcds;
}
LDEV void xcd_tile(int64_t &row, int &blk) {
  const int64_t p = xcd_linear();
  row = p / gridDim.x;
  blk = (int)(p % gridDim.x);
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
// Keys of second-level workgroup `blk` (< row_blocks): an equal share of
// the crowded bucket (S.band keys from S.set0 in the first level's keys),
// kRowLoads loads per thread in flight (the bucket may start anywhere, so
// no vectors).
template <class F>
LDEV void for_each_set_key(const BandArgs &a, int64_t row, int blk, F &&f) {
  constexpr int kRowLoads = 8;
  const RowState &S = a.st[row];
  const int64_t len = (int64_t)S.band;
  const int nbr = row_blocks(a, S);
  const int64_t chunk = (len + nbr - 1) / nbr;
  const int64_t c0 = (int64_t)blk * chunk, c1 = min(len, c0 + chunk);
  const uint32_t *src = a.src2 + row * a.cap + S.set0;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += (int64_t)kBT * kRowLoads) {
    uint32_t v[kRowLoads];
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
      const int64_t ii = i + (int64_t)u * kBT;
      v[u] = ii < c1 ? src[ii] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u)
      if (i + (int64_t)u * kBT < c1) f(v[u]);
  }
}

// Scores of full-row workgroup `blk`: its chunk, 16 bytes per thread and
// step on the vector path.
template <class F>
LDEV void for_each_row_key(const BandArgs &a, int64_t row, int blk, F &&f) {
  if (a.src2 != nullptr) {
    for_each_set_key(a, row, blk, f);
    return;
  }
  typedef float f4 __attribute__((ext_vector_type(4)));
  const float *rr = a.r + row * a.n;
  const int64_t c0 = (int64_t)blk * a.chunk, c1 = min(a.n, c0 + a.chunk);
  const bool vec = (a.n & 3) == 0 && (((uintptr_t)a.r & 15u) == 0);
  if (vec) {
    // kRowLoads loads in flight per thread and round (the chunk is a
    // multiple of 4 long, so a vector that starts inside it ends inside it)
    constexpr int kRowLoads = 4;
    for (int64_t i = c0 + 4 * (int64_t)threadIdx.x; i < c1; i += 4 * kBT * kRowLoads) {
      f4 v[kRowLoads];
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) {
        const int64_t ii = i + (int64_t)u * 4 * kBT;
        // ordinary (temporal) loads: the min/max, count and scatter passes
        // read the same chunk, so a later pass may find it in cache
        v[u] = ii < c1 ? *reinterpret_cast<const f4 *>(rr + ii) : f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int u = 0; u < kRowLoads; ++u) {
        if (i + (int64_t)u * 4 * kBT < c1) {
          f(key_of(v[u].x));
          f(key_of(v[u].y));
          f(key_of(v[u].z));
          f(key_of(v[u].w));
        }
      }
    }
  } else {
    for (int64_t i = c0 + threadIdx.x; i < c1; i += kBT) f(key_of(rr[i]));
  }
}
template <class F>
LDEV void for_each_band_key(const BandArgs &a, int64_t row, int blk, const uint32_t *sb, F &&f) {
  if (a.r != nullptr) {
    for_each_row_key(a, row, blk, f);
    return;
  }
  // band mode: this workgroup's slots hold the band positions sb[0] ..
  // sb[ns]; thread t takes positions t, t + kBT, ... of that range, U at a
  // time, every load issued before any key is used (a slot's keys are a
  // contiguous run, so positions map to slots by the bounds in sb)
  constexpr int U = 8;
  const int s0 = blk * a.group, ns = min(a.gx - s0, a.group);
  const uint32_t first = sb[0], total = sb[ns] - first;
  const uint32_t *src = a.slots + (row * a.gx + s0) * (int64_t)kBandSlot;
  for (uint32_t f0 = 0; f0 < total; f0 += U * kBT) {
    // slot of this thread's first position: the last i with sb[i] <= it
    const uint32_t g0 = first + min(f0 + threadIdx.x, total - 1u);
    int sl = 0, hi = ns - 1;
    while (sl < hi) {
      const int mid = (sl + hi + 1) >> 1;
      if (sb[mid] <= g0) sl = mid;
      else hi = mid - 1;
    }
    uint32_t key[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t fi = f0 + u * kBT + threadIdx.x;
      const bool in = fi < total;
      const uint32_t g = first + fi;
      if (in)
        while (sb[sl + 1] <= g) ++sl;  // positions only grow with u
      key[u] = src[in ? (int64_t)sl * kBandSlot + (g - sb[sl]) : 0];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (f0 + u * kBT + threadIdx.x < total) f(key[u]);
  }
}

// full-row mode: key minimum and maximum of each workgroup's chunk
// The first launch of the spread fallback's whole-row solve: the rows the
// band kernels left flagged FALLBACK (their bracket missed or their band
// overflowed; a row with an invalid per-row k or t already holds b = NaN)
// take part, each in a state of its own (flagged, with the row's k and t)
// that its first workgroup writes; every other row's state is cleared.
LDEV bool spread_begin(const BandArgs &a, int64_t row) {
  const RowState &P = a.st_out[row];
  const bool missed = (P.flags & LAPSUM_FLAG_FALLBACK) && !(P.flags & LAPSUM_FLAG_INVALID);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (missed) {
      reset_row_state(a.st, row, kFlagDeferred, 0, 0.0, 0.0);
      RowState &D = a.st[row];
      D.k = P.k;
      D.t = P.t;
      D.c = P.c;
      D.cf = P.cf;
    } else {
      a.st[row].flags = 0;
    }
  }
  return missed;
}

__global__ __launch_bounds__(kBT) void band_minmax_kernel(BandArgs a) {
  __shared__ uint32_t lmn[kBT / kWave], lmx[kBT / kWave];
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  if (a.need == kFlagDeferred ? !spread_begin(a, row) : band_skip(a, a.st[row])) return;
  lds_poison(lmn);
  lds_poison(lmx);
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for_each_row_key(a, row, blockIdx.x, [&](uint32_t k) {
    mn = min(mn, k);
    mx = max(mx, k);
  });
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, m, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, kWave));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lmn[w] = mn;
    lmx[w] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < kBT / kWave; ++i) {
      mn = min(mn, lmn[i]);
      mx = max(mx, lmx[i]);
    }
    a.mm[(row * a.nblk + blockIdx.x) * 2] = mn;
    a.mm[(row * a.nblk + blockIdx.x) * 2 + 1] = mx;
  }
}

__global__ __launch_bounds__(kBT) void band_count_kernel(BandArgs a) {
  __shared__ uint32_t h[kBandBuckets], hmn[kBandBuckets], hmx[kBandBuckets];
  __shared__ uint32_t soffs[kMaxFilterBlocks + 1];
  __shared__ uint32_t rng[2];
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const int blk = blockIdx.x;
  RowState &S = a.st[row];
  if (band_skip(a, S) || blk >= row_blocks(a, S)) return;
  lds_poison(h);
  lds_poison(hmn);
  lds_poison(hmx);
  lds_poison(soffs);
  lds_poison(rng);
  const int nb = 1 << a.bbits;
  for (int j = threadIdx.x; j < nb; j += kBT) {
    h[j] = 0u;
    hmn[j] = 0xFFFFFFFFu;
    hmx[j] = 0u;
  }
  RowState R;  // the key range and count this workgroup buckets by
  const uint32_t *sb = soffs;
  if (a.src2 != nullptr) {
    // second level: the crowded bucket's extremes and size, recorded by the
    // first level's locate
    R.kmin = S.kmin;
    R.kmax = S.kmax;
    R.band = S.band;
  } else if (a.r != nullptr) {
    // full-row mode: the row's key range from the min/max partials; the
    // first workgroup records it (and the key count) for the later kernels
    if (threadIdx.x < kWave) {
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      for (int i = threadIdx.x; i < a.nblk; i += kWave) {
        mn = min(mn, a.mm[(row * a.nblk + i) * 2]);
        mx = max(mx, a.mm[(row * a.nblk + i) * 2 + 1]);
      }
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, m, kWave));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, m, kWave));
      }
      if (threadIdx.x == 0) {
        rng[0] = mn;
        rng[1] = mx;
        if (blk == 0) {
          S.kmin = mn;
          S.kmax = mx;
          S.band = (unsigned long long)a.n;
        }
      }
    }
    __syncthreads();
    R.kmin = rng[0];
    R.kmax = rng[1];
    R.band = (unsigned long long)a.n;
  } else {
    // band mode: the streaming filter's partials of the row, added by every
    // workgroup in the same fixed order; the first one records the totals
    // and the slot offsets for the later kernels
    const FilterTotals T = filter_totals<kBT>(a.part + row * a.gx, a.gx, a.n, a.cap, soffs);
    if (blk == 0) {
      if (threadIdx.x == 0) store_filter_totals(S, T);
      uint32_t *ro = a.offs + row * (int64_t)(a.gx + 1);
      for (int i = threadIdx.x; i <= a.gx; i += kBT) ro[i] = soffs[i];
    }
    if (T.overflow) return;  // the row takes the fallback
    R.kmin = T.kmin;
    R.kmax = T.kmax;
    R.band = T.band;
    sb = soffs + blk * a.group;
  }
  const uint32_t kmin = R.kmin;
  const int shift = band_shift(R, a.bbits);
  uint32_t *dst = a.hist + (row * a.nblk + blk) * (int64_t)kBandBuckets;
  if (a.r != nullptr) {
    // full-row mode: counts and key extremes of the buckets in this chunk
    for_each_band_key(a, row, blk, sb, [&](uint32_t key) {
      const uint32_t j = (key - kmin) >> shift;
      atomicAdd(&h[j], 1u);
      atomicMin(&hmn[j], key);
      atomicMax(&hmx[j], key);
    });
    __syncthreads();
    uint32_t *ext = a.hext + (row * a.nblk + blk) * (int64_t)(2 * kBandBuckets);
    for (int j = threadIdx.x; j < nb; j += kBT) {
      dst[j] = h[j];
      ext[j] = hmn[j];
      ext[kBandBuckets + j] = hmx[j];
    }
  } else {
    for_each_band_key(a, row, blk, sb, [&](uint32_t key) { atomicAdd(&h[(key - kmin) >> shift], 1u); });
    __syncthreads();
    for (int j = threadIdx.x; j < nb; j += kBT) dst[j] = h[j];
  }
}

// One thread per bucket (band mode, and whole rows of at most
// kBandCountBlocks count workgroups): exclusive scan over the count
// workgroups, in place, kBandCountBlocks counts at a time (each batch loaded
// before any of it is used); for whole rows the bucket's key extremes over
// the workgroups and its fixed-point sums cleared for the aggregate kernel
// to add into
__global__ __launch_bounds__(kBT) void band_scan_kernel(BandArgs a) {
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const int j = blockIdx.x * kBT + threadIdx.x;
  if (j >= (1 << a.bbits) || band_skip(a, a.st[row])) return;
  uint32_t *h = a.hist + row * a.nblk * (int64_t)kBandBuckets + j;
  const uint32_t *ext = a.hext + row * a.nblk * (int64_t)(2 * kBandBuckets) + j;
  uint32_t v[kBandCountBlocks];
#pragma unroll
  for (int b = 0; b < kBandCountBlocks; ++b) v[b] = b < a.nblk ? h[(int64_t)b * kBandBuckets] : 0u;
  if (!band_active(a, a.st[row])) return;
  uint32_t run = 0u;
  for (int b0 = 0; b0 < a.nblk; b0 += kBandCountBlocks) {
    if (b0 > 0) {
#pragma unroll
      for (int b = 0; b < kBandCountBlocks; ++b)
        v[b] = b0 + b < a.nblk ? h[(int64_t)(b0 + b) * kBandBuckets] : 0u;
    }
#pragma unroll
    for (int b = 0; b < kBandCountBlocks; ++b) {
      if (b0 + b < a.nblk) h[(int64_t)(b0 + b) * kBandBuckets] = run;
      run += v[b];
    }
  }
  const int64_t o = row * kBandBuckets + j;
  a.btot[o] = run;
  if (a.r == nullptr) return;
  // full-row mode: key extremes over the workgroups (an empty share holds
  // ~0 and 0), a batch of loads at a time
  constexpr int kExtBatch = 16;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
  for (int b0 = 0; b0 < a.nblk; b0 += kExtBatch) {
    uint32_t lo[kExtBatch], hi[kExtBatch];
#pragma unroll
    for (int b = 0; b < kExtBatch; ++b) {
      const bool in = b0 + b < a.nblk;
      lo[b] = in ? ext[(int64_t)(b0 + b) * (2 * kBandBuckets)] : 0xFFFFFFFFu;
      hi[b] = in ? ext[(int64_t)(b0 + b) * (2 * kBandBuckets) + kBandBuckets] : 0u;
    }
#pragma unroll
    for (int b = 0; b < kExtBatch; ++b) {
      kmn = min(kmn, lo[b]);
      kmx = max(kmx, hi[b]);
    }
  }
  a.bkey[2 * o] = kmn;
  a.bkey[2 * o + 1] = kmx;
  a.bsum[2 * o] = 0ull;
  a.bsum[2 * o + 1] = 0ull;
}

// Whole rows of more count workgroups (up to kFullCountBlocksMax), and the
// second level (its row_blocks vary by row): a workgroup per kWave
// consecutive buckets, lane = bucket, so every load is one
// coalesced row of the per-workgroup records; each of its waves takes a
// contiguous share of the count workgroups.  Pass 1 adds each lane's share
// and its key extremes (an empty share holds ~0 and 0), the shares are
// combined across the waves through LDS, pass 2 rewrites the counts as
// exclusive offsets; the bucket's size, key extremes and cleared
// fixed-point sums (for the aggregate kernel to add into) follow.
constexpr int kScanT = 1024;
constexpr int kScanW = kScanT / kWave;
constexpr int kScanBatch = 16;  // count workgroups per batch of loads in pass 1 (3 loads each)
constexpr int kOffBatch = 32;   // and in pass 2

__global__ __launch_bounds__(kScanT) void band_scan_full_kernel(BandArgs a) {
  __shared__ uint32_t wt[kScanW][kWave], wmn[kScanW][kWave], wmx[kScanW][kWave];
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const RowState &S = a.st[row];
  if (!band_active(a, S)) return;
  lds_poison(wt);
  lds_poison(wmn);
  lds_poison(wmx);
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int j = blockIdx.x * kWave + lane;
  const bool jin = j < (1 << a.bbits);
  const int nbr = row_blocks(a, S);
  const int per = (nbr + kScanW - 1) / kScanW;
  const int b0 = min(w * per, nbr), b1 = min(nbr, b0 + per);
  uint32_t *h = a.hist + row * a.nblk * (int64_t)kBandBuckets + j;
  const uint32_t *ext = a.hext + row * a.nblk * (int64_t)(2 * kBandBuckets) + j;
  uint32_t sum = 0u, mn = 0xFFFFFFFFu, mx = 0u;
  for (int c = b0; c < b1; c += kScanBatch) {
    uint32_t v[kScanBatch], lo[kScanBatch], hi[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const bool in = jin && c + u < b1;
      const int64_t q = (int64_t)(c + u);
      v[u] = in ? h[q * kBandBuckets] : 0u;
      lo[u] = in ? ext[q * (2 * kBandBuckets)] : 0xFFFFFFFFu;
      hi[u] = in ? ext[q * (2 * kBandBuckets) + kBandBuckets] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      sum += v[u];
      mn = min(mn, lo[u]);
      mx = max(mx, hi[u]);
    }
  }
  wt[w][lane] = sum;
  wmn[w][lane] = mn;
  wmx[w][lane] = mx;
  __syncthreads();
  uint32_t run = 0u, tot = 0u;
  for (int i = 0; i < kScanW; ++i) {
    const uint32_t x = wt[i][lane];
    run += i < w ? x : 0u;
    tot += x;
  }
  for (int c = b0; c < b1; c += kOffBatch) {
    uint32_t v[kOffBatch];
#pragma unroll
    for (int u = 0; u < kOffBatch; ++u) v[u] = jin && c + u < b1 ? h[(int64_t)(c + u) * kBandBuckets] : 0u;
#pragma unroll
    for (int u = 0; u < kOffBatch; ++u) {
      if (jin && c + u < b1) h[(int64_t)(c + u) * kBandBuckets] = run;
      run += v[u];
    }
  }
  if (w == 0 && jin) {
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for (int i = 0; i < kScanW; ++i) {
      kmn = min(kmn, wmn[i][lane]);
      kmx = max(kmx, wmx[i][lane]);
    }
    const int64_t o = row * kBandBuckets + j;
    a.btot[o] = tot;
    a.bkey[2 * o] = kmn;
    a.bkey[2 * o + 1] = kmx;
    a.bsum[2 * o] = 0ull;
    a.bsum[2 * o + 1] = 0ull;
  }
}

__global__ __launch_bounds__(kBT) void band_scatter_kernel(BandArgs a) {
  __shared__ uint32_t base[kBandBuckets];
  __shared__ uint32_t wsum[kBT / kWave];
  __shared__ uint32_t sb[kMaxGroup + 1];
  int64_t row;
  int blk;
  if (a.src2 != nullptr) {
    // second level: only the first row_blocks workgroups of a row take
    // part, so they keep the launch order (spread over every XCD)
    row = grid_row();
    blk = blockIdx.x;
  } else {
    xcd_tile(row, blk);
  }
  if (row >= a.rows) return;
  const RowState &S = a.st[row];
  if (band_skip(a, S) || blk >= row_blocks(a, S)) return;
  lds_poison(base);
  lds_poison(wsum);
  lds_poison(sb);
  // bucket sizes (thread i owns buckets i*kBPT ..), this workgroup's offset
  // inside each bucket and its slot bounds, all loaded before any is used
  const int64_t o = row * kBandBuckets;
  const uint32_t *hin = a.hist + (row * a.nblk + blk) * (int64_t)kBandBuckets;
  const int nb = 1 << a.bbits;
  uint32_t v[kBPT], hv[kBPT];
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int j = threadIdx.x * kBPT + u;
    v[u] = j < nb ? a.btot[o + j] : 0u;
    hv[u] = j < nb ? hin[j] : 0u;
  }
  if (a.r == nullptr) load_slot_bounds(a, row, blk, sb);
  if (!band_active(a, S)) return;
  const uint32_t kmin = S.kmin;
  const int shift = band_shift(S, a.bbits);
  uint32_t sum = 0u;
#pragma unroll
  for (int u = 0; u < kBPT; ++u) sum += v[u];
  uint32_t run = wg_excl_scan<kBT>(sum, wsum);
#pragma unroll
  for (int u = 0; u < kBPT; ++u) {
    const int j = threadIdx.x * kBPT + u;
    if (j < nb) {
      base[j] = run + hv[u];
      if (blk == 0) a.bstart[o + j] = run;
    }
    run += v[u];
  }
  __syncthreads();
  uint32_t *dst = a.keys + row * a.cap;
  for_each_band_key(a, row, blk, sb, [&](uint32_t key) {
    const uint32_t pos = atomicAdd(&base[(key - kmin) >> shift], 1u);
    dst[pos] = key;
  });
}

// ------------------------------------------------------ bucket aggregates
LDEV void write_agg(TileAgg *out, Pre p, Suf s) {
  out->aP = p.a;
  out->sP = p.s;
  out->aS = s.a;
  out->sS = s.s;
}

// The anchored sums of a bucket need its extreme keys, not its order: the
// P-type sum is anchored at the largest key, the S-type sum at the smallest,
// and every term e^{-|x - anchor|/t} lies in [0, 1].  Each term is added as
// a 64-bit fixed-point number with `fb` fraction bits, fb chosen from the
// bucket size so that the sum stays below 2^62.  Integer sums do not depend
// on the order in which the scatter left the keys, so the aggregates (and
// everything computed from them) are bitwise reproducible.  A term loses at
// most 2^-(fb+1) to the rounding; fb >= 30 for any bucket.

LDEV void agg_write(TileAgg *out, uint32_t kmx, uint32_t kmn, unsigned long long sp, unsigned long long ss, int fb) {
  write_agg(out, Pre{value_of(kmx), fixed_value(sp, fb)}, Suf{value_of(kmn), fixed_value(ss, fb)});
}

// A team of LANES lanes aggregates one bucket, kAggE keys per lane and
// round, the round's loads issued together (a bucket of one round keeps its
// keys in registers for the second pass).
constexpr int kAggE = 8;
template <int LANES>
LDEV void bucket_agg(const uint32_t *kb, int cnt, double c, TileAgg *out) {
  constexpr int R = kAggE * LANES;  // keys per round
  WaveTeam<LANES> team;
  uint32_t key[kAggE];
  uint32_t kmx = 0u, kmn = 0xFFFFFFFFu;
  for (int i0 = 0; i0 < cnt; i0 += R) {
#pragma unroll
    for (int e = 0; e < kAggE; ++e) {
      const int i = i0 + e * LANES + team.lane;
      key[e] = i < cnt ? kb[i] : 0u;
    }
#pragma unroll
    for (int e = 0; e < kAggE; ++e) {
      if (i0 + e * LANES + team.lane < cnt) {
        kmx = max(kmx, key[e]);
        kmn = min(kmn, key[e]);
      }
    }
  }
  kmx = team.umax(kmx);
  kmn = team.umin(kmn);
  const int fb = agg_frac_bits((uint32_t)cnt);
  const double hi = (double)value_of(kmx), lo = (double)value_of(kmn);
  unsigned long long sp = 0ull, ss = 0ull;
  const bool reload = cnt > R;
  for (int i0 = 0; i0 < cnt; i0 += R) {
    if (reload) {
#pragma unroll
      for (int e = 0; e < kAggE; ++e) {
        const int i = i0 + e * LANES + team.lane;
        key[e] = i < cnt ? kb[i] : 0u;
      }
    }
#pragma unroll
    for (int e = 0; e < kAggE; ++e) {
      if (i0 + e * LANES + team.lane < cnt) {
        const double x = (double)value_of(key[e]);
        sp += fixed_term(wexp(x - hi, c), fb);
        ss += fixed_term(wexp(lo - x, c), fb);
      }
    }
  }
  sp = team.sum(sp);
  ss = team.sum(ss);
  if (team.lane == 0) agg_write(out, kmx, kmn, sp, ss, fb);
}

// Band mode (a band's buckets hold a few dozen keys each): each workgroup
// owns kAggGroup consecutive buckets of one row, one per 16-lane team; a
// bucket of more than kAggTeamMax keys is left to a whole wave, the
// workgroup's large buckets dealt out to its waves in turn.
constexpr int kAggTeam = 16;
constexpr int kAggGroup = kBT / kAggTeam;
constexpr int kAggTeamMax = 4 * kAggE * kAggTeam;

__global__ __launch_bounds__(kBT) void band_agg_buckets_kernel(BandArgs a) {
  __shared__ uint32_t big;  // the workgroup's buckets too large for a team
  int64_t row;
  int blk;
  xcd_tile(row, blk);
  if (row >= a.rows) return;
  const RowState &S = a.st[row];
  const int64_t o = row * kBandBuckets;
  const int q = (int)threadIdx.x / kAggTeam;
  const int j = blk * kAggGroup + q;
  const int cnt = (int)a.btot[o + j];
  const uint32_t bst = a.bstart[o + j];
  if (!band_active(a, S)) return;
  lds_poison(big);
  const int shift = band_shift(S, a.bbits);
  const uint32_t *kb = a.keys + row * a.cap + bst;
  TileAgg *out = a.bagg + o + j;
  const int tl = threadIdx.x & (kAggTeam - 1);
  double rk, rt, c;
  float rcf;
  band_row_params(a, S, rk, rt, c, rcf);
  if (threadIdx.x == 0) big = 0u;
  __syncthreads();
  if (cnt == 0) {
    if (tl == 0) write_agg(out, Pre{0.0f, 0.0}, Suf{0.0f, 0.0});
  } else if (shift == 0) {
    // the bucket holds one distinct key
    if (tl == 0) {
      const float x = value_of(kb[0]);
      write_agg(out, Pre{x, (double)cnt}, Suf{x, (double)cnt});
    }
  } else if (cnt <= kAggTeamMax) {
    bucket_agg<kAggTeam>(kb, cnt, c, out);
  } else if (tl == 0) {
    atomicOr(&big, 1u << q);
  }
  __syncthreads();
  const int w = threadIdx.x / kWave;
  int i = 0;
  for (uint32_t m = big; m != 0u; m &= m - 1u, ++i) {
    if ((i & (kBT / kWave - 1)) != w) continue;
    const int jj = blk * kAggGroup + __ffs((int)m) - 1;
    bucket_agg<kWave>(a.keys + row * a.cap + a.bstart[o + jj], (int)a.btot[o + jj], c, a.bagg + o + jj);
  }
}

// Full-row mode: the key bits of a whole row can put millions of scores in
// one bucket, so the work is split by key ranges, not by buckets.  Each
// workgroup takes kAggChunk consecutive bucketed keys (a window of
// consecutive buckets; 16 consecutive keys per thread, whose terms are
// summed in registers over each run of one bucket), adds the runs into LDS
// sums of the window and each window sum into the bucket's global sums with
// one integer atomic.  The anchors are the bucket extremes the count and
// scan recorded; integer sums make the order of the adds irrelevant.
constexpr int kAggKeysPerThread = 16;
constexpr int kAggChunk = kBT * kAggKeysPerThread;

__global__ __launch_bounds__(kBT) void band_agg_keys_kernel(BandArgs a) {
  __shared__ unsigned long long sp[kBandBuckets], ss[kBandBuckets];
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const int64_t row = grid_row();
  if (row >= a.rows) return;
  const RowState &S = a.st[row];
  if (!band_active(a, S)) return;
  const int64_t M = a.src2 != nullptr ? (int64_t)S.band : a.n;
  const int64_t c0 = (int64_t)blockIdx.x * kAggChunk;
  if (c0 >= M) return;
  lds_poison(sp);
  lds_poison(ss);
  const int64_t c1 = min(M, c0 + (int64_t)kAggChunk);
  double rk, rt, c;
  float rcf;
  band_row_params(a, S, rk, rt, c, rcf);
  const uint32_t kmin = S.kmin;
  const int shift = band_shift(S, a.bbits);
  const uint32_t *kb = a.keys + row * a.cap;
  const int64_t o = row * kBandBuckets;
  // this thread's keys, loaded first (the row stride is a multiple of 4 keys)
  constexpr int E = kAggKeysPerThread;
  const int64_t t0 = c0 + (int64_t)threadIdx.x * E;
  uint32_t key[E];
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    const u4 v = t0 + 4 * q < c1 ? *reinterpret_cast<const u4 *>(kb + t0 + 4 * q) : u4{0u, 0u, 0u, 0u};
    key[4 * q] = v.x;
    key[4 * q + 1] = v.y;
    key[4 * q + 2] = v.z;
    key[4 * q + 3] = v.w;
  }
  // the keys are in bucket order: the window is first key's bucket .. last key's
  const uint32_t jf = (kb[c0] - kmin) >> shift, jl = (kb[c1 - 1] - kmin) >> shift;
  for (uint32_t j = jf + threadIdx.x; j <= jl; j += kBT) {
    sp[j - jf] = 0ull;
    ss[j - jf] = 0ull;
  }
  __syncthreads();
  const int nv = (int)max(min(c1 - t0, (int64_t)E), (int64_t)0);
  if (nv > 0) {
    uint32_t cj = (key[0] - kmin) >> shift;
    uint32_t kn = a.bkey[2 * (o + cj)], kx = a.bkey[2 * (o + cj) + 1];
    int fb = agg_frac_bits(a.btot[o + cj]);
    unsigned long long accp = 0ull, accs = 0ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e < nv) {
        const uint32_t j = (key[e] - kmin) >> shift;
        if (j != cj) {  // a new run: flush the last one
          atomicAdd(&sp[cj - jf], accp);
          atomicAdd(&ss[cj - jf], accs);
          accp = accs = 0ull;
          cj = j;
          kn = a.bkey[2 * (o + j)];
          kx = a.bkey[2 * (o + j) + 1];
          fb = agg_frac_bits(a.btot[o + j]);
        }
        const double x = (double)value_of(key[e]);
        accp += fixed_term(wexp(x - (double)value_of(kx), c), fb);
        accs += fixed_term(wexp((double)value_of(kn) - x, c), fb);
      }
    }
    atomicAdd(&sp[cj - jf], accp);
    atomicAdd(&ss[cj - jf], accs);
  }
  __syncthreads();
  for (uint32_t j = jf + threadIdx.x; j <= jl; j += kBT) {
    const unsigned long long p = sp[j - jf], q = ss[j - jf];
    if (p != 0ull) atomicAdd(&a.bsum[2 * (o + j)], p);
    if (q != 0ull) atomicAdd(&a.bsum[2 * (o + j) + 1], q);
  }
}

// ---------------------------------------------------------------- locate
// One workgroup per row: 1024 threads for whole rows (crowded buckets are
// common there), 512 for bands, where a bucket beyond one wave is rare: a
// thread then has 256 registers instead of 128, and the bucket search and
// the one-wave solve no longer spill.  Its first kLocScanT threads
// (two waves per SIMD) search the buckets, kLocPer consecutive buckets each:
// a scan of the bucket aggregates between the tail seeds (DPP inside waves,
// the wave totals through LDS), the threshold curve at the bucket ends and
// the balancing bucket.  Only that bucket is sorted: by one wave in
// registers when it holds at most 1024 keys, else by the whole workgroup
// (radix passes in place, then tile aggregates), and the root is taken
// inside it.  A row whose root falls outside its bracket (or whose band
// overflowed) is then widened or solved in full by the same workgroup, so no
// separate launch is needed; whole rows have no bracket and never take it.
constexpr int kLocScanT = 512;                     // threads of the bucket search
constexpr int kLocScanW = kLocScanT / kWave;
constexpr int kLocPer = kBandBuckets / kLocScanT;  // buckets per search thread
static_assert(kLocPer * kLocScanT == kBandBuckets, "every bucket has a search thread");
static_assert(kLocScanW <= 16, "wave totals are scanned inside one DPP row");

template <int NT>
union BandLocLds {
  BlockTeamLds<NT, 1> team;
  SegLds<NT> fb;
};

template <bool FULL, int NT = FULL ? 1024 : 512>
__global__ __launch_bounds__(NT) void band_locate_kernel(BandArgs a, SegArgs fb) {
  static_assert(NT >= kLocScanT, "the bucket search needs kLocScanT threads");
  __shared__ BandLocLds<NT> L;
  __shared__ double sel_b;
  __shared__ int sel_fb;
  const int64_t row = xcd_linear();
  if (row >= a.rows) return;
  RowState &S = a.st[row];
  if (band_skip(a, S)) return;  // a launch for flagged rows only
  lds_poison(L);
  lds_poison(sel_b);
  lds_poison(sel_fb);
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t o = row * kBandBuckets;
  // The bucket search runs on the first kLocScanW waves only (two per SIMD):
  // each of their threads owns kLocPer consecutive buckets.  This thread's
  // bucket records are loaded before the row state is examined.
  const int j0 = threadIdx.x * kLocPer;
  TileAgg g[kLocPer];
  uint32_t cnt[kLocPer];
  const int nb = 1 << a.bbits;
  if (a.r == nullptr) {
#pragma unroll
    for (int u = 0; u < kLocPer; ++u) {
      const bool in = threadIdx.x < kLocScanT && j0 + u < nb;
      g[u] = in ? a.bagg[o + j0 + u] : TileAgg{0.0f, 0.0f, 0.0, 0.0};
      cnt[u] = in ? a.btot[o + j0 + u] : 0u;
    }
  } else {
    // full-row mode: P-type sums anchored at the largest key, S-type at the
    // smallest, from the fixed-point sums
#pragma unroll
    for (int u = 0; u < kLocPer; ++u) {
      const bool in = threadIdx.x < kLocScanT && j0 + u < nb;
      const int64_t q = o + j0 + u;
      cnt[u] = in ? a.btot[q] : 0u;
      const int fb = cnt[u] > 0u ? agg_frac_bits(cnt[u]) : 0;
      g[u] = cnt[u] > 0u ? TileAgg{value_of(a.bkey[2 * q + 1]), value_of(a.bkey[2 * q]),
                                   fixed_value(a.bsum[2 * q], fb), fixed_value(a.bsum[2 * q + 1], fb)}
                         : TileAgg{0.0f, 0.0f, 0.0, 0.0};
    }
  }
  const bool active = band_active(a, S);
  if (threadIdx.x == 0) sel_fb = active ? 0 : 1;  // overflow: the row is already flagged for the fallback
  if (active) {
    double rk, rt, c;
    float rcf;
    band_row_params(a, S, rk, rt, c, rcf);
    const int64_t M = (int64_t)S.band;
    const Pre seed_lo{(float)S.a_lo, S.count_lo ? S.tail_lo : 0.0};
    const Suf seed_hi{(float)S.a_hi, S.count_hi ? S.tail_hi : 0.0};
    const double cR = (double)S.count_hi;
    const BucketPick P = bucket_search<NT, kLocScanT, kLocPer>(g, cnt, seed_lo, seed_hi, cR, M, rk, c);
    const int J = P.J;
    const int64_t cJ = P.cnt, sJ = P.start;
    const Pre slo{P.lo_a, P.lo_s};
    const Suf shi{P.hi_a, P.hi_s};
    const double cR_eff = (double)(M - sJ - cJ) + cR;
    uint32_t *kb = a.keys + row * a.cap + sJ;
    PartInfo part;
    part.nvalid = 0;
    part.above = (double)cJ + cR_eff;
    part.seed_lo = slo;
    part.seed_hi = shi;
    part.first = P.first != 0;
    part.last = P.last != 0;
    if (cJ <= (int64_t)kWaveBucket) {
      if (w == 0) {
        const double bb = cJ <= 4 * kWave ? wave_sort_solve<4>(kb, (int)cJ, part, rk, rt, c, rcf)
                                          : wave_sort_solve<16>(kb, (int)cJ, part, rk, rt, c, rcf);
        if (lane == 0) sel_b = bb;
      }
    } else if (cJ <= (int64_t)kFallbackSort || band_shift(S, a.bbits) == 0) {
      // a bucket of several tiles: sorted in place by the workgroup, its tile
      // aggregates, then locate over them
      const int shift = band_shift(S, a.bbits);
      const double bb = sorted_range_solve<NT>(
          kb, a.tmp + row * a.cap + sJ, cJ, S.kmin + ((uint32_t)J << shift), shift, slo, shi, cR_eff, part.first,
          part.last, a.tagg + row * a.max_tiles, a.tpre + row * a.max_tiles, a.tsuf + row * a.max_tiles, rk, rt,
          c, rcf, L.fb);
      if (threadIdx.x == 0) sel_b = bb;
    } else if (FULL && a.nested) {
      // a crowded bucket of a whole row, left to the second bucket level:
      // its place, size and exact key extremes, and everything around it
      // (the first level has no seeds, so the keys below it are sJ of the
      // row's scores) into the row state
      __syncthreads();  // every thread has read the state the search used
      if (threadIdx.x == 0) {
        S.set0 = sJ;
        S.band = (unsigned long long)cJ;
        S.kmin = a.bkey[2 * (o + J)];
        S.kmax = a.bkey[2 * (o + J) + 1];
        S.a_lo = (double)slo.a;
        S.tail_lo = slo.s;
        S.count_lo = (unsigned long long)sJ;
        S.a_hi = (double)shi.a;
        S.tail_hi = shi.s;
        S.count_hi = (unsigned long long)cR_eff;
        S.flags |= kFlagNested;
      }
      return;
    } else {
      // a crowded bucket (the key bits of a whole row spread values over
      // binades, so one bucket can hold millions of keys): the nested bucket
      // selection of the fallback on its keys, seeded with everything around
      // it; gathers go to the scratch keys, then alternate with this row's
      // bucketed keys (the bucket is read only by the first gather)
      const int shift = band_shift(S, a.bbits);
      const uint32_t kb0 = S.kmin + ((uint32_t)J << shift);
      SegArgs sub = fb;
      sub.A = a.tmp;
      sub.B = a.keys;
      sub.stride = a.cap;
      sub.max_tiles = a.max_tiles;
      sub.tagg = a.tagg;
      sub.tpre = a.tpre;
      sub.tsuf = a.tsuf;
      sub.st = a.st;
      sub.k = rk;
      sub.t = rt;
      sub.c = c;
      sub.cf = rcf;
      const uint64_t top = (uint64_t)kb0 + ((1ull << shift) - 1ull);  // the bucket's key bound
      const uint32_t kb1 = top < (uint64_t)S.kmax ? (uint32_t)top : S.kmax;
      const double bb = bucket_set_solve<NT>(sub, (int)row, kb, cJ, 0, kb0, kb1, slo, shi, cR_eff, L.fb);
      if (threadIdx.x == 0) sel_b = bb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const double bb = (S.flags & LAPSUM_FLAG_INVALID) ? __builtin_nan("") : sel_b;
      S.b = bb;
      if (a.st_out != nullptr) a.st_out[row].b = bb;
      if (FULL && a.src2 != nullptr) {
        // second level done: the row state describes the whole row again
        S.a_lo = -INFINITY;
        S.a_hi = INFINITY;
        S.tail_lo = S.tail_hi = 0.0;
        S.count_lo = S.count_hi = 0ull;
        S.band = (unsigned long long)a.n;
        S.flags &= ~kFlagNested;
      }
      if (!FULL) {  // certification against the bracket
        const bool hit = (bb >= S.a_lo) && (bb < S.a_hi);
        S.flags |= hit ? LAPSUM_FLAG_HIT : LAPSUM_FLAG_FALLBACK;
        sel_fb = hit ? 0 : 1;
      }
    }
  }
  if constexpr (!FULL) {
    __syncthreads();
    if (sel_fb && !fb.defer) missed_row<NT>(fb, (int)row, L.fb);
  }
}

// Sizes of the records the host lays out in the workspace for the bucketed
// solve, the sorted-tile solve and the exact fallback.
size_t tile_agg_bytes() { return sizeof(TileAgg); }
size_t pre_bytes() { return sizeof(Pre); }
size_t suf_bytes() { return sizeof(Suf); }

int band_count_blocks(int gx, int *group) {
  const int nblk = gx < kBandCountBlocks ? gx : kBandCountBlocks;
  *group = (gx + nblk - 1) / nblk;
  return (gx + *group - 1) / *group;
}

int bucket_bits(int64_t keys) {
  int b = 4;
  while (b < kBandBucketBits && ((int64_t)32 << b) < keys) ++b;
  return b;
}

int full_count_blocks(int64_t n, int64_t *chunk) {
  // at least a tile per workgroup; up to kBandCountBlocks workgroups, more
  // for rows beyond 2^22 scores (a chunk of at most 2^16 scores each, so a
  // 1e8 row is bucketed by ~1500 workgroups instead of 64)
  int64_t nblk = (n + kTile - 1) / kTile;
  int64_t most = (n + kFullChunkMax - 1) / kFullChunkMax;
  if (most < kBandCountBlocks) most = kBandCountBlocks;
  if (most > kFullCountBlocksMax) most = kFullCountBlocksMax;
  if (nblk > most) nblk = most;
  if (nblk < 1) nblk = 1;
  int64_t c = (n + nblk - 1) / nblk;
  c = (c + 3) / 4 * 4;
  *chunk = c;
  return (int)((n + c - 1) / c);
}

// Whole rows of at least this many scores take the second bucket level: a
// crowded balancing bucket (more than kFallbackSort keys) is bucketed again
// by every count/scatter workgroup instead of one.  Its launches cost a few
// microseconds when no row needs them; shorter rows rarely crowd a bucket,
// and there one workgroup selects inside it.
constexpr int64_t kNestedMinN = (int64_t)1 << 22;

hipError_t launch_band_buckets(const BandArgs &a_in, const SegArgs &fb, hipStream_t s) {
  BandArgs a = a_in;
  a.src2 = nullptr;
  a.nested = a.r != nullptr && a.n >= kNestedMinN ? 1 : 0;
  const dim3 blk = rows_grid((unsigned)a.nblk, a.rows);
  if (a.r != nullptr) hipLaunchKernelGGL(band_minmax_kernel, blk, dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_count_kernel, blk, dim3(kBT), 0, s, a);
  const int nb = 1 << a.bbits;
  if (a.nblk > kBandCountBlocks)
    hipLaunchKernelGGL(band_scan_full_kernel, rows_grid((unsigned)((nb + kWave - 1) / kWave), a.rows), dim3(kScanT),
                       0, s, a);
  else
    hipLaunchKernelGGL(band_scan_kernel, rows_grid((unsigned)((nb + kBT - 1) / kBT), a.rows), dim3(kBT), 0, s, a);
  hipLaunchKernelGGL(band_scatter_kernel, blk, dim3(kBT), 0, s, a);
  const dim3 agg_keys = rows_grid((unsigned)((a.n + kAggChunk - 1) / kAggChunk), a.rows);
  if (a.r != nullptr)
    hipLaunchKernelGGL(band_agg_keys_kernel, agg_keys, dim3(kBT), 0, s, a);
  else
    hipLaunchKernelGGL(band_agg_buckets_kernel, rows_grid((unsigned)((nb + kAggGroup - 1) / kAggGroup), a.rows),
                       dim3(kBT), 0, s, a);
  if (a.r != nullptr)
    hipLaunchKernelGGL(band_locate_kernel<true>, rows_grid(1u, a.rows), dim3(1024), 0, s, a, fb);
  else
    hipLaunchKernelGGL(band_locate_kernel<false>, rows_grid(1u, a.rows), dim3(512), 0, s, a, fb);
  if (a.nested) {
    // second level over the crowded buckets the locate recorded: the first
    // level's bucketed keys are the input, its scratch the output, and the
    // bucket records are reused (rows without a crowded bucket return at once)
    BandArgs a2 = a;
    a2.nested = 0;
    a2.need = kFlagNested;
    a2.src2 = a.keys;
    a2.keys = a.tmp;
    a2.tmp = a.keys;
    a2.bbits = kBandBucketBits;
    const int nb2 = 1 << a2.bbits;
    hipLaunchKernelGGL(band_count_kernel, blk, dim3(kBT), 0, s, a2);
    hipLaunchKernelGGL(band_scan_full_kernel, rows_grid((unsigned)((nb2 + kWave - 1) / kWave), a.rows),
                       dim3(kScanT), 0, s, a2);
    hipLaunchKernelGGL(band_scatter_kernel, blk, dim3(kBT), 0, s, a2);
    hipLaunchKernelGGL(band_agg_keys_kernel, agg_keys, dim3(kBT), 0, s, a2);
    hipLaunchKernelGGL(band_locate_kernel<true>, rows_grid(1u, a.rows), dim3(1024), 0, s, a2, fb);
  }
  return hipGetLastError();
}

}  // namespace lapsum
