// Internal interface between the C-ABI host runtime (api.cpp) and the HIP
// kernel files.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lapsum.h"

namespace lapsum {

struct RowState;
struct TileAgg;
struct Pre;
struct Suf;

constexpr int kTile = 4096;          // keys per tile of the large-row sort and scan
constexpr int kSelectCap = 1024;     // direct-selection capacity of the bracket select
constexpr int kStreamThreads = 256;  // threads per workgroup of the streaming kernels
constexpr int kUnroll = 4;           // independent 16 B loads per thread per stream and iteration
constexpr int kBandSlot = 2048;      // band keys one filter workgroup may keep
constexpr int kMaxFilterBlocks = 4096;  // filter workgroups per row, at most

// Launch grids over rows.  Kernels with several workgroups per row put the
// row's workgroups in grid.x and the rows in grid.y and grid.z (a launch
// dimension other than x holds at most 65535 workgroups here); kernels with
// one workgroup per row use the same folding with grid.x = 1, so no launch
// exceeds 2^32 work-items in a dimension.  Device side: grid_row() in
// lapsum_device.hpp; a workgroup whose row is past the last one returns.
constexpr int64_t kGridDimMax = 65535;
inline dim3 rows_grid(unsigned gx, int64_t rows) {
  const int64_t z = (rows + kGridDimMax - 1) / kGridDimMax;
  const int64_t y = (rows + z - 1) / z;
  return dim3(gx, (unsigned)y, (unsigned)z);
}

// Optional per-row budget and temperature (device arrays [rows], NULL: the
// call's scalars).
struct RowParams {
  const double *k;
  const double *t;
  __host__ __device__ bool any() const { return k != nullptr || t != nullptr; }
};

// Arguments of the one-workgroup treatment of a row whose bracket missed
// (or whose band overflowed): up to `nwiden` widened brackets, each the
// sample's order statistics of ranks wlo[i], whi[i] (1-based; 0 and m + 1
// mean open ends), then the exact solve over all the row's scores.
constexpr int kMaxWiden = 4;
struct SegArgs {
  int rows;
  int64_t n;            // row length
  const float *r;       // [rows][n] scores
  uint32_t *A, *B;      // [rows][stride] key ping-pong buffers
  int64_t stride;       // per-row stride of A/B, a multiple of kTile
  int max_tiles;        // stride / kTile
  TileAgg *tagg;        // [rows][max_tiles] tile aggregates
  Pre *tpre;            // [rows][max_tiles] prefix before each tile
  Suf *tsuf;            // [rows][max_tiles] suffix after each tile
  RowState *st;         // [rows]
  double k, t, c;       // c = log2(e)/t
  float cf;
  const float *samples; // [rows][m] noised sample of the bracketing path, or NULL (no widening)
  int64_t m;
  int nwiden;           // widening steps (0: none)
  int64_t wlo[kMaxWiden], whi[kMaxWiden];
  int per_row;          // rows carry their own k, t, c, cf (in RowState): the fallback uses those
  int defer;            // a missed row is left flagged for the whole-row bucket solve launched after
                        // the band kernels (the spread fallback), not solved here
};

// Bucketed solve (bands too large for one workgroup, and whole rows of the
// full-sort path): the keys are spread over up to kBandBuckets buckets by
// their leading bits above the smallest key, the threshold curve is located
// over the bucket aggregates, and only the bucket that holds the root is
// sorted.
constexpr int kBandBucketBits = 11;
constexpr int kBandBuckets = 1 << kBandBucketBits;
constexpr int kBandCountBlocks = 64;  // count/scatter workgroups per row (band mode), at most
constexpr int64_t kFullChunkMax = 1 << 16;  // full-row mode: scores per count/scatter workgroup beyond that
constexpr int64_t kFullCountBlocksMax = 4096;

struct FilterPartial;

struct BandArgs {
  int rows;
  int gx;               // band mode: filter workgroups (slots) per row
  int group;            // band mode: slots per count/scatter workgroup
  int nblk;             // count/scatter workgroups per row
  int bbits;            // buckets per row = 2^bbits <= kBandBuckets (about 32 keys per bucket)
  const uint32_t *slots; // band mode: [rows][gx][kBandSlot] band keys per filter workgroup
  uint32_t *offs;        // band mode: [rows][gx + 1] slot offsets (written by the count kernel)
  const FilterPartial *part;  // band mode: [rows][gx] streaming-filter partials
  const float *r;       // full-row mode (non-null): the scores [rows][n], every one a key
  int64_t n;            // row length
  int64_t chunk;        // full-row mode: scores per count/scatter workgroup (a multiple of 4)
  uint32_t *mm;         // full-row mode: [rows][nblk][2] key minimum and maximum per workgroup
  RowState *st;         // [rows]
  uint32_t *keys;       // [rows][cap] bucketed band keys (the balancing bucket sorted by the locate)
  uint32_t *tmp;        // [rows][cap] scratch of the large-bucket sort
  uint32_t *hist;       // [rows][nblk][kBandBuckets] counts -> offsets inside buckets
  uint32_t *hext;       // full-row mode: [rows][nblk][2][kBandBuckets] key minimum / maximum per count
                        // workgroup and bucket
  uint32_t *btot;       // [rows][kBandBuckets] bucket sizes
  uint32_t *bstart;     // [rows][kBandBuckets] bucket starts
  TileAgg *bagg;        // band mode: [rows][kBandBuckets] anchored aggregates of the buckets
  uint32_t *bkey;       // full-row mode: [rows][kBandBuckets][2] smallest and largest key of each bucket
  unsigned long long *bsum;  // full-row mode: [rows][kBandBuckets][2] fixed-point sums anchored at the
                             // largest / smallest key
  TileAgg *tagg;        // [rows][max_tiles] tile aggregates of a large balancing bucket
  Pre *tpre;            // [rows][max_tiles]
  Suf *tsuf;            // [rows][max_tiles]
  int64_t cap;          // per-row stride of keys/tmp (a multiple of kTile)
  int max_tiles;        // cap / kTile
  double k, t, c;
  float cf;
  RowParams rp;         // per-row k and t (full-row mode), overriding k, t, c, cf
  int nested;           // full-row mode: a crowded balancing bucket is recorded in the row state and left
                        // to a second, multi-workgroup bucket level (else one workgroup selects inside it)
  const uint32_t *src2; // second level (non-null): the first level's bucketed keys [rows][cap]; each flagged
                        // row's set is its crowded bucket, keys / tmp are this level's buffers
  int32_t need;         // only rows whose state flags hold these bits take part (0: every row)
  RowState *st_out;     // non-null: each final b is also written to this state array (the whole-row
                        // solve of rows whose bracket missed, run on a state array of its own)
};

// Whole-row radix sort and the solve over the sorted rows (sort.hip): pass
// outputs alternate A, B, A, B, so the sorted keys end in B.
struct SortArgs {
  int64_t rows, n;
  const float *r;        // [rows][n] scores
  uint32_t *A, *B;       // [rows][stride] key buffers
  int64_t stride;        // per-row stride of A and B (a multiple of the solve tile)
  int ntiles;            // sort tiles per row
  uint32_t *cnt;         // [rows][256][ntiles] digit counts -> offsets inside the digit
  uint32_t *dtot;        // [rows][256] digit totals
  int nst;               // solve tiles per row
  TileAgg *ta;           // [rows][nst] anchored aggregates of the solve tiles
  Pre *tp;               // [rows][nst] scratch of the locate
  Suf *ts;               // [rows][nst]
  RowState *st;          // [rows]: b
  double k, t;
  RowParams rp;
};
hipError_t launch_row_sort(const SortArgs &a, hipStream_t s);
hipError_t launch_row_sort_solve(const SortArgs &a, hipStream_t s);
int sort_tiles(int64_t n);
int solve_tiles(int64_t n);
int64_t sort_stride(int64_t n);
// DFTopK midpoint on the sorted rows (kk-th and (kk+1)-th largest) and the
// Laplace mass there.
hipError_t launch_midpoint(const SortArgs &a, int64_t kk, double *b_mid, double *mass, void *partials, int gx,
                           hipStream_t s);
int midpoint_grid_x(int64_t rows, int64_t n);
size_t midpoint_partial_bytes(int64_t rows, int gx);

// Bisection baseline (bisect.hip).
bool bisect_onchip(int64_t n);
hipError_t launch_bisect_onchip(const float *r, int64_t rows, int64_t n, double k, double t, RowParams rp, float *p,
                                double *b, hipStream_t s);
hipError_t launch_bisect_stream(const float *r, int64_t rows, int64_t n, double k, double t, RowParams rp,
                                void *state, void *partials, int gx, RowState *st, hipStream_t s);
int bisect_grid_x(int64_t rows, int64_t n);
size_t bisect_state_bytes(int64_t rows);
size_t bisect_partial_bytes(int64_t rows, int gx);

// Launchers (each returns the first HIP error, or hipSuccess).
hipError_t launch_init_rows(RowState *st, int64_t rows, int32_t flags, const double *override2, int64_t n,
                            double k, double t, RowParams rp, hipStream_t s);
hipError_t launch_onchip_forward(const float *r, int64_t rows, int n, double k, double t, RowParams rp, float *p,
                                 double *b, lapsum_row_stats *stats, hipStream_t s);
hipError_t launch_onchip_backward(const float *g, const float *p, int64_t rows, int n, double t, RowParams rp,
                                  float *dr, float *dk, lapsum_row_stats *stats, hipStream_t s);
bool onchip_backward_supported(int64_t n);
hipError_t launch_sample(const float *r, int64_t rows, int64_t n, double t, int64_t m, uint64_t seed,
                         float *samples, uint16_t *starts, RowState *st, int32_t flags, uint32_t *tail, int Q,
                         const double *t_rows, hipStream_t s);
// Per-row bracket indices (and the rows' k, t, c, validity) into the row
// state, after the sample kernel reset it; the selection then reads them
// (lo < 0 asks for that).
hipError_t launch_bracket_rows(const double *k_rows, const double *t_rows, double k, double t, int64_t rows,
                               int64_t n, int64_t m, double delta, RowState *st, hipStream_t s);
// Top-side selection of the bracket: the depth Q of the per-group top lists
// (0: not applicable), their size, and the selection over them.
int tail_depth(int64_t m, int64_t lo, int64_t hi);
size_t tail_bytes(int64_t rows, int64_t m, int Q);
hipError_t launch_select_tail(const uint32_t *tail, int64_t rows, int64_t m, int Q, int64_t lo, int64_t hi,
                              RowState *st, hipStream_t s);
size_t sample_start_bytes(int64_t rows, int64_t m);
hipError_t launch_select(const float *samples, const uint16_t *starts, int64_t rows, int64_t m, int64_t lo,
                         int64_t hi, RowState *st, hipStream_t s);
hipError_t launch_filter(const float *r, int64_t rows, int64_t n, double t, RowState *st, uint32_t *slots,
                         void *partials, int grid_x, bool per_row, hipStream_t s);
int filter_grid_x(int64_t rows, int64_t n, int64_t cap);
size_t filter_partial_bytes(int64_t rows, int grid_x);
size_t band_slot_bytes(int64_t rows, int grid_x);
size_t band_offs_bytes(int64_t rows, int grid_x);
hipError_t launch_band_onchip(const uint32_t *slots, const void *partials, int gx, int64_t rows, int64_t n,
                              int64_t cap, RowState *st, double k, double t, const SegArgs &fb, hipStream_t s);
hipError_t launch_band_buckets(const BandArgs &a, const SegArgs &fallback, hipStream_t s);
int band_count_blocks(int gx, int *group);
int full_count_blocks(int64_t n, int64_t *chunk);
int bucket_bits(int64_t keys);
hipError_t launch_apply(const float *r, int64_t rows, int64_t n, const RowState *st, double t, RowParams rp,
                        float *p, double *b, hipStream_t s);
hipError_t launch_bwd_reduce(const float *g, const float *p, int64_t rows, int64_t n, void *partials, int grid_x,
                             hipStream_t s);
hipError_t launch_bwd_apply(const float *g, const float *p, int64_t rows, int64_t n, const void *partials,
                            int npart, double t, RowParams rp, float *dr, float *dk, lapsum_row_stats *stats,
                            hipStream_t s);
int bwd_grid_x(int64_t rows, int64_t n);
size_t bwd_partial_bytes(int64_t rows, int grid_x);
// Device address of the fixed no-alloc scratch (LAPSUM_NOALLOC_SCRATCH_BYTES)
// on the current device.
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_copy_stats(const RowState *st, int64_t rows, lapsum_row_stats *stats, hipStream_t s);

size_t row_state_bytes();
size_t tile_agg_bytes();
size_t pre_bytes();
size_t suf_bytes();

}  // namespace lapsum
