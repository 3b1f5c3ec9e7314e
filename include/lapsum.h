/*
 * lapsum.h -- C ABI of the MI355X (gfx950) Fast LapSum exact soft top-k library.
 *
 * Operator ("Fast LapSum: Exact Differentiable Top-k at Million Scale",
 * section 2.1, eqs. (1)-(2)): for each row of scores r_1..r_n, a budget k with
 * 0 < k < n and a temperature t > 0 (the Laplace scale),
 *     p_i = F((r_i - b)/t),   F(z) = e^z/2 (z < 0),  1 - e^-z/2 (z >= 0),
 * where the threshold b is the unique root of  sum_i p_i = k.  The backward
 * pass is the analytic vector-Jacobian product (same section): with
 * d_i = min(p_i, 1 - p_i)/t (the Laplace density at the score),
 *     dk   = sum_i g_i d_i / sum_i d_i,     dr_i = d_i (g_i - dk).
 *
 * Solvers (section 2.2): a full sort of the row followed by one stable
 * prefix/suffix scan, an index lookup of the balancing interval and a
 * closed-form root; and, for million-scale rows, probabilistic bracketing
 * (sample, binomial order-statistic bracket, one streaming pass that folds
 * out-of-bracket scores into tail sums and keeps the middle band, an exact
 * solve on the band, and certification; a bracket that fails it is widened
 * and tried again).  The full-sort solver exists as written (the SORT path:
 * every score of the row radix-sorted) and in a form that sorts only what
 * the root needs (the BUCKET path: one bucket pass over the row or band
 * locates the balancing bucket from order-free bucket sums, and only that
 * bucket is sorted).  A missed bracket is widened (wider order statistics
 * of the same sample, one pass over the row by the workgroup that found the
 * miss, the same bucket selection on the wider band); if every widened
 * bracket fails too, a deterministic fallback nests the bucket selection
 * over the whole row.  The iterative bisection that the full-sort solver
 * replaces is available as a baseline (the BISECT path).
 *
 * Conventions shared by every entry point
 *   - Array arguments marked "device" are device pointers on the current HIP
 *     device; "host" pointers are read during the call only.
 *   - r, p, g, dr are contiguous row-major [rows, n] fp32; b is fp64 [rows];
 *     dk is fp32 [rows].  k and t are shared by all rows.
 *   - The caller owns every buffer, including the workspace.  The library
 *     never allocates or frees device memory, never synchronises the stream
 *     and keeps no state between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Outputs are valid once the stream reaches the call's end.
 *   - The returned status covers host-side argument checks and launch errors
 *     only.  Each call first clears any non-sticky HIP error left pending on
 *     the calling thread by earlier runtime calls.  Per-row outcomes (bracket
 *     hit/miss, widening, fallback, degenerate backward) are reported through
 *     the optional `stats` array.
 *   - Scores must be finite; non-finite scores give unspecified outputs (the
 *     kernels still terminate).
 *   - Results are deterministic: the same inputs, options and seed give
 *     bitwise identical outputs.
 */
#ifndef LAPSUM_H
#define LAPSUM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lapsum_status {
    LAPSUM_OK = 0,
    LAPSUM_ERR_NULL = 1,      /* a required pointer is NULL */
    LAPSUM_ERR_SHAPE = 2,     /* rows < 1, n < 1, n > LAPSUM_MAX_N, rows > LAPSUM_MAX_ROWS */
    LAPSUM_ERR_K = 3,         /* k not finite or not in (0, n) */
    LAPSUM_ERR_T = 4,         /* t not finite or t <= 0 */
    LAPSUM_ERR_WORKSPACE = 5, /* workspace smaller than lapsum_workspace_bytes() or not 256-byte aligned */
    LAPSUM_ERR_PATH = 6,      /* the requested path cannot run this shape */
    LAPSUM_ERR_OPTION = 7,    /* an option is out of range */
    LAPSUM_ERR_HIP = 8,       /* a HIP launch or runtime query failed */
    LAPSUM_ERR_SCRATCH = 9    /* lapsum_backward_noalloc: the call needs more scratch than the
                                 library's fixed buffer (LAPSUM_NOALLOC_SCRATCH_BYTES) holds */
} lapsum_status;

/* Longest row: sample indices use 32x32-bit products and tile counts fit int32.
 * Most rows per call: every path accepts up to 2^24 rows (launches fold rows
 * over two grid dimensions, so no launch dimension exceeds its limit); the
 * practical limit is device memory for r, p and the workspace. */
#define LAPSUM_MAX_N ((int64_t)1 << 31)
#define LAPSUM_MAX_ROWS ((int64_t)1 << 24)
/* Longest row the on-chip (LDS/register) sort path takes. */
#define LAPSUM_ONCHIP_MAX_N 8192

typedef enum lapsum_path {
    LAPSUM_PATH_AUTO = 0,     /* n <= 8192: ONCHIP; n <= 2^20: BUCKET; else BRACKET (also with
                                 per-row k or t) */
    LAPSUM_PATH_ONCHIP = 1,   /* fused per-row bitonic sort + scan + root + apply (n <= 8192) */
    LAPSUM_PATH_BUCKET = 2,   /* the full-sort solver sorting only the balancing bucket: one radix
                                 (bucket) pass over the row, order-free bucket sums, locate, sort of
                                 that bucket, root + streaming apply */
    LAPSUM_PATH_BRACKET = 3,  /* probabilistic bracketing; a missed bracket is widened, then an
                                 exact whole-row fallback */
    LAPSUM_PATH_SORT = 4,     /* the full-sort solver as the pages state it: a radix sort of every
                                 score of the row (4 passes of 8-bit digits), the threshold curve
                                 over the sorted row, locate, root + streaming apply */
    LAPSUM_PATH_BISECT = 5    /* baseline: bisection of the monotone budget f(b) in fp64, no sort
                                 (on chip up to 16384 scores, else one streaming pass per halving) */
} lapsum_path;

/* Per-row flags in lapsum_row_stats.flags. */
#define LAPSUM_FLAG_BRACKET 0x1     /* the bracketing path ran for this row */
#define LAPSUM_FLAG_HIT 0x2         /* the first bracket held (certified) */
#define LAPSUM_FLAG_FALLBACK 0x4    /* b came from the exact whole-row fallback */
#define LAPSUM_FLAG_OVERFLOW 0x8    /* the first band exceeded its capacity (counted as a miss) */
#define LAPSUM_FLAG_DEGENERATE 0x10 /* backward: every d_i was 0 in fp32, so dr = 0 and dk = 0 */
#define LAPSUM_FLAG_WIDENED 0x20    /* the first bracket missed (or overflowed) and a widened
                                       bracket held (certified); the stats describe it */
#define LAPSUM_FLAG_INVALID 0x40    /* the row's per-row k or t was out of range: its outputs are NaN */

/* Optional per-row diagnostics, written by lapsum_forward (all fields) and
 * lapsum_backward (flags |= LAPSUM_FLAG_DEGENERATE only).  Device memory. */
typedef struct lapsum_row_stats {
    double a_lo, a_hi;       /* bracket [a_L, a_R); -inf / +inf when open */
    double tail_lo, tail_hi; /* S_L = sum_{r<a_L} e^{(r-a_L)/t},  S_R = sum_{r>=a_R} e^{-(r-a_R)/t} */
    int64_t count_lo;        /* c_L = #{r < a_L} */
    int64_t count_hi;        /* c_R = #{r >= a_R} */
    int64_t band;            /* M = #{a_L <= r < a_R} (may exceed the capacity) */
    int32_t flags;           /* LAPSUM_FLAG_* */
    int32_t reserved;
} lapsum_row_stats;

/* Stage ids for optional per-stage timing (lapsum_options.stage_events). */
enum {
    LAPSUM_STAGE_ONCHIP_FWD = 0, /* fused on-chip forward */
    LAPSUM_STAGE_INIT = 1,       /* per-call state reset */
    LAPSUM_STAGE_SAMPLE = 2,     /* kernel-noised sample */
    LAPSUM_STAGE_SELECT = 3,     /* order statistics -> bracket */
    LAPSUM_STAGE_FILTER = 4,     /* streaming tail sums + band compaction */
    LAPSUM_STAGE_BAND = 5,       /* band solve + certification (+ widening / fallback of a missed row) */
    LAPSUM_STAGE_BUCKET = 6,     /* bucketed solve of whole rows (BUCKET path) */
    LAPSUM_STAGE_APPLY = 7,      /* streaming Laplace-CDF apply */
    LAPSUM_STAGE_ONCHIP_BWD = 8, /* fused on-chip backward */
    LAPSUM_STAGE_BWD_REDUCE = 9, /* streaming backward reductions (D, G) */
    LAPSUM_STAGE_BWD_APPLY = 10, /* streaming backward elementwise dr */
    LAPSUM_STAGE_SORT = 11,      /* SORT path: radix sort of every row */
    LAPSUM_STAGE_SOLVE = 12,     /* SORT path: threshold curve, locate and root over the sorted rows */
    LAPSUM_STAGE_BISECT = 13,    /* BISECT path: the bisection (on chip it also writes p) */
    LAPSUM_STAGE_COUNT = 14
};

typedef struct lapsum_options {
    int32_t path;          /* lapsum_path; LAPSUM_PATH_AUTO picks by n */
    int32_t sample_log2;   /* bracketing sample size m = 2^sample_log2 (4..20);
                              0 = min(16, max(4, floor(log2(n/16)))) */
    double delta;          /* bracket miss probability bound in (0, 1); 0 = 1e-6 */
    uint64_t seed;         /* Philox-4x32-10 key of the sample */
    int64_t band_capacity; /* 0 = derived from (n, k, m, delta); else an override >= 1 */
    const double *bracket_override; /* host [2] or NULL: force (a_L, a_R) on every row
                                       instead of sampling (used to test the fallback) */
    lapsum_row_stats *stats;        /* device [rows] or NULL */
    void *const *stage_events;      /* host array of 2*LAPSUM_STAGE_COUNT hipEvent_t or NULL;
                                       entries 2s and 2s+1 (if non-NULL) are recorded on the
                                       stream before and after stage s */
    int32_t widen_steps;   /* bracketing: widened brackets tried after a miss before the
                              whole-row fallback (section 2.2, step 4); step i uses the
                              bracket indices for delta * 1e-6^i, skipped where they are
                              no wider.  0 = 2, -1 = none, at most 4.  Rows whose bracket
                              came from bracket_override have no sample and go straight
                              to the fallback. */
    int32_t spread_fallback; /* bracketing: 1 = a row whose bracket misses (or whose band
                              overflows) is solved exactly by the whole-row bucket solve,
                              launched after the band solve and spread over every workgroup
                              (no widening; its b is the bucket path's for that row); 0 (the
                              default) = widening, then the exact fallback, both inside the
                              one workgroup that found the miss.  The extra launches cost a
                              few microseconds each when every row hits, and the workspace
                              grows by the bucket solve's (about 8 bytes per score). */
    const double *k_rows;  /* device [rows] or NULL: a budget per row (the k argument is then
                              not used).  Values must satisfy 0 < k_i < n; a row whose value
                              does not gets NaN outputs and LAPSUM_FLAG_INVALID. */
    const double *t_rows;  /* device [rows] or NULL: a temperature per row (the t argument is
                              then not used), 0 < t_i < inf, likewise.  lapsum_backward reads
                              it too.  On the bracketing path with k_rows or t_rows each row's
                              order-statistic indices come from its own k (computed on the
                              device, from the same binomial definition), its sample is noised
                              with its own t, the band is sized for the widest bracket (that of
                              k = n/2) and solved by the bucketed band solve, and a row whose
                              bracket misses goes straight to the exact whole-row fallback (no
                              widening: the widened indices would depend on k). */
} lapsum_options;

/* Resolved plan of a call (host-only query, no GPU needed). */
typedef struct lapsum_plan_info {
    int32_t path;          /* resolved lapsum_path */
    int32_t sample_log2;   /* bracketing: log2(m) */
    int64_t m;             /* bracketing: sample size */
    int64_t lo, hi;        /* bracketing: 1-based order-statistic indices; lo = 0 means
                              a_L = -inf, hi = m + 1 means a_R = +inf; both -1 when every
                              row has its own (per-row budgets or temperatures) */
    int64_t band_capacity; /* bracketing: band buffer length per row */
    int32_t band_onchip;   /* bracketing: 1 if the band is solved on chip (capacity <= 8192) */
    int32_t filter_groups; /* bracketing: streaming-filter workgroups per row; their band slots
                              (2048 keys each) hold at least twice the band capacity when the row
                              is long enough to give each of them a full load */
    uint64_t forward_bytes;  /* workspace bytes lapsum_forward needs */
    uint64_t backward_bytes; /* workspace bytes lapsum_backward needs */
} lapsum_plan_info;

/* Fill *opt with defaults (AUTO path, default m and delta, seed 0, no
 * diagnostics).  A NULL options pointer means the same defaults. */
void lapsum_options_init(lapsum_options *opt);

/* Human-readable name of a status code (static string). */
const char *lapsum_status_string(lapsum_status st);

/* Host-only: resolve the path, sample size, bracket indices, band capacity
 * and workspace sizes for a call with these arguments.  Same argument
 * checks as lapsum_forward. */
lapsum_status lapsum_plan(int64_t rows, int64_t n, double k, double t, const lapsum_options *opt,
                          lapsum_plan_info *out);

/* Host-only: the equal-tailed binomial order-statistic indices of the
 * localisation step (section 2.2, probabilistic bracketing, step 1).  With
 * N ~ Bin(m, 1 - k/n) the number of noised samples at or below b,
 *   lo = max{l in [0, m]   : P(N <= l-1) <= delta/2},
 *   hi = min{h in [1, m+1] : P(N >= h)   <= delta/2},
 * so P(X_(lo) > b) <= delta/2 and P(X_(hi) <= b) <= delta/2. */
lapsum_status lapsum_bracket_indices(int64_t n, double k, int64_t m, double delta, int64_t *lo, int64_t *hi);

/* Workspace bytes sufficient for both lapsum_forward and lapsum_backward
 * with these arguments (the maximum of the two; 0 when neither needs any). */
size_t lapsum_workspace_bytes(int64_t rows, int64_t n, double k, double t, const lapsum_options *opt);

/* Forward (section 2.1 eqs. (1)-(2); solvers of section 2.2).
 *   r  device [rows, n] fp32 scores (read only)
 *   p  device [rows, n] fp32 output probabilities (must not alias r)
 *   b  device [rows]    fp64 output thresholds
 *   workspace, workspace_bytes: device scratch of at least
 *       lapsum_workspace_bytes() bytes, 256-byte aligned (may be NULL when
 *       that size is 0); its contents need no initialisation.
 *   opt may be NULL.  Errors: LAPSUM_ERR_NULL, _SHAPE, _K, _T, _WORKSPACE,
 *   _PATH, _OPTION (nothing launched), LAPSUM_ERR_HIP (launch failed). */
lapsum_status lapsum_forward(const float *r, int64_t rows, int64_t n, double k, double t, float *p, double *b,
                             void *workspace, size_t workspace_bytes, const lapsum_options *opt, void *stream);

/* Backward: the analytic VJP of the forward (section 2.1).
 *   g  device [rows, n] fp32 upstream gradient w.r.t. p
 *   p  device [rows, n] fp32 probabilities from lapsum_forward
 *   b  device [rows]    fp64 thresholds from lapsum_forward (accepted for
 *      symmetry with the forward; the VJP needs only p and t because
 *      min(p, 1 - p) is the Laplace density at the score)
 *   dr device [rows, n] fp32 output (may alias g, not p)
 *   dk device [rows]    fp32 output
 *   Only opt->stats, opt->stage_events and opt->t_rows (a temperature per
 *   row, as in the forward) are read.  Errors as forward. */
lapsum_status lapsum_backward(const float *g, const float *p, const double *b, int64_t rows, int64_t n, double t,
                              float *dr, float *dk, void *workspace, size_t workspace_bytes,
                              const lapsum_options *opt, void *stream);

/* DFTopK diagnostic (section 2.3, relation to DFTopK; section 4.1, budget
 * accuracy): DFTopK fixes the threshold at the midpoint of the k-th and the
 * (k+1)-th largest score instead of solving the budget equation, and is
 * LapSum's zero-temperature limit.  For each row this computes that fixed
 * threshold and the mass the Laplace kernel of temperature t assigns at it,
 *     b_mid = (s_(k) + s_(k+1)) / 2,   mass = sum_i F((r_i - b_mid)/t),
 * so mass / k - 1 is the budget drift of the fixed midpoint (LapSum's own
 * threshold gives exactly k).  The order statistics come from the SORT
 * path's radix sort of the row; mass is an exact count of the scores above
 * b_mid plus fp64 sums of the terms e^{-|r - b_mid|/t}/2.
 *   r      device [rows, n] fp32 scores
 *   k      integer budget, 1 <= k <= n - 1 (else LAPSUM_ERR_K; n >= 2)
 *   t      temperature, finite and > 0
 *   b_mid  device [rows] fp64 output
 *   mass   device [rows] fp64 output
 *   workspace: lapsum_midpoint_workspace_bytes(rows, n) bytes, 256-byte
 *   aligned.  Errors as lapsum_forward. */
size_t lapsum_midpoint_workspace_bytes(int64_t rows, int64_t n);
lapsum_status lapsum_midpoint_mass(const float *r, int64_t rows, int64_t n, int64_t k, double t, double *b_mid,
                                   double *mass, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the fixed device buffer lapsum_backward_noalloc uses instead of a
 * workspace: one per device, held until the process ends. */
#define LAPSUM_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

/* Backward without any allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and results (bitwise) as
 * lapsum_backward, with the streaming pass's partial sums kept in a fixed
 * device buffer of the library (LAPSUM_NOALLOC_SCRATCH_BYTES per device,
 * looked up on the first call on each device) instead of a caller
 * workspace.  The caller still passes every input and output.  Nothing is
 * allocated or freed, by the library or by any routine it calls.
 *   Arguments, layouts and opt fields read: as lapsum_backward (minus the
 *   workspace).  Rows of at most 1024 scores need no scratch; longer rows
 *   need 16 bytes per streaming workgroup, i.e. at most
 *   16 * max(4096, rows) bytes, so up to 65536 rows of any length fit.
 *   Errors: as lapsum_backward, plus LAPSUM_ERR_SCRATCH (nothing launched)
 *   when the call needs more than the fixed buffer.
 *   Concurrency: every call on one device shares that device's buffer, and
 *   the buffer keeps whatever the last call left in it; calls that overlap
 *   on one device (other streams, other threads) race and must be ordered
 *   by the caller. */
lapsum_status lapsum_backward_noalloc(const float *g, const float *p, const double *b, int64_t rows, int64_t n,
                                      double t, float *dr, float *dk, const lapsum_options *opt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LAPSUM_H */
