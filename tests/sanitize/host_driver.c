/* Drives the host-only logic of the C-ABI library (argument checks, plans,
 * bracket indices, workspace sizes, status strings, and every entry point's
 * early error returns) over a grid of shapes and options.  Built and run by
 * tests/test_sanitize.py against a host-only AddressSanitizer +
 * UndefinedBehaviorSanitizer build of the library; no call here reaches the
 * GPU.  Exits non-zero on the first unexpected status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lapsum.h"

static int failures = 0;

#define EXPECT(cond, ...)                       \
    do {                                        \
        if (!(cond)) {                          \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);       \
            fprintf(stderr, "\n");              \
            ++failures;                         \
        }                                       \
    } while (0)

static void check_plan(int64_t rows, int64_t n, double k, double t, const lapsum_options *o) {
    lapsum_plan_info info;
    memset(&info, 0xAB, sizeof info);
    const lapsum_status st = lapsum_plan(rows, n, k, t, o, &info);
    const size_t ws = lapsum_workspace_bytes(rows, n, k, t, o);
    if (st != LAPSUM_OK) {
        EXPECT(ws == 0, "workspace bytes %zu for a rejected call (status %d)", ws, (int)st);
        return;
    }
    EXPECT(info.path >= LAPSUM_PATH_ONCHIP && info.path <= LAPSUM_PATH_BISECT, "path %d", info.path);
    EXPECT(ws >= info.forward_bytes && ws >= info.backward_bytes, "workspace %zu below the plan", ws);
    if (info.path == LAPSUM_PATH_BRACKET) {
        EXPECT(info.m == ((int64_t)1 << info.sample_log2), "m %lld", (long long)info.m);
        EXPECT(info.lo >= 0 && info.lo <= info.hi && info.hi <= info.m + 1, "indices %lld %lld",
               (long long)info.lo, (long long)info.hi);
        EXPECT(info.band_capacity >= 1, "capacity %lld", (long long)info.band_capacity);
        EXPECT(info.filter_groups >= 1, "filter groups %d", info.filter_groups);
    }
}

static void grid_of_plans(void) {
    const int64_t rows_list[] = {1, 3, 32, 70000};
    const int64_t n_list[] = {1, 2, 17, 256, 1024, 8192, 8193, 65536, 1 << 20, (1 << 20) + 1, 3317760,
                              100000000, (int64_t)1 << 31};
    const double t_list[] = {1e-3, 0.05, 1.0};
    for (size_t a = 0; a < sizeof rows_list / sizeof rows_list[0]; ++a)
        for (size_t c = 0; c < sizeof n_list / sizeof n_list[0]; ++c)
            for (size_t d = 0; d < sizeof t_list / sizeof t_list[0]; ++d)
                for (int path = LAPSUM_PATH_AUTO; path <= LAPSUM_PATH_BISECT; ++path) {
                    const int64_t rows = rows_list[a], n = n_list[c];
                    if (rows * n > ((int64_t)1 << 34)) continue;  /* keep the sizes plausible */
                    const double ks[] = {0.5, 0.25 * (double)n, 0.5 * (double)n, (double)n - 0.5, 600.0, 1e5};
                    for (size_t e = 0; e < sizeof ks / sizeof ks[0]; ++e) {
                        lapsum_options o;
                        lapsum_options_init(&o);
                        o.path = path;
                        check_plan(rows, n, ks[e], t_list[d], &o);
                        o.sample_log2 = 4 + (int)((c + e) % 17);
                        o.delta = 0.1;
                        o.widen_steps = (int)(e % 6) - 1;
                        check_plan(rows, n, ks[e], t_list[d], &o);
                        o.band_capacity = 16;
                        check_plan(rows, n, ks[e], t_list[d], &o);
                        o.spread_fallback = 1;
                        check_plan(rows, n, ks[e], t_list[d], &o);
                    }
                }
    check_plan(1, 1000, 10.0, 0.1, NULL);
}

static void rejected_arguments(void) {
    lapsum_options o;
    lapsum_plan_info info;
    lapsum_options_init(&o);
    EXPECT(lapsum_plan(0, 10, 1.0, 1.0, &o, &info) == LAPSUM_ERR_SHAPE, "rows 0");
    EXPECT(lapsum_plan(1, 0, 1.0, 1.0, &o, &info) == LAPSUM_ERR_SHAPE, "n 0");
    EXPECT(lapsum_plan(1, LAPSUM_MAX_N + 1, 1.0, 1.0, &o, &info) == LAPSUM_ERR_SHAPE, "n too large");
    EXPECT(lapsum_plan(LAPSUM_MAX_ROWS + 1, 2, 1.0, 1.0, &o, &info) == LAPSUM_ERR_SHAPE, "rows too many");
    EXPECT(lapsum_plan(1, 10, 0.0, 1.0, &o, &info) == LAPSUM_ERR_K, "k 0");
    EXPECT(lapsum_plan(1, 10, 10.0, 1.0, &o, &info) == LAPSUM_ERR_K, "k n");
    EXPECT(lapsum_plan(1, 10, NAN, 1.0, &o, &info) == LAPSUM_ERR_K, "k nan");
    EXPECT(lapsum_plan(1, 10, 1.0, 0.0, &o, &info) == LAPSUM_ERR_T, "t 0");
    EXPECT(lapsum_plan(1, 10, 1.0, -1.0, &o, &info) == LAPSUM_ERR_T, "t negative");
    EXPECT(lapsum_plan(1, 10, 1.0, INFINITY, &o, &info) == LAPSUM_ERR_T, "t inf");
    EXPECT(lapsum_plan(1, 10, 1.0, 1.0, &o, NULL) == LAPSUM_ERR_NULL, "plan out NULL");
    o.path = 99;
    EXPECT(lapsum_plan(1, 10, 1.0, 1.0, &o, &info) != LAPSUM_OK, "path 99");
    lapsum_options_init(&o);
    o.sample_log2 = 3;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "sample_log2 3");
    o.sample_log2 = 21;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "sample_log2 21");
    lapsum_options_init(&o);
    o.delta = 1.5;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "delta 1.5");
    lapsum_options_init(&o);
    o.widen_steps = 5;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "widen 5");
    lapsum_options_init(&o);
    o.band_capacity = -1;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "capacity -1");
    lapsum_options_init(&o);
    o.spread_fallback = 2;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_ERR_OPTION, "spread fallback 2");
    /* per-row parameters: bracketing reports its indices as per row (the
     * pointer is only compared with NULL on the host) */
    lapsum_options_init(&o);
    static const double fake_rows[1] = {1.0};
    o.k_rows = fake_rows;
    o.path = LAPSUM_PATH_BRACKET;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_OK && info.lo == -1 && info.hi == -1,
           "per-row bracket");
    o.path = LAPSUM_PATH_AUTO;
    EXPECT(lapsum_plan(1, 1 << 22, 1.0, 1.0, &o, &info) == LAPSUM_OK && info.path == LAPSUM_PATH_BRACKET,
           "per-row auto");
}

static void bracket_index_grid(void) {
    const int64_t n_list[] = {2, 100, 1 << 20, 3317760, 100000000};
    const double delta_list[] = {1e-6, 1e-3, 0.5};
    for (size_t a = 0; a < sizeof n_list / sizeof n_list[0]; ++a)
        for (int lg = 4; lg <= 20; lg += 4)
            for (size_t d = 0; d < sizeof delta_list / sizeof delta_list[0]; ++d) {
                const int64_t n = n_list[a], m = (int64_t)1 << lg;
                const double ks[] = {0.5, 1.0, 0.5 * (double)n, (double)n - 1.0};
                for (size_t e = 0; e < sizeof ks / sizeof ks[0]; ++e) {
                    int64_t lo = -7, hi = -7;
                    const lapsum_status st = lapsum_bracket_indices(n, ks[e], m, delta_list[d], &lo, &hi);
                    if (ks[e] <= 0.0 || ks[e] >= (double)n) continue;
                    EXPECT(st == LAPSUM_OK, "bracket indices status %d", (int)st);
                    EXPECT(lo >= 0 && lo <= hi && hi <= m + 1, "indices %lld %lld (m %lld)", (long long)lo,
                           (long long)hi, (long long)m);
                }
            }
    int64_t lo, hi;
    EXPECT(lapsum_bracket_indices(100, 10.0, 64, 1e-6, NULL, &hi) == LAPSUM_ERR_NULL, "indices NULL");
    EXPECT(lapsum_bracket_indices(100, 10.0, 64, 0.0, &lo, &hi) != LAPSUM_OK, "delta 0");
}

static void early_returns(void) {
    /* every entry point checks its arguments before it touches the GPU */
    float fbuf[8];
    double dbuf[4];
    char ws_raw[1024 + 256];
    void *ws = (void *)(((uintptr_t)ws_raw + 255) & ~(uintptr_t)255);
    lapsum_options o;
    lapsum_options_init(&o);
    EXPECT(lapsum_forward(NULL, 1, 4, 1.0, 1.0, fbuf, dbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_NULL, "fwd r NULL");
    EXPECT(lapsum_forward(fbuf, 1, 4, 1.0, 1.0, NULL, dbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_NULL, "fwd p NULL");
    EXPECT(lapsum_forward(fbuf, 1, 4, 1.0, 1.0, fbuf, NULL, ws, 1024, &o, NULL) == LAPSUM_ERR_NULL, "fwd b NULL");
    EXPECT(lapsum_forward(fbuf, 1, 4, 5.0, 1.0, fbuf, dbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_K, "fwd k");
    EXPECT(lapsum_forward(fbuf, 0, 4, 1.0, 1.0, fbuf, dbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_SHAPE, "fwd rows");
    /* a streaming path needs a workspace: missing, short, misaligned */
    const int64_t big = (int64_t)1 << 22;
    const size_t need = lapsum_workspace_bytes(1, big, 10.0, 0.1, &o);
    EXPECT(need > 1024, "workspace %zu", need);
    EXPECT(lapsum_forward(fbuf, 1, big, 10.0, 0.1, fbuf, dbuf, NULL, 0, &o, NULL) == LAPSUM_ERR_NULL, "fwd ws NULL");
    EXPECT(lapsum_forward(fbuf, 1, big, 10.0, 0.1, fbuf, dbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_WORKSPACE,
           "fwd ws short");
    EXPECT(lapsum_forward(fbuf, 1, big, 10.0, 0.1, fbuf, dbuf, (char *)ws + 4, need, &o, NULL) ==
               LAPSUM_ERR_WORKSPACE, "fwd ws misaligned");
    EXPECT(lapsum_backward(NULL, fbuf, dbuf, 1, 4, 1.0, fbuf, fbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_NULL,
           "bwd g NULL");
    EXPECT(lapsum_backward(fbuf, fbuf, dbuf, 1, 4, 0.0, fbuf, fbuf, ws, 1024, &o, NULL) == LAPSUM_ERR_T, "bwd t");
    EXPECT(lapsum_backward(fbuf, fbuf, dbuf, 1, big, 0.1, fbuf, fbuf, ws, 8, &o, NULL) == LAPSUM_ERR_WORKSPACE,
           "bwd ws short");
    EXPECT(lapsum_backward_noalloc(fbuf, fbuf, NULL, 1, 4, 1.0, fbuf, fbuf, &o, NULL) == LAPSUM_ERR_NULL,
           "noalloc NULL");
    EXPECT(lapsum_backward_noalloc(fbuf, fbuf, dbuf, (int64_t)1 << 22, 4096, 1.0, fbuf, fbuf, &o, NULL) ==
               LAPSUM_ERR_SCRATCH, "noalloc scratch");
    EXPECT(lapsum_midpoint_mass(NULL, 1, 100, 10, 0.1, dbuf, dbuf, ws, 1024, NULL) != LAPSUM_OK, "midpoint NULL");
    EXPECT(lapsum_midpoint_mass(fbuf, 1, 100, 0, 0.1, dbuf, dbuf, ws, 1024, NULL) != LAPSUM_OK, "midpoint k 0");
    EXPECT(lapsum_midpoint_mass(fbuf, 1, 100, 100, 0.1, dbuf, dbuf, ws, 1024, NULL) != LAPSUM_OK, "midpoint k n");
    EXPECT(lapsum_midpoint_workspace_bytes(3, 1 << 20) > 0, "midpoint workspace");
}

int main(void) {
    for (int st = 0; st <= 12; ++st) {
        const char *s = lapsum_status_string((lapsum_status)st);
        EXPECT(s != NULL && strlen(s) > 0, "status string %d", st);
    }
    grid_of_plans();
    rejected_arguments();
    bracket_index_grid();
    early_returns();
    if (failures) {
        fprintf(stderr, "%d unexpected results\n", failures);
        return 1;
    }
    printf("host driver: all checks passed\n");
    return 0;
}
