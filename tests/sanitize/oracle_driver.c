/* Drives every entry point of the C oracle (oracle/lapsum_oracle.c) over
 * small and edge-case inputs: single scores, budgets next to 0 and n, runs of
 * ties, tiny and huge temperatures, infinite bracket ends and the invalid
 * arguments.  Built with AddressSanitizer + UndefinedBehaviorSanitizer and
 * run by tests/test_sanitize.py; it checks that every call returns and that
 * the results satisfy sum p = k, not the values themselves (the oracle's own
 * tests pin those).  Exits non-zero on the first unexpected result. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_laplace_cdf(double z);
double oracle_laplace_quantile(double u);
double oracle_budget(const double *r, int64_t n, double b, double t, int threads);
int oracle_forward(const double *r, int64_t rows, int64_t n, double k, double t, double *p, double *b, int threads);
int oracle_backward(const double *r, const double *b, const double *g, int64_t rows, int64_t n, double t, double *dr,
                    double *dk, int threads);
int oracle_solve_sorted(const double *r, int64_t n, double k, double t, double *b_out, int64_t *j_out);
void oracle_tail_sums(const double *r, int64_t n, double aL, double aR, double t, double *SL, double *SR,
                      int64_t *cL, int64_t *cR, int64_t *M);
int oracle_midpoint_mass(const double *r, int64_t rows, int64_t n, int64_t k, double t, double *b_mid,
                         double *mass, int threads);

static int failures = 0;
#define EXPECT(cond, ...)                                         \
    do {                                                          \
        if (!(cond)) {                                            \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
            fprintf(stderr, __VA_ARGS__);                         \
            fprintf(stderr, "\n");                                \
            ++failures;                                           \
        }                                                         \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return ((double)(z >> 11) + 0.5) * 0x1p-53;
}

static void one_case(const double *r, int64_t rows, int64_t n, double k, double t, int threads) {
    double *p = malloc(sizeof(double) * (size_t)(rows * n));
    double *g = malloc(sizeof(double) * (size_t)(rows * n));
    double *dr = malloc(sizeof(double) * (size_t)(rows * n));
    double *b = malloc(sizeof(double) * (size_t)rows);
    double *dk = malloc(sizeof(double) * (size_t)rows);
    for (int64_t i = 0; i < rows * n; ++i) g[i] = uniform01() - 0.5;
    const int rc = oracle_forward(r, rows, n, k, t, p, b, threads);
    EXPECT(rc == 0, "forward rc %d (n %lld k %g t %g)", rc, (long long)n, k, t);
    if (rc == 0) {
        for (int64_t row = 0; row < rows; ++row) {
            double s = 0.0;
            for (int64_t i = 0; i < n; ++i) s += p[row * n + i];
            EXPECT(fabs(s - k) <= 1e-6 * (k + 1.0), "sum p %.17g vs k %g (n %lld t %g)", s, k, (long long)n, t);
            double bs;
            int64_t j;
            if (oracle_solve_sorted(r + row * n, n, k, t, &bs, &j) == 0)
                EXPECT(j >= -1 && j < n, "located knot %lld", (long long)j);
            (void)oracle_budget(r + row * n, n, b[row], t, threads);
            double SL, SR;
            int64_t cL, cR, M;
            oracle_tail_sums(r + row * n, n, b[row] - t, b[row] + t, t, &SL, &SR, &cL, &cR, &M);
            EXPECT(cL + cR + M == n, "tail counts");
            oracle_tail_sums(r + row * n, n, -INFINITY, INFINITY, t, &SL, &SR, &cL, &cR, &M);
            EXPECT(M == n, "open bracket");
        }
        const int rb = oracle_backward(r, b, g, rows, n, t, dr, dk, threads);
        EXPECT(rb == 0, "backward rc %d", rb);
        if (n >= 2 && k >= 1.0 && k <= (double)n - 1.0) {
            double *bm = malloc(sizeof(double) * (size_t)rows), *ms = malloc(sizeof(double) * (size_t)rows);
            EXPECT(oracle_midpoint_mass(r, rows, n, (int64_t)k, t, bm, ms, threads) == 0, "midpoint");
            free(bm);
            free(ms);
        }
    }
    free(p);
    free(g);
    free(dr);
    free(b);
    free(dk);
}

int main(void) {
    for (int i = -50; i <= 50; ++i) (void)oracle_laplace_cdf(0.37 * i);
    for (int i = 1; i < 100; ++i) (void)oracle_laplace_quantile(i / 100.0);
    const int64_t ns[] = {1, 2, 3, 17, 256, 1000, 5000};
    const double ts[] = {1e-6, 1e-2, 1.0, 1e3};
    for (size_t a = 0; a < sizeof ns / sizeof ns[0]; ++a) {
        const int64_t n = ns[a], rows = n < 1000 ? 3 : 1;
        double *r = malloc(sizeof(double) * (size_t)(rows * n));
        for (int kind = 0; kind < 3; ++kind) {
            for (int64_t i = 0; i < rows * n; ++i) {
                const double u = uniform01();
                r[i] = kind == 0 ? 4.0 * u - 2.0 : (kind == 1 ? floor(8.0 * u) : 0.5); /* spread, ties, constant */
            }
            for (size_t d = 0; d < sizeof ts / sizeof ts[0]; ++d) {
                const double ks[] = {1e-3, 0.5, 1.0, 0.5 * (double)n, (double)n - 1.0, (double)n - 1e-3};
                for (size_t e = 0; e < sizeof ks / sizeof ks[0]; ++e) {
                    if (!(ks[e] > 0.0 && ks[e] < (double)n)) continue;
                    one_case(r, rows, n, ks[e], ts[d], e % 2 ? 1 : 4);
                }
            }
        }
        free(r);
    }
    double r1[4] = {0.0, 1.0, 2.0, 3.0}, p1[4], b1[1], dk1[1];
    EXPECT(oracle_forward(r1, 1, 4, 0.0, 1.0, p1, b1, 1) != 0, "k 0 accepted");
    EXPECT(oracle_forward(r1, 1, 4, 4.0, 1.0, p1, b1, 1) != 0, "k n accepted");
    EXPECT(oracle_forward(r1, 1, 4, 1.0, 0.0, p1, b1, 1) != 0, "t 0 accepted");
    EXPECT(oracle_forward(r1, 0, 4, 1.0, 1.0, p1, b1, 1) != 0, "rows 0 accepted");
    EXPECT(oracle_backward(r1, b1, r1, 1, 4, -1.0, p1, dk1, 1) != 0, "backward t < 0 accepted");
    EXPECT(oracle_midpoint_mass(r1, 1, 4, 4, 1.0, b1, dk1, 1) != 0, "midpoint k n accepted");
    if (failures) {
        fprintf(stderr, "%d unexpected results\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
