/*
 * Plain fp64 CPU oracle for the Fast LapSum exact soft top-k operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library: it is written from the method's definition so that a reader can
 * check it against the text by eye, not for speed.
 *
 * Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale"
 * (Struski et al., gist.science summaries, five language versions).
 *
 *   - LapSum operator, section 2.1, eq. (1): p_i = sigma((r_i - b)/t) with
 *     sigma the Laplace CDF, and eq. (2): sum_i p_i = k fixes b uniquely.
 *   - Section 2.1 also states that the backward pass is an analytic
 *     vector-Jacobian product; its formula is derived here by implicit
 *     differentiation of eq. (2) (the pages do not print it).
 *   - Section 2.2 "Full-Sort Solver": sort, one numerically stable
 *     prefix/suffix scan giving the threshold curve, an index lookup of the
 *     interval where the budget balances and a closed-form root there.
 *   - Section 2.2 "Probabilistic Bracketing", step 2: elements outside the
 *     bracket [a_L, a_R) fold into tail sums through Laplace-CDF identities.
 *
 * Readings where the pages are silent:
 *   - t is the Laplace scale, sigma is the unit-scale CDF
 *     F(z) = e^z / 2 for z < 0 and 1 - e^-z / 2 for z >= 0;
 *   - k is real with 0 < k < n; the budget sums over all n elements;
 *   - every floating-point quantity is fp64, sums use long double.
 *
 * Functions:
 *   oracle_forward        b by bisection on the monotone budget f(b) (the
 *                         definition written out), then p = F((r - b)/t).
 *   oracle_backward       the analytic VJP: dr, dk.
 *   oracle_solve_sorted   the full-sort solver's steps (sort, scans, locate,
 *                         closed-form root), a second independent route.
 *   oracle_budget         f(b) itself.
 *   oracle_tail_sums      the bracketing tail sums for a given bracket.
 *   oracle_midpoint_mass  the DFTopK threshold (midpoint of the k-th and
 *                         (k+1)-th largest scores, section 2.3) and the mass
 *                         the Laplace kernel assigns at it.
 *
 * Parity pins (tests/test_oracle_*.py): brute force over all "above" sets at
 * n <= 8 in 50-digit arithmetic, closed forms for n = 1 and constant rows,
 * shift/scale/complement symmetries, the zero-temperature limit (midpoint of
 * the k-th and (k+1)-th largest scores), central finite differences of the
 * forward for the VJP, and agreement of the two routes to b.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Unit-scale Laplace CDF (section 2.1, eq. (1)). */
static double laplace_cdf(double z)
{
    if (z < 0.0)
        return 0.5 * exp(z);
    return 1.0 - 0.5 * exp(-z);
}

/* Its inverse: the Laplace quantile function. */
static double laplace_quantile(double u)
{
    if (u <= 0.5)
        return log(2.0 * u);
    return -log(2.0 * (1.0 - u));
}

double oracle_laplace_cdf(double z) { return laplace_cdf(z); }
double oracle_laplace_quantile(double u) { return laplace_quantile(u); }

/* f(b) = sum_i F((r_i - b)/t), the budget function of eq. (2).  Summed in
 * long double over fixed chunks so the result does not depend on the thread
 * count's scheduling: chunk c always covers the same indices and the chunk
 * partials are added in index order. */
#define ORACLE_CHUNK 65536
double oracle_budget(const double *r, int64_t n, double b, double t, int threads)
{
    int64_t nchunks = (n + ORACLE_CHUNK - 1) / ORACLE_CHUNK;
    long double *part = (long double *)calloc((size_t)(nchunks > 0 ? nchunks : 1), sizeof(long double));
    if (!part)
        return NAN;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) if (threads > 1 && nchunks > 1)
#endif
    for (int64_t c = 0; c < nchunks; ++c) {
        int64_t lo = c * ORACLE_CHUNK, hi = lo + ORACLE_CHUNK < n ? lo + ORACLE_CHUNK : n;
        long double s = 0.0L;
        for (int64_t i = lo; i < hi; ++i)
            s += laplace_cdf((r[i] - b) / t);
        part[c] = s;
    }
    long double total = 0.0L;
    for (int64_t c = 0; c < nchunks; ++c)
        total += part[c];
    free(part);
    return (double)total;
}

/* The residual f(b) - k of eq. (2), computed so that it keeps its sign
 * where f is flat (t far below the gaps between scores).  Writing
 * F(z) = 1 - e^{-z}/2 for the scores above b and F(z) = e^{z}/2 for the
 * others gives
 *     f(b) - k = (#{r_i > b} - k) + sum_{r_i <= b} e^{(r_i-b)/t}/2
 *                                 - sum_{r_i >  b} e^{-(r_i-b)/t}/2,
 * an exact integer-minus-k term plus two sums of small positive terms, so
 * nothing small is absorbed into a 1.  Long double (x87, 64-bit mantissa and
 * a wide exponent range) is used for the terms and the sums. */
static long double budget_residual(const double *r, int64_t n, double b, double k, double t, int threads)
{
    int64_t nchunks = (n + ORACLE_CHUNK - 1) / ORACLE_CHUNK;
    long double *lo_part = (long double *)calloc((size_t)(nchunks > 0 ? nchunks : 1), sizeof(long double));
    long double *hi_part = (long double *)calloc((size_t)(nchunks > 0 ? nchunks : 1), sizeof(long double));
    int64_t *cnt = (int64_t *)calloc((size_t)(nchunks > 0 ? nchunks : 1), sizeof(int64_t));
    if (!lo_part || !hi_part || !cnt) {
        free(lo_part); free(hi_part); free(cnt);
        return NAN;
    }
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) if (threads > 1 && nchunks > 1)
#endif
    for (int64_t c = 0; c < nchunks; ++c) {
        int64_t lo = c * ORACLE_CHUNK, hi = lo + ORACLE_CHUNK < n ? lo + ORACLE_CHUNK : n;
        long double sb = 0.0L, sa = 0.0L;
        int64_t above = 0;
        for (int64_t i = lo; i < hi; ++i) {
            long double z = ((long double)r[i] - (long double)b) / (long double)t;
            if (r[i] > b) {
                above++;
                sa += expl(-z);
            } else {
                sb += expl(z);
            }
        }
        lo_part[c] = sb;
        hi_part[c] = sa;
        cnt[c] = above;
    }
    long double sb = 0.0L, sa = 0.0L;
    int64_t above = 0;
    for (int64_t c = 0; c < nchunks; ++c) {
        sb += lo_part[c];
        sa += hi_part[c];
        above += cnt[c];
    }
    free(lo_part); free(hi_part); free(cnt);
    return ((long double)above - (long double)k) + 0.5L * sb - 0.5L * sa;
}

/* The threshold of eq. (2) by bisection.  f is continuous and strictly
 * decreasing from n to 0, so for 0 < k < n the root is unique.  Starting
 * bracket: with q = k/n, every r_i >= min r gives f(min r - t F^-1(q)) >= k,
 * and every r_i <= max r gives f(max r - t F^-1(q)) <= k.  Halve until the
 * midpoint no longer moves (fp64 resolution of b). */
static double bisect_threshold(const double *r, int64_t n, double k, double t, int threads)
{
    double rmin = r[0], rmax = r[0];
    for (int64_t i = 1; i < n; ++i) {
        if (r[i] < rmin) rmin = r[i];
        if (r[i] > rmax) rmax = r[i];
    }
    double q = laplace_quantile(k / (double)n);
    double lo = rmin - t * q, hi = rmax - t * q;
    /* widen by a few ulps in case rounding put the root just outside */
    lo -= fabs(lo) * 1e-15 + 1e-300;
    hi += fabs(hi) * 1e-15 + 1e-300;
    for (int it = 0; it < 4000; ++it) {
        double mid = lo + 0.5 * (hi - lo);
        if (!(mid > lo && mid < hi))
            break;
        long double res = budget_residual(r, n, mid, k, t, threads);
        if (res > 0.0L)
            lo = mid;      /* f(mid) > k: root lies above mid */
        else if (res < 0.0L)
            hi = mid;
        else
            return mid;
    }
    long double rlo = budget_residual(r, n, lo, k, t, threads);
    long double rhi = budget_residual(r, n, hi, k, t, threads);
    return fabsl(rlo) <= fabsl(rhi) ? lo : hi;
}

double oracle_budget_residual(const double *r, int64_t n, double b, double k, double t, int threads)
{
    return (double)budget_residual(r, n, b, k, t, threads);
}

/* Forward: rows x n scores (row-major, fp64), one budget k and scale t for
 * all rows.  Writes p [rows*n] and b [rows].  Returns 0, or -1 on invalid
 * arguments (n < 1, k outside (0, n), t <= 0). */
int oracle_forward(const double *r, int64_t rows, int64_t n, double k, double t,
                   double *p, double *b, int threads)
{
    if (rows < 1 || n < 1 || !(k > 0.0) || !(k < (double)n) || !(t > 0.0))
        return -1;
    int inner = rows >= threads ? 1 : threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1) if (rows > 1 && threads > 1)
#endif
    for (int64_t row = 0; row < rows; ++row) {
        const double *rr = r + row * n;
        double bb = bisect_threshold(rr, n, k, t, inner);
        b[row] = bb;
        for (int64_t i = 0; i < n; ++i)
            p[row * n + i] = laplace_cdf((rr[i] - bb) / t);
    }
    return 0;
}

/* Backward (section 2.1: analytic VJP).  Implicit differentiation of
 * sum_i F((r_i - b)/t) = k gives, with d_i = F'((r_i - b)/t)/t
 * = exp(-|r_i - b|/t) / (2t):
 *     db/dr_j = d_j / D,  db/dk = -1/D,  D = sum_i d_i,
 * hence for an upstream gradient g on p
 *     dk   = sum_i g_i d_i / D,
 *     dr_j = d_j (g_j - dk).
 * dk is a weighted mean of g, so it is formed with weights rescaled by the
 * largest one (exactly the same ratio, no underflow when t is tiny). */
int oracle_backward(const double *r, const double *b, const double *g, int64_t rows, int64_t n,
                    double t, double *dr, double *dk, int threads)
{
    if (rows < 1 || n < 1 || !(t > 0.0))
        return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1) if (rows > 1 && threads > 1)
#endif
    for (int64_t row = 0; row < rows; ++row) {
        const double *rr = r + row * n, *gg = g + row * n;
        double bb = b[row];
        double amin = INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double a = fabs(rr[i] - bb);
            if (a < amin) amin = a;
        }
        long double wsum = 0.0L, gwsum = 0.0L;
        for (int64_t i = 0; i < n; ++i) {
            double w = exp(-(fabs(rr[i] - bb) - amin) / t);
            wsum += w;
            gwsum += (long double)gg[i] * w;
        }
        double dkk = (double)(gwsum / wsum);
        dk[row] = dkk;
        for (int64_t i = 0; i < n; ++i) {
            double d = 0.5 * exp(-fabs(rr[i] - bb) / t) / t;
            dr[row * n + i] = d * (gg[i] - dkk);
        }
    }
    return 0;
}

static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

/* Section 2.2, full-sort solver, on one row, in the pages' order:
 *  1. sort the scores ascending: s_0 <= ... <= s_{n-1};
 *  2. one stable prefix scan and one stable suffix scan of shifted
 *     exponentials (every multiplier is <= 1, so nothing overflows):
 *        P_j = sum_{i<=j} exp((s_i - s_j)/t)   (P_j = P_{j-1} e^{-(s_j-s_{j-1})/t} + 1)
 *        S_j = sum_{i>=j} exp(-(s_i - s_j)/t)  (S_j = S_{j+1} e^{-(s_{j+1}-s_j)/t} + 1)
 *     giving the threshold curve at the knots,
 *        g_j = f(s_j) = (P_j - 1)/2 + (n - j) - S_j/2,  non-increasing in j;
 *  3. index lookup: the largest j with g_j >= k, so b lies in [s_j, s_{j+1});
 *     b < s_0 when k > g_0 and b >= s_{n-1} when g_{n-1} >= k;
 *  4. closed-form root in that interval.  With y = exp((b - s_j)/t),
 *     A = P_j/2, B = (S_j - 1)/2 = exp(-(s_{j+1}-s_j)/t) S_{j+1}/2 and
 *     c = n - j - 1, the budget reads A/y + c - B y = k, a quadratic
 *     B y^2 - (c - k) y - A = 0 whose positive root is taken in a
 *     cancellation-free form.
 * Writes b and the located index j (-1 when b < s_0).  Returns 0 or -1. */
int oracle_solve_sorted(const double *r, int64_t n, double k, double t, double *b_out, int64_t *j_out)
{
    if (n < 1 || !(k > 0.0) || !(k < (double)n) || !(t > 0.0))
        return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *P = (double *)malloc(sizeof(double) * (size_t)n);
    double *S = (double *)malloc(sizeof(double) * (size_t)n);
    if (!s || !P || !S) {
        free(s); free(P); free(S);
        return -1;
    }
    memcpy(s, r, sizeof(double) * (size_t)n);
    qsort(s, (size_t)n, sizeof(double), cmp_double);

    P[0] = 1.0;
    for (int64_t j = 1; j < n; ++j)
        P[j] = P[j - 1] * exp(-(s[j] - s[j - 1]) / t) + 1.0;
    S[n - 1] = 1.0;
    for (int64_t j = n - 2; j >= 0; --j)
        S[j] = S[j + 1] * exp(-(s[j + 1] - s[j]) / t) + 1.0;

    int64_t j = -1;
    for (int64_t i = 0; i < n; ++i) {
        double g = 0.5 * (P[i] - 1.0) + (double)(n - i) - 0.5 * S[i];
        if (g >= k)
            j = i;   /* g is non-increasing: keep the last index that passes */
    }

    double bb;
    if (j < 0) {
        /* every score above b: n - S_0 e^{(b - s_0)/t} / 2 = k */
        bb = s[0] + t * log(2.0 * ((double)n - k) / S[0]);
    } else if (j == n - 1) {
        /* every score below b: P_{n-1} e^{(s_{n-1} - b)/t} / 2 = k */
        bb = s[n - 1] + t * log(P[n - 1] / (2.0 * k));
    } else {
        double delta = (s[j + 1] - s[j]) / t;
        double A = 0.5 * P[j];
        double lnB = log(0.5 * S[j + 1]) - delta;     /* B = S_{j+1} e^{-delta} / 2 */
        double e = (double)(n - j - 1) - k;
        /* ln of |e| + sqrt(e^2 + 4AB), with 4AB possibly far below e^2 or far above */
        double lh = 0.5 * (log(4.0 * A) + lnB);       /* ln sqrt(4AB) */
        double le = e != 0.0 ? log(fabs(e)) : -INFINITY;
        double m = le > lh ? le : lh;
        double lsum = m + log(exp(le - m) + sqrt(exp(2.0 * (le - m)) + exp(2.0 * (lh - m))));
        double lny;
        if (e >= 0.0)
            lny = lsum - log(2.0) - lnB;              /* y = (e + sqrt(.)) / (2B) */
        else
            lny = log(2.0 * A) - lsum;                /* y = 2A / (-e + sqrt(.)) */
        bb = s[j] + t * lny;
        if (bb < s[j]) bb = s[j];
        if (bb > s[j + 1]) bb = s[j + 1];
    }
    *b_out = bb;
    if (j_out)
        *j_out = j;
    free(s); free(P); free(S);
    return 0;
}

/* Section 2.2, bracketing step 2, for a given bracket [aL, aR) (either end
 * may be infinite): counts and tail sums shifted to the bracket ends,
 *   c_L = #{r < aL},  S_L = sum_{r < aL} exp((r - aL)/t),
 *   c_R = #{r >= aR}, S_R = sum_{r >= aR} exp(-(r - aR)/t),
 *   M   = #{aL <= r < aR}  (the uncertain middle band). */
void oracle_tail_sums(const double *r, int64_t n, double aL, double aR, double t,
                      double *SL, double *SR, int64_t *cL, int64_t *cR, int64_t *M)
{
    long double sl = 0.0L, sr = 0.0L;
    int64_t nl = 0, nr = 0, nm = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (r[i] < aL) {
            nl++;
            sl += exp((r[i] - aL) / t);
        } else if (r[i] >= aR) {
            nr++;
            sr += exp(-(r[i] - aR) / t);
        } else {
            nm++;
        }
    }
    *SL = (double)sl;
    *SR = (double)sr;
    *cL = nl;
    *cR = nr;
    *M = nm;
}

/* Section 2.3, relation to DFTopK: DFTopK fixes the threshold at the
 * midpoint between the k-th and the (k+1)-th largest score instead of
 * solving the budget equation, and the pages show it is the zero-temperature
 * limit of LapSum.  At a positive temperature the mass the Laplace kernel
 * assigns at that fixed threshold,
 *     mass = sum_i F((r_i - b_mid)/t),   b_mid = (s_(k) + s_(k+1)) / 2,
 * drifts away from k (the budget error the pages report for DFTopK).  Here
 * k is an integer with 1 <= k <= n - 1, so both order statistics exist;
 * with the scores sorted ascending, s_(k) = s[n-k] and s_(k+1) = s[n-k-1].
 * Writes b_mid [rows] and mass [rows] (long double sum).  Returns 0 or -1. */
int oracle_midpoint_mass(const double *r, int64_t rows, int64_t n, int64_t k, double t,
                         double *b_mid, double *mass, int threads)
{
    if (rows < 1 || n < 2 || k < 1 || k > n - 1 || !(t > 0.0))
        return -1;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1) if (rows > 1 && threads > 1)
#endif
    for (int64_t row = 0; row < rows; ++row) {
        const double *rr = r + row * n;
        double *s = (double *)malloc(sizeof(double) * (size_t)n);
        if (!s) {
            failed = 1;
            continue;
        }
        memcpy(s, rr, sizeof(double) * (size_t)n);
        qsort(s, (size_t)n, sizeof(double), cmp_double);
        const double bm = 0.5 * (s[n - k] + s[n - k - 1]);
        free(s);
        long double m = 0.0L;
        for (int64_t i = 0; i < n; ++i)
            m += laplace_cdf((rr[i] - bm) / t);
        b_mid[row] = bm;
        mass[row] = (double)m;
    }
    return failed ? -1 : 0;
}
