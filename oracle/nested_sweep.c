/*
 * Oracle (test infrastructure only): plain sequential float64 GPTQ-2D sweep.
 *
 * Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
 * build, load or call this file.  It shares no code with the GPU library.
 *
 * What it computes.  Two-sided adaptive rounding rounds a real m x n matrix W to
 * Q = diag(s) Z, Z integer in [lo, hi], under the metric tr(A E B E^T), E = W - Q
 * ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", Abstract and Technical
 * contributions; mind-verse.de article "Neue Ansaetze ... durch GPTQ-2D", section
 * "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung": non-singular bases act
 * on both sides of the residual and errors travel through triangular feedback).
 * Row-major vectorisation turns the metric into one quadratic form with Gram
 * matrix A (x) B (article section "Geometrische Grundlagen ..."), and the result is
 * defined as the trajectory of the naive vectorised sweep: one-dimensional GPTQ
 * over the mn coordinates (article section "Die algorithmische Neuerung ...";
 * arXiv page, Results).  The upper Cholesky factor of (A (x) B)^-1 is Ua (x) Ub,
 * so with unit-diagonal factors Ua', Ub' that sweep is, for each coordinate (k,l)
 * in row-major order:
 *     z = clamp(rint(x[k,l] / s_k), lo, hi);  d = x[k,l] - s_k z;
 *     x[i,j] -= d * Ua'[k,i] * Ub'[l,j]      for all i >= k, j >= l, (i,j) != (k,l).
 * Grouping the updates by row gives the cubic "nested" form used here (the
 * feedback is rank-one and separable: arXiv page, Results and Technical
 * contributions):
 *     for each row k in order:
 *         g[l] = W[k,l] - sum_{i<k} Ua'[i,k] R[i,l]          (rows above, i ascending)
 *         t = g;  for l in order: round t[l], push d * Ub'[l, l2] into t[l2 > l]
 *         R[k,l] = g[l] - Q[k,l]
 * R[i,:] is exactly the error row i passes on to the rows below, because the
 * sum over j <= l of d[i,j] Ub'[j,l] equals g_i[l] - Q[i,l].
 *
 * Readings where the pages are silent: natural order (row 0, column 0 first);
 * rint is IEEE round-half-to-even of the IEEE quotient t/s_k; the clamp follows
 * the rint; scales are fixed inputs.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * The optional OpenMP loop only splits the vertical gather over columns; each
 * element's subtraction order (i ascending) is unchanged, so every thread count
 * gives bit-identical output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double round_clamp(double t, double s, int lo, int hi) {
    double z = nearbyint(t / s); /* default rounding mode: to nearest, ties to even */
    if (z < (double)lo) z = (double)lo;
    if (z > (double)hi) z = (double)hi;
    return z;
}

/*
 * W (m x n), Ua (m x m, unit upper), Ub (n x n, unit upper), s (m): float64, row-major.
 * Z (m x n) int32 and Q (m x n) float64 are outputs.  R (m x n float64) is
 * caller-provided scratch that holds the vertical residual on return.  Delta
 * (m x n float64, optional, may be NULL) receives the per-entry step error t - q.
 * Returns the number of OpenMP threads used (1 without OpenMP), or -1 on bad
 * arguments / allocation failure.
 */
int oracle_gptq2d_sweep(int64_t m, int64_t n, const double* W, const double* Ua,
                        const double* Ub, const double* s, int lo, int hi,
                        int32_t* Z, double* Q, double* R, double* Delta, int nthreads) {
    if (m <= 0 || n <= 0 || !W || !Ua || !Ub || !s || !Z || !Q || !R) return -1;
    double* g = (double*)malloc((size_t)n * sizeof(double));
    double* t = (double*)malloc((size_t)n * sizeof(double));
    if (!g || !t) { free(g); free(t); return -1; }
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    used = nthreads;
#else
    (void)nthreads;
#endif
    for (int64_t k = 0; k < m; ++k) {
        /* vertical feedback: the residuals of all rows above, i ascending */
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
        for (int64_t l0 = 0; l0 < n; l0 += 256) {
            int64_t l1 = l0 + 256 < n ? l0 + 256 : n;
            for (int64_t l = l0; l < l1; ++l) g[l] = W[k * n + l];
            for (int64_t i = 0; i < k; ++i) {
                double c = Ua[i * m + k];
                const double* Ri = R + i * n;
                for (int64_t l = l0; l < l1; ++l) g[l] -= c * Ri[l];
            }
        }
        /* horizontal feedback: one-dimensional GPTQ along the row with Ub' */
        memcpy(t, g, (size_t)n * sizeof(double));
        const double sk = s[k];
        for (int64_t l = 0; l < n; ++l) {
            double z = round_clamp(t[l], sk, lo, hi);
            double q = sk * z;
            double d = t[l] - q;
            Z[k * n + l] = (int32_t)z;
            Q[k * n + l] = q;
            if (Delta) Delta[k * n + l] = d;
            const double* Ubl = Ub + l * n;
            for (int64_t l2 = l + 1; l2 < n; ++l2) t[l2] -= d * Ubl[l2];
        }
        for (int64_t l = 0; l < n; ++l) R[k * n + l] = g[l] - Q[k * n + l];
    }
    free(g);
    free(t);
    return used;
}
