/*
 * qknorm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference for layerwise QK-Norm. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product library never links or calls it, and it shares no code, header or
 * constant with the HIP sources.
 *
 * What it computes (SwiftQK technical review, "Prerequisites", Eq. 1):
 *     y_j = x_j / sqrt( (1/H) * sum_{i=1..H} x_i^2 + eps ) * gamma_j
 * for every token row of the projected query and, separately, the projected
 * key ("Layerwise vs. headwise QK-Norm": one statistic over the whole
 * projected width of each tensor).
 *
 * The sum of squares is kept in the slice structure of the review's
 * section 4b worked example (Eqs. 3-5): the row is cut into K equal,
 * contiguous column slices, slice 0 holding the first columns; each slice
 * yields one partial sum, and the partials are added in ascending slice
 * order. The inverse RMS divides by the FULL width (Eq. 6) and adds eps to
 * the mean inside the square root (Eq. 1 and Eq. 6 agree on both points).
 *
 * Precision: inputs arrive as float (exact for bf16 and fp32 data) and are
 * widened to double before any arithmetic; every sum, the square root and
 * the scaling are done in double. No blocking, fusion or reordering beyond
 * the slice structure above: sums run in ascending column order.
 *
 * Threads: the token loop may run on several OpenMP threads (tokens are
 * independent; each row's arithmetic is identical whatever the thread count).
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

/* Number of threads the token loops use (>= 1). Returns the value now in force. */
int oracle_set_threads(int n)
{
    g_threads = n < 1 ? 1 : n;
    return g_threads;
}

int oracle_get_threads(void) { return g_threads; }

/*
 * Per-slice sums of squares (review section 4b, Eqs. 3-4: each shard's
 * "local sum of squares").
 *   x      : T rows; row t starts at x + t*ldx; the first W columns are used
 *   W      : columns in the row part handed in (W % K == 0)
 *   K      : number of equal contiguous slices the W columns are cut into
 *   P      : out, P[s*T + t] = sum over columns j in slice s of x[t][j]^2
 */
void oracle_slice_sumsq(const float *x, int64_t T, int64_t W, int64_t ldx,
                        int K, double *P)
{
    const int64_t w = W / K; /* slice width */
    int64_t t;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (t = 0; t < T; ++t) {
        const float *row = x + t * ldx;
        for (int s = 0; s < K; ++s) {
            double acc = 0.0;
            for (int64_t j = s * w; j < (s + 1) * w; ++j) {
                const double v = (double)row[j];
                acc += v * v;
            }
            P[(int64_t)s * T + t] = acc;
        }
    }
}

/*
 * Combine the slice statistics and normalise (review Eqs. 5-6, then Eq. 1).
 *   x       : T rows of at least W columns (row t at x + t*ldx); the columns
 *             to normalise (a whole row, or one slice of it)
 *   P       : K partial sums per token, P[s*T + t]
 *   gamma   : W weights matching the columns of x
 *   H_total : width of the FULL row the partials cover (the mean divides by it)
 *   eps     : added to the mean inside the square root
 *   y       : out, T rows of W doubles, row t at y + t*ldy
 */
void oracle_apply(const float *x, int64_t T, int64_t W, int64_t ldx,
                  const double *P, int K, const float *gamma,
                  int64_t H_total, double eps, double *y, int64_t ldy)
{
    int64_t t;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (t = 0; t < T; ++t) {
        double S = 0.0;
        for (int s = 0; s < K; ++s) /* Eq. 5: ascending slice order */
            S += P[(int64_t)s * T + t];
        const double rms = sqrt(S / (double)H_total + eps); /* Eq. 1 / Eq. 6 */
        const float *row = x + t * ldx;
        double *out = y + t * ldy;
        for (int64_t j = 0; j < W; ++j)
            out[j] = (double)row[j] / rms * (double)gamma[j]; /* Eq. 1 order */
    }
}

/*
 * Whole forward for one tensor (q or k): the slice sums of all K slices over
 * the full row, then the combine-and-normalise step over the full row.
 * P is caller scratch of K*T doubles and holds the partials on return.
 */
void oracle_forward(const float *x, int64_t T, int64_t H, int64_t ldx,
                    const float *gamma, double eps, int K, double *P,
                    double *y, int64_t ldy)
{
    oracle_slice_sumsq(x, T, H, ldx, K, P);
    oracle_apply(x, T, H, ldx, P, K, gamma, H, eps, y, ldy);
}

/*
 * Headwise QK-Norm (review, "Layerwise vs. headwise QK-Norm": one
 * normalisation factor per attention head instead of one per projected
 * row). Each row's H columns hold H / D heads of D contiguous columns, head
 * 0 first. Head h uses only its own columns: its sum of squares (ascending
 * column order), its mean over D, eps inside the square root as in Eq. 1,
 * and the D weights of gamma, which every head shares.
 *   x     : T rows of H columns (row t at x + t*ldx); H % D == 0
 *   gamma : D weights
 *   y     : out, T rows of H doubles, row t at y + t*ldy
 */
void oracle_headwise(const float *x, int64_t T, int64_t H, int64_t ldx,
                     int64_t D, const float *gamma, double eps,
                     double *y, int64_t ldy)
{
    int64_t t;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (t = 0; t < T; ++t) {
        const float *row = x + t * ldx;
        double *out = y + t * ldy;
        for (int64_t h0 = 0; h0 < H; h0 += D) {
            double S = 0.0;
            for (int64_t j = 0; j < D; ++j) {
                const double v = (double)row[h0 + j];
                S += v * v;
            }
            const double rms = sqrt(S / (double)D + eps);
            for (int64_t j = 0; j < D; ++j)
                out[h0 + j] = (double)row[h0 + j] / rms * (double)gamma[j];
        }
    }
}

/*
 * The per-token inverse RMS alone (review Eq. 6; the statistic a consumer
 * applies itself when the scaling is deferred to it). The sum of squares is
 * formed as in oracle_forward: K slice sums in ascending column order, added
 * in ascending slice order (Eq. 5); the mean divides by the full width H.
 *   r : out, r[t] = 1 / sqrt( S_t / H + eps )
 * P is caller scratch of K*T doubles and holds the partials on return.
 */
void oracle_inv_rms(const float *x, int64_t T, int64_t H, int64_t ldx,
                    int K, double eps, double *P, double *r)
{
    oracle_slice_sumsq(x, T, H, ldx, K, P);
    int64_t t;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (t = 0; t < T; ++t) {
        double S = 0.0;
        for (int s = 0; s < K; ++s)
            S += P[(int64_t)s * T + t];
        r[t] = 1.0 / sqrt(S / (double)H + eps);
    }
}
