/*
 * Plain C, fp64 CPU oracle for FAVOR+ attention.
 *
 * TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library.
 *
 * It follows the definitions on the pages, written out as plain loops:
 *   - positive random features phi(x)_i = m^-1/2 exp(omega_i.x - |x|^2/2)
 *     ("Performer" digest, irregular6612.github.io: core components and key
 *     formulas; Su Jianlin, "From Performer to Linear Attention": Simple
 *     Derivation);
 *   - bidirectional FAVOR+: KV = sum_s phi(k_s) v_s^T, z = sum_s phi(k_s),
 *     out_t = phi(q_t).KV / phi(q_t).z (digest: key formulas, flowchart);
 *   - causal FAVOR+ by the prefix-sum recurrence G_t = sum_{s<=t} phi(k_s)
 *     v_s^T, z_t = sum_{s<=t} phi(k_s) (digest: Methods and core components;
 *     paperlayer.ai summary of arXiv:2009.14794v4, A.2 unidirectional
 *     attention).
 * No stabiliser (fp64 exp has the range needed), no epsilon in the
 * normaliser, inclusive causal mask.
 *
 * Layouts: q, k, v, out are [B, H, L, d] row-major doubles; omega is [m, d]
 * (omega_per_head = 0) or [H, m, d] (omega_per_head = 1), the same for every
 * batch element.  Heads run in parallel with OpenMP; everything inside a head
 * is sequential.
 */
#include <math.h>
#include <stdlib.h>

static const double *head_omega(const double *omega, int omega_per_head, int h, int m, int d) {
    return omega_per_head ? omega + (size_t)h * m * d : omega;
}

/* phi(x) for one row x[d] into phi[m]. */
static void feature_row(const double *x, const double *om, int d, int m, double *phi) {
    double sq = 0.0;
    for (int j = 0; j < d; ++j) sq += x[j] * x[j];
    double scale = 1.0 / sqrt((double)m);
    for (int i = 0; i < m; ++i) {
        double p = 0.0;
        for (int j = 0; j < d; ++j) p += om[(size_t)i * d + j] * x[j];
        phi[i] = scale * exp(p - 0.5 * sq);
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* phi for n_rows rows x[n_rows, d] with one omega[m, d]; phi is [n_rows, m]. */
void oracle_features(long n_rows, int d, int m, const double *x, const double *omega, double *phi) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < n_rows; ++r) feature_row(x + (size_t)r * d, omega, d, m, phi + (size_t)r * m);
}

int oracle_bidir(int B, int H, int L, int d, int m, const double *q, const double *k, const double *v,
                 const double *omega, int omega_per_head, double *out) {
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int bh = 0; bh < B * H; ++bh) {
        int h = bh % H;
        const double *om = head_omega(omega, omega_per_head, h, m, d);
        size_t base = (size_t)bh * L * d;
        double *kv = calloc((size_t)m * d, sizeof(double));
        double *z = calloc((size_t)m, sizeof(double));
        double *phi = malloc((size_t)m * sizeof(double));
        if (!kv || !z || !phi) {
            failed = 1;
        } else {
            for (int s = 0; s < L; ++s) {
                feature_row(k + base + (size_t)s * d, om, d, m, phi);
                const double *vs = v + base + (size_t)s * d;
                for (int i = 0; i < m; ++i) {
                    z[i] += phi[i];
                    for (int j = 0; j < d; ++j) kv[(size_t)i * d + j] += phi[i] * vs[j];
                }
            }
            for (int t = 0; t < L; ++t) {
                feature_row(q + base + (size_t)t * d, om, d, m, phi);
                double den = 0.0;
                for (int i = 0; i < m; ++i) den += phi[i] * z[i];
                double *o = out + base + (size_t)t * d;
                for (int j = 0; j < d; ++j) {
                    double num = 0.0;
                    for (int i = 0; i < m; ++i) num += phi[i] * kv[(size_t)i * d + j];
                    o[j] = num / den;
                }
            }
        }
        free(kv);
        free(z);
        free(phi);
    }
    return failed ? -1 : 0;
}

int oracle_causal(int B, int H, int L, int d, int m, const double *q, const double *k, const double *v,
                  const double *omega, int omega_per_head, double *out) {
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int bh = 0; bh < B * H; ++bh) {
        int h = bh % H;
        const double *om = head_omega(omega, omega_per_head, h, m, d);
        size_t base = (size_t)bh * L * d;
        double *G = calloc((size_t)m * d, sizeof(double));
        double *z = calloc((size_t)m, sizeof(double));
        double *phik = malloc((size_t)m * sizeof(double));
        double *phiq = malloc((size_t)m * sizeof(double));
        if (!G || !z || !phik || !phiq) {
            failed = 1;
        } else {
            for (int t = 0; t < L; ++t) {
                /* G_t = G_{t-1} + phi(k_t) v_t^T ; z_t = z_{t-1} + phi(k_t) */
                feature_row(k + base + (size_t)t * d, om, d, m, phik);
                const double *vt = v + base + (size_t)t * d;
                for (int i = 0; i < m; ++i) {
                    z[i] += phik[i];
                    for (int j = 0; j < d; ++j) G[(size_t)i * d + j] += phik[i] * vt[j];
                }
                /* out_t = phi(q_t).G_t / phi(q_t).z_t */
                feature_row(q + base + (size_t)t * d, om, d, m, phiq);
                double den = 0.0;
                for (int i = 0; i < m; ++i) den += phiq[i] * z[i];
                double *o = out + base + (size_t)t * d;
                for (int j = 0; j < d; ++j) {
                    double num = 0.0;
                    for (int i = 0; i < m; ++i) num += phiq[i] * G[(size_t)i * d + j];
                    o[j] = num / den;
                }
            }
        }
        free(G);
        free(z);
        free(phik);
        free(phiq);
    }
    return failed ? -1 : 0;
}
