/* Sanitizer driver for the plain-C oracle (favor_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (single-threaded: the
 * OpenMP pragmas are ignored without -fopenmp).  Every buffer is an
 * exactly-sized heap allocation; a few shapes, both projection layouts.
 * Test infrastructure only. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_features(long n_rows, int d, int m, const double *x, const double *omega, double *phi);
int oracle_bidir(int B, int H, int L, int d, int m, const double *q, const double *k, const double *v,
                 const double *omega, int omega_per_head, double *out);
int oracle_causal(int B, int H, int L, int d, int m, const double *q, const double *k, const double *v,
                  const double *omega, int omega_per_head, double *out);

static double *fill(size_t n, unsigned *state) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        *state = *state * 1103515245u + 12345u;
        p[i] = ((double)((*state >> 8) & 0xFFFF) / 65536.0 - 0.5) * 0.8;
    }
    return p;
}

int main(void) {
    const int shapes[][5] = {{1, 1, 1, 2, 1}, {1, 2, 17, 4, 3}, {2, 3, 64, 16, 32}, {1, 1, 5, 3, 8}};
    unsigned st = 1;
    int bad = 0;
    for (int c = 0; c < 4; ++c) {
        const int B = shapes[c][0], H = shapes[c][1], L = shapes[c][2], d = shapes[c][3], m = shapes[c][4];
        const size_t n = (size_t)B * H * L * d;
        double *q = fill(n, &st), *k = fill(n, &st), *v = fill(n, &st);
        double *om = fill((size_t)H * m * d, &st);
        double *o1 = malloc(n * sizeof(double)), *o2 = malloc(n * sizeof(double));
        double *phi = malloc((size_t)B * H * L * m * sizeof(double));
        for (int per_head = 0; per_head < 2; ++per_head) {
            if (oracle_bidir(B, H, L, d, m, q, k, v, om, per_head, o1) != 0) bad = 1;
            if (oracle_causal(B, H, L, d, m, q, k, v, om, per_head, o2) != 0) bad = 1;
            /* last causal row = last bidirectional row; all finite */
            for (int bh = 0; bh < B * H; ++bh)
                for (int j = 0; j < d; ++j) {
                    const size_t i = ((size_t)bh * L + L - 1) * d + j;
                    if (!(fabs(o1[i] - o2[i]) <= 1e-12 * (1.0 + fabs(o1[i])))) bad = 1;
                }
            for (size_t i = 0; i < n; ++i)
                if (!isfinite(o1[i]) || !isfinite(o2[i])) bad = 1;
        }
        oracle_features((long)B * H * L, d, m, q, om, phi);
        free(q); free(k); free(v); free(om); free(o1); free(o2); free(phi);
    }
    printf("oracle_driver: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
