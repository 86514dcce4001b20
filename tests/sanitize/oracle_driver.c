/* Drives every entry point of the C oracle (oracle/race_oracle.c) on small
 * inputs in all three input types, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (tests/test_sanitizers.py). Exit status 0
 * when every call returns 0 and every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_forward(const void *Q, const void *K, const void *V, int in_dtype, const double *W, int64_t BH,
                   int64_t N, int d, int P, int L, double beta, int causal, const int64_t *sample,
                   int64_t n_sample, double *O, double *Dout);
int oracle_backward(const void *Q, const void *K, const void *V, const void *dO, int in_dtype, const double *W,
                    int64_t BH, int64_t N, int d, int P, int L, double beta, int causal, const int64_t *sample,
                    int64_t n_sample, double *dQ, double *dK, double *dV);
int oracle_hash(const void *X, int in_dtype, const double *W, int64_t rows, int d, int P, int L, int32_t *ids,
                int64_t *near_zero);

static uint64_t state = 88172645463325252ull;
static double uniform(void) {   /* xorshift64 */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

/* n values of type dtype (0 float32, 1 bf16 bits, 2 float64) in a fresh buffer */
static void *make(int dtype, size_t n) {
    size_t es = dtype == 0 ? 4 : dtype == 1 ? 2 : 8;
    unsigned char *p = malloc(n * es);
    for (size_t i = 0; i < n; ++i) {
        double v = uniform();
        if (dtype == 0) { float f = (float)v; memcpy(p + 4 * i, &f, 4); }
        else if (dtype == 1) { float f = (float)v; uint32_t u; memcpy(&u, &f, 4); uint16_t h = (uint16_t)(u >> 16); memcpy(p + 2 * i, &h, 2); }
        else memcpy(p + 8 * i, &v, 8);
    }
    return p;
}

static int finite_all(const double *x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    int bad = 0;
    const int shapes[][4] = {{5, 8, 1, 3}, {33, 16, 4, 5}, {17, 8, 6, 2}, {1, 4, 2, 1}};
    for (int dt = 0; dt < 3; ++dt)
        for (size_t si = 0; si < sizeof(shapes) / sizeof(shapes[0]); ++si) {
            const int N = shapes[si][0], d = shapes[si][1], P = shapes[si][2], L = shapes[si][3];
            const int64_t BH = 2;
            const size_t n = (size_t)BH * N * d;
            void *Q = make(dt, n), *K = make(dt, n), *V = make(dt, n), *dO = make(dt, n);
            double *W = make(2, (size_t)L * P * d);
            double *O = malloc(n * 8), *D = malloc((size_t)BH * N * 8);
            double *dQ = malloc(n * 8), *dK = malloc(n * 8), *dV = malloc(n * 8);
            int64_t smp[2] = {0, N - 1};
            for (int causal = 0; causal < 2; ++causal) {
                bad |= oracle_forward(Q, K, V, dt, W, BH, N, d, P, L, 1.3, causal, NULL, 0, O, D);
                bad |= !finite_all(O, n);
                bad |= oracle_backward(Q, K, V, dO, dt, W, BH, N, d, P, L, 0.7, causal, NULL, 0, dQ, dK, dV);
                bad |= !finite_all(dQ, n) | !finite_all(dK, n) | !finite_all(dV, n);
                const int64_t ns = N > 1 ? 2 : 1;
                bad |= oracle_forward(Q, K, V, dt, W, BH, N, d, P, L, 1.0, causal, smp, ns, O, D);
                bad |= oracle_backward(Q, K, V, dO, dt, W, BH, N, d, P, L, 1.0, causal, smp, ns, dQ, dK, dV);
            }
            int32_t *ids = malloc((size_t)BH * N * L * 4);
            int64_t nz = 0;
            bad |= oracle_hash(Q, dt, W, BH * N, d, P, L, ids, &nz);
            for (size_t i = 0; i < (size_t)BH * N * L; ++i) bad |= ids[i] < 0 || ids[i] >= (1 << P);
            /* bad arguments are refused */
            bad |= oracle_forward(Q, K, V, dt, W, BH, N, 0, P, L, 1.0, 0, NULL, 0, O, D) == 0;
            bad |= oracle_hash(Q, dt, W, BH * N, d, 0, L, ids, &nz) == 0;
            free(Q); free(K); free(V); free(dO); free(W); free(O); free(D); free(dQ); free(dK); free(dV); free(ids);
        }
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad ? 1 : 0;
}
