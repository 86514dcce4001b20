/*
 * Streaming float64 RACE Attention oracle — TEST INFRASTRUCTURE ONLY.
 * Only tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load this library; the GPU library shares no code with it.
 *
 * Computes, for every (batch, head) sequence independently, the RACE
 * Attention forward output and the gradients of <dO, O>, in float64, with a
 * plain per-token recurrence over the sequence (the causal mode is the prefix
 * sum of the Japanese gist.science page, section 2.2). Sources on arXiv
 * 2510.04008 "RACE Attention: A Strictly Linear-Time Attention for
 * Long-Sequence Training":
 *   soft_bucket():   Italian gist.science page, Sommario tecnico section 2,
 *                    Concetti Chiave 2 (random hyperplanes, tanh, softmax over
 *                    hypercube vertices); Korean page, 기술 요약 section 2
 *                    (L tables of P hyperplanes, R = 2^P buckets); Japanese
 *                    page, section 2.2 (temperature beta);
 *   state update:    mass and value sums per bucket (Italian page, section 2,
 *                    Algoritmo; Japanese page, section 2.1);
 *   readout:         normalised weighted average over the L tables (Italian
 *                    page, section 2, Algoritmo; Japanese page, section 2.1).
 *   backward:        exact gradient of the above (the pages state the soft
 *                    sketch is differentiable end to end: Japanese page,
 *                    section 2.2), by the chain rule.
 *
 * Readings where the pages are silent: x_hat = x / max(|x|, 1e-12), V not
 * normalised; corner r has sign +1 on plane p when bit p of r is set, else -1;
 * logits are beta * sum_p sign * tanh(h_p); tables combine as a ratio of sums;
 * causal sums include the diagonal j <= i; W [L, P, d] is shared by queries,
 * keys and all heads; hard id = sum_p [h_p > 0] 2^p.
 *
 * Layouts: Q, K, V, dO are [BH, N, d] row-major in `in_dtype` (0 = float32,
 * 1 = bf16 bit patterns, 2 = float64); W is [L, P, d] float64. `sample`
 * (sorted token indices, shared by every head) selects which rows are written
 * to the outputs ([BH, n_sample, d]); NULL means every row (n_sample = N).
 * Return value: 0 on success, 1 on a bad argument, 2 on allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define EPS 1e-12
#define NEAR_ZERO 1e-5
#define MAXD 256
#define MAXLP 65536
#define MAXLR 65536

static inline double load_in(const void *p, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float *)p)[i];
    if (dtype == 1) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return ((const double *)p)[i];
}

typedef struct {
    int d, P, L, R;
    double beta;
    const double *W;
} cfg_t;

/* Per-row cache of the soft assignment and what its backward needs. */
typedef struct {
    double xh[MAXD];
    double nrm;
    double u[MAXLP];
    double a[MAXLR];
} sb_t;

static inline double corner_sign(int r, int p) { return ((r >> p) & 1) ? 1.0 : -1.0; }

/* Steps 1-3: normalise, project, tanh, corner softmax (per table). */
static void soft_bucket(const cfg_t *c, const void *X, int dtype, size_t row, sb_t *s) {
    const int d = c->d, P = c->P, L = c->L, R = c->R;
    double ss = 0.0;
    for (int k = 0; k < d; ++k) {
        double v = load_in(X, dtype, row * (size_t)d + (size_t)k);
        s->xh[k] = v;
        ss += v * v;
    }
    s->nrm = sqrt(ss);
    double den = s->nrm > EPS ? s->nrm : EPS;
    for (int k = 0; k < d; ++k) s->xh[k] /= den;
    for (int l = 0; l < L; ++l) {
        for (int p = 0; p < P; ++p) {
            const double *w = c->W + ((size_t)l * P + p) * d;
            double h = 0.0;
            for (int k = 0; k < d; ++k) h += w[k] * s->xh[k];
            s->u[l * P + p] = tanh(h);
        }
        double *a = s->a + (size_t)l * R;
        double mx = -INFINITY;
        for (int r = 0; r < R; ++r) {
            double lg = 0.0;
            for (int p = 0; p < P; ++p) lg += corner_sign(r, p) * s->u[l * P + p];
            a[r] = c->beta * lg;
            if (a[r] > mx) mx = a[r];
        }
        double tot = 0.0;
        for (int r = 0; r < R; ++r) { a[r] = exp(a[r] - mx); tot += a[r]; }
        for (int r = 0; r < R; ++r) a[r] /= tot;
    }
}

/* Chain rule from dA [L*R] back to dx [d] through steps 3, 2, 1. */
static void soft_bucket_backward(const cfg_t *c, const sb_t *s, const double *dA, double *dx) {
    const int d = c->d, P = c->P, L = c->L, R = c->R;
    double dxh[MAXD];
    for (int k = 0; k < d; ++k) dxh[k] = 0.0;
    for (int l = 0; l < L; ++l) {
        const double *a = s->a + (size_t)l * R;
        const double *g = dA + (size_t)l * R;
        double mean = 0.0;
        for (int r = 0; r < R; ++r) mean += a[r] * g[r];
        for (int p = 0; p < P; ++p) {
            double du = 0.0;
            for (int r = 0; r < R; ++r) du += corner_sign(r, p) * a[r] * (g[r] - mean);
            du *= c->beta;
            double u = s->u[l * P + p];
            double dh = du * (1.0 - u * u);
            const double *w = c->W + ((size_t)l * P + p) * d;
            for (int k = 0; k < d; ++k) dxh[k] += dh * w[k];
        }
    }
    if (s->nrm > EPS) {
        double radial = 0.0;
        for (int k = 0; k < d; ++k) radial += s->xh[k] * dxh[k];
        for (int k = 0; k < d; ++k) dx[k] = (dxh[k] - s->xh[k] * radial) / s->nrm;
    } else {
        for (int k = 0; k < d; ++k) dx[k] = dxh[k] / EPS;
    }
}

/* State: S [L*R, d] value sums and z [L*R] masses. */
static void state_add(const cfg_t *c, double *S, double *z, const double *a, const void *V,
                      int dtype, size_t row) {
    const int d = c->d, LR = c->L * c->R;
    double v[MAXD];
    for (int k = 0; k < d; ++k) v[k] = load_in(V, dtype, row * (size_t)d + (size_t)k);
    for (int f = 0; f < LR; ++f) {
        z[f] += a[f];
        double *s = S + (size_t)f * d;
        for (int k = 0; k < d; ++k) s[k] += a[f] * v[k];
    }
}

static double readout(const cfg_t *c, const double *S, const double *z, const double *a,
                      double *num) {
    const int d = c->d, LR = c->L * c->R;
    for (int k = 0; k < d; ++k) num[k] = 0.0;
    double den = 0.0;
    for (int f = 0; f < LR; ++f) {
        den += a[f] * z[f];
        const double *s = S + (size_t)f * d;
        for (int k = 0; k < d; ++k) num[k] += a[f] * s[k];
    }
    return den;
}

static int check(int d, int P, int L) {
    return d >= 1 && d <= MAXD && P >= 1 && P <= 12 && L >= 1 && L * P <= MAXLP &&
           L * (1 << P) <= MAXLR;
}

int oracle_forward(const void *Q, const void *K, const void *V, int in_dtype, const double *W,
                   int64_t BH, int64_t N, int d, int P, int L, double beta, int causal,
                   const int64_t *sample, int64_t n_sample, double *O, double *Dout) {
    if (!check(d, P, L) || BH < 0 || N < 0) return 1;
    cfg_t c = {d, P, L, 1 << P, beta, W};
    const int64_t n_out = sample ? n_sample : N;
    int status = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const size_t LR = (size_t)L << P;
        double *S = calloc(LR * d, sizeof(double));
        double *z = calloc(LR, sizeof(double));
        sb_t *sb = malloc(sizeof(sb_t));
        double num[MAXD];
        if (!S || !z || !sb) { status = 2; free(S); free(z); free(sb); continue; }
        const size_t base = (size_t)bh * (size_t)N;
        int64_t next = 0;  /* index into sample */
        if (!causal) {
            for (int64_t j = 0; j < N; ++j) {
                soft_bucket(&c, K, in_dtype, base + j, sb);
                state_add(&c, S, z, sb->a, V, in_dtype, base + j);
            }
        }
        for (int64_t i = 0; i < N; ++i) {
            if (causal) {
                soft_bucket(&c, K, in_dtype, base + i, sb);
                state_add(&c, S, z, sb->a, V, in_dtype, base + i);
            }
            int64_t slot = -1;
            if (!sample) slot = i;
            else if (next < n_sample && sample[next] == i) slot = next++;
            if (slot < 0) continue;
            soft_bucket(&c, Q, in_dtype, base + i, sb);
            double den = readout(&c, S, z, sb->a, num);
            double *o = O + ((size_t)bh * n_out + slot) * d;
            for (int k = 0; k < d; ++k) o[k] = num[k] / den;
            if (Dout) Dout[(size_t)bh * n_out + slot] = den;
        }
        free(S); free(z); free(sb);
    }
    return status;
}

int oracle_backward(const void *Q, const void *K, const void *V, const void *dO, int in_dtype,
                    const double *W, int64_t BH, int64_t N, int d, int P, int L, double beta,
                    int causal, const int64_t *sample, int64_t n_sample, double *dQ, double *dK,
                    double *dV) {
    if (!check(d, P, L) || BH < 0 || N < 0) return 1;
    cfg_t c = {d, P, L, 1 << P, beta, W};
    const int64_t n_out = sample ? n_sample : N;
    int status = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const size_t LR = (size_t)L << P;
        const size_t E = (size_t)d + 1;
        double *S = calloc(LR * d, sizeof(double));
        double *z = calloc(LR, sizeof(double));
        double *T = calloc(LR * E, sizeof(double));   /* [L*R, d+1]: sums of a_Q [g | e] */
        double *Dv = malloc((size_t)N * sizeof(double) + 1);
        double *ev = malloc((size_t)N * sizeof(double) + 1);
        double *dA = malloc(LR * sizeof(double));
        sb_t *sb = malloc(sizeof(sb_t));
        if (!S || !z || !T || !Dv || !ev || !dA || !sb) {
            status = 2;
            free(S); free(z); free(T); free(Dv); free(ev); free(dA); free(sb);
            continue;
        }
        const size_t base = (size_t)bh * (size_t)N;
        double num[MAXD], g[MAXD], v[MAXD], dx[MAXD];
        if (!causal) {
            for (int64_t j = 0; j < N; ++j) {
                soft_bucket(&c, K, in_dtype, base + j, sb);
                state_add(&c, S, z, sb->a, V, in_dtype, base + j);
            }
        }
        /* pass 1, sequence order: O, D, e and the query-side gradient */
        int64_t next = 0;
        for (int64_t i = 0; i < N; ++i) {
            if (causal) {
                soft_bucket(&c, K, in_dtype, base + i, sb);
                state_add(&c, S, z, sb->a, V, in_dtype, base + i);
            }
            soft_bucket(&c, Q, in_dtype, base + i, sb);
            double den = readout(&c, S, z, sb->a, num);
            double dot = 0.0;
            for (int k = 0; k < d; ++k) {
                double go = load_in(dO, in_dtype, (base + i) * (size_t)d + k);
                g[k] = go / den;
                dot += go * (num[k] / den);
            }
            double e = -dot / den;
            Dv[i] = den;
            ev[i] = e;
            if (!causal) {
                for (size_t f = 0; f < LR; ++f) {
                    double *t = T + f * E;
                    for (int k = 0; k < d; ++k) t[k] += sb->a[f] * g[k];
                    t[d] += sb->a[f] * e;
                }
            }
            int64_t slot = -1;
            if (!sample) slot = i;
            else if (next < n_sample && sample[next] == i) slot = next++;
            if (slot < 0) continue;
            for (size_t f = 0; f < LR; ++f) {
                const double *s = S + f * d;
                double acc = z[f] * e;
                for (int k = 0; k < d; ++k) acc += s[k] * g[k];
                dA[f] = acc;
            }
            soft_bucket_backward(&c, sb, dA, dx);
            memcpy(dQ + ((size_t)bh * n_out + slot) * d, dx, sizeof(double) * d);
        }
        /* pass 2, reverse order (causal) or any order (non-causal): key side */
        int64_t prev = n_sample - 1;
        for (int64_t j = N - 1; j >= 0; --j) {
            /* every sampled row is written: the earlier tokens change nothing
               that is returned */
            if (sample && prev < 0) break;
            if (causal) {
                soft_bucket(&c, Q, in_dtype, base + j, sb);
                for (int k = 0; k < d; ++k)
                    g[k] = load_in(dO, in_dtype, (base + j) * (size_t)d + k) / Dv[j];
                for (size_t f = 0; f < LR; ++f) {
                    double *t = T + f * E;
                    for (int k = 0; k < d; ++k) t[k] += sb->a[f] * g[k];
                    t[d] += sb->a[f] * ev[j];
                }
            }
            int64_t slot = -1;
            if (!sample) slot = j;
            else if (prev >= 0 && sample[prev] == j) slot = prev--;
            if (slot < 0) continue;
            soft_bucket(&c, K, in_dtype, base + j, sb);
            for (int k = 0; k < d; ++k) v[k] = load_in(V, in_dtype, (base + j) * (size_t)d + k);
            double *dv = dV + ((size_t)bh * n_out + slot) * d;
            for (int k = 0; k < d; ++k) dv[k] = 0.0;
            for (size_t f = 0; f < LR; ++f) {
                const double *t = T + f * E;
                double acc = t[d];
                for (int k = 0; k < d; ++k) {
                    dv[k] += sb->a[f] * t[k];
                    acc += t[k] * v[k];
                }
                dA[f] = acc;
            }
            soft_bucket_backward(&c, sb, dA, dx);
            memcpy(dK + ((size_t)bh * n_out + slot) * d, dx, sizeof(double) * d);
        }
        free(S); free(z); free(T); free(Dv); free(ev); free(dA); free(sb);
    }
    return status;
}

/* Hard-hash diagnostic: ids [rows, L] and the number of |h| < 1e-5 projections. */
int oracle_hash(const void *X, int in_dtype, const double *W, int64_t rows, int d, int P, int L,
                int32_t *ids, int64_t *near_zero) {
    if (d < 1 || d > MAXD || P < 1 || P > 30 || L < 1 || rows < 0) return 1;
    int64_t nz = 0;
    #pragma omp parallel for schedule(static) reduction(+ : nz)
    for (int64_t n = 0; n < rows; ++n) {
        double xh[MAXD], ss = 0.0;
        for (int k = 0; k < d; ++k) {
            xh[k] = load_in(X, in_dtype, (size_t)n * d + k);
            ss += xh[k] * xh[k];
        }
        double den = sqrt(ss) > EPS ? sqrt(ss) : EPS;
        for (int k = 0; k < d; ++k) xh[k] /= den;
        for (int l = 0; l < L; ++l) {
            int32_t id = 0;
            for (int p = 0; p < P; ++p) {
                const double *w = W + ((size_t)l * P + p) * d;
                double h = 0.0;
                for (int k = 0; k < d; ++k) h += w[k] * xh[k];
                if (h > 0.0) id |= 1 << p;
                if (fabs(h) < NEAR_ZERO) ++nz;
            }
            ids[(size_t)n * L + l] = id;
        }
    }
    *near_zero = nz;
    return 0;
}
