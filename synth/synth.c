/*
 * Seeded synthetic inputs (host side).
 *
 * This module draws the random inputs that both the CPU oracle and the GPU
 * library consume. It holds none of the attention method's arithmetic: it only
 * turns (seed, tensor id, flat element index) into numbers.
 *
 * Generator: Philox-4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11),
 * written here from that definition:
 *   round:  (hi0,lo0) = mulhilo(0xD2511F53, c0); (hi1,lo1) = mulhilo(0xCD9E8D57, c2)
 *           c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
 *   key schedule between rounds: k0 += 0x9E3779B9, k1 += 0xBB67AE85
 *   10 rounds.
 *
 * Stream definition (shared with the device generator):
 *   key     = (seed & 0xffffffff, tensor_id)
 *   counter = (m & 0xffffffff, m >> 32, 0, 0) for pair index m = i / 2
 *   u1 = ((x1:x0) >> 11) + 0.5) * 2^-53,  u2 = ((x3:x2) >> 11) + 0.5) * 2^-53
 *   Box-Muller in double: r = sqrt(-2 ln u1); element 2m = r cos(2 pi u2),
 *   element 2m+1 = r sin(2 pi u2); multiplied by `scale`.
 *   Rounding: double -> float (round to nearest even) -> bf16 (round to
 *   nearest even) for bf16 tensors.
 *
 * Mixture stream (the clustered query/key workload): 64 centres g_m drawn
 * from tensor id 5 with standard deviation `centre_sd` (shared by every
 * batch/head); the cluster of row n is (x0 of Philox(counter=(n_lo,n_hi,0,0),
 * key=(seed, id_tensor))) mod n_centres; the row is the centre plus
 * noise_sd times the row's own normal stream, then scaled to unit length
 * in double before rounding.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct { uint32_t v[4]; } p4;

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

static p4 philox4x32_10(p4 c, uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(0xD2511F53u, c.v[0], &hi0, &lo0);
        mulhilo(0xCD9E8D57u, c.v[2], &hi1, &lo1);
        p4 o;
        o.v[0] = hi1 ^ c.v[1] ^ k0;
        o.v[1] = lo1;
        o.v[2] = hi0 ^ c.v[3] ^ k1;
        o.v[3] = lo0;
        c = o;
    }
    return c;
}

/* Raw Philox block, exposed for the known-answer test. */
void synth_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    p4 c = {{ctr[0], ctr[1], ctr[2], ctr[3]}};
    p4 o = philox4x32_10(c, key[0], key[1]);
    memcpy(out, o.v, sizeof(o.v));
}

static inline void normal_pair(uint64_t seed, uint32_t tid, uint64_t m, double *n0, double *n1) {
    p4 c = {{(uint32_t)m, (uint32_t)(m >> 32), 0u, 0u}};
    p4 x = philox4x32_10(c, (uint32_t)seed, tid);
    uint64_t a = ((uint64_t)x.v[1] << 32) | x.v[0];
    uint64_t b = ((uint64_t)x.v[3] << 32) | x.v[2];
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53;
    double u2 = ((double)(b >> 11) + 0.5) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    *n0 = r * cos(t);
    *n1 = r * sin(t);
}

static inline double normal_at(uint64_t seed, uint32_t tid, uint64_t i) {
    double n0, n1;
    normal_pair(seed, tid, i >> 1, &n0, &n1);
    return (i & 1) ? n1 : n0;
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  /* NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

/* Fill n elements starting at flat index `start`; dtype 0 = f32, 1 = bf16, 2 = f64. */
void synth_normal(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, double scale,
                  int dtype, void *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        double v = scale * normal_at(seed, tid, start + (uint64_t)j);
        if (dtype == 0) ((float *)out)[j] = (float)v;
        else if (dtype == 1) ((uint16_t *)out)[j] = f32_to_bf16_rne((float)v);
        else ((double *)out)[j] = v;
    }
}

/* Mixture rows: rows [row0, row0+nrows) of a [*, d] tensor whose rows are
 * unit-length draws around one of n_centres centres. */
void synth_mixture(uint64_t seed, uint32_t tid_noise, uint32_t tid_ids, uint32_t tid_centres,
                   int n_centres, double centre_sd, double noise_sd, int d,
                   uint64_t row0, uint64_t nrows, int dtype, void *out) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)nrows; ++j) {
        uint64_t n = row0 + (uint64_t)j;
        p4 c = {{(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u}};
        p4 x = philox4x32_10(c, (uint32_t)seed, tid_ids);
        uint32_t cid = x.v[0] % (uint32_t)n_centres;
        double row[1024];
        double ss = 0.0;
        for (int e = 0; e < d; ++e) {
            double g = centre_sd * normal_at(seed, tid_centres, (uint64_t)cid * (uint64_t)d + (uint64_t)e);
            double v = g + noise_sd * normal_at(seed, tid_noise, n * (uint64_t)d + (uint64_t)e);
            row[e] = v;
            ss += v * v;
        }
        double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        for (int e = 0; e < d; ++e) {
            double v = row[e] * inv;
            size_t o = (size_t)j * (size_t)d + (size_t)e;
            if (dtype == 0) ((float *)out)[o] = (float)v;
            else if (dtype == 1) ((uint16_t *)out)[o] = f32_to_bf16_rne((float)v);
            else ((double *)out)[o] = v;
        }
    }
}
