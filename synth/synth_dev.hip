// Seeded synthetic inputs (device side): the same Philox-4x32-10 stream and
// Box-Muller definition as synth.c, used to fill HBM directly at sizes where a
// host round trip would dominate. Holds no attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct P4 { uint32_t v[4]; };

__device__ inline P4 philox10(P4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint32_t lo0 = 0xD2511F53u * c.v[0];
        uint32_t hi0 = __umulhi(0xD2511F53u, c.v[0]);
        uint32_t lo1 = 0xCD9E8D57u * c.v[2];
        uint32_t hi1 = __umulhi(0xCD9E8D57u, c.v[2]);
        P4 o;
        o.v[0] = hi1 ^ c.v[1] ^ k0;
        o.v[1] = lo1;
        o.v[2] = hi0 ^ c.v[3] ^ k1;
        o.v[3] = lo0;
        c = o;
    }
    return c;
}

__device__ inline double normal_at(uint64_t seed, uint32_t tid, uint64_t i) {
    uint64_t m = i >> 1;
    P4 c = {{(uint32_t)m, (uint32_t)(m >> 32), 0u, 0u}};
    P4 x = philox10(c, (uint32_t)seed, tid);
    uint64_t a = ((uint64_t)x.v[1] << 32) | x.v[0];
    uint64_t b = ((uint64_t)x.v[3] << 32) | x.v[2];
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53;
    double u2 = ((double)(b >> 11) + 0.5) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ inline void store(void* out, uint64_t o, double v, int dtype) {
    if (dtype == 0) reinterpret_cast<float*>(out)[o] = (float)v;
    else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne((float)v);
}

__global__ void k_normal(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, double scale,
                         int dtype, void* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride)
        store(out, j, scale * normal_at(seed, tid, start + j), dtype);
}

__global__ void k_mixture(uint64_t seed, uint32_t tid_noise, uint32_t tid_ids, uint32_t tid_c,
                          int n_centres, double centre_sd, double noise_sd, int d,
                          uint64_t row0, uint64_t nrows, int dtype, void* out) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nrows; j += stride) {
        uint64_t n = row0 + j;
        P4 c = {{(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u}};
        P4 x = philox10(c, (uint32_t)seed, tid_ids);
        uint32_t cid = x.v[0] % (uint32_t)n_centres;
        double ss = 0.0;
        for (int e = 0; e < d; ++e) {
            double v = centre_sd * normal_at(seed, tid_c, (uint64_t)cid * d + e) +
                       noise_sd * normal_at(seed, tid_noise, n * (uint64_t)d + e);
            ss += v * v;
        }
        double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
        for (int e = 0; e < d; ++e) {
            double v = centre_sd * normal_at(seed, tid_c, (uint64_t)cid * d + e) +
                       noise_sd * normal_at(seed, tid_noise, n * (uint64_t)d + e);
            store(out, j * (uint64_t)d + e, v * inv, dtype);
        }
    }
}

}  // namespace

extern "C" int synth_dev_normal(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n,
                                double scale, int dtype, void* out, void* stream) {
    if (n == 0) return 0;
    if (!out || (dtype != 0 && dtype != 1)) return 1;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_normal, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       seed, tid, start, n, scale, dtype, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int synth_dev_mixture(uint64_t seed, uint32_t tid_noise, uint32_t tid_ids,
                                 uint32_t tid_c, int n_centres, double centre_sd, double noise_sd,
                                 int d, uint64_t row0, uint64_t nrows, int dtype, void* out,
                                 void* stream) {
    if (nrows == 0) return 0;
    if (!out || d <= 0 || n_centres <= 0 || (dtype != 0 && dtype != 1)) return 1;
    uint64_t blocks = (nrows + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_mixture, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       seed, tid_noise, tid_ids, tid_c, n_centres, centre_sd, noise_sd, d, row0,
                       nrows, dtype, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
