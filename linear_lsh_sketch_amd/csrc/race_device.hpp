// Device building blocks shared by the RACE Attention kernels (gfx950).
//
// Matrix-core layout used throughout (16x16 output tiles, 64-lane waves):
//   lane l, ln = l % 16, g = l / 16.
//   A operand (M x K): lane holds row ln, K positions 8g .. 8g+7 of a 32-wide chunk.
//   B operand (K x N): lane holds column ln, K positions 8g .. 8g+7.
//   C/D (M x N): lane holds rows 4g .. 4g+3 of column ln.
// bf16 uses v_mfma_f32_16x16x32_bf16 directly. float32 uses eight
// v_mfma_f32_16x16x4_f32 per 32-wide chunk: MFMA j contracts the j-th value
// of every lane group, so the same per-lane layout covers all 32 positions.
//
// Feature ("canonical f") order. L tables of R = 2^P corners give
// F = L_pad * R features. The hash projection computes H^T = W' X^T, so a lane
// of a projection tile t holds rows 4g..4g+3 (= P' consecutive planes of one
// table when P' = 4, or several whole tables when P' < 4) for one token. The
// features the lane derives from them are numbered f = 32 kc + 8 g + j with
// kc = t * KB + kb: every lane owns complete tables, and the same numbering is
// a valid A/B operand for any contraction over f. Accumulators whose rows are
// features use the row order rho = 32 kc + 16 h + 4 g + i <-> f = 32 kc + 8 g
// + 4 h + i, so two 16-row tiles (h = 0, 1) pack straight into one operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace race {

constexpr int DH = 64;       // head dimension
constexpr int TB = 64;       // tokens per sub-block
constexpr int NW = 4;        // waves per workgroup
constexpr int NT = NW * 64;  // threads per workgroup
constexpr int EA = 96;       // augmented width: 64 values, 1 mass column, zero padding
constexpr int ZR = 80;       // rows of the transposed value tile: 64 values + mass tile
constexpr float NORM_EPS = 1e-12f;
constexpr float NEAR_ZERO = 1e-5f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// precision policy
// ---------------------------------------------------------------------------
template <bool F32>
struct Prec;

template <>
struct Prec<false> {
    using elem = __bf16;
    using frag = bf16x8;
    using half = bf16x4;
    static constexpr int PAD = 8;  // 16 bytes
};

template <>
struct Prec<true> {
    using elem = float;
    using frag = f32x8;
    using half = f32x4;
    static constexpr int PAD = 8;  // 32 bytes
};

__device__ inline f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 mma(const f32x8& a, const f32x8& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

template <bool F32>
__device__ inline typename Prec<F32>::elem to_elem(float x) {
    return (typename Prec<F32>::elem)x;
}

template <bool F32>
__device__ inline typename Prec<F32>::frag zero_frag() {
    typename Prec<F32>::frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = to_elem<F32>(0.f);
    return f;
}

// Operand from two accumulator tiles (rows 4g..4g+3 of tile h = 0 and h = 1).
template <bool F32>
__device__ inline typename Prec<F32>::frag pack(const f32x4& lo, const f32x4& hi) {
    typename Prec<F32>::frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_elem<F32>(lo[i]);
        f[4 + i] = to_elem<F32>(hi[i]);
    }
    return f;
}

template <bool F32>
__device__ inline typename Prec<F32>::frag pack8(const float* v) {
    typename Prec<F32>::frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = to_elem<F32>(v[j]);
    return f;
}

template <bool F32>
__device__ inline typename Prec<F32>::frag ld_frag(const typename Prec<F32>::elem* p) {
    return *reinterpret_cast<const typename Prec<F32>::frag*>(p);
}

// Operand whose 8 K positions are two runs of 4 (permuted K order).
template <bool F32>
__device__ inline typename Prec<F32>::frag ld_frag2(const typename Prec<F32>::elem* p0,
                                                   const typename Prec<F32>::elem* p1) {
    using H = typename Prec<F32>::half;
    H a = *reinterpret_cast<const H*>(p0);
    H b = *reinterpret_cast<const H*>(p1);
    typename Prec<F32>::frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = a[i];
        f[4 + i] = b[i];
    }
    return f;
}

template <bool F32>
__device__ inline void st_frag(typename Prec<F32>::elem* p, const typename Prec<F32>::frag& f) {
    *reinterpret_cast<typename Prec<F32>::frag*>(p) = f;
}

template <bool F32>
__device__ inline void st_half(typename Prec<F32>::elem* p, const f32x4& v) {
    typename Prec<F32>::half h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = to_elem<F32>(v[i]);
    *reinterpret_cast<typename Prec<F32>::half*>(p) = h;
}

template <bool F32>
__device__ inline float elem_f(typename Prec<F32>::elem x) {
    return (float)x;
}

// ---------------------------------------------------------------------------
// layout helpers
// ---------------------------------------------------------------------------

// feature (canonical f, relative to a chunk base) of accumulator row rho within
// a pair of 16-row tiles: rho = 16 h + 4 g + i  ->  8 g + 4 h + i
__device__ inline int canon_of_row(int h, int m) { return 8 * (m >> 2) + 4 * h + (m & 3); }

// Transcendentals on the hardware units: v_exp_f32 (2^x) and v_rcp_f32, each
// about 1 ulp; no IEEE division sequences on the hot path.
__device__ inline float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;

// tanh(x) = sign(x) (1 - e^{-2|x|}) / (1 + e^{-2|x|})
__device__ inline float fast_tanh(float x) {
    const float t = exp2_(-2.f * LOG2E * fabsf(x));
    return copysignf((1.f - t) * rcp_(1.f + t), x);
}

// sigmoid(x) = 1 / (1 + e^{-x})
__device__ inline float sigmoidf_(float x) { return rcp_(1.f + exp2_(-LOG2E * x)); }

// Sum over the four lane groups holding the same column (lanes ln, ln+16, ...).
__device__ inline float sum_groups(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Sum over the 16 lanes of a lane group.
__device__ inline float sum_row16(float v) {
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// ---------------------------------------------------------------------------
// shape configuration
// ---------------------------------------------------------------------------
template <int P_, int MT_, bool F32_, int FBK_OVERRIDE = 0>
struct Cfg {
    static constexpr int P = P_;
    static constexpr int MT = MT_;          // projection tiles of 16 rows
    static constexpr bool F32 = F32_;
    static constexpr int Pp = (P == 3) ? 4 : P;   // planes per table, padded
    static constexpr int R = 1 << P;
    static constexpr int TPL = 4 / Pp;            // tables per lane group per tile
    static constexpr int TPT = 16 / Pp;           // tables per tile
    static constexpr int KB = (P == 4) ? 2 : 1;   // 32-wide feature chunks per tile
    static constexpr int NKC = MT * KB;           // feature chunks
    static constexpr int F = 32 * NKC;            // padded feature count
    static constexpr int FBK0 = FBK_OVERRIDE ? FBK_OVERRIDE : (F32 ? KB : 4);  // chunks per feature block
    static constexpr int FBK = FBK0 < NKC ? FBK0 : NKC;
    static constexpr int TPB = FBK / KB;          // tiles per block
    static constexpr int NBLK = NKC / FBK;
    // Mass column: in feature block fb, wave w < FBK owns chunk w of the block
    // (global chunk fb * FBK + w); its accumulators are Zacc[2 fb + h].
    static constexpr int NOWN = NBLK;
    static constexpr int NPAIR = (MT + 1) / 2;    // 32-row pairs of projection tiles
    static constexpr int PAD = Prec<F32>::PAD;
    static constexpr int ROWF = FBK * 32 + PAD;   // row stride of token x feature tiles
    static constexpr int ROWT = TB + PAD;         // row stride of feature x token tiles
    static constexpr int ROWE = EA + PAD;         // row stride of token x augmented tiles
    static constexpr int ROWD = DH + PAD;
    static_assert(NKC % FBK == 0, "feature blocks must tile the features");
    static_assert(FBK % KB == 0, "feature blocks hold whole tables");
};

// table / plane of row `ri` (0..15) of projection tile t
template <class C>
__device__ inline void row_table(int t, int ri, int& table, int& plane) {
    const int g = ri >> 2, i = ri & 3;
    table = t * C::TPT + g * C::TPL + i / C::Pp;
    plane = i % C::Pp;
}

// Soft bucket features of one lane for projection tile t.
// hs[i] = normalised projection for rows 4g+i; writes phi[KB*8] (canonical
// order within the lane's chunks), u[4] = tanh(h), s[4] = sigmoid(2 beta u).
template <class C>
__device__ inline void soft_features(int t, int g, const float hs[4], float beta, int L,
                                     float phi[C::KB * 8], float u[4], float s[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u[i] = fast_tanh(hs[i]);
        s[i] = sigmoidf_(2.f * beta * u[i]);
    }
    if constexpr (C::P == 4) {
        const bool ok = (t * C::TPT + g) < L;
        float lo[4], hi[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            lo[b] = ((b & 1) ? s[0] : 1.f - s[0]) * ((b & 2) ? s[1] : 1.f - s[1]);
            hi[b] = ((b & 1) ? s[2] : 1.f - s[2]) * ((b & 2) ? s[3] : 1.f - s[3]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) phi[r] = ok ? lo[r & 3] * hi[r >> 2] : 0.f;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tl = j / C::R, r = j % C::R;
            const bool ok = (t * C::TPT + g * C::TPL + tl) < L;
            float v = 1.f;
#pragma unroll
            for (int p = 0; p < C::P; ++p) {
                const float sp = s[tl * C::Pp + p];
                v *= ((r >> p) & 1) ? sp : 1.f - sp;
            }
            phi[j] = ok ? v : 0.f;
        }
    }
}

// Chain rule of soft_features: given dA (same layout as phi) return dh[4]
// (gradient wrt the normalised projections of rows 4g..4g+3).
template <class C>
__device__ inline void soft_features_backward(const float phi[C::KB * 8], const float dA[C::KB * 8],
                                              const float u[4], float beta, float dh[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[i] = 0.f;
    constexpr int TABLES = (C::P == 4) ? 1 : C::TPL;
    constexpr int RR = C::R;
#pragma unroll
    for (int tl = 0; tl < TABLES; ++tl) {
        float mean = 0.f;
#pragma unroll
        for (int r = 0; r < RR; ++r) mean += phi[tl * RR + r] * dA[tl * RR + r];
#pragma unroll
        for (int p = 0; p < C::P; ++p) {
            float du = 0.f;
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                const float w = phi[tl * RR + r] * (dA[tl * RR + r] - mean);
                du += ((r >> p) & 1) ? w : -w;
            }
            const int i = tl * C::Pp + p;
            dh[i] = beta * du * (1.f - u[i] * u[i]);
        }
    }
}

}  // namespace race
