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
// Feature ("canonical f") order. L tables of R = 2^P features (the monomials
// of the table's planes) give F = L_pad * R features. The hash projection computes H^T = W' X^T, so a lane
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
constexpr float NORM_EPS = 1e-12f;
constexpr float NEAR_ZERO = 1e-5f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// precision policy
// ---------------------------------------------------------------------------
template <bool F32>
struct Prec;

// ucache / uvec: how the per-plane soft values u = tanh(h) are kept between
// passes (float16 for bf16 inputs: |u| <= 1, so the rounding error is below
// 2.5e-4, far under the bf16 operand rounding; float32 otherwise).
template <>
struct Prec<false> {
    using elem = __bf16;
    using frag = bf16x8;
    using half = bf16x4;
    using ucache = _Float16;
    using uvec = f16x4;
    static constexpr int PAD = 16;  // 32 bytes
};

template <>
struct Prec<true> {
    using elem = float;
    using frag = f32x8;
    using half = f32x4;
    using ucache = float;
    using uvec = f32x4;
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

template <bool F32>
__device__ inline void st_frag(typename Prec<F32>::elem* p, const typename Prec<F32>::frag& f) {
    *reinterpret_cast<typename Prec<F32>::frag*>(p) = f;
}

// Store element j of f at base + off[j] (8 scattered 2- or 4-byte writes);
// bf16 elements are written from the packed register pairs (low and high
// halves), so no value is converted twice.
template <bool F32>
__device__ inline void st_scatter(typename Prec<F32>::elem* base, const int (&off)[8],
                                  const typename Prec<F32>::frag& f) {
    if constexpr (F32) {
#pragma unroll
        for (int j = 0; j < 8; ++j) base[off[j]] = f[j];
    } else {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 w = __builtin_bit_cast(u32x4, f);
        unsigned short* b = reinterpret_cast<unsigned short*>(base);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[off[2 * j]] = (unsigned short)(w[j] & 0xffffu);
            b[off[2 * j + 1]] = (unsigned short)(w[j] >> 16);
        }
    }
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

// Tiles whose rows are features (transposed features, sketch rows) store
// feature f = 8 g + j of a 32-feature chunk at its accumulator row
// rho = 16 (j / 4) + 4 g + j % 4. A matrix-core operand that reads rows
// 16 h + ln then yields, in output rows 4 g + i, the features 8 g + 4 h + i a
// lane owns, and its 16 lanes read consecutive rows (no LDS bank conflicts).
__device__ inline int acc_row(int g, int j) { return 16 * (j >> 2) + 4 * g + (j & 3); }

// Tiles whose columns are the 64 tokens of a sub-block (transposed features,
// transposed values, intra scores) store token b = 32 m + 16 h + 4 g + i at
// column 32 m + 8 g + 4 h + i: the order in which two accumulator tiles of a
// token contraction pack into one operand, so every token-contraction operand
// is one contiguous 16-byte LDS read.
__device__ inline int tok_pos(int b) { return (b & 32) + 8 * ((b >> 2) & 3) + 4 * ((b >> 4) & 1) + (b & 3); }

// Transcendentals on the hardware units: v_exp_f32 (2^x) and v_rcp_f32, each
// about 1 ulp; no IEEE division sequences on the hot path.
__device__ inline float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ inline float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;

// Reciprocals of four values with one hardware reciprocal: 1/q_i = (product
// of the other three) / (product of all four). For q_i in [1, 2] (the only
// use here) the products stay in [1, 16], so this costs a few ulp.
__device__ inline void rcp4(const float q[4], float r[4]) {
    const float a = q[0] * q[1], b = q[2] * q[3];
    const float z = rcp_(a * b);
    const float za = z * b, zb = z * a;   // 1/a, 1/b
    r[0] = za * q[1];
    r[1] = za * q[0];
    r[2] = zb * q[3];
    r[3] = zb * q[2];
}

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
    // planes per table, padded: 1, 2, 4, or 8 (P = 5, 6: a table spans two
    // lane groups, planes 0-3 in the even one and 4-7 in the odd one)
    static constexpr int Pp = P <= 2 ? P : (P <= 4 ? 4 : 8);
    static constexpr int R = 1 << P;
    static constexpr int TPL = Pp <= 4 ? 4 / Pp : 0;   // tables per lane group per tile (Pp = 8: half a table)
    static constexpr int TPT = 16 / Pp;           // tables per tile
    // 32-wide feature chunks per tile: a lane group holds 8 KB features of
    // each of its tables (P = 5, 6: half of the table's 2^P monomials)
    static constexpr int KB = P == 6 ? 4 : (P == 4 || P == 5) ? 2 : 1;
    static constexpr int NKC = MT * KB;           // feature chunks
    static constexpr int F = 32 * NKC;            // padded feature count
    static constexpr int FBK0 = FBK_OVERRIDE ? FBK_OVERRIDE : (F32 ? KB : 4);  // chunks per feature block
    static constexpr int FBK = FBK0 < NKC ? FBK0 : NKC;
    static constexpr int TPB = FBK / KB;          // tiles per block
    static constexpr int NBLK = NKC / FBK;
    // Mass column: feature chunk c is owned by wave c % NW, in its
    // accumulators Zacc[2 (c / NW) + h]. In feature block fb the owners are
    // waves own_base(fb) .. own_base(fb) + FBK - 1 (local chunk w - own_base),
    // all at accumulator pair zidx(fb); a block of more than NW chunks gives
    // wave w its local chunks w + NW j, at pairs zidx(fb) + j.
    static constexpr int NOWN = (NKC + NW - 1) / NW;
    static constexpr int own_base(int fb) { return (fb * FBK) % NW; }
    static constexpr int zidx(int fb) { return fb * FBK / NW; }
    static constexpr int NPAIR = (MT + 1) / 2;    // 32-row pairs of projection tiles
    static constexpr int NPL = MT * 16;           // projection rows (planes incl. padding) per token
    static constexpr int PAD = Prec<F32>::PAD;
    static constexpr int ROWF = FBK * 32 + PAD;   // row stride of token x feature tiles
    static constexpr int ROWT = TB + PAD;         // row stride of token-column tiles (intra scores)
    static constexpr int ROWE = EA + PAD;         // row stride of token x augmented tiles
    static constexpr int ROWD = DH + PAD;
    static_assert(NKC % FBK == 0, "feature blocks must tile the features");
    static_assert(FBK % KB == 0, "feature blocks hold whole tables");
    static_assert(NW % FBK == 0 || FBK % NW == 0, "a feature block's mass chunks have distinct owner waves");
};

// table / plane of row `ri` (0..15) of projection tile t
template <class C>
__device__ inline void row_table(int t, int ri, int& table, int& plane) {
    const int g = ri >> 2, i = ri & 3;
    if constexpr (C::Pp == 8) {
        table = t * C::TPT + (g >> 1);
        plane = 4 * (g & 1) + i;
    } else {
        table = t * C::TPT + g * C::TPL + i / C::Pp;
        plane = i % C::Pp;
    }
}

// P = 5, 6: the plane values of the partner lane group (the other half of the
// lane's tables: lanes l and l ^ 16 hold the same token).
__device__ inline float partner(float x) { return __shfl_xor(x, 16); }

// tanh(x) = 1 - 2 / (1 + e^{2x}), with the exponent scale c = 2 log2(e)
// times any factor folded into x: e^{2x} overflows to +inf for large x (then
// tanh = 1) and underflows to 0 for very negative x (tanh = -1); near 0 the
// absolute error is about one float32 ulp of 1. One exponential, one
// reciprocal and three plain operations, no sign handling.
__device__ inline float tanh_scaled(float x, float c) { return fmaf(-2.f, rcp_(1.f + exp2_(c * x)), 1.f); }

// u = tanh(acc * inv) for the four rows a lane holds.
__device__ inline void tanh4(const float acc[4], float inv, float u[4]) {
    const float c = 2.f * LOG2E * inv;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = tanh_scaled(acc[i], c);
}

// The stored form of four u values, and back. Every pass derives the soft
// assignment of a token from the stored form, so all passes see the same
// features bit for bit.
template <bool F32>
__device__ inline typename Prec<F32>::uvec round_u(const float u[4]) {
    typename Prec<F32>::uvec v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (typename Prec<F32>::ucache)u[i];
    return v;
}

// Feature basis. The kernels contract monomial features instead of the
// corner probabilities: with t_p = tanh(beta u_p) each plane's factor is
// sigmoid(2 beta c u_p) = (1 + c t_p) / 2, so the per-table kernel
// sum_r a_r(q) a_r(k) = prod_p (1 + t_p(q) t_p(k)) / 2
//                     = 2^-P sum_{T subset of planes} psi_T(q) psi_T(k),
// psi_T = prod_{p in T} t_p. Feature r of a table is psi_T with T = the set
// bits of r. The common factor 2^-P cancels in the output O = num / den and
// in the gradients, so it is dropped. psi_{} = 1 for every table: the state
// rows of that feature are the same for all tables (the plain sums of
// [v | 1]), and only the forward read-out needs them exactly (it adds them
// in float32); every other monomial averages to zero over random planes, so
// no large common offset rides on the bf16 operands.

// Per-plane values of one lane's four rows from the stored u: t = tanh(beta u)
// and gt = (1 - t^2) (1 - u^2), which is dt/dh / beta (the factor beta is
// applied once per gradient row, where the normalisation's chain rule scales
// it).
template <bool F32>
__device__ inline void tplanes(const typename Prec<F32>::uvec& uv, float beta, float t[4], float gt[4]) {
    const float c = 2.f * LOG2E * beta;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float u = (float)uv[i];
        t[i] = tanh_scaled(u, c);
        gt[i] = (1.f - t[i] * t[i]) * (1.f - u * u);
    }
}

// Monomial features of projection tile t for one lane: phi[j] = psi of the
// table and subset that lane feature j stands for (P = 4: the lane's table,
// subset r = j + 8 kb; P < 4: table j / R of the lane, subset j % R).
// Nothing is masked here. Padded tables (index >= L) have all-zero projection
// rows, so t = 0 and only their empty subset is non-zero (1): the kernels
// discount those where they enter (the forward leaves every empty subset out
// of its state operands; the in-sub-block scores start from -n_pad; the dV
// read-out subtracts n_pad times the empty-subset row). Tokens past the end
// of the chunk load zero plane values (finite features); their value and
// mass rows are zero and the in-sub-block terms mask them.
// P = 5, 6 (two lane groups per table): the even group holds the subsets
// without the top plane P - 1, the odd group those with it; within a group
// feature jj is the subset jj (+ 2^(P-1) in the odd group), i.e. the
// monomial over planes 0-3 of jj % 16, times t_4 when P = 6 and jj >= 16,
// times t_(P-1) in the odd group. tA: planes 0-3, tB: planes 4, 5.
template <class C>
__device__ inline void split_planes(const float tt[4], int g, float tA[4], float tB[2]) {
    float pt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pt[i] = partner(tt[i]);
    const bool odd = g & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) tA[i] = odd ? pt[i] : tt[i];
    tB[0] = odd ? tt[0] : pt[0];
    tB[1] = odd ? tt[1] : pt[1];
}

template <class C>
__device__ inline void quad_monomials(const float t[4], float A[16]) {
    const float lo[4] = {1.f, t[0], t[1], t[0] * t[1]};   // subsets of planes {0, 1}
    const float hi[4] = {1.f, t[2], t[3], t[2] * t[3]};   // subsets of planes {2, 3}
#pragma unroll
    for (int r = 0; r < 16; ++r) A[r] = (r >> 2) == 0 ? lo[r & 3] : (r & 3) == 0 ? hi[r >> 2] : lo[r & 3] * hi[r >> 2];
}

template <class C>
__device__ inline void monomial_features(const float tt[4], float phi[C::KB * 8], int g = 0) {
    if constexpr (C::Pp == 8) {
        float tA[4], tB[2], A[16];
        split_planes<C>(tt, g, tA, tB);
        quad_monomials<C>(tA, A);
        const float top = (g & 1) ? (C::P == 6 ? tB[1] : tB[0]) : 1.f;
#pragma unroll
        for (int jj = 0; jj < C::KB * 8; ++jj) phi[jj] = A[jj & 15] * (C::P == 6 && jj >= 16 ? tB[0] * top : top);
    } else if constexpr (C::P == 4) {
        const float lo[4] = {1.f, tt[0], tt[1], tt[0] * tt[1]};   // subsets of planes {0, 1}
        const float hi[4] = {1.f, tt[2], tt[3], tt[2] * tt[3]};   // subsets of planes {2, 3}
#pragma unroll
        for (int r = 0; r < 16; ++r)
            phi[r] = (r >> 2) == 0 ? lo[r & 3] : (r & 3) == 0 ? hi[r >> 2] : lo[r & 3] * hi[r >> 2];
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tl = j / C::R, r = j % C::R;
            float v = 1.f;
#pragma unroll
            for (int p = 0; p < C::P; ++p)
                if ((r >> p) & 1) v *= tt[tl * C::Pp + p];
            phi[j] = v;
        }
    }
}

// Number of padded tables (projection tiles hold MT * TPT table slots).
template <class C>
__device__ inline int padded_tables(int L) { return C::MT * C::TPT - L; }

// Chain rule of monomial_features: given dA (gradient wrt the lane's
// features, same layout as phi) return dh[4], the gradient wrt the
// normalised projections of rows 4g..4g+3: dL/dt_p = sum over subsets T
// containing p of dA_T prod_{q in T, q != p} t_q, times gt_p. The empty
// subset carries no gradient.
template <class C>
__device__ inline void monomial_backward(const float dA[C::KB * 8], const float tt[4], const float gt[4],
                                         float dh[4], int g = 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dh[i] = 0.f;
    if constexpr (C::Pp == 8) {
        // this lane's features give part of dL/dt for planes 0-5; the partner
        // lane's give the rest; each lane keeps its own rows' sum
        float tA[4], tB[2], A[16];
        split_planes<C>(tt, g, tA, tB);
        quad_monomials<C>(tA, A);
        const bool odd = g & 1;
        const float top = odd ? (C::P == 6 ? tB[1] : tB[0]) : 1.f;
        // e[a] = d/dA_a of this lane's features; S0, S1 = sums against A
        float e[16], S0 = 0.f, S1 = 0.f;
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const float d0 = dA[a];
            const float d1 = C::P == 6 ? dA[a + 16] : 0.f;
            e[a] = (d0 + d1 * tB[0]) * top;
            S0 += d0 * A[a];
            S1 += d1 * A[a];
        }
        // planes 0-3: the P = 4 chain rule of the quad monomials against e
        const float t01 = tA[0] * tA[1], t23 = tA[2] * tA[3];
        float Ra[4], Cb[4];
#pragma unroll
        for (int a = 1; a < 4; ++a) Ra[a] = e[a] + e[a + 4] * tA[2] + e[a + 8] * tA[3] + e[a + 12] * t23;
#pragma unroll
        for (int b = 1; b < 4; ++b) Cb[b] = e[4 * b] + e[4 * b + 1] * tA[0] + e[4 * b + 2] * tA[1] + e[4 * b + 3] * t01;
        float dt[6];
        dt[0] = Ra[1] + Ra[3] * tA[1];
        dt[1] = Ra[2] + Ra[3] * tA[0];
        dt[2] = Cb[1] + Cb[3] * tA[3];
        dt[3] = Cb[2] + Cb[3] * tA[2];
        if constexpr (C::P == 6) {
            dt[4] = S1 * top;                          // features with plane 4 (jj >= 16)
            dt[5] = odd ? S0 + S1 * tB[0] : 0.f;       // the odd group's features all hold plane 5
        } else {
            dt[4] = odd ? S0 : 0.f;                    // the odd group's features all hold plane 4
            dt[5] = 0.f;
        }
        float tot[6];
#pragma unroll
        for (int p = 0; p < 6; ++p) tot[p] = dt[p] + partner(dt[p]);
        if (odd) {
            dh[0] = tot[4] * gt[0];
            dh[1] = C::P == 6 ? tot[5] * gt[1] : 0.f;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) dh[i] = tot[i] * gt[i];
        }
    } else if constexpr (C::P == 4) {
        // subset r = a + 4 b, a over planes {0, 1}, b over planes {2, 3}
        const float t01 = tt[0] * tt[1], t23 = tt[2] * tt[3];
        float Ra[4], Cb[4];   // Ra[a] = sum_b dA[a + 4b] hi_b, Cb[b] = sum_a dA[a + 4b] lo_a
#pragma unroll
        for (int a = 1; a < 4; ++a) Ra[a] = dA[a] + dA[a + 4] * tt[2] + dA[a + 8] * tt[3] + dA[a + 12] * t23;
#pragma unroll
        for (int b = 1; b < 4; ++b)
            Cb[b] = dA[4 * b] + dA[4 * b + 1] * tt[0] + dA[4 * b + 2] * tt[1] + dA[4 * b + 3] * t01;
        dh[0] = (Ra[1] + Ra[3] * tt[1]) * gt[0];
        dh[1] = (Ra[2] + Ra[3] * tt[0]) * gt[1];
        dh[2] = (Cb[1] + Cb[3] * tt[3]) * gt[2];
        dh[3] = (Cb[2] + Cb[3] * tt[2]) * gt[3];
    } else {
#pragma unroll
        for (int tl = 0; tl < C::TPL; ++tl) {
#pragma unroll
            for (int p = 0; p < C::P; ++p) {
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < C::R; ++r) {
                    if (!((r >> p) & 1)) continue;
                    float prod = dA[tl * C::R + r];
#pragma unroll
                    for (int q = 0; q < C::P; ++q)
                        if (q != p && ((r >> q) & 1)) prod *= tt[tl * C::Pp + q];
                    acc += prod;
                }
                dh[tl * C::Pp + p] = acc * gt[tl * C::Pp + p];
            }
        }
    }
}

// True when lane feature (h, i) of accumulator tile pair kc (feature
// j = 4 h + i of the chunk) in lane group g is the empty subset of its table.
template <class C>
__device__ constexpr bool is_empty_subset(int kc, int g, int h, int i) {
    if constexpr (C::Pp == 8) return (g & 1) == 0 && (kc % C::KB) == 0 && h == 0 && i == 0;
    return C::P == 4 ? ((kc % C::KB) == 0 && h == 0 && i == 0) : ((4 * h + i) % C::R) == 0;
}

}  // namespace race
