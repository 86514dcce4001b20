// RACE Attention kernels for gfx950.
//
// Method (arXiv 2510.04008 summaries): unit-normalise q and k, project on L
// tables of P Gaussian hyperplanes, soften with tanh, softmax over the 2^P
// hypercube corners (Italian gist.science page, Sommario tecnico section 2;
// Korean page, 기술 요약 section 2); keys add mass and value sums per bucket;
// queries read their own buckets; causal mode uses prefix sums (Japanese
// page, sections 2.1 and 2.2). The kernels contract, instead of the 2^P
// corner probabilities of a table, the 2^P monomials prod_{p in T} tanh(beta
// u_p) over the subsets T of its planes: a table's soft-collision kernel is
// 2^-P times their inner product, and the constant cancels in the output and
// the gradients (see the feature basis in race_device.hpp).
//
// Decomposition (per (batch, head), the sequence cut into chunks of `chunk`
// tokens, one workgroup per chunk, sub-blocks of 64 tokens inside a chunk):
//   k_totals : per-chunk sketch  M_c = sum_{b in c} phi(x_b)^T [z_b | m_b]
//   k_scan   : exclusive prefix (causal), reverse exclusive prefix (backward
//              key side) or total (non-causal) over chunks; for few heads of
//              long sequences k_scan_segsum + k_scan_segapply do the same in
//              segments
//   k_fwd    : per sub-block readout of the queries against the running key
//              sketch plus the intra-sub-block causal term, then the sketch
//              update -> O (and the per-token denominator D)
//   k_bwd_q  : y = [dO/D | e], e = -<dO, O>/D; dA_Q = (key sketch) y plus the
//              intra term; chain rule of the monomials and tanh,
//              back-projection -> dQ
//   k_bwd_k  : against the reverse sketch of the queries' [dO/D | e]: the dV
//              readout (one launch) and dA_K = T [v | 1] with the chain rule
//              and back-projection -> dK (a second launch)
// "a" is the side that reads the sketch, "b" the side that writes it. Sketch
// states are held in float32 accumulators, split by value columns over the
// four waves (wave w owns columns 16w..16w+15; the mass column is split by
// feature chunk).
#pragma once

#include <type_traits>

#include "race_device.hpp"

namespace race {

enum { SCAN_EXCL = 0, SCAN_REV_EXCL = 1, SCAN_TOTAL = 2 };

// ---------------------------------------------------------------------------
// Back-projection operand table: W'^T in the paired-tile K order (row 4g+j
// of tile 2m for j < 4, row 4g+j-4 of tile 2m+1 otherwise).
// ---------------------------------------------------------------------------
// One table per head of W (blockIdx.y; heads w_hs elements apart in W and
// wt_hs apart in WTp: 0 and 0 when W is shared). ndt 16-column tiles per
// tile pair: 4 (head dimension 64 or 32) or 8 (128).
template <class C>
__global__ void k_prep(const typename Prec<C::F32>::elem* __restrict__ W, int L,
                       typename Prec<C::F32>::elem* __restrict__ WTp, int64_t w_hs, int64_t wt_hs, int dh,
                       int ndt) {
    using elem = typename Prec<C::F32>::elem;
    W += blockIdx.y * w_hs;
    WTp += blockIdx.y * wt_hs;
    const int n2 = C::NPAIR * ndt * 64 * 8;
    for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < n2; k += gridDim.x * blockDim.x) {
        elem v = to_elem<C::F32>(0.f);
        const int m = k / (ndt * 512), dt = (k / 512) % ndt, l = (k / 8) & 63, j = k & 7;
        const int d = 16 * dt + (l & 15);
        const int tile = 2 * m + (j >> 2);
        const int ri = 4 * (l >> 4) + (j & 3);
        if (tile < C::MT) {
            int table, plane;
            row_table<C>(tile, ri, table, plane);
            if (table < L && plane < C::P && d < dh) v = W[((size_t)table * C::P + plane) * dh + d];
        }
        WTp[k] = v;
    }
}

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------
template <bool F32>
struct In {
    using T = typename std::conditional<F32, float, __bf16>::type;
};

// Global loads are issued one sub-block ahead ("raw" registers) and consumed
// by the next iteration, so their latency overlaps the current sub-block.

// Row stride of value tiles [z | mass] read only through transpose reads:
// 64 values, the mass and 15 zeros (a stride the transpose reads hit without
// LDS bank conflicts).
constexpr int ZV = 80;

// Per-chunk tensor access through buffer resources: a workgroup addresses the
// rows [row0, row0 + nrows) of its chunk with 32-bit byte offsets; loads of
// rows past the end return zeros and stores there are dropped, so the ragged
// last sub-block of a sequence needs no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline rsrc_t rows_rsrc(const void* base, size_t row0, int64_t nrows, int row_bytes) {
    char* p = base ? const_cast<char*>(reinterpret_cast<const char*>(base)) + row0 * (size_t)row_bytes : nullptr;
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, base ? (int)(nrows * row_bytes) : 0, 0x00020000);
}
__device__ inline u32x4 bload128(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ inline u32x2 bload64(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }
__device__ inline float bload_f32(rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void bstore128(rsrc_t r, int off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
__device__ inline void bstore64(rsrc_t r, int off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0); }
__device__ inline void bstore_f32(rsrc_t r, int off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, off, 0, 0);
}

// One 8-element operand (bf16: 16 bytes, float32: 32 bytes) at byte offset off.
template <bool F32>
__device__ inline typename Prec<F32>::frag bload_frag(rsrc_t r, int off) {
    if constexpr (F32) {
        const u32x4 a = bload128(r, off), b = bload128(r, off + 16);
        const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
        return f32x8{fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
    } else {
        return __builtin_bit_cast(bf16x8, bload128(r, off));
    }
}

template <bool F32>
__device__ inline void bstore_frag(rsrc_t r, int off, const typename Prec<F32>::frag& f) {
    if constexpr (F32) {
        // whole-vector casts (a vector built from per-element bit casts
        // compiled to a single-element load here)
        const f32x4 lo = __builtin_shufflevector(f, f, 0, 1, 2, 3), hi = __builtin_shufflevector(f, f, 4, 5, 6, 7);
        bstore128(r, off, __builtin_bit_cast(u32x4, lo));
        bstore128(r, off + 16, __builtin_bit_cast(u32x4, hi));
    } else {
        bstore128(r, off, __builtin_bit_cast(u32x4, f));
    }
}

// Bytes of a [*, dh] row of the input type. The kernels work on 64 columns;
// a head dimension dh = 32 leaves columns 32..63 zero on load (the norms,
// projections and value sums are then those of the 32 real columns) and
// unwritten on store.
template <bool F32>
__device__ inline int row_bytes(int dh) { return dh * (F32 ? 4 : 2); }

// This lane's projection operand of in-chunk row rowi: K positions 32 s + 8 g .. +7.
// (rs: elements between rows; dh: columns of the row that exist.)
template <bool F32>
__device__ inline void load_row_b(rsrc_t r, int rowi, int g, typename Prec<F32>::frag x[2], int rs, int dh) {
    constexpr int es = F32 ? 4 : 2;
#pragma unroll
    for (int s = 0; s < 2; ++s)
        x[s] = 32 * s < dh ? bload_frag<F32>(r, rowi * row_bytes<F32>(rs) + (32 * s + 8 * g) * es) : zero_frag<F32>();
}

// Columns 16 q .. 16 q + 15 of in-chunk row rowi.
template <bool F32>
__device__ inline void load_q16_b(rsrc_t r, int rowi, int q, typename Prec<F32>::frag v[2], int rs, int dh) {
    constexpr int es = F32 ? 4 : 2;
    if (16 * q < dh) {
        v[0] = bload_frag<F32>(r, rowi * row_bytes<F32>(rs) + 16 * q * es);
        v[1] = bload_frag<F32>(r, rowi * row_bytes<F32>(rs) + (16 * q + 8) * es);
    } else {
        v[0] = zero_frag<F32>();
        v[1] = zero_frag<F32>();
    }
}

// This lane's projection operand of one token row: K positions 32 s + 8 g .. +7.
template <bool F32>
__device__ inline void load_row_raw(const void* X, size_t row, bool valid, int g,
                                    typename Prec<F32>::frag x[2], int dh) {
    using T = typename In<F32>::T;
    const T* p = reinterpret_cast<const T*>(X) + row * dh + 8 * g;
#pragma unroll
    for (int s = 0; s < 2; ++s)
        x[s] = (valid && 32 * s < dh) ? *reinterpret_cast<const typename Prec<F32>::frag*>(p + 32 * s)
                                      : zero_frag<F32>();
}

// 1 / max(|x|, eps) of the row held by load_row_b / load_row_raw (same in all
// four lane groups): the sum of squares (bf16: two-element dot products, exact
// products, float32 sums) and one hardware reciprocal square root of
// max(|x|^2, eps^2).
template <bool F32>
__device__ inline float row_sumsq(const typename Prec<F32>::frag x[2]) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if constexpr (F32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ss += x[s][j] * x[s][j];
        } else {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 p = {x[s][2 * j], x[s][2 * j + 1]};
                ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
            }
        }
    }
    return ss;
}
template <bool F32>
__device__ inline float row_inv_norm(const typename Prec<F32>::frag x[2]) {
    const float ss = sum_groups(row_sumsq<F32>(x));
    return __builtin_amdgcn_rsqf(fmaxf(ss, NORM_EPS * NORM_EPS));
}


// <a, b> over the 16 values of two q16 row quarters (bf16: packed dot
// products with float32 sums, no conversions).
template <bool F32>
__device__ inline float dot16(const typename Prec<F32>::frag a[2], const typename Prec<F32>::frag b[2]) {
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if constexpr (F32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += a[s][j] * b[s][j];
        } else {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 pa = {a[s][2 * j], a[s][2 * j + 1]}, pb = {b[s][2 * j], b[s][2 * j + 1]};
                acc = __builtin_amdgcn_fdot2_f32_bf16(pa, pb, acc, false);
            }
        }
    }
    return acc;
}

template <bool F32>
__device__ inline float q16_at(const typename Prec<F32>::frag v[2], int c) {
    return (float)v[c >> 3][c & 7];
}

// Projection operands W' (rows in tile order) in LDS, laid out per lane:
// [tile][K half s][lane][8], filled once per workgroup.
template <class C>
__device__ inline void stage_w(const typename Prec<C::F32>::elem* __restrict__ W, int L,
                               typename Prec<C::F32>::elem* s_w, int dh) {
    for (int idx = threadIdx.x; idx < C::MT * 1024; idx += NT) {
        const int t = idx / 1024, s = (idx / 512) & 1, l = (idx / 8) & 63, j = idx & 7;
        int table, plane;
        row_table<C>(t, l & 15, table, plane);
        typename Prec<C::F32>::elem v = to_elem<C::F32>(0.f);
        const int col = 32 * s + 8 * (l >> 4) + j;
        if (table < L && plane < C::P && col < dh) v = W[((size_t)table * C::P + plane) * dh + col];
        s_w[idx] = v;
    }
}

// H^T tile t (rows 4g..4g+3 of column = this lane's token) from LDS-staged W'.
template <class C>
__device__ inline f32x4 project_lds(const typename Prec<C::F32>::elem* s_w, int t, int lane,
                                    const typename Prec<C::F32>::frag xf[2]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) acc = mma(ld_frag<C::F32>(s_w + ((t * 2 + s) * 64 + lane) * 8), xf[s], acc);
    return acc;
}

// Same from W in global memory (used where LDS is full, and by the hash kernel).
template <class C>
__device__ inline f32x4 project_global(const typename Prec<C::F32>::elem* __restrict__ W, int L, int t, int ln,
                                       int g, const typename Prec<C::F32>::frag xf[2], int dh) {
    int table, plane;
    row_table<C>(t, ln, table, plane);
    const bool ok = table < L && plane < C::P;
    const typename Prec<C::F32>::elem* wr = W + ((size_t)(ok ? table * C::P + plane : 0)) * dh + 8 * g;
    typename Prec<C::F32>::frag wf[2] = {zero_frag<C::F32>(), zero_frag<C::F32>()};
    if (ok) {
        wf[0] = ld_frag<C::F32>(wr);
        if (dh > 32) wf[1] = ld_frag<C::F32>(wr + 32);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mma(wf[0], xf[0], acc);
    acc = mma(wf[1], xf[1], acc);
    return acc;
}

// Source of the projection operands: LDS-staged when STAGED (the choice is
// made at compile time from the LDS budget, so no dead path is emitted).
template <class C, bool STAGED = true>
struct WSrc {
    const typename Prec<C::F32>::elem* s_w;
    const typename Prec<C::F32>::elem* W;
    int L;
    int dh;
    __device__ inline f32x4 project(int t, int lane, int ln, int g, const typename Prec<C::F32>::frag xf[2]) const {
        if constexpr (STAGED) return project_lds<C>(s_w, t, lane, xf);
        else return project_global<C>(W, L, t, ln, g, xf, dh);
    }
};

// Per-token plane values of one side (queries or keys), written by the pass
// that projects the rows and read by the later passes instead of projecting
// again: u = tanh(h) for every projection row (tile-row order, NPL per
// token) in Prec::ucache, and 1 / max(|x|, eps) per token in float32.
struct PlaneCache {
    void* u;      // [rows][NPL] of Prec::ucache
    float* inv;   // [rows]
};

// The stored u of the own token for the tiles of one feature block.
template <class C>
struct Planes {
    typename Prec<C::F32>::uvec u[C::TPB];
};

// Chunk-local view of one side's plane cache: the u rows and the inverse
// norms of the chunk's tokens (no cache: every access out of range).
struct PlaneRows {
    rsrc_t u, inv;
};

template <class C>
__device__ inline PlaneRows plane_rows(const PlaneCache& pc, size_t row0, int64_t nrows) {
    constexpr int ub = C::NPL * (int)sizeof(typename Prec<C::F32>::ucache);
    return PlaneRows{rows_rsrc(pc.u, row0, pc.u ? nrows : 0, ub), rows_rsrc(pc.inv, row0, pc.inv ? nrows : 0, 4)};
}

// Byte offset of the u values of projection tile t, lane group g, in-chunk row rowi.
template <class C>
__device__ inline int u_offset(int rowi, int t, int g) {
    constexpr int us = (int)sizeof(typename Prec<C::F32>::ucache);
    return (rowi * C::NPL + 16 * t + 4 * g) * us;
}

template <class C>
__device__ inline void load_planes(const PlaneRows& pr, int rowi, int fb, int g, Planes<C>& p) {
#pragma unroll
    for (int tb = 0; tb < C::TPB; ++tb) {
        const int off = u_offset<C>(rowi, fb * C::TPB + tb, g);
        if constexpr (C::F32) p.u[tb] = __builtin_bit_cast(f32x4, bload128(pr.u, off));
        else p.u[tb] = __builtin_bit_cast(f16x4, bload64(pr.u, off));
    }
}

template <class C>
__device__ inline void store_u(const PlaneRows& pr, int rowi, int t, int g, const typename Prec<C::F32>::uvec& uq) {
    const int off = u_offset<C>(rowi, t, g);
    if constexpr (C::F32) bstore128(pr.u, off, __builtin_bit_cast(u32x4, uq));
    else bstore64(pr.u, off, __builtin_bit_cast(u32x2, uq));
}

// Write the value tile of the 64 tokens (this thread: row th/4, quarter th%4)
// into Zrow [64][ROWE] (token rows): z = [x * scale | mass]. With Zlo set, also
// the rows of the rounding residual z - elem(z) (so that hi + lo carries z to
// float32 precision). Columns 65.. stay zero from zero_pads.
template <class C, int ZS = C::ROWE, bool UNIT = false>
__device__ inline void write_aug(const typename Prec<C::F32>::frag zr[2], float scale, float mass,
                                 typename Prec<C::F32>::elem* Zrow, typename Prec<C::F32>::elem* Zlo = nullptr) {
    const int th = threadIdx.x, r = th >> 2, q = th & 3;
    if constexpr (UNIT) {
        // scale 1: the loaded rows are stored as they are
        st_frag<C::F32>(Zrow + r * ZS + 16 * q, zr[0]);
        st_frag<C::F32>(Zrow + r * ZS + 16 * q + 8, zr[1]);
        if (q == 0) Zrow[r * ZS + 64] = to_elem<C::F32>(mass);
        return;
    }
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = q16_at<C::F32>(zr, c) * scale;
    const typename Prec<C::F32>::frag h0 = pack8<C::F32>(v), h1 = pack8<C::F32>(v + 8);
    st_frag<C::F32>(Zrow + r * ZS + 16 * q, h0);
    st_frag<C::F32>(Zrow + r * ZS + 16 * q + 8, h1);
    const typename Prec<C::F32>::elem mh = to_elem<C::F32>(mass);
    if (q == 0) Zrow[r * ZS + 64] = mh;
    if (Zlo) {
        float lo[16];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            lo[c] = v[c] - elem_f<C::F32>(h0[c]);
            lo[8 + c] = v[8 + c] - elem_f<C::F32>(h1[c]);
        }
        st_frag<C::F32>(Zlo + r * ZS + 16 * q, pack8<C::F32>(lo));
        st_frag<C::F32>(Zlo + r * ZS + 16 * q + 8, pack8<C::F32>(lo + 8));
        if (q == 0) Zlo[r * ZS + 64] = to_elem<C::F32>(mass - elem_f<C::F32>(mh));
    }
}

// Zero the constant padding (columns 65 .. min(ZS, 96) - 1) of token-row value
// tiles of row stride ZS.
template <class C, int ZS = C::ROWE>
__device__ inline void zero_pads(typename Prec<C::F32>::elem* rows_a, typename Prec<C::F32>::elem* rows_b) {
    constexpr int NZ = (ZS < EA ? ZS : EA) - 65;
    if (rows_a)
        for (int idx = threadIdx.x; idx < NZ * TB; idx += NT) rows_a[(idx / NZ) * ZS + 65 + idx % NZ] = to_elem<C::F32>(0.f);
    if (rows_b)
        for (int idx = threadIdx.x; idx < NZ * TB; idx += NT) rows_b[(idx / NZ) * ZS + 65 + idx % NZ] = to_elem<C::F32>(0.f);
}

// State block of one (bh, chunk): value sums [F][64] then masses [F], float32.
// Sketch states between the passes. float32 inputs: [F x 64 value sums |
// F masses], float32. bf16 inputs (the compact form, half the bytes of the
// value sums, which the passes round to bf16 operands anyway): the F x 64
// value sums in bf16 (row f at bf16 index 64 f), then the F masses in
// float32 (float index 32 F: exact counts for the hard buckets), then the
// 64 value sums of the empty subset in float32 (float index 33 F: the
// forward's exact float32 term; it is the row of every table's empty subset,
// so the same for all). Either form sits in a slot of F * 65 floats.
template <class C>
struct StateForm {
    static constexpr bool compact = !C::F32;
    static constexpr int mass = compact ? 32 * C::F : DH * C::F;   // float index of the masses
    static constexpr int empty = 33 * C::F;                        // compact: the empty subset's row
};

__device__ inline float bf16_at(const float* st, int i) {
    return (float)reinterpret_cast<const __bf16*>(st)[i];
}

template <class C>
__device__ inline void load_state(const float* __restrict__ st, int w, int ln, int g,
                                  f32x4 Macc[C::NKC * 2], f32x4 Zacc[C::NOWN * 2]) {
    using SF = StateForm<C>;
    if constexpr (SF::compact) {
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = 32 * kc + 8 * g + 4 * h + i;
                    Macc[2 * kc + h][i] = bf16_at(st, f * DH + 16 * w + ln);
                }
        // feature 0 (table 0's empty subset) from its float32 copy
        if (g == 0) Macc[0][0] = st[SF::empty + 16 * w + ln];
#pragma unroll
        for (int j = 0; j < C::NOWN; ++j) {
            const int kc = NW * j + w;
            const bool owner = kc < C::NKC && ln == 0;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = 32 * (owner ? kc : 0) + 8 * g + 4 * h + i;
                    Zacc[2 * j + h][i] = owner ? st[SF::mass + f] : 0.f;
                }
        }
        return;
    }
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 32 * kc + 8 * g + 4 * h + i;
                Macc[2 * kc + h][i] = st[(size_t)f * DH + 16 * w + ln];
            }
#pragma unroll
    for (int j = 0; j < C::NOWN; ++j) {
        const int kc = NW * j + w;             // the chunk this wave owns
        const bool owner = kc < C::NKC && ln == 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 32 * (owner ? kc : 0) + 8 * g + 4 * h + i;
                float v = 0.f;
                if (owner) v = st[(size_t)C::F * DH + f];
                Zacc[2 * j + h][i] = v;
            }
    }
}

// The same state in the transposed accumulator layout (TR): tile (kc, h)
// holds value columns 16 w + 4 g + i (rows) of accumulator rows 32 kc + 16 h +
// ln (columns; feature 32 kc + 8 (ln / 4) + 4 h + ln % 4), so a lane reads
// four consecutive floats, and later writes four consecutive columns of one
// sketch row. The mass of the chunks a wave owns sits at (g, i) = (0, 0).
template <class C>
__device__ inline void load_state_t(const float* __restrict__ st, int w, int ln, int g,
                                    f32x4 Macc[C::NKC * 2], f32x4 Zacc[C::NOWN * 2]) {
    using SF = StateForm<C>;
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int f = 32 * kc + 8 * (ln >> 2) + 4 * h + (ln & 3);
            if constexpr (SF::compact) {
                const bf16x4 v = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(st) + f * DH +
                                                                  16 * w + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[2 * kc + h][i] = (float)v[i];
            } else {
                Macc[2 * kc + h] = *reinterpret_cast<const f32x4*>(st + (size_t)f * DH + 16 * w + 4 * g);
            }
        }
#pragma unroll
    for (int j = 0; j < C::NOWN; ++j) {
        const int kc = NW * j + w;
        const bool owner = kc < C::NKC && g == 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int f = 32 * (owner ? kc : 0) + 8 * (ln >> 2) + 4 * h + (ln & 3);
            Zacc[2 * j + h] = f32x4{owner ? st[SF::mass + f] : 0.f, 0.f, 0.f, 0.f};
        }
    }
}

// COMPACT: the compact form for bf16 inputs (else float32).
template <class C, bool COMPACT = StateForm<C>::compact>
__device__ inline void store_state(float* __restrict__ st, int w, int ln, int g,
                                   const f32x4 Macc[C::NKC * 2], const f32x4 Zacc[C::NOWN * 2]) {
    if constexpr (COMPACT) {
        using SF = StateForm<C>;
        __bf16* sv = reinterpret_cast<__bf16*>(st);
#pragma unroll
        for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = 32 * kc + 8 * g + 4 * h + i;
                    sv[f * DH + 16 * w + ln] = (__bf16)Macc[2 * kc + h][i];
                }
        if (g == 0) st[SF::empty + 16 * w + ln] = Macc[0][0];
#pragma unroll
        for (int j = 0; j < C::NOWN; ++j) {
            const int kc = NW * j + w;
            if (kc < C::NKC && ln == 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[SF::mass + 32 * kc + 8 * g + 4 * h + i] = Zacc[2 * j + h][i];
            }
        }
        return;
    }
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = 32 * kc + 8 * g + 4 * h + i;
                st[(size_t)f * DH + 16 * w + ln] = Macc[2 * kc + h][i];
            }
#pragma unroll
    for (int j = 0; j < C::NOWN; ++j) {
        const int kc = NW * j + w;
        if (kc < C::NKC && ln == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int f = 32 * kc + 8 * g + 4 * h + i;
                    st[(size_t)C::F * DH + f] = Zacc[2 * j + h][i];
                }
        }
    }
}

// Matrix-core A operand of a token contraction, read from a token-row feature
// tile rows[64][ROWF] (token b, feature 32 kcl + f of the block): lane
// (ln, g) gets, for accumulator row 16 h + ln of feature chunk kcl (feature
// 8 (ln / 4) + 4 h + ln % 4), the tokens at K positions 32 s + 8 g + j in
// tok_pos order, i.e. tokens 32 s + 16 (j / 4) + 4 g + j % 4. bf16 uses two
// LDS transpose reads (ds_read_b64_tr_b16): lane j of a 16-lane group points
// at 4 consecutive features of one token, and the group receives the 4 x 16
// block transposed, lane l holding element l % 4 of the lanes l / 4 + 4 i.
template <class C>
__device__ inline typename Prec<C::F32>::frag feat_operand(const typename Prec<C::F32>::elem* rows, int kcl, int h,
                                                          int s, int ln, int g) {
    typename Prec<C::F32>::frag f;
    if constexpr (C::F32) {
        const int fo = 32 * kcl + 8 * (ln >> 2) + 4 * h + (ln & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = rows[(32 * s + 16 * (j >> 2) + 4 * g + (j & 3)) * C::ROWF + fo];
    } else {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const typename Prec<C::F32>::elem* p =
            rows + (32 * s + 4 * g + (ln >> 2)) * C::ROWF + 32 * kcl + 8 * (ln & 3) + 4 * h;
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * C::ROWF));
        const bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = ab[i];
            f[4 + i] = bb[i];
        }
    }
    return f;
}

// Matrix-core B operand of a token contraction, read from a token-row value
// tile Zrow[64][ROWE]: lane (ln, g) gets column cb + ln and the tokens at K
// positions 32 s + 8 g + j in tok_pos order (as feat_operand). bf16: two LDS
// transpose reads, lane j of a 16-lane group pointing at columns
// cb + 4 (j % 4) .. +3 of one token.
template <class C, int ZS = C::ROWE>
__device__ inline typename Prec<C::F32>::frag val_operand(const typename Prec<C::F32>::elem* Zrow, int cb, int s,
                                                         int ln, int g) {
    typename Prec<C::F32>::frag f;
    if constexpr (C::F32) {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = Zrow[(32 * s + 16 * (j >> 2) + 4 * g + (j & 3)) * ZS + cb + ln];
    } else {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const typename Prec<C::F32>::elem* p = Zrow + (32 * s + 4 * g + (ln >> 2)) * ZS + cb + 4 * (ln & 3);
        const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * ZS));
        const bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = ab[i];
            f[4 + i] = bb[i];
        }
    }
    return f;
}

// Sketch update for feature block fb from the b-side features (token-row tile
// `brow`) and the value tile Zrow: value columns of wave w, then the mass
// accumulators of the chunk wave w owns in this block.
template <class C, bool MASS = true, int ZS = C::ROWE, bool PIPE = false, bool TR = false>
__device__ inline void sketch_update(int fb, int w, int ln, int g, const typename Prec<C::F32>::elem* brow,
                                     const typename Prec<C::F32>::elem* Zrow, f32x4 Macc[C::NKC * 2],
                                     f32x4 Zacc[C::NOWN * 2]) {
    using frag = typename Prec<C::F32>::frag;
    frag zt[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) zt[s] = val_operand<C, ZS>(Zrow, 16 * w, s, ln, g);
    static_assert(!(PIPE && TR), "the pipelined update uses the plain layout");
    if constexpr (PIPE && !C::F32) {
        // Operand reads run D products ahead of the matrix cores, pinned by
        // scheduling groups (4 reads for the value operands and 2 D for the
        // first feature operands, then one product and the next operand's 2
        // reads at a time): the register-pressure schedule otherwise waits
        // out every read's latency before its product.
        constexpr int NM = C::FBK * 4, D = 4;
        frag A[NM];
#pragma unroll
        for (int j = 0; j < D; ++j) A[j] = feat_operand<C>(brow, j >> 2, (j >> 1) & 1, j & 1, ln, g);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 + 2 * D, 0);
#pragma unroll
        for (int j = 0; j < NM; ++j) {
            if (j + D < NM) A[j + D] = feat_operand<C>(brow, (j + D) >> 2, ((j + D) >> 1) & 1, (j + D) & 1, ln, g);
            const int kc = fb * C::FBK + (j >> 2), h = (j >> 1) & 1, s2 = j & 1;
            Macc[2 * kc + h] = mma(A[j], zt[s2], Macc[2 * kc + h]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (j + D < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    } else {
#pragma unroll
        for (int kcl = 0; kcl < C::FBK; ++kcl) {
            const int kc = fb * C::FBK + kcl;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    if constexpr (TR)
                        Macc[2 * kc + h] = mma(zt[s], feat_operand<C>(brow, kcl, h, s, ln, g), Macc[2 * kc + h]);
                    else
                        Macc[2 * kc + h] = mma(feat_operand<C>(brow, kcl, h, s, ln, g), zt[s], Macc[2 * kc + h]);
                }
            }
        }
    }
    if constexpr (MASS && C::FBK > NW) {
        // blocks wider than the workgroup: wave w owns local chunks w + NW j
        frag zm[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) zm[s] = val_operand<C, ZS>(Zrow, 64, s, ln, g);
#pragma unroll
        for (int j = 0; j < C::FBK / NW; ++j) {
            const int kw = w + NW * j;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    f32x4& acc = Zacc[2 * (C::zidx(fb) + j) + h];
                    if constexpr (TR) acc = mma(zm[s], feat_operand<C>(brow, kw, h, s, ln, g), acc);
                    else acc = mma(feat_operand<C>(brow, kw, h, s, ln, g), zm[s], acc);
                }
            }
        }
        return;
    }
    const int kw = w - C::own_base(fb);        // local chunk whose mass this wave owns
    if (MASS && kw >= 0 && kw < C::FBK) {
        frag zm[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) zm[s] = val_operand<C, ZS>(Zrow, 64, s, ln, g);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if constexpr (TR)
                    Zacc[2 * C::zidx(fb) + h] =
                        mma(zm[s], feat_operand<C>(brow, kw, h, s, ln, g), Zacc[2 * C::zidx(fb) + h]);
                else
                    Zacc[2 * C::zidx(fb) + h] =
                        mma(feat_operand<C>(brow, kw, h, s, ln, g), zm[s], Zacc[2 * C::zidx(fb) + h]);
            }
        }
    }
}

// Pack the lane's features of tile tb of the block and write them to the
// token-row tile `rows`; KEEP also returns the operands.
template <class C, bool KEEP>
__device__ inline void emit_tile(int tb, int w, int ln, int g, const float phi[C::KB * 8],
                                 typename Prec<C::F32>::elem* rows, typename Prec<C::F32>::frag (&phi_frag)[C::FBK]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
        const int kcl = tb * C::KB + kb;
        const typename Prec<C::F32>::frag fr = pack8<C::F32>(phi + kb * 8);
        if constexpr (KEEP) phi_frag[kcl] = fr;
        st_frag<C::F32>(rows + (16 * w + ln) * C::ROWF + 32 * kcl + 8 * g, fr);
    }
}

// Project the own 16-token tile for the tiles of feature block fb and write
// the features to the token-row tile `rows`; when KEEP,
// also return the lane's operands (one per chunk of the block) in phi_frag.
// The plane values are stored to `out` (in-chunk row rowi; rows past the
// chunk, or every row when there is no cache, are dropped) for later passes.
template <class C, bool KEEP, class WS>
__device__ inline void block_features(const WS& wsrc, int fb, int lane, int w, int ln, int g,
                                      const typename Prec<C::F32>::frag xf[2], float inv, float beta,
                                      typename Prec<C::F32>::elem* rows /* [64][ROWF] */,
                                      typename Prec<C::F32>::frag (&phi_frag)[C::FBK], const PlaneRows& out,
                                      int rowi) {
#pragma unroll
    for (int tb = 0; tb < C::TPB; ++tb) {
        const int t = fb * C::TPB + tb;
        const f32x4 acc = wsrc.project(t, lane, ln, g, xf);
        float hs[4], u[4], phi[C::KB * 8], tt[4], gt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[i] = acc[i];
        tanh4(hs, inv, u);
        const typename Prec<C::F32>::uvec uq = round_u<C::F32>(u);
        tplanes<C::F32>(uq, beta, tt, gt);
        monomial_features<C>(tt, phi, g);
        store_u<C>(out, rowi, t, g, uq);
        emit_tile<C, KEEP>(tb, w, ln, g, phi, rows, phi_frag);
    }
}

// The same from stored plane values (no projection); when KEEP, also return
// per tile the plane values t and dt/dh for the chain rule.
template <class C, bool KEEP>
__device__ inline void block_features_cached(const Planes<C>& pl, int w, int ln, int g, float beta,
                                             typename Prec<C::F32>::elem* rows,
                                             typename Prec<C::F32>::frag (&phi_frag)[C::FBK],
                                             float (&t_keep)[C::TPB][4], float (&gt_keep)[C::TPB][4]) {
#pragma unroll
    for (int tb = 0; tb < C::TPB; ++tb) {
        float tt[4], gt[4], phi[C::KB * 8];
        tplanes<C::F32>(pl.u[tb], beta, tt, gt);
        monomial_features<C>(tt, phi, g);
        if constexpr (KEEP) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t_keep[tb][i] = tt[i];
                gt_keep[tb][i] = gt[i];
            }
        }
        emit_tile<C, KEEP>(tb, w, ln, g, phi, rows, phi_frag);
    }
}

// ---------------------------------------------------------------------------
// per-chunk sketch totals
// ---------------------------------------------------------------------------
struct TotArgs {
    const void* Xb;      // keys (projected here); unused for the gradient sketch
    const void* Z;       // V, or dO for the gradient sketch
    const float* Dv;     // gradient sketch: per-token D
    const float* Ev;     // gradient sketch: per-token e
    const void* W;       // [L, P, d] (this group's tables; per head: W of head h at + h * w_hs bytes)
    PlaneCache pc;       // keys: where their plane values go; gradient sketch: the queries' plane values
    float* out;          // [BH][NC][F*65]
    int64_t N;
    int chunk;
    int nchunks;
    int L;
    float beta;
    int H;               // heads (W of sequence bh: W + (bh % H) * w_hs bytes)
    int64_t w_hs;        // bytes between the heads' hyperplanes; 0: one W for all
    int dh;              // columns of a row the kernels use: 64, or 32 (columns 32..63 zero)
    int rs;              // elements between consecutive rows (the head dimension)
    int ezero;           // gradient sketch: e taken as 0 (the second value half of d = 128)
    int f32form;         // bf16 inputs: write the float32 form (the running decode state's source)
};

template <class C, bool CACHED>
struct TotLds {
    using elem = typename Prec<C::F32>::elem;
    static constexpr int n_rows = TB * C::ROWF;   // features of the block, token rows
    static constexpr int n_zr = TB * ZV;          // [z | mass], token rows
    static constexpr int n_w = CACHED ? 0 : C::MT * 1024;
    static constexpr int n_elem = n_rows + n_zr + n_w;
    static_assert(n_elem * (int)sizeof(elem) <= 160 * 1024, "LDS budget");
};

// CACHED = false: sketch of the keys, [v | 1], projecting K (and storing the
// keys' plane values), or with PG from the keys' plane values computed
// beforehand (head dimension 128); CACHED = true: gradient sketch of the
// queries, [dO/D | e] (e taken as 0 when a.ezero), from the queries' stored
// plane values.
template <class C, bool CACHED, bool PG = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 3))) void k_totals(TotArgs a) {
    using elem = typename Prec<C::F32>::elem;
    using frag = typename Prec<C::F32>::frag;
    constexpr bool FC = CACHED || PG;   // features from stored plane values
    using LD = TotLds<C, FC>;
    __shared__ __attribute__((aligned(32))) elem lds[LD::n_elem];
    elem* s_rows = lds;
    elem* s_zr = lds + LD::n_rows;
    elem* s_w = s_zr + LD::n_zr;

    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    // wave index as a scalar: every branch on it is wave-uniform, so no MFMA is
    // ever issued under a partial or empty EXEC mask
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int th = threadIdx.x, tr = th >> 2, tq = th & 3;
    const int bh = blockIdx.y, c = blockIdx.x;
    const int64_t seg0 = (int64_t)c * a.chunk;
    const int64_t seg1 = seg0 + a.chunk < a.N ? seg0 + a.chunk : a.N;
    const size_t base = (size_t)bh * a.N;
    const int nsub = (int)((seg1 - seg0 + TB - 1) / TB);
    const int my = 16 * w + ln;
    const elem* Wh = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.W) + (bh % a.H) * a.w_hs);
    if (!FC) stage_w<C>(Wh, a.L, s_w, a.dh);
    zero_pads<C, ZV>(s_zr, nullptr);
    __syncthreads();   // W' and the padding are written by all waves, read by each
    const WSrc<C> wsrc{s_w, Wh, a.L, a.dh};
    const int64_t nrows = seg1 - seg0;
    const size_t row0 = base + seg0;
    const rsrc_t rX = rows_rsrc(FC ? nullptr : a.Xb, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rZ = rows_rsrc(a.Z, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rD = rows_rsrc(CACHED ? a.Dv : nullptr, row0, nrows, 4);
    const rsrc_t rE = rows_rsrc(CACHED ? a.Ev : nullptr, row0, nrows, 4);
    const PlaneRows pr = plane_rows<C>(a.pc, row0, nrows);

    f32x4 Macc[C::NKC * 2], Zacc[C::NOWN * 2];
#pragma unroll
    for (int i = 0; i < C::NKC * 2; ++i) Macc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < C::NOWN * 2; ++i) Zacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // loads issued one sub-block (plane values: one feature block) ahead
    frag nx[2], nz[2];
    float nd = 1.f, ne = 0.f;
    Planes<C> pn;
    auto nv_of = [&](int it2) {
        const int64_t t0 = seg0 + (int64_t)it2 * TB;
        return (int)(seg1 - t0 < TB ? seg1 - t0 : TB);
    };
    auto issue = [&](int it2) {
        const int r0 = it2 * TB;
        if (!FC) load_row_b<C::F32>(rX, r0 + my, g, nx, a.rs, a.dh);
        load_q16_b<C::F32>(rZ, r0 + tr, tq, nz, a.rs, a.dh);
        if (CACHED) {
            nd = bload_f32(rD, (r0 + tr) * 4);
            ne = bload_f32(rE, (r0 + tr) * 4);
        }
    };
    auto issue_planes = [&](int it2, int fb2) { load_planes<C>(pr, it2 * TB + my, fb2, g, pn); };
    issue(0);
    if (FC) issue_planes(0, 0);
    for (int it = 0; it < nsub; ++it) {
        const int nv = nv_of(it);
        const int rowi = it * TB + my;
        frag xf[2] = {nx[0], nx[1]}, zr[2] = {nz[0], nz[1]};
        const float dz = nd, ez = ne;
        if (it + 1 < nsub) issue(it + 1);
        float inv = 0.f;
        if (!FC) {
            inv = row_inv_norm<C::F32>(xf);
            if (g == 0) bstore_f32(pr.inv, rowi * 4, inv);
        }
        const bool ok = tr < nv;
        if (!CACHED) write_aug<C, ZV, true>(zr, 1.f, ok ? 1.f : 0.f, s_zr);
        else write_aug<C, ZV>(zr, ok ? rcp_(dz) : 0.f, (ok && !a.ezero) ? ez : 0.f, s_zr);
#pragma unroll
        for (int fb = 0; fb < C::NBLK; ++fb) {
            frag unused[C::FBK];
            if constexpr (FC) {
                const Planes<C> pl = pn;
                if (fb + 1 < C::NBLK) issue_planes(it, fb + 1);
                else if (it + 1 < nsub) issue_planes(it + 1, 0);
                float us[C::TPB][4], ug[C::TPB][4];
                block_features_cached<C, false>(pl, w, ln, g, a.beta, s_rows, unused, us, ug);
            } else {
                block_features<C, false>(wsrc, fb, lane, w, ln, g, xf, inv, a.beta, s_rows, unused,
                                         pr, rowi);
            }
            __syncthreads();
            sketch_update<C, true, ZV, true>(fb, w, ln, g, s_rows, s_zr, Macc, Zacc);
            __syncthreads();
        }
    }
    float* out = a.out + ((size_t)bh * a.nchunks + c) * (size_t)(C::F * 65);
    if (StateForm<C>::compact && a.f32form) store_state<C, false>(out, w, ln, g, Macc, Zacc);
    else store_state<C>(out, w, ln, g, Macc, Zacc);
}

// ---------------------------------------------------------------------------
// scans over chunks (one thread per state element, fixed order: deterministic)
// ---------------------------------------------------------------------------
// Running sum over logical chunk positions [c0, c1) of one state word
// (position c is chunk c, or chunk nchunks - 1 - c for the reverse scan),
// starting from run; with WRITE each position first receives the sum of the
// positions before it. A word is one float32 value, or (PAIR: the value sums
// of the compact form) two bf16 values summed in two float32 runs, each
// prefix rounded once to bf16. The loads of the next batch are issued before
// the sums and stores of the current one, so about 2 * BATCH loads per lane
// stay in flight; the order of the additions is fixed (deterministic).
struct Run2 {
    float a, b;
};

template <int KIND, bool WRITE, bool PAIR>
__device__ inline Run2 scan_range(float* p, int nchunks, int stride, int c0, int c1, Run2 run) {
    constexpr int BATCH = 16;
    auto at = [&](int c) -> float* {
        return p + (size_t)((KIND == SCAN_REV_EXCL) ? nchunks - 1 - c : c) * stride;
    };
    auto load = [&](int b0, float (&v)[BATCH]) {
#pragma unroll
        for (int k = 0; k < BATCH; ++k) v[k] = *at(b0 + k < c1 ? b0 + k : c1 - 1);
    };
    if (c0 >= c1) return run;
    float cur[BATCH], nxt[BATCH];
    load(c0, cur);
    for (int b0 = c0; b0 < c1; b0 += BATCH) {
        if (b0 + BATCH < c1) load(b0 + BATCH, nxt);
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            if (b0 + k < c1) {
                if constexpr (PAIR) {
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    if constexpr (WRITE) *at(b0 + k) = __builtin_bit_cast(float, bf16x2{(__bf16)run.a, (__bf16)run.b});
                    const bf16x2 v = __builtin_bit_cast(bf16x2, cur[k]);
                    run.a += (float)v[0];
                    run.b += (float)v[1];
                } else {
                    if constexpr (WRITE) *at(b0 + k) = run.a;
                    run.a += cur[k];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) cur[k] = nxt[k];
    }
    return run;
}

// Words of one chunk slot (stride floats apart): the first npair hold bf16
// pairs (the compact form's value sums; 0 for the float32 form), the rest up
// to nwords one float32 each. Segment sums keep two floats per pair word:
// word e < npair at 2 e, 2 e + 1, word e >= npair at npair + e.
struct ScanShape {
    int nchunks, stride, nwords, npair;
};

// One pass over all chunks (one thread per state word): exclusive prefix
// (causal), reverse exclusive prefix (backward) or the total (non-causal).
// The total of head bh goes to total + bh * total_stride (same form).
template <int KIND>
__global__ __launch_bounds__(256) void k_scan(float* __restrict__ st, float* __restrict__ total, ScanShape sh,
                                              int64_t total_stride) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= sh.nwords) return;
    float* p = st + (size_t)bh * sh.nchunks * sh.stride + e;
    constexpr bool W = KIND != SCAN_TOTAL;
    Run2 run{0.f, 0.f};
    if (e < sh.npair) {
        run = scan_range<KIND, W, true>(p, sh.nchunks, sh.stride, 0, sh.nchunks, run);
        if constexpr (KIND == SCAN_TOTAL) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            total[(size_t)bh * (size_t)total_stride + e] =
                __builtin_bit_cast(float, bf16x2{(__bf16)run.a, (__bf16)run.b});
        }
    } else {
        run = scan_range<KIND, W, false>(p, sh.nchunks, sh.stride, 0, sh.nchunks, run);
        if constexpr (KIND == SCAN_TOTAL) total[(size_t)bh * (size_t)total_stride + e] = run.a;
    }
}

// Total of the chunk states of one head and table group (float32 form) into
// its part of a running decode state: the F x 64 value sums in float32 at
// vals + bh * head_floats, and the F masses summed and stored in float64 at
// mass_off floats after that (mass_off < 0: not stored; the second value
// half at head dimension 128), so that counts beyond 2^24 keys stay exact.
template <int KIND = SCAN_TOTAL>
__global__ __launch_bounds__(256) void k_state_total(const float* __restrict__ st, float* __restrict__ vals,
                                                     int nchunks, int F, int64_t head_floats, int64_t mass_off) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= F * 65) return;
    const float* p = st + (size_t)bh * nchunks * (size_t)(F * 65) + e;
    float* out = vals + (size_t)bh * (size_t)head_floats;
    if (e < F * DH) {
        out[e] = scan_range<SCAN_TOTAL, false, false>(const_cast<float*>(p), nchunks, F * 65, 0, nchunks,
                                                       Run2{0.f, 0.f}).a;
    } else if (mass_off >= 0) {
        double z = 0.0;
        for (int c = 0; c < nchunks; ++c) z += (double)p[(size_t)c * (F * 65)];
        reinterpret_cast<double*>(out + mass_off)[e - F * DH] = z;
    }
}

// Segmented form of the (reverse) exclusive prefix, for grids too small to
// keep the memory busy (few heads): the logical chunk positions are split
// into segs segments; k_scan_segsum sums each segment, k_scan_segapply starts
// each segment from the sum of the segments before it (fixed order).
// segsum: per head and segment npair + nwords floats (ScanShape).
template <int KIND>
__global__ __launch_bounds__(256) void k_scan_segsum(const float* __restrict__ st, float* __restrict__ segsum,
                                                     ScanShape sh, int segs) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int bh = blockIdx.y / segs, sg = blockIdx.y % segs;
    if (e >= sh.nwords) return;
    const int len = (sh.nchunks + segs - 1) / segs;
    const int c0 = sg * len, c1 = min(sh.nchunks, c0 + len);
    float* p = const_cast<float*>(st) + (size_t)bh * sh.nchunks * sh.stride + e;
    float* out = segsum + ((size_t)bh * segs + sg) * (size_t)(sh.npair + sh.nwords);
    if (e < sh.npair) {
        const Run2 r = scan_range<KIND, false, true>(p, sh.nchunks, sh.stride, c0, c1, Run2{0.f, 0.f});
        out[2 * e] = r.a;
        out[2 * e + 1] = r.b;
    } else {
        out[sh.npair + e] = scan_range<KIND, false, false>(p, sh.nchunks, sh.stride, c0, c1, Run2{0.f, 0.f}).a;
    }
}

template <int KIND>
__global__ __launch_bounds__(256) void k_scan_segapply(float* __restrict__ st, const float* __restrict__ segsum,
                                                       ScanShape sh, int segs) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    const int bh = blockIdx.y / segs, sg = blockIdx.y % segs;
    if (e >= sh.nwords) return;
    const int len = (sh.nchunks + segs - 1) / segs;
    const int c0 = sg * len, c1 = min(sh.nchunks, c0 + len);
    const size_t per = (size_t)(sh.npair + sh.nwords);
    const bool pair = e < sh.npair;
    Run2 run{0.f, 0.f};
    for (int s2 = 0; s2 < sg; ++s2) {
        const float* in = segsum + ((size_t)bh * segs + s2) * per;
        if (pair) {
            run.a += in[2 * e];
            run.b += in[2 * e + 1];
        } else {
            run.a += in[sh.npair + e];
        }
    }
    float* p = st + (size_t)bh * sh.nchunks * sh.stride + e;
    if (pair) scan_range<KIND, true, true>(p, sh.nchunks, sh.stride, c0, c1, run);
    else scan_range<KIND, true, false>(p, sh.nchunks, sh.stride, c0, c1, run);
}

// ---------------------------------------------------------------------------
// sub-block passes
// ---------------------------------------------------------------------------
struct PassArgs {
    const void* Xa;        // readout-side rows (FWD, BWD_Q: Q; BWD_K: K)
    PlaneCache ca;         // readout side's plane values: FWD stores them (if ca.u), BWD_Q / BWD_K read them
    PlaneCache cb;         // sketch side's plane values (read)
    const void* Zsrc;      // FWD, BWD_Q: V; BWD_K: dO
    const void* Ysrc;      // BWD_Q: dO; BWD_K: V
    const void* Osrc;      // BWD_Q: the forward output O
    const void* W;         // [L, P, d] (this group's tables; per head: W of head h at + h * w_hs bytes)
    const void* WTp;       // back-projection operands (k_prep)
    const float* state;    // sketch before the chunk (causal) or the total
    int64_t state_bh_stride;
    int64_t state_chunk_stride;
    float* Dv;             // per-token D: FWD writes it when set; BWD_Q, BWD_K read it
    float* Ev;             // per-token e: BWD_Q writes it, BWD_K reads it
    void* out0;            // FWD: O; BWD_Q: dQ; BWD_K: dK
    void* out1;            // BWD_K: dV
    int64_t N;
    int chunk;
    int L;
    float beta;
    int causal;
    int hard;              // FWD: hard buckets (beta = HARD_BETA): a denominator below 2^(P-1) is 0
    // Table groups: a pass over one group of the tables adds its part of the
    // output to the partial of the groups before it (ACC_IN) and/or leaves
    // the sum as the next group's partial (ACC_OUT) instead of finishing the
    // output. acc: [rows][64] float32 (O's numerators, or dQ, dK before the
    // normalisation's chain rule, or dV); accD: the forward's denominators.
    float* acc;
    float* accD;
    int gmode;
    int H;                 // heads: W of sequence bh at W + (bh % H) * w_hs bytes, its
    int64_t w_hs;          // back-projection table at WTp + (bh % H) * wt_hs bytes
    int64_t wt_hs;         // (both 0 when one W serves every head)
    int dh;                // columns of a row the kernels use: 64, or 32 (columns 32..63 zero)
    int rs;                // elements between consecutive rows (the head dimension)
    // Head dimension 128 (the H2 forms of the gradient passes): the pass
    // covers value half `half` (64 columns); e comes from Ev in half 0 and is
    // 0 in half 1 (the mass terms count once), and instead of dQ or dK the
    // pass leaves the gradient wrt each normalised projection in dhb
    // ([rows][NPL] float32 of this group; half 1 adds to half 0's).
    float* dhb;
    int half;
};

enum { ACC_IN = 1, ACC_OUT = 2 };

// Head dimension 128: the per-plane gradient (dh / beta, as monomial_backward
// gives it) of projection tile t of in-chunk row rowi, stored, or added to the
// first value half's, in the group's [rows][NPL] float32 table.
template <class C>
__device__ inline void put_dh(rsrc_t rdh, int rowi, int t, int g, const float dh[4], bool add) {
    const int off = (rowi * C::NPL + 16 * t + 4 * g) * 4;
    f32x4 v = {dh[0], dh[1], dh[2], dh[3]};
    if (add) {
        const f32x4 prev = __builtin_bit_cast(f32x4, bload128(rdh, off));
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += prev[i];
    }
    bstore128(rdh, off, __builtin_bit_cast(u32x4, v));
}

// Partial output rows of one lane in the transposed read-out layout
// (columns cb + 4 g .. +3 of rows r0 + 16 at + ln), float32.
__device__ inline void acc_load_t(rsrc_t racc, int r0, int cb, int ln, int g, f32x4 (&Y)[4]) {
#pragma unroll
    for (int at = 0; at < 4; ++at) {
        const f32x4 v = __builtin_bit_cast(f32x4, bload128(racc, ((r0 + 16 * at + ln) * DH + cb + 4 * g) * 4));
        Y[at] += v;
    }
}
__device__ inline void acc_store_t(rsrc_t racc, int r0, int cb, int ln, int g, const f32x4 (&Y)[4]) {
#pragma unroll
    for (int at = 0; at < 4; ++at)
        bstore128(racc, ((r0 + 16 * at + ln) * DH + cb + 4 * g) * 4, __builtin_bit_cast(u32x4, Y[at]));
}
// The same for one own-token gradient row (columns 16 dt + 4 g .. +3 of row rowi).
__device__ inline void acc_load_row(rsrc_t racc, int rowi, int g, f32x4 (&dX)[4]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        dX[dt] += __builtin_bit_cast(f32x4, bload128(racc, (rowi * DH + 16 * dt + 4 * g) * 4));
}
__device__ inline void acc_store_row(rsrc_t racc, int rowi, int g, const f32x4 (&dX)[4]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) bstore128(racc, (rowi * DH + 16 * dt + 4 * g) * 4, __builtin_bit_cast(u32x4, dX[dt]));
}

// Sketch rows of feature block fb for the gradient contraction dA = M y:
// [FBK*32][ROWE], value columns of wave w and the mass column (64) from the
// wave that owns it. (In the monomial basis only the empty subset's rows carry
// the large plain sums, and its dA is not used.)
template <class C, bool TR = false>
__device__ inline void write_sketch_rows(int fb, int w, int ln, int g, const f32x4 Macc[C::NKC * 2],
                                         const f32x4 Zacc[C::NOWN * 2], typename Prec<C::F32>::elem* s_ms) {
    if constexpr (TR) {
        // transposed accumulators: four consecutive columns of one row per tile
#pragma unroll
        for (int kcl = 0; kcl < C::FBK; ++kcl)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                st_half<C::F32>(s_ms + (32 * kcl + 16 * h + ln) * C::ROWE + 16 * w + 4 * g,
                                Macc[2 * (fb * C::FBK + kcl) + h]);
        const int kw = w - C::own_base(fb);
        if (kw >= 0 && kw < C::FBK && g == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                s_ms[(32 * kw + 16 * h + ln) * C::ROWE + 64] = to_elem<C::F32>(Zacc[2 * C::zidx(fb) + h][0]);
        }
        return;
    }
#pragma unroll
    for (int kcl = 0; kcl < C::FBK; ++kcl)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 32 * kcl + 16 * h + 4 * g + i;
                s_ms[rl * C::ROWE + 16 * w + ln] = to_elem<C::F32>(Macc[2 * (fb * C::FBK + kcl) + h][i]);
            }
    const int kw = w - C::own_base(fb);
    if (kw >= 0 && kw < C::FBK && ln == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_ms[(32 * kw + 16 * h + 4 * g + i) * C::ROWE + 64] = to_elem<C::F32>(Zacc[2 * C::zidx(fb) + h][i]);
    }
}

// Zero the padding columns 65..95 of `nbuf` consecutive sketch-row tiles.
template <class C>
__device__ inline void zero_sketch_pads(typename Prec<C::F32>::elem* s_ms, int nbuf = 1) {
    for (int idx = threadIdx.x; idx < nbuf * C::FBK * 32 * 31; idx += NT)
        s_ms[(idx / 31) * C::ROWE + 65 + idx % 31] = to_elem<C::F32>(0.f);
}

// dA of feature block fb for the own token: the sketch part M y (three
// 32-wide K steps over the augmented width) plus, when causal, the
// intra-sub-block part phi_b^T Cc. G[2 kcl + h] holds canonical features
// 32 kcl + 8 g + 4 h + i of the block, matching the lane's feature order.
template <class C>
__device__ inline void block_grad(int ln, int g, const typename Prec<C::F32>::elem* s_ms,
                                  const typename Prec<C::F32>::frag yf[3], const typename Prec<C::F32>::elem* s_brow,
                                  const typename Prec<C::F32>::frag Cf[2], bool causal, f32x4 (&G)[C::FBK * 2]) {
#pragma unroll
    for (int m = 0; m < C::FBK * 2; ++m) {
        const int kcl = m >> 1, h = m & 1;
        const int fl = 32 * kcl + 16 * h + ln;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 3; ++s) acc = mma(ld_frag<C::F32>(s_ms + fl * C::ROWE + 32 * s + 8 * g), yf[s], acc);
        if (causal) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                acc = mma(feat_operand<C>(s_brow, kcl, h, s2, ln, g), Cf[s2], acc);
        }
        G[m] = acc;
    }
}

// True when projection tile t completes a pair of tiles (the back-projection
// operand covers two tiles).
template <class C>
__device__ constexpr bool completes_pair(int t) { return (t & 1) == 1 || t == C::MT - 1; }

// Back-projection operands (W'^T, four 16-column tiles) of the tile pair that
// tile t completes, from the table k_prep writes; loaded early in a block so
// the memory latency overlaps the block's matrix-core work.
template <class C>
__device__ inline void load_wtp(int t, int lane, const typename Prec<C::F32>::elem* WTp,
                                typename Prec<C::F32>::frag (&wf)[4]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) wf[dt] = ld_frag<C::F32>(WTp + ((size_t)((t >> 1) * 4 + dt) * 64 + lane) * 8);
}

// Chain rule of the monomial features for projection tile t of the own token
// (dA in the lane's feature order, t and dt/dh of its planes as tplanes gives
// them), then, when t completes a tile pair, the back-projection
// dX += W'^T dh with the operands wf of load_wtp.
template <class C>
__device__ inline void chain_backproject(int t, int g, const float dA[C::KB * 8], const float tt[4],
                                         const float gt[4], const typename Prec<C::F32>::frag (&wf)[4],
                                         f32x4 (&dhp)[2], f32x4 (&dX)[4]) {
    float dh[4];
    monomial_backward<C>(dA, tt, gt, dh, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) dhp[t & 1][i] = dh[i];
    if (completes_pair<C>(t)) {
        const typename Prec<C::F32>::frag df = pack<C::F32>(dhp[0], (t & 1) ? dhp[1] : f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dX[dt] = mma(wf[dt], df, dX[dt]);
        dhp[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        dhp[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Intra-sub-block operand of the gradient contraction: Cc[b][a] = z_b . y_a
// over the augmented width (y = hi + lo when YLO, z = hi + lo when ZLO; the
// lo x lo term is below float32 resolution), kept where sketch-side token b is
// visible from the own token a (b <= a, or b >= a when REV) and b < nv;
// returned as the two B operands of phi_b^T Cc (K index = b). The split
// matters where z_b . y_a nearly cancels: a query against its only key, so it
// is applied (lo = true) in the sub-block that starts the sequence.
template <class C, bool REV, bool YLO, bool ZLO>
__device__ inline void intra_operand(const typename Prec<C::F32>::elem* s_zr, const typename Prec<C::F32>::elem* s_zlo,
                                     const typename Prec<C::F32>::elem* s_yr, const typename Prec<C::F32>::elem* s_ylo,
                                     bool lo, int ln, int g, int my, int nv,
                                     typename Prec<C::F32>::frag (&Cf)[2]) {
    using frag = typename Prec<C::F32>::frag;
    f32x4 Cc[4];
    frag yf[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) yf[s] = ld_frag<C::F32>(s_yr + my * C::ROWE + 32 * s + 8 * g);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
        // every tile is formed (the mask below keeps the visible entries), so
        // all waves run the same instruction stream (skipping the tiles the
        // mask empties measured slower here)
        Cc[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const frag zf = ld_frag<C::F32>(s_zr + (16 * bt + ln) * C::ROWE + 32 * s + 8 * g);
            Cc[bt] = mma(zf, yf[s], Cc[bt]);
            if (YLO && lo) Cc[bt] = mma(zf, ld_frag<C::F32>(s_ylo + my * C::ROWE + 32 * s + 8 * g), Cc[bt]);
            if (ZLO && lo)
                Cc[bt] = mma(ld_frag<C::F32>(s_zlo + (16 * bt + ln) * C::ROWE + 32 * s + 8 * g), yf[s], Cc[bt]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 16 * bt + 4 * g + i;
            const bool v2 = (REV ? (b >= my) : (b <= my)) && b < nv;
            if (!v2) Cc[bt][i] = 0.f;
        }
    }
    Cf[0] = pack<C::F32>(Cc[0], Cc[1]);
    Cf[1] = pack<C::F32>(Cc[2], Cc[3]);
}

// The own token's row values that store_dx needs (columns 16 dt + 4 g .. +3),
// loaded early so the memory latency overlaps the sub-block's work.
template <class C>
__device__ inline void load_dx_row(rsrc_t rX, int rowi, int g, typename Prec<C::F32>::half (&xr)[4], int rs, int dh) {
    constexpr int es = C::F32 ? 4 : 2;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const int off = rowi * row_bytes<C::F32>(rs) + (16 * dt + 4 * g) * es;
        if (16 * dt >= dh) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[dt][i] = to_elem<C::F32>(0.f);
        } else if constexpr (C::F32) {
            xr[dt] = __builtin_bit_cast(f32x4, bload128(rX, off));
        } else {
            xr[dt] = __builtin_bit_cast(bf16x4, bload64(rX, off));
        }
    }
}

// dx = (dx_hat - x_hat <x_hat, dx_hat>) / |x| for the own token row (the chain
// rule of x_hat = x / max(|x|, eps); below eps the map is a plain scaling, and
// inv = 1 / max(|x|, eps) tells which case holds). dX[dt] holds columns
// 16 dt + 4 g .. +3 of dx_hat / beta (tplanes leaves beta out of dt/dh), so
// the final scaling is beta / max(|x|, eps).
template <class C>
__device__ inline void store_dx(const typename Prec<C::F32>::half (&xr)[4], rsrc_t rOut, int rowi, int g, float inv,
                                float beta, const f32x4 dX[4], int rs, int dh) {
    constexpr int es = C::F32 ? 4 : 2;
    float xv[4][4];
    float radial = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[dt][i] = (float)xr[dt][i];
            radial += xv[dt][i] * inv * dX[dt][i];
        }
    }
    radial = sum_groups(radial);
    const bool tangent = inv < rcp_(NORM_EPS);
    const float binv = beta * inv;   // dX carries dt/dh without its factor beta
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        if (16 * dt >= dh) break;
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (tangent ? dX[dt][i] - xv[dt][i] * inv * radial : dX[dt][i]) * binv;
        const int off = rowi * row_bytes<C::F32>(rs) + (16 * dt + 4 * g) * es;
        if constexpr (C::F32) {
            bstore128(rOut, off, __builtin_bit_cast(u32x4, o));
        } else {
            bf16x4 ob;
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i] = (__bf16)o[i];
            bstore64(rOut, off, __builtin_bit_cast(u32x2, ob));
        }
    }
}

// Store the transposed read-out tile Yt (C layout with rows = the wave's 16
// columns, columns = tokens: lane (ln, g) holds columns cb + 4 g .. +3 of
// token 16 at + ln) to in-chunk rows r0 + 16 at + ln of the output, scaling
// token rows by rs[at] and adding add[i] per column (rows past the chunk are
// dropped).
template <class C>
__device__ inline void store_rows_t(rsrc_t out, int r0, int cb, int ln, int g, const f32x4 (&Yt)[4],
                                    const float (&rsc)[4], const float (&add)[4], int rs, int dh) {
    constexpr int es = C::F32 ? 4 : 2;
    if (cb >= dh) return;   // columns past the head dimension (wave-uniform)
#pragma unroll
    for (int at = 0; at < 4; ++at) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (Yt[at][i] + add[i]) * rsc[at];
        const int off = (r0 + 16 * at + ln) * row_bytes<C::F32>(rs) + (cb + 4 * g) * es;
        if constexpr (C::F32) {
            bstore128(out, off, __builtin_bit_cast(u32x4, o));
        } else {
            bf16x4 ob;
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i] = (__bf16)o[i];
            bstore64(out, off, __builtin_bit_cast(u32x2, ob));
        }
    }
}


// LDS budget: W' is staged when it fits next to the tiles at the target
// number of workgroups per CU, else the projections read it from global memory.
template <class elem, int BASE, int NFLOAT, int MT, int OCC>
struct WStage {
    static constexpr int n_w0 = MT * 1024;
    static constexpr bool on = ((BASE + n_w0) * (int)sizeof(elem) + NFLOAT * 4) * OCC <= 160 * 1024;
    static constexpr int n_w = on ? n_w0 : 0;
    static constexpr int n_elem = BASE + n_w;
    static constexpr int bytes = n_elem * (int)sizeof(elem) + NFLOAT * 4;
    static_assert(bytes * OCC <= 160 * 1024, "LDS budget");
};

// ---------------------------------------------------------------------------
// forward pass: O = (sum_f phi_a,f M_f) / (sum_f phi_a,f z_f) with M, z the
// sketch of the keys before the sub-block plus the intra-sub-block causal term;
// then the sketch update. Also writes the per-token denominator D when Dv is set.
// ---------------------------------------------------------------------------
// Matrix-core operand of state tile pair kc with the rows of the empty subset
// set to zero (the forward read-out adds their contribution in float32).
template <class C>
__device__ inline typename Prec<C::F32>::frag pack_nonempty(int kc, int g, f32x4 lo, f32x4 hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (is_empty_subset<C>(kc, g, 0, i)) lo[i] = 0.f;
        if (is_empty_subset<C>(kc, g, 1, i)) hi[i] = 0.f;
    }
    return pack<C::F32>(lo, hi);
}

template <class C>
struct FwdLds {
    using elem = typename Prec<C::F32>::elem;
    static constexpr int n_rows = TB * C::ROWF;                 // a-side features [64][ROWF]
    static constexpr int n_brow = TB * C::ROWF;                 // b-side features [64][ROWF]
    static constexpr int ZS = ZV;                               // value-tile row stride
    static constexpr int n_zr = TB * ZS;                        // [z_b | mass], token rows
    static constexpr int n_sc = TB * C::ROWT;                   // intra scores [a][b]
    static constexpr int n_float = 4 * TB + TB + TB;            // Dpart, Dint, 1 / D
    // Feature tiles of a block, double-buffered where they fit: block fb uses
    // buffer fb % 2, so one barrier per block separates its writes from its
    // reads. A single buffer (float32, P = 6: 136-float rows) takes a second
    // barrier per block before the next block's writes.
    static constexpr int NB =
        ((2 * n_rows + 2 * n_brow + n_zr + n_sc) * (int)sizeof(elem) + n_float * 4 <= 160 * 1024) ? 2 : 1;
    static_assert(NB == 2 || (C::F32 && C::P == 6), "single buffers for float32 P = 6 only");
    static constexpr int o_rows = 0;                            // [NB][rows]
    static constexpr int o_brow = o_rows + NB * n_rows;         // [NB][brow]
    static constexpr int o_zr = o_brow + NB * n_brow;
    static constexpr int o_sc = o_zr + n_zr;
    static constexpr int o_w = o_sc + n_sc;
    // two workgroups per CU (VGPR budget 256: two waves share each SIMD) where
    // the tiles fit twice in the LDS
    static constexpr int OCC =
        (!C::F32 && C::NKC <= 8 && (o_w * (int)sizeof(elem) + n_float * 4) * 2 <= 160 * 1024) ? 2 : 1;
    using WS = WStage<elem, o_w, n_float, C::MT, OCC>;
};

// PG (head dimension 128): the queries' plane values come from ca (computed
// beforehand from the whole rows) instead of a projection of Q. HARD (bf16
// inputs, hard buckets): the exact denominator read-out below; a separate
// instantiation, so that the soft kernels keep their registers.
template <class C, bool CAUSAL, bool PG = false, bool HARD = false>
__global__ __launch_bounds__(NT, (FwdLds<C>::OCC))
__attribute__((amdgpu_waves_per_eu(FwdLds<C>::OCC, FwdLds<C>::OCC))) void k_fwd(PassArgs a) {
    using elem = typename Prec<C::F32>::elem;
    using frag = typename Prec<C::F32>::frag;
    using LD = FwdLds<C>;
    __shared__ __attribute__((aligned(32))) elem lds[LD::WS::n_elem];
    __shared__ float ldf[LD::n_float];
    elem* s_rows = lds + LD::o_rows;
    elem* s_brow = lds + LD::o_brow;
    elem* s_zr = lds + LD::o_zr;
    elem* s_sc = lds + LD::o_sc;
    float* f_Dpart = ldf;               // [4][64]
    float* f_Dint = ldf + 4 * TB;       // [64]
    float* f_rD = ldf + 5 * TB;         // [64]

    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    // wave index as a scalar: every branch on it is wave-uniform, so no MFMA is
    // ever issued under a partial or empty EXEC mask
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int th = threadIdx.x, tr = th >> 2, tq = th & 3;   // tile-row role of this thread
    const int bh = blockIdx.y, c = blockIdx.x;
    const int64_t seg0 = (int64_t)c * a.chunk;
    const int64_t seg1 = seg0 + a.chunk < a.N ? seg0 + a.chunk : a.N;
    const size_t base = (size_t)bh * a.N;
    const elem* W = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.W) + (bh % a.H) * a.w_hs);
    constexpr bool causal = CAUSAL;
    elem* s_w = LD::WS::on ? lds + LD::o_w : nullptr;
    if (LD::WS::on && !PG) stage_w<C>(W, a.L, s_w, a.dh);
    zero_pads<C, ZV>(s_zr, nullptr);
    __syncthreads();   // W' and the padding are written by all waves, read by each
    const WSrc<C, LD::WS::on> wsrc{s_w, W, a.L, a.dh};
    const int64_t nrows = seg1 - seg0;
    const size_t row0 = base + seg0;
    const rsrc_t rXa = rows_rsrc(a.Xa, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rZ = rows_rsrc(a.Zsrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rO = rows_rsrc(a.out0, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rD = rows_rsrc(a.Dv, row0, nrows, 4);
    const rsrc_t rAcc = rows_rsrc(a.acc, row0, nrows, DH * 4);
    const rsrc_t rAD = rows_rsrc(a.accD, row0, nrows, 4);
    const PlaneRows pra = plane_rows<C>(a.ca, row0, nrows), prb = plane_rows<C>(a.cb, row0, nrows);

    f32x4 Macc[C::NKC * 2], Zacc[C::NOWN * 2];
    load_state<C>(a.state + bh * a.state_bh_stride + c * a.state_chunk_stride, w, ln, g, Macc, Zacc);

    const int nsub = (int)((seg1 - seg0 + TB - 1) / TB);
    // Own 16-token tile of wave w in sub-block it: (w + it) mod 4. The tiles
    // rotate so that the in-sub-block score work, which shrinks with the
    // tile (keys after the own tokens are skipped), evens out over the SIMDs.
    auto own_tok = [&](int it2) { return 16 * ((w + it2) & 3) + ln; };

    // loads issued one sub-block (plane values: one feature block) ahead
    frag n_xa[2], n_z[2];
    Planes<C> pn, pq;
    auto nv_of = [&](int it2) {
        const int64_t t0 = seg0 + (int64_t)it2 * TB;
        return (int)(seg1 - t0 < TB ? seg1 - t0 : TB);
    };
    auto issue = [&](int it2) {
        if (!PG) load_row_b<C::F32>(rXa, it2 * TB + own_tok(it2), g, n_xa, a.rs, a.dh);
        load_q16_b<C::F32>(rZ, it2 * TB + tr, tq, n_z, a.rs, a.dh);
    };
    auto issue_planes = [&](int it2, int fb2) {
        if (causal) load_planes<C>(prb, it2 * TB + own_tok(it2), fb2, g, pn);
        if (PG) load_planes<C>(pra, it2 * TB + own_tok(it2), fb2, g, pq);
    };
    issue(0);
    if (causal || PG) issue_planes(0, 0);

    for (int it = 0; it < nsub; ++it) {
        const int64_t t0 = seg0 + (int64_t)it * TB;
        const int nv = nv_of(it);
        const bool tok = tr < nv;
        const int ow = (w + it) & 3;             // own tile (wave-uniform)
        const int my = 16 * ow + ln;             // own token within the sub-block
        const int rowi = it * TB + my;
        frag xa[2] = {n_xa[0], n_xa[1]}, zr[2] = {n_z[0], n_z[1]};
        if (it + 1 < nsub) issue(it + 1);

        const float inv_a = PG ? 0.f : row_inv_norm<C::F32>(xa);
        if (!PG && g == 0) bstore_f32(pra.inv, rowi * 4, inv_a);   // dropped without a cache
        write_aug<C, ZV, true>(zr, 1.f, tok ? 1.f : 0.f, s_zr);

        // The empty subset's state rows (plain sums of the keys' [v | 1], the
        // same for every valid table) enter the read-out exactly, in float32:
        // L times the value sums of this wave's columns (held by lane group 0
        // as table 0's first feature, before this sub-block's updates) and L
        // times the number of keys in the state.
        float y_empty[4];   // columns 16 w + 4 g + i of the transposed read-out
#pragma unroll
        for (int i = 0; i < 4; ++i) y_empty[i] = (float)a.L * __shfl(Macc[0][0], 4 * g + i);
        const float d_empty = (float)a.L * (float)(causal ? t0 : a.N);

        // the scores start at -n_pad: each padded table adds 1 (its empty
        // subset) to every query-key feature product
        const float sc0 = -(float)padded_tables<C>(a.L);
        f32x4 Y[4], Dacc[4], Sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Y[i] = f32x4{y_empty[0], y_empty[1], y_empty[2], y_empty[3]};   // the read-out adds to it
            Dacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            Sc[i] = f32x4{sc0, sc0, sc0, sc0};
        }
        // Software-pipelined feature blocks: after the barrier that publishes
        // block fb, a wave computes and writes the features of block fb + 1
        // (other buffer) while its matrix-core work on block fb proceeds.
        // With a single buffer the features of block fb are written after
        // the reads of block fb - 1.
        auto buf = [](int fb) { return LD::NB == 2 ? (fb & 1) : 0; };
        auto features = [&](int fb) {
            frag unused[C::FBK];
            elem* rows_b = s_rows + buf(fb) * LD::n_rows;
            elem* brow_b = s_brow + buf(fb) * LD::n_brow;
            const Planes<C> pl = pn, ql = pq;
            if (causal || PG) {
                if (fb + 1 < C::NBLK) issue_planes(it, fb + 1);
                else if (it + 1 < nsub) issue_planes(it + 1, 0);
            }
            if constexpr (PG) {
                float us[C::TPB][4], ug[C::TPB][4];
                block_features_cached<C, false>(ql, ow, ln, g, a.beta, rows_b, unused, us, ug);
            } else {
                block_features<C, false>(wsrc, fb, lane, ow, ln, g, xa, inv_a, a.beta, rows_b, unused, pra,
                                         rowi);
            }
            if (causal) {
                float us[C::TPB][4], ug[C::TPB][4];
                block_features_cached<C, false>(pl, ow, ln, g, a.beta, brow_b, unused, us, ug);
            }
        };
        if (LD::NB == 2) features(0);
#pragma unroll
        for (int fb = 0; fb < C::NBLK; ++fb) {
            const elem* rows_b = s_rows + buf(fb) * LD::n_rows;
            const elem* brow_b = s_brow + buf(fb) * LD::n_brow;
            if (LD::NB == 1) {
                if (fb > 0) __syncthreads();   // block fb - 1's tiles are read
                features(fb);
            }
            __syncthreads();
            if (LD::NB == 2 && fb + 1 < C::NBLK) features(fb + 1);
            if (causal) {
                // own features from the tile (not kept in registers); key
                // tiles after the own one are all masked and skipped
                frag pa[C::FBK];
#pragma unroll
                for (int kcl = 0; kcl < C::FBK; ++kcl) pa[kcl] = ld_frag<C::F32>(rows_b + my * C::ROWF + 32 * kcl + 8 * g);
#pragma unroll
                for (int bt = 0; bt < 4; ++bt) {
                    if (bt > ow) break;
#pragma unroll
                    for (int kcl = 0; kcl < C::FBK; ++kcl)
                        Sc[bt] = mma(ld_frag<C::F32>(brow_b + (16 * bt + ln) * C::ROWF + 32 * kcl + 8 * g), pa[kcl],
                                     Sc[bt]);
                }
            }
#pragma unroll
            for (int kcl = 0; kcl < C::FBK; ++kcl) {
                const int kc = fb * C::FBK + kcl;
                const frag mf = pack_nonempty<C>(kc, g, Macc[2 * kc], Macc[2 * kc + 1]);
#pragma unroll
                for (int at = 0; at < 4; ++at)
                    Y[at] = mma(mf, ld_frag<C::F32>(rows_b + (16 * at + ln) * C::ROWF + 32 * kcl + 8 * g), Y[at]);
            }
            const int kw = w - C::own_base(fb);
            if (kw >= 0 && kw < C::FBK) {
                const int kcz = fb * C::FBK + kw;
                f32x4 zl = Zacc[2 * C::zidx(fb)], zh = Zacc[2 * C::zidx(fb) + 1];
                const frag zf = pack_nonempty<C>(kcz, g, zl, zh);
                frag fa[4];
#pragma unroll
                for (int at = 0; at < 4; ++at) {
                    fa[at] = ld_frag<C::F32>(rows_b + (16 * at + ln) * C::ROWF + 32 * kw + 8 * g);
                    Dacc[at] = mma(fa[at], zf, Dacc[at]);
                }
                if constexpr (!C::F32) {
                    // hard buckets, bf16 operands: the masses are integers (below
                    // 2^24) and the features 0 or +-1, so the mass operand goes in
                    // as three bf16 parts of 8 significant bits each, and the
                    // denominator comes out exact
                    if constexpr (HARD) {
                        frag zp = zf;
#pragma unroll
                        for (int part = 0; part < 2; ++part) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                zl[i] -= (float)zp[i];
                                zh[i] -= (float)zp[4 + i];
                            }
                            zp = pack_nonempty<C>(kcz, g, zl, zh);
#pragma unroll
                            for (int at = 0; at < 4; ++at) Dacc[at] = mma(fa[at], zp, Dacc[at]);
                        }
                    }
                }
            }
            if (causal) sketch_update<C, true, ZV, true>(fb, w, ln, g, brow_b, s_zr, Macc, Zacc);
        }
        // intra-sub-block term: scores of visible keys b <= a. The value
        // readout multiplies the scores rounded to the operand type, so the
        // denominator sums the same rounded scores: O is then exactly a
        // weighted mean of the values (a lone key gives O = v, and the
        // backward's g.v + e cancels to float32 precision).
        if (causal) {
            float dint = 0.f;
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) {
                typename Prec<C::F32>::half hv;   // the rounded scores, packed once
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int b = 16 * bt + 4 * g + i;
                    hv[i] = to_elem<C::F32>((b <= my && b < nv) ? Sc[bt][i] : 0.f);
                }
                *reinterpret_cast<typename Prec<C::F32>::half*>(s_sc + my * C::ROWT + tok_pos(16 * bt + 4 * g)) = hv;
#pragma unroll
                for (int i = 0; i < 4; ++i) dint += elem_f<C::F32>(hv[i]);
            }
            dint = sum_groups(dint);
            if (g == 0) f_Dint[my] = dint;
        }
        if (ln == 0) {
#pragma unroll
            for (int at = 0; at < 4; ++at)
#pragma unroll
                for (int i = 0; i < 4; ++i) f_Dpart[w * TB + 16 * at + 4 * g + i] = Dacc[at][i];
        }
        __syncthreads();
        // one thread per token sums the denominator parts, stores D and
        // publishes 1 / D for the output normalisation
        if (tq == 0) {
            float d = f_Dpart[tr] + f_Dpart[TB + tr] + f_Dpart[2 * TB + tr] + f_Dpart[3 * TB + tr] + d_empty;
            if (causal) d += f_Dint[tr];
            if (a.gmode & ACC_IN) d += bload_f32(rAD, (it * TB + tr) * 4);
            if (a.gmode & ACC_OUT) {
                bstore_f32(rAD, (it * TB + tr) * 4, d);
            } else {
                bstore_f32(rD, (it * TB + tr) * 4, d);
                // hard buckets: D is 2^P times a collision count, so anything
                // below half a unit is an exact zero, and O = 0 for that query
                f_rD[tr] = (a.hard && fabsf(d) < (float)(1 << (C::P - 1))) ? 0.f : rcp_(d);
            }
        }
        if (causal) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const frag zt = val_operand<C, LD::ZS>(s_zr, 16 * w, s, ln, g);
#pragma unroll
                for (int at = 0; at < 4; ++at)   // queries 0..31 see no key of the second half
                    if (s == 0 || at >= 2)
                        Y[at] = mma(zt, ld_frag<C::F32>(s_sc + (16 * at + ln) * C::ROWT + 32 * s + 8 * g), Y[at]);
            }
        }
        if (a.gmode & ACC_IN) acc_load_t(rAcc, it * TB, 16 * w, ln, g, Y);
        __syncthreads();
        if (a.gmode & ACC_OUT) {
            acc_store_t(rAcc, it * TB, 16 * w, ln, g, Y);
        } else {
            float rd[4];
#pragma unroll
            for (int at = 0; at < 4; ++at) rd[at] = f_rD[16 * at + ln];
            const float none[4] = {-0.f, -0.f, -0.f, -0.f};   // x + -0 = x: nothing added
            store_rows_t<C>(rO, it * TB, 16 * w, ln, g, Y, rd, none, a.rs, a.dh);
        }
    }
}

// ---------------------------------------------------------------------------
// query-side backward: y = [dO/D | e] with e = -<dO, O>/D from the saved D and
// the forward output; dA_Q = M y (sketch of the keys before the sub-block, plus
// the intra-sub-block causal term), the chain rule of the monomials and tanh,
// the back-projection and the normalisation's chain rule -> dQ; also writes e.
// ---------------------------------------------------------------------------
template <class C>
struct BwdQLds {
    using elem = typename Prec<C::F32>::elem;
    // bf16 residual of the y rows: the intra-sub-block product g.v + e
    // cancels for a query against the first keys of a sequence, so in that
    // sub-block it is formed from y = hi + lo with float32 accumulation
    static constexpr bool YLO = !C::F32;
    static constexpr int n_ms = C::FBK * 32 * C::ROWE;          // sketch rows
    static constexpr int n_cols = TB * C::ROWF;                 // key features, token rows
    static constexpr int n_zr = TB * C::ROWE;                   // [v | 1] rows
    static constexpr int n_yr = TB * C::ROWE;                   // y rows (hi)
    static constexpr int n_ylo = YLO ? TB * C::ROWE : 0;        // y rows (lo)
    // The per-block tiles (sketch rows, key features) are double-buffered
    // where they fit: block fb uses buffer fb % 2, so one barrier per block
    // separates writes from reads (a single buffer, float32 P = 6, takes a
    // second barrier per block). The y lo rows (first sub-block of a sequence
    // only, read before the block loop) share the feature buffers where they
    // fit.
    static constexpr int NB = ((2 * n_ms + 2 * n_cols + n_zr + n_yr) * (int)sizeof(elem) <= 160 * 1024) ? 2 : 1;
    static_assert(NB == 2 || (C::F32 && C::P == 6), "single buffers for float32 P = 6 only");
    static constexpr bool YLO_SHARED = n_ylo <= NB * n_cols;
    static constexpr int o_ms = 0;
    static constexpr int o_cols = o_ms + NB * n_ms;
    static constexpr int o_zr = o_cols + NB * n_cols;
    static constexpr int o_yr = o_zr + n_zr;
    static constexpr int o_end = o_yr + n_yr;
    static constexpr int o_ylo = YLO_SHARED ? o_cols : o_end;
    static constexpr int n_elem = o_end + (YLO_SHARED ? 0 : n_ylo);
    // two workgroups per CU where registers (bf16, up to 8 feature chunks) and
    // LDS allow
    static constexpr int OCC =
        (!C::F32 && C::NKC <= 8 && n_elem * (int)sizeof(elem) * 2 <= 160 * 1024) ? 2 : 1;
    static_assert(n_elem * (int)sizeof(elem) * OCC <= 160 * 1024, "LDS budget");
};

template <class C, bool CAUSAL, bool H2 = false>
__global__ __launch_bounds__(NT, (BwdQLds<C>::OCC))
__attribute__((amdgpu_waves_per_eu(BwdQLds<C>::OCC, BwdQLds<C>::OCC))) void k_bwd_q(PassArgs a) {
    using elem = typename Prec<C::F32>::elem;
    using frag = typename Prec<C::F32>::frag;
    using LD = BwdQLds<C>;
    __shared__ __attribute__((aligned(32))) elem lds[LD::n_elem];
    elem* s_ms = lds + LD::o_ms;
    elem* s_cols = lds + LD::o_cols;
    elem* s_zr = lds + LD::o_zr;
    elem* s_yr = lds + LD::o_yr;
    elem* s_ylo = lds + LD::o_ylo;

    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int th = threadIdx.x, tr = th >> 2, tq = th & 3;
    const int bh = blockIdx.y, c = blockIdx.x;
    const int64_t seg0 = (int64_t)c * a.chunk;
    const int64_t seg1 = seg0 + a.chunk < a.N ? seg0 + a.chunk : a.N;
    const size_t base = (size_t)bh * a.N;
    const elem* WTp = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.WTp) + (bh % a.H) * a.wt_hs);
    constexpr bool causal = CAUSAL;
    zero_sketch_pads<C>(s_ms, LD::NB);
    zero_pads<C>(s_zr, s_yr);
    if (LD::YLO) zero_pads<C>(s_ylo, nullptr);
    __syncthreads();   // the padding is written by all waves, read by each

    f32x4 Macc[C::NKC * 2], Zacc[C::NOWN * 2];
    // bf16: the state in the transposed accumulator layout (sketch rows are
    // then written four columns at a time)
    constexpr bool TR = !C::F32;
    if constexpr (TR) load_state_t<C>(a.state + bh * a.state_bh_stride + c * a.state_chunk_stride, w, ln, g, Macc, Zacc);
    else load_state<C>(a.state + bh * a.state_bh_stride + c * a.state_chunk_stride, w, ln, g, Macc, Zacc);

    const int nsub = (int)((seg1 - seg0 + TB - 1) / TB);
    const int my = 16 * w + ln;
    const int64_t nrows = seg1 - seg0;
    const size_t row0 = base + seg0;
    const rsrc_t rZ = rows_rsrc(a.Zsrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rY = rows_rsrc(a.Ysrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rOs = rows_rsrc(a.Osrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rXa = rows_rsrc(a.Xa, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rOut = rows_rsrc(a.out0, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rD = rows_rsrc(a.Dv, row0, nrows, 4);
    const rsrc_t rE = rows_rsrc(a.Ev, row0, nrows, 4);
    const rsrc_t rAcc = rows_rsrc(a.acc, row0, nrows, DH * 4);
    const rsrc_t rdh = rows_rsrc(H2 ? a.dhb : nullptr, row0, nrows, C::NPL * 4);
    const PlaneRows pra = plane_rows<C>(a.ca, row0, nrows), prb = plane_rows<C>(a.cb, row0, nrows);

    // the plane values of queries and keys are loaded one feature block ahead;
    // the value, gradient and output rows at the top of their sub-block
    // (register budget)
    Planes<C> pa, pb;
    auto nv_of = [&](int it2) {
        const int64_t t0 = seg0 + (int64_t)it2 * TB;
        return (int)(seg1 - t0 < TB ? seg1 - t0 : TB);
    };
    auto issue_planes = [&](int it2, int fb2) {
        load_planes<C>(pra, it2 * TB + my, fb2, g, pa);
        if (causal) load_planes<C>(prb, it2 * TB + my, fb2, g, pb);
    };
    issue_planes(0, 0);

    for (int it = 0; it < nsub; ++it) {
        const int64_t t0 = seg0 + (int64_t)it * TB;
        const int nv = nv_of(it);
        const bool valid = my < nv;
        const int rowi = it * TB + my, rowt = it * TB + tr;
        const bool tok = tr < nv;
        frag zr[2], yr[2], orow[2];
        if (causal) load_q16_b<C::F32>(rZ, rowt, tq, zr, a.rs, a.dh);
        load_q16_b<C::F32>(rY, rowt, tq, yr, a.rs, a.dh);
        if (!H2) load_q16_b<C::F32>(rOs, rowt, tq, orow, a.rs, a.dh);
        const float dd = tok ? bload_f32(rD, rowt * 4) : 1.f;
        const float e_in = (H2 && a.half == 0) ? bload_f32(rE, rowt * 4) : 0.f;
        const float inv_a = (!H2 && valid) ? bload_f32(pra.inv, rowi * 4) : 1.f;
        typename Prec<C::F32>::half xr[4];
        if (!H2) load_dx_row<C>(rXa, rowi, g, xr, a.rs, a.dh);
        const bool first = t0 == 0;   // the sub-block that starts the sequence
        if (causal) write_aug<C, C::ROWE, true>(zr, 1.f, tok ? 1.f : 0.f, s_zr);
        // y = [dO / D | e], e = -<dO, O> / D; this thread holds 16 columns of row tr
        {
            const float rD = tok ? rcp_(dd) : 0.f;
            float e;
            if constexpr (H2) {
                e = tok ? e_in : 0.f;   // over all 128 columns, computed beforehand
            } else {
                float delta = dot16<C::F32>(yr, orow);
                delta += __shfl_xor(delta, 1);
                delta += __shfl_xor(delta, 2);
                e = -delta * rD;
            }
            float v[16];
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) v[cc] = q16_at<C::F32>(yr, cc) * rD;
            const frag h0 = pack8<C::F32>(v), h1 = pack8<C::F32>(v + 8);
            st_frag<C::F32>(s_yr + tr * C::ROWE + 16 * tq, h0);
            st_frag<C::F32>(s_yr + tr * C::ROWE + 16 * tq + 8, h1);
            if (LD::YLO && first) {
                float lo[16];
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    lo[cc] = v[cc] - elem_f<C::F32>(h0[cc]);
                    lo[8 + cc] = v[8 + cc] - elem_f<C::F32>(h1[cc]);
                }
                st_frag<C::F32>(s_ylo + tr * C::ROWE + 16 * tq, pack8<C::F32>(lo));
                st_frag<C::F32>(s_ylo + tr * C::ROWE + 16 * tq + 8, pack8<C::F32>(lo + 8));
            }
            if (tq == 0) {
                const elem eh = to_elem<C::F32>(e);
                s_yr[tr * C::ROWE + 64] = eh;
                if (LD::YLO && first) s_ylo[tr * C::ROWE + 64] = to_elem<C::F32>(e - elem_f<C::F32>(eh));
                if (!H2) bstore_f32(rE, rowt * 4, e);
            }
        }
        __syncthreads();
        frag Cf[2];
        if (causal)
            intra_operand<C, false, LD::YLO, false>(s_zr, nullptr, s_yr, s_ylo, first, ln, g, my, nv, Cf);
        if (LD::YLO && LD::YLO_SHARED && causal && first)
            __syncthreads();   // the y lo rows are read; their space becomes the feature tiles
        f32x4 dX[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) dX[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 dhp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int fb = 0; fb < C::NBLK; ++fb) {
            frag wf[C::TPB][4];
            if constexpr (!H2) {
#pragma unroll
                for (int tb = 0; tb < C::TPB; ++tb)
                    if (completes_pair<C>(fb * C::TPB + tb)) load_wtp<C>(fb * C::TPB + tb, lane, WTp, wf[tb]);
            }
            const Planes<C> qa = pa, kb_ = pb;
            if (fb + 1 < C::NBLK) issue_planes(it, fb + 1);
            else if (it + 1 < nsub) issue_planes(it + 1, 0);
            const int bsel = LD::NB == 2 ? (fb & 1) : 0;
            elem* ms_b = s_ms + bsel * LD::n_ms;
            elem* cols_b = s_cols + bsel * LD::n_cols;
            write_sketch_rows<C, TR>(fb, w, ln, g, Macc, Zacc, ms_b);
            if (causal) {
                frag unused[C::FBK];
                float us[C::TPB][4], ug[C::TPB][4];
                block_features_cached<C, false>(kb_, w, ln, g, a.beta, cols_b, unused, us, ug);
            }
            __syncthreads();
            frag yf[3];
#pragma unroll
            for (int s = 0; s < 3; ++s) yf[s] = ld_frag<C::F32>(s_yr + my * C::ROWE + 32 * s + 8 * g);
            f32x4 G[C::FBK * 2];
            block_grad<C>(ln, g, ms_b, yf, cols_b, Cf, causal, G);
#pragma unroll
            for (int tb = 0; tb < C::TPB; ++tb) {
                const int t = fb * C::TPB + tb;
                float tt[4], gt[4], dA[C::KB * 8];
                tplanes<C::F32>(qa.u[tb], a.beta, tt, gt);
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb) {
                    const int kcl = tb * C::KB + kb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        dA[kb * 8 + i] = G[2 * kcl][i];
                        dA[kb * 8 + 4 + i] = G[2 * kcl + 1][i];
                    }
                }
                if constexpr (H2) {
                    float dh[4];
                    monomial_backward<C>(dA, tt, gt, dh, g);
                    put_dh<C>(rdh, rowi, t, g, dh, a.half != 0);
                } else {
                    chain_backproject<C>(t, g, dA, tt, gt, wf[tb], dhp, dX);
                }
            }
            if (causal) sketch_update<C, true, C::ROWE, false, TR>(fb, w, ln, g, cols_b, s_zr, Macc, Zacc);
            if (LD::NB == 1) __syncthreads();   // single buffer: read before the next block's writes
        }
        __syncthreads();   // the next sub-block rewrites the y and z rows
        if constexpr (!H2) {
            if (a.gmode & ACC_IN) acc_load_row(rAcc, rowi, g, dX);
            if (a.gmode & ACC_OUT) acc_store_row(rAcc, rowi, g, dX);
            else store_dx<C>(xr, rOut, rowi, g, inv_a, a.beta, dX, a.rs, a.dh);
        }
    }
}

// ---------------------------------------------------------------------------
// key-side backward (sub-blocks in reverse), against the reverse sketch
// T = sum_b phi_b^T [dO_b / D_b | e_b] of the queries after the sub-block:
//   dV_a  = phi_a^T T_g  (+ intra: sum_{b >= a} <phi_b, phi_a> g_b)
//   dA_K  = T [v_a | 1]  (+ intra: phi_b^T Cc, Cc[b][a] = g_b . v_a + e_b)
// then the chain rule -> dK. PART selects dV (KPART_DV) or dK (KPART_DK),
// two launches: split, the dV pass fits three workgroups per CU and the dK
// pass two.
// ---------------------------------------------------------------------------
enum { KPART_DV = 1, KPART_DK = 2 };

template <class C, int PART>
struct BwdKLds {
    using elem = typename Prec<C::F32>::elem;
    static constexpr bool DV = PART == KPART_DV;
    static constexpr bool DK = PART == KPART_DK;
    static constexpr int n_rows = DV ? TB * C::ROWF : 0;        // key features [64][ROWF]
    static constexpr int n_brow = DV ? TB * C::ROWF : 0;        // query features [64][ROWF]
    static constexpr int n_cols = DK ? TB * C::ROWF : 0;        // query features, token rows
    static constexpr int n_ms = DK ? C::FBK * 32 * C::ROWE : 0; // sketch rows
    // per-sub-block tiles
    static constexpr int n_sc = DV ? TB * C::ROWT : 0;          // intra scores [a][b]
    // [g | e] rows: the dK pass also reads them as intra-product rows over the
    // augmented width, the dV pass only through transpose reads
    static constexpr int ZS = DK ? C::ROWE : ZV;
    static constexpr int n_zr = TB * ZS;
    // bf16 residual of the [g | e] rows: the intra-sub-block product g.v + e
    // cancels for a query against its only key
    static constexpr bool ZLO = DK && !C::F32;
    static constexpr int n_zlo = ZLO ? TB * C::ROWE : 0;
    static constexpr int n_yr = DK ? TB * C::ROWE : 0;          // [v | 1] rows
    // per-block tiles, double-buffered where they fit: block fb uses buffer
    // fb % 2, so one barrier per block separates writes from reads (a single
    // buffer, float32 P = 6, takes a second barrier per block)
    static constexpr int NB =
        ((2 * (n_rows + n_brow + n_cols + n_ms) + TB * ZS + n_yr) * (int)sizeof(elem) <= 160 * 1024) ? 2 : 1;
    static_assert(NB == 2 || (C::F32 && C::P == 6), "single buffers for float32 P = 6 only");
    // Tiles live outside the block loop share the block buffers where they
    // fit: the intra scores the first query-feature buffer (dV) or the feature
    // buffers (dK), the residual rows the feature buffers.
    static constexpr bool SC_SHARED = DV ? n_sc <= n_brow : n_sc <= NB * n_cols;
    static constexpr bool ZLO_SHARED = n_zlo <= NB * n_cols;
    static constexpr int o_rows = 0;                            // [NB][rows | brow]
    static constexpr int o_brow = o_rows + n_rows;
    static constexpr int RB = n_rows + n_brow;                  // stride of the row-feature buffers
    static constexpr int o_cols = NB * RB;                      // [NB][cols]
    static constexpr int o_ms = o_cols + NB * n_cols;           // [NB][ms]
    static constexpr int o_zr = o_ms + NB * n_ms;
    static constexpr int o_yr = o_zr + n_zr;
    static constexpr int o_x0 = o_yr + n_yr;                    // unshared tiles follow
    static constexpr int o_sc = SC_SHARED ? (DV ? o_brow : o_cols) : o_x0;
    static constexpr int o_x1 = o_x0 + (SC_SHARED ? 0 : n_sc);
    static constexpr int o_x2 = o_x1;
    static constexpr int o_zlo = ZLO_SHARED ? o_cols : o_x2;
    static constexpr int n_elem = o_x2 + (ZLO_SHARED ? 0 : n_zlo);
    // workgroups per CU where registers (bf16, up to 8 feature chunks) and LDS
    // allow: three for the dV pass, two for the dK pass
    static constexpr int BYTES = n_elem * (int)sizeof(elem);
    static constexpr int OCC = (C::F32 || C::NKC > 8) ? 1
                               : (DV && BYTES * 3 <= 160 * 1024) ? 3
                               : (BYTES * 2 <= 160 * 1024) ? 2 : 1;
    static_assert(BYTES * OCC <= 160 * 1024, "LDS budget");
};

// H2 (head dimension 128, the dK part only): see PassArgs::dhb.
template <class C, bool CAUSAL, int PART, bool H2 = false>
__global__ __launch_bounds__(NT, (BwdKLds<C, PART>::OCC))
__attribute__((amdgpu_waves_per_eu(BwdKLds<C, PART>::OCC, BwdKLds<C, PART>::OCC))) void k_bwd_k(PassArgs a) {
    static_assert(!H2 || PART == KPART_DK, "the dV part has no head-dimension-128 form");
    using elem = typename Prec<C::F32>::elem;
    using frag = typename Prec<C::F32>::frag;
    using LD = BwdKLds<C, PART>;
    constexpr bool DV = LD::DV, DK = LD::DK;
    __shared__ __attribute__((aligned(32))) elem lds[LD::n_elem];
    elem* s_rows = lds + LD::o_rows;
    elem* s_brow = lds + LD::o_brow;
    elem* s_cols = lds + LD::o_cols;
    elem* s_ms = lds + LD::o_ms;
    elem* s_sc = lds + LD::o_sc;
    elem* s_zr = lds + LD::o_zr;
    elem* s_yr = lds + LD::o_yr;
    elem* s_zlo = lds + LD::o_zlo;

    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int th = threadIdx.x, tr = th >> 2, tq = th & 3;
    const int bh = blockIdx.y, c = blockIdx.x;
    const int64_t seg0 = (int64_t)c * a.chunk;
    const int64_t seg1 = seg0 + a.chunk < a.N ? seg0 + a.chunk : a.N;
    const size_t base = (size_t)bh * a.N;
    const elem* WTp = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.WTp) + (bh % a.H) * a.wt_hs);
    constexpr bool causal = CAUSAL;
    if (DK) zero_sketch_pads<C>(s_ms, LD::NB);
    zero_pads<C, LD::ZS>(s_zr, DK ? s_yr : nullptr);
    if (LD::ZLO) zero_pads<C>(s_zlo, nullptr);
    __syncthreads();   // the padding is written by all waves, read by each

    f32x4 Macc[C::NKC * 2], Zacc[C::NOWN * 2];
    // dK, bf16: the state in the transposed accumulator layout (sketch rows are
    // then written four columns at a time); the dV read-out needs the plain one
    constexpr bool TR = DK && !C::F32;
    if constexpr (TR) load_state_t<C>(a.state + bh * a.state_bh_stride + c * a.state_chunk_stride, w, ln, g, Macc, Zacc);
    else load_state<C>(a.state + bh * a.state_bh_stride + c * a.state_chunk_stride, w, ln, g, Macc, Zacc);

    const int nsub = (int)((seg1 - seg0 + TB - 1) / TB);
    // Own 16-token tile: w (rotating it, as the forward does, measured slower
    // here: the register budget of three workgroups per CU has no room left).
    const int my = 16 * w + ln;

    // global loads are issued one sub-block (plane values: one feature block)
    // ahead; in the split passes the rows at the top of their sub-block
    constexpr bool PREFETCH = LD::OCC == 1;
    frag n_z[2], n_y[2];
    float n_d = 1.f, n_e = 0.f, n_inv = 1.f;
    Planes<C> pa, pb;
    auto t0_of = [&](int it2) { return seg0 + (int64_t)(nsub - 1 - it2) * TB; };
    auto nv_of = [&](int it2) {
        const int64_t t0 = t0_of(it2);
        return (int)(seg1 - t0 < TB ? seg1 - t0 : TB);
    };
    const int64_t nrows = seg1 - seg0;
    const size_t row0 = base + seg0;
    const rsrc_t rZ = rows_rsrc(a.Zsrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rY = rows_rsrc(a.Ysrc, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rXa = rows_rsrc(a.Xa, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rOut0 = rows_rsrc(a.out0, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rOut1 = rows_rsrc(a.out1, row0, nrows, row_bytes<C::F32>(a.rs));
    const rsrc_t rD = rows_rsrc(a.Dv, row0, nrows, 4);
    const rsrc_t rE = rows_rsrc(a.Ev, row0, nrows, 4);
    const rsrc_t rAcc = rows_rsrc(a.acc, row0, nrows, DH * 4);
    const rsrc_t rdh = rows_rsrc(H2 ? a.dhb : nullptr, row0, nrows, C::NPL * 4);
    const PlaneRows pra = plane_rows<C>(a.ca, row0, nrows), prb = plane_rows<C>(a.cb, row0, nrows);
    auto r0_of = [&](int it2) { return (nsub - 1 - it2) * TB; };   // first in-chunk row of a sub-block
    auto issue = [&](int it2) {
        const int r0 = r0_of(it2);
        if (DK && !H2) n_inv = my < nv_of(it2) ? bload_f32(pra.inv, (r0 + my) * 4) : 1.f;
        if (causal) {
            load_q16_b<C::F32>(rZ, r0 + tr, tq, n_z, a.rs, a.dh);
            n_d = bload_f32(rD, (r0 + tr) * 4);
            n_e = (H2 && a.half != 0) ? 0.f : bload_f32(rE, (r0 + tr) * 4);
        }
        if (DK) load_q16_b<C::F32>(rY, r0 + tr, tq, n_y, a.rs, a.dh);
    };
    auto issue_planes = [&](int it2, int fb2) {
        load_planes<C>(pra, r0_of(it2) + my, fb2, g, pa);
        if (causal) load_planes<C>(prb, r0_of(it2) + my, fb2, g, pb);
    };
    if (PREFETCH) issue(0);
    issue_planes(0, 0);

    for (int it = 0; it < nsub; ++it) {
        const int64_t t0 = t0_of(it);
        const int nv = nv_of(it);
        const bool tok = tr < nv;
        if (!PREFETCH) issue(it);
        frag zr[2] = {n_z[0], n_z[1]}, yr[2] = {n_y[0], n_y[1]};
        const float zd = n_d, ze = n_e, inv_a = n_inv;
        if (PREFETCH && it + 1 < nsub) issue(it + 1);

        typename Prec<C::F32>::half xr[4];
        if constexpr (DK && !H2) load_dx_row<C>(rXa, r0_of(it) + my, g, xr, a.rs, a.dh);
        const bool first = t0 == 0;   // the sub-block that starts the sequence
        if (causal)
            write_aug<C, LD::ZS>(zr, tok ? rcp_(zd) : 0.f, tok ? ze : 0.f, s_zr,
                         (LD::ZLO && first) ? s_zlo : nullptr);
        if constexpr (DK) {
            // y rows = [v | 1]
            float v[16];
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) v[cc] = q16_at<C::F32>(yr, cc);
            st_frag<C::F32>(s_yr + tr * C::ROWE + 16 * tq, pack8<C::F32>(v));
            st_frag<C::F32>(s_yr + tr * C::ROWE + 16 * tq + 8, pack8<C::F32>(v + 8));
            if (tq == 0) s_yr[tr * C::ROWE + 64] = to_elem<C::F32>(tok ? 1.f : 0.f);
        }
        __syncthreads();
        frag Cf[2];
        if (DK && causal)
            intra_operand<C, true, false, LD::ZLO>(s_zr, s_zlo, s_yr, nullptr, first, ln, g, my, nv, Cf);
        if (LD::ZLO && LD::ZLO_SHARED && causal && first)
            __syncthreads();   // the residual rows are read; their space becomes the feature tiles
        // Padded tables: their empty subset (1) adds 1 to every feature
        // product, so the dV scores start at -n_pad, and n_pad times the
        // empty-subset row of the gradient sketch (the same for every table;
        // table 0's, held by lane group 0, before this sub-block's updates) is
        // taken off the dV read-out (columns 16 w + 4 g + i).
        const int npad = padded_tables<C>(a.L);
        float y0[4] = {0.f, 0.f, 0.f, 0.f};
        if (DV && npad > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) y0[i] = -(float)npad * __shfl(Macc[0][0], 4 * g + i);
        }
        f32x4 Y[4], Sc[4], dX[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Y[i] = f32x4{y0[0], y0[1], y0[2], y0[3]};
            Sc[i] = f32x4{-(float)npad, -(float)npad, -(float)npad, -(float)npad};
            dX[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 dhp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int fb = 0; fb < C::NBLK; ++fb) {
            frag unused[C::FBK];
            float us[C::TPB][4], ug[C::TPB][4];
            frag wf[C::TPB][4];
            if constexpr (DK && !H2) {
#pragma unroll
                for (int tb = 0; tb < C::TPB; ++tb)
                    if (completes_pair<C>(fb * C::TPB + tb)) load_wtp<C>(fb * C::TPB + tb, lane, WTp, wf[tb]);
            }
            const Planes<C> ka = pa, qb = pb;
            if (fb + 1 < C::NBLK) issue_planes(it, fb + 1);
            else if (it + 1 < nsub) issue_planes(it + 1, 0);
            const int bsel = LD::NB == 2 ? (fb & 1) : 0;
            elem* rows_b = s_rows + bsel * LD::RB;
            elem* brow_b = s_brow + bsel * LD::RB;
            elem* cols_b = s_cols + bsel * LD::n_cols;
            elem* ms_b = s_ms + bsel * LD::n_ms;
            if constexpr (DV) {
                block_features_cached<C, false>(ka, w, ln, g, a.beta, rows_b, unused, us, ug);
                if (causal)
                    block_features_cached<C, false>(qb, w, ln, g, a.beta, brow_b, unused, us, ug);
            } else if (causal) {
                block_features_cached<C, false>(qb, w, ln, g, a.beta, cols_b, unused, us, ug);
            }
            if constexpr (DK) write_sketch_rows<C, TR>(fb, w, ln, g, Macc, Zacc, ms_b);
            __syncthreads();
            if constexpr (DV) {
                if (causal) {
                    // own features from the tile (not kept in registers); query
                    // tiles before the own one are all masked and skipped
#pragma unroll
                    for (int kcl = 0; kcl < C::FBK; ++kcl) {
                        const frag pa = ld_frag<C::F32>(rows_b + my * C::ROWF + 32 * kcl + 8 * g);
#pragma unroll
                        for (int bt = 0; bt < 4; ++bt)
                            if (bt >= w)
                                Sc[bt] = mma(ld_frag<C::F32>(brow_b + (16 * bt + ln) * C::ROWF + 32 * kcl + 8 * g),
                                             pa, Sc[bt]);
                    }
                }
                // dV readout of the value columns of this wave (before this block's update)
#pragma unroll
                for (int kcl = 0; kcl < C::FBK; ++kcl) {
                    const int kc = fb * C::FBK + kcl;
                    const frag mf = pack<C::F32>(Macc[2 * kc], Macc[2 * kc + 1]);
#pragma unroll
                    for (int at = 0; at < 4; ++at)
                        Y[at] = mma(mf, ld_frag<C::F32>(rows_b + (16 * at + ln) * C::ROWF + 32 * kcl + 8 * g), Y[at]);
                }
            }
            if constexpr (DK) {
                frag yf[3];
#pragma unroll
                for (int s = 0; s < 3; ++s) yf[s] = ld_frag<C::F32>(s_yr + my * C::ROWE + 32 * s + 8 * g);
                f32x4 G[C::FBK * 2];
                block_grad<C>(ln, g, ms_b, yf, cols_b, Cf, causal, G);
#pragma unroll
                for (int tb = 0; tb < C::TPB; ++tb) {
                    const int t = fb * C::TPB + tb;
                    float dA[C::KB * 8], tt[4], gt[4];
                    tplanes<C::F32>(ka.u[tb], a.beta, tt, gt);
#pragma unroll
                    for (int kb = 0; kb < C::KB; ++kb) {
                        const int kcl = tb * C::KB + kb;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            dA[kb * 8 + i] = G[2 * kcl][i];
                            dA[kb * 8 + 4 + i] = G[2 * kcl + 1][i];
                        }
                    }
                    if constexpr (H2) {
                        float dh[4];
                        monomial_backward<C>(dA, tt, gt, dh, g);
                        put_dh<C>(rdh, r0_of(it) + my, t, g, dh, a.half != 0);
                    } else {
                        chain_backproject<C>(t, g, dA, tt, gt, wf[tb], dhp, dX);
                    }
                }
            }
            if (causal) sketch_update<C, DK, LD::ZS, DV, TR>(fb, w, ln, g, DV ? brow_b : cols_b, s_zr, Macc, Zacc);
            if (LD::NB == 1) __syncthreads();   // single buffer: read before the next block's writes
        }
        __syncthreads();   // the block tiles are read; the sub-block tiles below reuse them
        if constexpr (DV) {
            // intra-sub-block dV: queries b >= a
            if (causal) {
#pragma unroll
                for (int bt = 0; bt < 4; ++bt) {
                    f32x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int b = 16 * bt + 4 * g + i;
                        v[i] = (b >= my && b < nv) ? Sc[bt][i] : 0.f;
                    }
                    st_half<C::F32>(s_sc + my * C::ROWT + tok_pos(16 * bt + 4 * g), v);
                }
                __syncthreads();
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const frag zt = val_operand<C, LD::ZS>(s_zr, 16 * w, s, ln, g);
#pragma unroll
                    for (int at = 0; at < 4; ++at)   // keys 32..63 see no query of the first half
                        if (s == 1 || at < 2)
                            Y[at] = mma(zt, ld_frag<C::F32>(s_sc + (16 * at + ln) * C::ROWT + 32 * s + 8 * g), Y[at]);
                }
                __syncthreads();   // the value rows and scores are read before the next sub-block rewrites them
            }
            if (a.gmode & ACC_IN) acc_load_t(rAcc, r0_of(it), 16 * w, ln, g, Y);
            if (a.gmode & ACC_OUT) {
                acc_store_t(rAcc, r0_of(it), 16 * w, ln, g, Y);
            } else {
                const float one[4] = {1.f, 1.f, 1.f, 1.f}, zero[4] = {-0.f, -0.f, -0.f, -0.f};   // x + -0 = x
                store_rows_t<C>(rOut1, r0_of(it), 16 * w, ln, g, Y, one, zero, a.rs, a.dh);
            }
        }
        if constexpr (DK && !H2) {
            if (a.gmode & ACC_IN) acc_load_row(rAcc, r0_of(it) + my, g, dX);
            if (a.gmode & ACC_OUT) acc_store_row(rAcc, r0_of(it) + my, g, dX);
            else store_dx<C>(xr, rOut0, r0_of(it) + my, g, inv_a, a.beta, dX, a.rs, a.dh);
        }
    }
}

// ---------------------------------------------------------------------------
// hard-hash diagnostic
// ---------------------------------------------------------------------------
// ids: row r's entry for table l (of the L tables of this group) at
// ids[r * ld + l]. Block (x, y) takes rows 64 x .. 64 x + 63 of sequence y
// (N rows each), so a wave's 16 rows share one head's hyperplanes.
template <class C>
__global__ __launch_bounds__(NT) void k_hash(const void* X, const void* Wv, int64_t N, int L, int ld, int H,
                                             int64_t w_hs, int dh, int32_t* __restrict__ ids,
                                             unsigned long long* near_zero) {
    using elem = typename Prec<C::F32>::elem;
    using frag = typename Prec<C::F32>::frag;
    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    // wave index as a scalar: every branch on it is wave-uniform, so no MFMA is
    // ever issued under a partial or empty EXEC mask
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.y;
    const int64_t n = ((int64_t)blockIdx.x * NW + w) * 16 + ln;
    const bool valid = n < N;
    const int64_t r = bh * N + n;
    const elem* W = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(Wv) + (bh % H) * w_hs);
    // head dimension 128: columns 64..127 as a second pair of K chunks
    frag xf[4];
    load_row_raw<C::F32>(X, valid ? (size_t)r : 0, valid, g, xf, dh);
    if (dh > 64) {
        load_row_raw<C::F32>(reinterpret_cast<const typename In<C::F32>::T*>(X) + 64, valid ? (size_t)r : 0,
                             valid, g, xf + 2, dh);
    }
    const float ss = row_sumsq<C::F32>(xf) + (dh > 64 ? row_sumsq<C::F32>(xf + 2) : 0.f);
    const float inv = __builtin_amdgcn_rsqf(fmaxf(sum_groups(ss), NORM_EPS * NORM_EPS));
    unsigned int nz = 0;
#pragma unroll
    for (int t = 0; t < C::MT; ++t) {
        f32x4 acc = project_global<C>(W, L, t, ln, g, xf, dh);
        if (dh > 64) {
            const f32x4 a2 = project_global<C>(W + 64, L, t, ln, g, xf + 2, dh);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += a2[i];
        }
        if constexpr (C::Pp == 8) {
            // a table's planes 0-3 in the even lane group, 4-7 in the odd one
            const int table = t * C::TPT + (g >> 1);
            int bits = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int plane = 4 * (g & 1) + i;
                if (plane >= C::P) continue;
                const float h = acc[i];
                if (h > 0.f) bits |= 1 << plane;
                if (valid && table < L && fabsf(h * inv) < NEAR_ZERO) ++nz;
            }
            const int id = bits | __shfl_xor(bits, 16);
            if (valid && table < L && (g & 1) == 0) ids[(size_t)r * ld + table] = id;
            continue;
        }
#pragma unroll
        for (int tl = 0; tl < C::TPL; ++tl) {
            const int table = t * C::TPT + g * C::TPL + tl;
            int id = 0;
#pragma unroll
            for (int p = 0; p < C::P; ++p) {
                const float h = acc[tl * C::Pp + p];
                if (h > 0.f) id |= 1 << p;
                if (valid && table < L && fabsf(h * inv) < NEAR_ZERO) ++nz;
            }
            if (valid && table < L) ids[(size_t)r * ld + table] = id;
        }
    }
    // wave-level sum of the near-zero count, one atomic per wave
    unsigned int tot = nz;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
    if (lane == 0 && tot) atomicAdd(near_zero, (unsigned long long)tot);
}

}  // namespace race
