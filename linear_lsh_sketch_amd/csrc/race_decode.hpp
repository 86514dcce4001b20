// Causal decode against a running sketch (gfx950).
//
// T new tokens per (batch, head), in order: each token's key and value join
// the sketch, then its query reads the sketch out (causal sums include the
// diagonal). The
// sketch replaces the key-value cache: L * 2^P * (d + 1) floats per head,
// whatever the length of the sequence so far (efficient key-value caching
// at inference: Japanese gist.science page, section 6; Korean page,
// section 5). temperature = +inf selects the hard buckets of the original
// discrete hash (Japanese gist.science page, section 2.2): t_p = sign(h_p),
// so each table's monomials are those of a one-hot corner; a query that
// collides with no key then reads a zero denominator (exactly: the masses
// and the denominator are float64) and outputs zeros.
//
// The state has the layout of the kernels' sketch states: F x 64 value sums
// (row f = canonical feature f) then F masses, F = 32 * MT * KB. Padded
// tables (index >= L) keep the convention of the sketch kernels: their empty
// subset is 1 for every key (so their state rows stay the plain sums of
// [v | 1]) and every other feature is 0; the read-out leaves them out.
//
// Work per head: one read of the state into registers, then per token one
// projection of q and of k on the L * P planes, the features, the update of
// the rows in registers and the read-out from them, and one write of the
// state at the end: 2 * F * (64 VH * 4 + 8) bytes per call (the bound for T = 1).
// No matrix cores: a head's update is an outer product of one feature row
// and one value row, and the read-out a vector-matrix product over F rows.
#pragma once

#include <hip/hip_runtime.h>

#include "race_device.hpp"

namespace race {

constexpr int DEC_NT = 512;      // threads per workgroup (one head)
constexpr int DEC_RG = DEC_NT / 16;   // row groups: 16 lanes cover one 64-float row
constexpr int DEC_MAXF = 512;    // largest F of one table group
static_assert(DEC_MAXF <= DEC_NT, "one thread per feature and mass");

// The running state of a head holds its table groups one after the other,
// each as [VH halves of F_g x 64 float32 value sums | F_g float64 masses]
// (RW = 64 VH + 2 floats per feature; rows in the feature order of the sketch
// kernels' states): the masses count keys exactly beyond 2^24. VH = 2 at head
// dimension 128 (value columns 0..63, then 64..127), else 1. Full groups have
// F features and Lg tables, the last Fl and L - (G - 1) Lg.
//
// Head dimension 128: the planes project the whole 128-column q and k rows,
// and each launch updates and reads out one value half; the second half runs
// first and leaves the masses as they were (it counts the new keys in its
// registers), then the first half updates them too and stores them.
struct DecodeArgs {
    const void *q, *k, *v, *W;
    float* state;   // [BH][((G - 1) F + Fl) RW]
    void* o;        // [BH][T][dh]
    int T;          // new tokens per head (rows of a head in q, k, v, o), processed in order
    int tok;        // k_decode_one: the token of this launch (0 <= tok < T)
    int P, L, F, KB, TPT, TPL;
    int G, Lg, Fl;
    float beta;
    int hard;
    int H;          // heads: W of head bh at W + (bh % H) * w_hs bytes (0: one W for all)
    int64_t w_hs;
    int dh;         // head dimension (row length of q, k, v, o and W): 32, 64 or 128
    int VH;         // value halves of the state (2 at head dimension 128, else 1)
    int half;       // the value half of this launch
    int store_mass; // store the updated masses (0: the second half, before the first)
};

// Table and subset of canonical feature f (lane group g of 32-feature chunk
// kc holds features 8 g .. 8 g + 7 of the tables of its projection rows).
// P = 5, 6: a table spans two lane groups, the even one holding the subsets
// without the top plane, the odd one those with it.
__device__ inline void feature_table_subset(int f, int P, int KB, int TPT, int TPL, int& table, int& subset) {
    const int kc = f >> 5, g = (f >> 3) & 3, j = f & 7;
    const int jj = j + 8 * (kc % KB);
    const int R = 1 << P;
    if (P >= 5) {
        table = (kc / KB) * TPT + (g >> 1);
        subset = jj + (g & 1) * (R >> 1);
        return;
    }
    table = (kc / KB) * TPT + g * TPL + jj / R;
    subset = jj % R;
}

// Lanes per projection row: a group's 2 L P rows (the query's and the key's
// planes; L P <= 128 per group) spread over the workgroup, two consecutive
// lanes per row (each over 32 columns), combined by a shuffle. (Four lanes
// per row measured slower at every head count, one lane per row slower for
// few heads.)
__device__ inline int dec_parts(int) { return 2; }

// The parts' partial projections and squared norms summed over the row's
// lanes (every lane of the workgroup takes part), then the plane value
// t = tanh(beta tanh(h / |x|)), or the sign of h with hard buckets, with the
// sketch kernels' hardware tanh and reciprocal square root.
__device__ inline float dec_plane_t(float h, float ss, int parts, float beta, int hard) {
    for (int m = 1; m < parts; m <<= 1) {
        h += __shfl_xor(h, m);
        ss += __shfl_xor(ss, m);
    }
    h *= __builtin_amdgcn_rsqf(fmaxf(ss, NORM_EPS * NORM_EPS));
    if (hard) return h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
    return tanh_scaled(tanh_scaled(h, 2.f * LOG2E), 2.f * LOG2E * beta);
}

// This thread's read-out partial (columns 4 cq .. +3 over its rows) summed
// over the four row groups of its wave (lanes 16 apart), into s_num[wave].
__device__ inline void dec_reduce_num(f32x4 acc, float (*s_num)[DH + 4], int wv, int lane, int cq) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] += __shfl_xor(acc[j], 16);
        acc[j] += __shfl_xor(acc[j], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) s_num[wv][4 * cq + j] = acc[j];
    }
}

// More than one table group: one token per launch (token a.tok of each
// head), every table group in turn: the group's state rows are updated and
// written back as soon as the features are known, and the read-outs of the
// groups are summed. NR = F / 32 state rows per thread of a full group (a
// compile-time count).
// XW: projection width (64, or 128 at head dimension 128).
template <bool F32, int NR, int XW>
__global__ __launch_bounds__(DEC_NT) void k_decode_one(DecodeArgs a) {
    using elem = typename Prec<F32>::elem;
    __shared__ float s_x[2][XW];             // q, k of this head
    __shared__ float s_v[DH];                // this launch's value half
    __shared__ float s_t[2][128];            // t_p of each table plane, [q | k][l * P + p]
    __shared__ float s_phi[2][DEC_MAXF];     // features of q and of k
    __shared__ float s_num[DEC_NT / 64][DH + 4];  // partial read-outs per wave
    __shared__ double s_den[DEC_NT / 64];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int64_t r = bh * a.T + a.tok;      // row of this token in q, k, v, o
    const int RW = DH * a.VH + 2;
    const int64_t head_floats = ((int64_t)(a.G - 1) * a.F + a.Fl) * RW;
    float* st_head = a.state + (size_t)bh * (size_t)head_floats;
    const int cq = tid & 15, rg = tid >> 4;
    const int vcols = a.dh < DH ? a.dh : DH, vc0 = DH * a.half;   // this half's value columns
    constexpr int WV = 16 / sizeof(elem);   // elements per 16-byte load
    typedef elem wvec __attribute__((ext_vector_type(WV)));

    if (tid < 2 * XW) {
        const int which = tid / XW, c = tid % XW;
        const void* src = which == 0 ? a.q : a.k;
        s_x[which][c] = c < a.dh ? (float)reinterpret_cast<const elem*>(src)[r * a.dh + c] : 0.f;
    }
    if (tid < DH) s_v[tid] = tid < vcols ? (float)reinterpret_cast<const elem*>(a.v)[r * a.dh + vc0 + tid] : 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};   // read-out of columns 4 cq .. +3 over this thread's rows
    double den = 0.0;                   // and over its masses

    for (int gi = 0; gi < a.G; ++gi) {
        const bool lastg = gi == a.G - 1;
        const int F = lastg ? a.Fl : a.F;
        const int Lgr = lastg ? a.L - (a.G - 1) * a.Lg : a.Lg;
        const int LP = Lgr * a.P;
        float* stg = st_head + (size_t)gi * (size_t)a.F * RW;
        float* st = stg + (size_t)a.half * F * DH;   // this half's value sums
        double* zs = reinterpret_cast<double*>(stg + (size_t)a.VH * F * DH);
        // The state rows do not depend on this token: their loads are issued
        // first, so their latency overlaps the projections and features.
        f32x4 s[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i)
            if (rg + DEC_RG * i < F) s[i] = *reinterpret_cast<const f32x4*>(st + (size_t)(rg + DEC_RG * i) * DH + 4 * cq);
        const double z_old = tid < F ? zs[tid] : 0.0;
        // so are the hyperplane rows: projection row pr = side * L P + l * P + p
        // of the group takes `parts` lanes, part pi holding columns
        // pi * ncol .. + ncol - 1 of its weights, loaded 16 bytes at a time
        const int parts = dec_parts(LP), ncol = XW / parts;
        const int pr = tid / parts, pi = tid % parts, side = pr / LP, row = pr % LP, c0 = pi * ncol;
        wvec wr[XW / WV / 2];
        if (pr < 2 * LP) {
            const wvec* w = reinterpret_cast<const wvec*>(
                reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.W) + (bh % a.H) * a.w_hs) +
                ((size_t)gi * a.Lg * a.P + row) * a.dh + c0);
#pragma unroll
            for (int j = 0; j < XW / WV / 2; ++j) {
                if (j * WV < ncol && c0 + j * WV < a.dh) {
                    wr[j] = w[j];
                } else {
#pragma unroll
                    for (int e = 0; e < WV; ++e) wr[j][e] = (elem)0.f;
                }
            }
        }
        __syncthreads();   // s_x is written; the previous group's s_t and s_phi are read

        // projections; each part also sums its columns' squares (the same
        // order in both decode kernels)
        {
            float h = 0.f, ss = 0.f;
            if (pr < 2 * LP) {
#pragma unroll
                for (int j = 0; j < XW / WV / 2; ++j) {
                    if (j * WV >= ncol) break;
#pragma unroll
                    for (int e = 0; e < WV; ++e) {
                        const float x = s_x[side][c0 + WV * j + e];
                        h = fmaf((float)wr[j][e], x, h);
                        ss = fmaf(x, x, ss);
                    }
                }
            }
            const float t = dec_plane_t(h, ss, parts, a.beta, a.hard);
            if (pr < 2 * LP && pi == 0) s_t[side][row] = t;
        }
        __syncthreads();

        if (tid < F) {
            const int f = tid;
            int table, subset;
            feature_table_subset(f, a.P, a.KB, a.TPT, a.TPL, table, subset);
            float pq = 0.f, pk = subset == 0 ? 1.f : 0.f;   // padded table
            if (table < Lgr) {
                pq = 1.f;
                pk = 1.f;
                for (int p = 0; p < a.P; ++p)
                    if ((subset >> p) & 1) {
                        pq *= s_t[0][table * a.P + p];
                        pk *= s_t[1][table * a.P + p];
                    }
            }
            s_phi[0][f] = pq;
            s_phi[1][f] = pk;
        }
        __syncthreads();

        // value sums: lane quad cq owns columns 4 cq .. 4 cq + 3 of rows rg, rg + 32, ...
        {
            const f32x4 vq = {s_v[4 * cq], s_v[4 * cq + 1], s_v[4 * cq + 2], s_v[4 * cq + 3]};
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int f = rg + DEC_RG * i;
                if (f >= F) continue;
                const float pk = s_phi[1][f], pq = s_phi[0][f];
                s[i] += pk * vq;
                if (pk != 0.f) *reinterpret_cast<f32x4*>(st + (size_t)f * DH + 4 * cq) = s[i];
                acc += pq * s[i];
            }
        }
        // masses (F <= DEC_NT: one per thread), and the denominator, in
        // float64: with hard buckets the features are 0 or +-1 and the masses
        // integers, so the sum is exact and a query that collides with no key
        // reads exactly 0.
        if (tid < F) {
            const float pk = s_phi[1][tid];
            const double z = z_old + (double)pk;
            if (pk != 0.f && a.store_mass) zs[tid] = z;
            den += (double)s_phi[0][tid] * z;
        }
    }
    dec_reduce_num(acc, s_num, wv, lane, cq);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m);
    if (lane == 0) s_den[wv] = den;
    __syncthreads();
    if (tid < DH) {
        float num = 0.f;
        double dsum = 0.0;
#pragma unroll
        for (int rr = 0; rr < DEC_NT / 64; ++rr) num += s_num[rr][tid];
#pragma unroll
        for (int w = 0; w < DEC_NT / 64; ++w) dsum += s_den[w];
        const float o = (a.hard && dsum == 0.0) ? 0.f : num / (float)dsum;
        if (tid < vcols) reinterpret_cast<elem*>(a.o)[r * a.dh + vc0 + tid] = (elem)o;
    }
}

// One table group, any T: the state rows stay in registers across the
// tokens and are written back during the last token; the hyperplanes sit in
// LDS and each token's q, k, v rows are loaded while the previous token is
// processed (100 registers at F = 256 in bf16: two workgroups per CU; the
// one-launch-per-token kernel above needs 184 with its group loop, one
// workgroup per CU, and took 745 us against 407 us for 16,384 heads).
template <bool F32, int NR, int XW>
__global__ __launch_bounds__(DEC_NT) void k_decode_multi(DecodeArgs a) {
    using elem = typename Prec<F32>::elem;
    __shared__ float s_x[2][XW];             // q, k of the current token
    __shared__ float s_v[DH];                // its value half
    __shared__ float s_t[2][128];            // t_p of each table plane, [q | k][l * P + p]
    __shared__ float s_phi[2][DEC_MAXF];     // features of q and of k
    __shared__ float s_num[DEC_NT / 64][DH + 4];  // partial read-outs per wave
    __shared__ double s_den[DEC_NT / 64];
    __shared__ float s_w[128][XW + 1];       // hyperplane rows (padded: conflict-free row reads)

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int F = a.F, LP = a.L * a.P;
    float* sth = a.state + (size_t)bh * (size_t)F * (DH * a.VH + 2);
    float* st = sth + (size_t)a.half * F * DH;   // this half's value sums
    double* zs = reinterpret_cast<double*>(sth + (size_t)a.VH * F * DH);

    // The state rows do not depend on the new tokens: their loads are issued
    // first, so their latency overlaps the first token's projections. They
    // stay in registers for all T tokens and are written back once.
    const int cq = tid & 15, rg = tid >> 4;
    f32x4 s[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
        s[i] = *reinterpret_cast<const f32x4*>(st + (size_t)(rg + DEC_RG * i) * DH + 4 * cq);
    double z = tid < F ? zs[tid] : 0.0;
    // the hyperplanes, once, into LDS (read there for every token), 16 bytes
    // per load
    const elem* Wh = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.W) + (bh % a.H) * a.w_hs);
    {
        constexpr int WV = 16 / sizeof(elem);
        typedef elem wvec __attribute__((ext_vector_type(WV)));
        for (int e = tid; e < LP * (XW / WV); e += DEC_NT) {
            const int wrow = e / (XW / WV), c = (e % (XW / WV)) * WV;
            wvec v;
            if (c < a.dh) {
                v = *reinterpret_cast<const wvec*>(Wh + (size_t)wrow * a.dh + c);
            } else {
#pragma unroll
                for (int j = 0; j < WV; ++j) v[j] = (elem)0.f;
            }
#pragma unroll
            for (int j = 0; j < WV; ++j) s_w[wrow][c + j] = (float)v[j];
        }
    }
    const int parts = dec_parts(LP), ncol = XW / parts;
    const int pr = tid / parts, pi = tid % parts, side = pr / LP, row = pr % LP, c0 = pi * ncol;
    // q, k, v rows are loaded one token ahead: thread tid < 2 XW + 64 holds
    // one element (of q, of k, or of the value half) of the next token while
    // the current one is processed
    const int vcols = a.dh < DH ? a.dh : DH;
    const bool isv = tid >= 2 * XW;
    const int which = isv ? 2 : tid / XW, col = isv ? tid - 2 * XW : tid % XW;
    const elem* src = reinterpret_cast<const elem*>(which == 0 ? a.q : which == 1 ? a.k : a.v) +
                      (isv ? DH * a.half : 0);
    float* dst = isv ? &s_v[col < DH ? col : 0] : &s_x[which][col];
    const bool loads = tid < 2 * XW + DH;
    const int64_t r0 = bh * a.T;   // first row of this head's q, k, v, o
    float nx = 0.f;
    const bool in_col = col < (isv ? vcols : a.dh);
    if (loads) {
        *dst = in_col ? (float)src[r0 * a.dh + col] : 0.f;
        if (a.T > 1 && in_col) nx = (float)src[(r0 + 1) * a.dh + col];
    }
    __syncthreads();

    // Four barriers per token: projections | features | update and read-out
    // | output and the next token's rows (nothing reads s_x in that phase).
    for (int tok = 0; tok < a.T; ++tok) {
        const int64_t r = r0 + tok;
        // projections, each part with its columns' squares (as in k_decode_one)
        {
            float h = 0.f, ss = 0.f;
            if (pr < 2 * LP) {
#pragma unroll 8
                for (int c = c0; c < c0 + ncol; ++c) {
                    const float x = s_x[side][c];
                    h = fmaf(s_w[row][c], x, h);
                    ss = fmaf(x, x, ss);
                }
            }
            const float t = dec_plane_t(h, ss, parts, a.beta, a.hard);
            if (pr < 2 * LP && pi == 0) s_t[side][row] = t;
        }
        __syncthreads();

        if (tid < F) {
            const int f = tid;
            int table, subset;
            feature_table_subset(f, a.P, a.KB, a.TPT, a.TPL, table, subset);
            float pq = 0.f, pk = subset == 0 ? 1.f : 0.f;   // padded table
            if (table < a.L) {
                pq = 1.f;
                pk = 1.f;
                for (int p = 0; p < a.P; ++p)
                    if ((subset >> p) & 1) {
                        pq *= s_t[0][table * a.P + p];
                        pk *= s_t[1][table * a.P + p];
                    }
            }
            s_phi[0][f] = pq;
            s_phi[1][f] = pk;
        }
        __syncthreads();

        // value sums: lane quad cq owns columns 4 cq .. 4 cq + 3 of rows rg, rg + 32, ...
        // After the last token each row is written back as soon as it is
        // final, so the stores overlap the read-out's reduction.
        const bool last = tok == a.T - 1;
        {
            const f32x4 vq = {s_v[4 * cq], s_v[4 * cq + 1], s_v[4 * cq + 2], s_v[4 * cq + 3]};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int f = rg + DEC_RG * i;
                s[i] += s_phi[1][f] * vq;
                if (last) *reinterpret_cast<f32x4*>(st + (size_t)f * DH + 4 * cq) = s[i];
                acc += s_phi[0][f] * s[i];
            }
            dec_reduce_num(acc, s_num, wv, lane, cq);
        }
        // masses (F <= DEC_NT: one per thread) and the denominator in float64:
        // with hard buckets the features are 0 or +-1 and the masses integers,
        // so the sum is exact and a query that collides with no key reads
        // exactly 0.
        {
            double den = 0.0;
            if (tid < F) {
                z += (double)s_phi[1][tid];
                if (last && a.store_mass) zs[tid] = z;
                den = (double)s_phi[0][tid] * z;
            }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m);
            if (lane == 0) s_den[wv] = den;
        }
        __syncthreads();
        if (tid < DH) {
            float num = 0.f;
            double den = 0.0;
#pragma unroll
            for (int rr = 0; rr < DEC_NT / 64; ++rr) num += s_num[rr][tid];
#pragma unroll
            for (int w = 0; w < DEC_NT / 64; ++w) den += s_den[w];
            const float o = (a.hard && den == 0.0) ? 0.f : num / (float)den;
            if (tid < vcols) reinterpret_cast<elem*>(a.o)[r * a.dh + DH * a.half + tid] = (elem)o;
        }
        if (loads && tok + 1 < a.T) {
            *dst = nx;
            if (tok + 2 < a.T && in_col) nx = (float)src[(r + 2) * a.dh + col];
        }
        __syncthreads();
    }

}

}  // namespace race
