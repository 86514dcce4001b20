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
// collides with no key then reads a zero denominator (exactly, for fewer
// than 2^24 keys in the state) and outputs zeros.
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
// state at the end: 2 * F * 65 * 4 bytes per call (the bound for T = 1).
// No matrix cores: a head's update is an outer product of one feature row
// and one value row, and the read-out a vector-matrix product over F rows.
#pragma once

#include <hip/hip_runtime.h>

#include "race_device.hpp"

namespace race {

constexpr int DEC_NT = 512;      // threads per workgroup (one head)
constexpr int DEC_RG = DEC_NT / 16;   // row groups: 16 lanes cover one 64-float row
constexpr int DEC_MAXF = 512;    // largest F (MT = 8, KB = 2)
static_assert(DEC_MAXF <= DEC_NT, "one thread per feature and mass");

struct DecodeArgs {
    const void *q, *k, *v, *W;
    float* state;   // [BH][F * 65]
    void* o;        // [BH][T][64]
    int T;          // new tokens per head, processed in order
    int P, L, F, KB, TPT, TPL;
    float beta;
    int hard;
};

// Table and subset of canonical feature f (lane group g of 32-feature chunk
// kc holds features 8 g .. 8 g + 7 of the tables of its projection rows).
__device__ inline void feature_table_subset(int f, int P, int KB, int TPT, int TPL, int& table, int& subset) {
    const int kc = f >> 5, g = (f >> 3) & 3, j = f & 7;
    const int jj = j + 8 * (kc % KB);
    const int R = 1 << P;
    table = (kc / KB) * TPT + g * TPL + jj / R;
    subset = jj % R;
}

// T = 1: the state rows are updated and written back as soon as the
// features are known. NR = F / 32 state rows per thread (a compile-time
// count, so the registers match the state: 95 at F = 256 in bf16).
template <bool F32, int NR>
__global__ __launch_bounds__(DEC_NT) void k_decode_one(DecodeArgs a) {
    using elem = typename Prec<F32>::elem;
    __shared__ float s_x[3][DH];             // q, k, v of this head
    __shared__ float s_t[2][128];            // t_p of each table plane, [q | k][l * P + p]
    __shared__ float s_phi[2][DEC_MAXF];     // features of q and of k
    __shared__ float s_num[DEC_RG][DH + 4];  // partial read-outs per row group
    __shared__ double s_den[DEC_NT / 64];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int F = a.F, LP = a.L * a.P;
    float* st = a.state + (size_t)bh * (size_t)F * 65;

    // The state rows do not depend on this token: their loads are issued
    // first, so their latency overlaps the projections and features.
    const int cq = tid & 15, rg = tid >> 4;
    f32x4 s[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
        s[i] = *reinterpret_cast<const f32x4*>(st + (size_t)(rg + DEC_RG * i) * DH + 4 * cq);
    const float z_old = tid < F ? st[(size_t)F * DH + tid] : 0.f;
    // so are the hyperplane rows: thread (side, row), row = l * P + p, holds
    // all 64 weights of its row, loaded 16 bytes at a time
    const int side = tid / LP, row = tid % LP;
    constexpr int WV = 16 / sizeof(elem);   // elements per 16-byte load
    typedef elem wvec __attribute__((ext_vector_type(WV)));
    wvec wr[DH / WV];
    if (tid < 2 * LP) {
        const wvec* w = reinterpret_cast<const wvec*>(reinterpret_cast<const elem*>(a.W) + (size_t)row * DH);
#pragma unroll
        for (int j = 0; j < DH / WV; ++j) wr[j] = w[j];
    }

    if (tid < 3 * DH) {
        const int which = tid / DH, c = tid % DH;
        const void* src = which == 0 ? a.q : which == 1 ? a.k : a.v;
        s_x[which][c] = (float)reinterpret_cast<const elem*>(src)[bh * DH + c];
    }
    __syncthreads();

    // projections; each projection thread also sums its row's squares (the
    // same order in both decode kernels, so they agree bit for bit)
    if (tid < 2 * LP) {
        float h = 0.f, ss = 0.f;
#pragma unroll
        for (int j = 0; j < DH / WV; ++j)
#pragma unroll
            for (int e = 0; e < WV; ++e) {
                const float x = s_x[side][WV * j + e];
                h = fmaf((float)wr[j][e], x, h);
                ss = fmaf(x, x, ss);
            }
        h *= 1.f / fmaxf(sqrtf(ss), NORM_EPS);
        float t;
        if (a.hard) t = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
        else t = tanhf(a.beta * tanhf(h));
        s_t[side][row] = t;
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
    {
        const f32x4 vq = {s_x[2][4 * cq], s_x[2][4 * cq + 1], s_x[2][4 * cq + 2], s_x[2][4 * cq + 3]};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int f = rg + DEC_RG * i;
            const float pk = s_phi[1][f], pq = s_phi[0][f];
            s[i] += pk * vq;
            if (pk != 0.f) *reinterpret_cast<f32x4*>(st + (size_t)f * DH + 4 * cq) = s[i];
            acc += pq * s[i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s_num[rg][4 * cq + j] = acc[j];
    }
    // masses (F <= DEC_NT: one per thread). The denominator is summed in
    // float64: with hard buckets the features are 0 or +-1 and the masses
    // integers (exact in float32 below 2^24 keys), so the sum is exact and a
    // query that collides with no key reads exactly 0.
    {
        double den = 0.0;
        if (tid < F) {
            const float pk = s_phi[1][tid];
            const float z = z_old + pk;
            if (pk != 0.f) st[(size_t)F * DH + tid] = z;
            den = (double)s_phi[0][tid] * (double)z;
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m);
        if (lane == 0) s_den[wv] = den;
    }
    __syncthreads();
    if (tid < DH) {
        float num = 0.f;
        double den = 0.0;
#pragma unroll 8
        for (int r = 0; r < DEC_RG; ++r) num += s_num[r][tid];
#pragma unroll
        for (int w = 0; w < DEC_NT / 64; ++w) den += s_den[w];
        const float o = (a.hard && den == 0.0) ? 0.f : num / (float)den;
        reinterpret_cast<elem*>(a.o)[bh * DH + tid] = (elem)o;
    }
}

// T > 1: the state rows stay in registers across the tokens and are written
// back during the last token; the hyperplanes sit in LDS and each token's
// q, k, v rows are loaded while the previous token is processed (116
// registers at F = 256 in bf16: two workgroups per CU).
template <bool F32, int NR>
__global__ __launch_bounds__(DEC_NT) void k_decode_multi(DecodeArgs a) {
    using elem = typename Prec<F32>::elem;
    __shared__ float s_x[3][DH];             // q, k, v of the current token
    __shared__ float s_t[2][128];            // t_p of each table plane, [q | k][l * P + p]
    __shared__ float s_phi[2][DEC_MAXF];     // features of q and of k
    __shared__ float s_num[DEC_RG][DH + 4];  // partial read-outs per row group
    __shared__ double s_den[DEC_NT / 64];
    __shared__ float s_w[128][DH + 1];       // hyperplane rows (padded: conflict-free row reads)

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int F = a.F, LP = a.L * a.P;
    float* st = a.state + (size_t)bh * (size_t)F * 65;

    // The state rows do not depend on the new tokens: their loads are issued
    // first, so their latency overlaps the first token's projections. They
    // stay in registers for all T tokens and are written back once.
    const int cq = tid & 15, rg = tid >> 4;
    f32x4 s[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
        s[i] = *reinterpret_cast<const f32x4*>(st + (size_t)(rg + DEC_RG * i) * DH + 4 * cq);
    float z = tid < F ? st[(size_t)F * DH + tid] : 0.f;
    // the hyperplanes, once, into LDS (read there for every token)
    for (int e = tid; e < LP * DH; e += DEC_NT) s_w[e / DH][e % DH] = (float)reinterpret_cast<const elem*>(a.W)[e];
    const int side = tid / LP, row = tid % LP;
    // q, k, v rows are loaded one token ahead: thread tid < 3 * 64 holds one
    // element of the next token while the current one is processed
    const int which = tid / DH, col = tid % DH;
    const elem* src = reinterpret_cast<const elem*>(which == 0 ? a.q : which == 1 ? a.k : a.v);
    const int64_t r0 = bh * a.T;   // first row of this head's q, k, v, o
    float nx = 0.f;
    if (tid < 3 * DH) {
        s_x[which][col] = (float)src[r0 * DH + col];
        if (a.T > 1) nx = (float)src[(r0 + 1) * DH + col];
    }
    __syncthreads();

    // Four barriers per token: projections | features | update and read-out
    // | output and the next token's rows (nothing reads s_x in that phase).
    for (int tok = 0; tok < a.T; ++tok) {
        const int64_t r = r0 + tok;
        // projections, each thread with its row's norm (as in k_decode_one)
        if (tid < 2 * LP) {
            float h = 0.f, ss = 0.f;
#pragma unroll 16
            for (int c = 0; c < DH; ++c) {
                const float x = s_x[side][c];
                h = fmaf(s_w[row][c], x, h);
                ss = fmaf(x, x, ss);
            }
            h *= 1.f / fmaxf(sqrtf(ss), NORM_EPS);
            float t;
            if (a.hard) t = h > 0.f ? 1.f : (h < 0.f ? -1.f : 0.f);
            else t = tanhf(a.beta * tanhf(h));
            s_t[side][row] = t;
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
            const f32x4 vq = {s_x[2][4 * cq], s_x[2][4 * cq + 1], s_x[2][4 * cq + 2], s_x[2][4 * cq + 3]};
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                const int f = rg + DEC_RG * i;
                s[i] += s_phi[1][f] * vq;
                if (last) *reinterpret_cast<f32x4*>(st + (size_t)f * DH + 4 * cq) = s[i];
                acc += s_phi[0][f] * s[i];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) s_num[rg][4 * cq + j] = acc[j];
        }
        // masses (F <= DEC_NT: one per thread). The denominator is summed in
        // float64: with hard buckets the features are 0 or +-1 and the masses
        // integers (exact in float32 below 2^24 keys), so the sum is exact and
        // a query that collides with no key reads exactly 0.
        {
            double den = 0.0;
            if (tid < F) {
                const float pk = s_phi[1][tid];
                z += pk;
                if (last) st[(size_t)F * DH + tid] = z;
                den = (double)s_phi[0][tid] * (double)z;
            }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m);
            if (lane == 0) s_den[wv] = den;
        }
        __syncthreads();
        if (tid < DH) {
            float num = 0.f;
            double den = 0.0;
#pragma unroll 8
            for (int rr = 0; rr < DEC_RG; ++rr) num += s_num[rr][tid];
#pragma unroll
            for (int w = 0; w < DEC_NT / 64; ++w) den += s_den[w];
            const float o = (a.hard && den == 0.0) ? 0.f : num / (float)den;
            reinterpret_cast<elem*>(a.o)[r * DH + tid] = (elem)o;
        }
        if (tid < 3 * DH && tok + 1 < a.T) {
            s_x[which][col] = nx;
            if (tok + 2 < a.T) nx = (float)src[(r + 2) * DH + col];
        }
        __syncthreads();
    }

}

}  // namespace race
