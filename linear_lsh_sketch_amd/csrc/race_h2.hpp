// Head dimension 128: the forward and backward launch sequences and the three
// kernels only they use.
//
// The soft hash of a token depends on the whole row (its normalised
// projections onto the hyperplanes, "RACE Attention", the soft-hashing
// section), while the sketch passes are linear in the value columns (the
// bucket sums of the aggregation step, and the gradients of the read-out).
// So the plane values of queries and keys are computed once from the 128
// columns (k_planes), and every sketch pass runs twice, once per half of
// 64 value columns, on the same features:
//   - the forward's two halves give the two halves of O (the denominator,
//     the mass column, is the same in both);
//   - the gradient wrt a token's features is the sum of the two halves'
//     (each half reads only its own columns of V, dO and O); the mass terms
//     (e = -<dO, O>/D over all 128 columns, k_erow) enter the first half
//     only. The chain rule through the features is linear in that gradient,
//     so each half leaves its per-plane gradient and the second adds to the
//     first's; then k_backproject maps the sum back through the hyperplanes
//     and the normalisation onto the 128 columns of dQ and dK.
#pragma once

#include "race_dispatch.hpp"

namespace race {

constexpr int D128 = 128;

// 1 / max(|x|, eps) of a 128-column row held as four K chunks (lane group g:
// columns 32 s + 8 g .. +7), the same sums as row_inv_norm.
template <bool F32>
__device__ inline float inv_norm128(const typename Prec<F32>::frag x[4]) {
    const float ss = sum_groups(row_sumsq<F32>(x) + row_sumsq<F32>(x + 2));
    return __builtin_amdgcn_rsqf(fmaxf(ss, NORM_EPS * NORM_EPS));
}

// ---------------------------------------------------------------------------
// plane values of one side
// ---------------------------------------------------------------------------
struct PlanesArgs {
    const void* X;     // [BH][N][128] queries or keys
    const void* W;     // [L, P, 128], or [H, L, P, 128] (w_hs bytes between heads)
    char* u;           // group 0's plane values [rows][NPL]; group g at u + g * ustep bytes
    size_t ustep;
    float* inv;        // [rows] 1 / max(|x|, eps)
    int64_t N;
    int L, P, Pp, G, Lg, MT, MTl;
    int H;
    int64_t w_hs;
};

// Block (x, y): tokens 64 x .. 64 x + 63 of sequence y, wave w the 16 from
// 64 x + 16 w; lane (ln, g) projects token ln of its wave onto rows
// 4 g .. 4 g + 3 of each 16-row projection tile (row r of a group's tiles is
// plane r % P' of the group's table r / P'; rows of padded planes or tables
// have no hyperplane and give u = 0), with the matrix cores: H^T = W' X^T.
template <bool F32>
__global__ __launch_bounds__(NT) void k_planes(PlanesArgs a) {
    using elem = typename Prec<F32>::elem;
    using frag = typename Prec<F32>::frag;
    using ucache = typename Prec<F32>::ucache;
    using uvec = typename Prec<F32>::uvec;
    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.y;
    const int64_t n = ((int64_t)blockIdx.x * NW + w) * 16 + ln;
    const bool valid = n < a.N;
    const size_t r = (size_t)bh * a.N + (valid ? n : 0);
    const elem* xrow = reinterpret_cast<const elem*>(a.X) + r * D128 + 8 * g;
    frag xf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xf[s] = valid ? ld_frag<F32>(xrow + 32 * s) : zero_frag<F32>();
    const float inv = inv_norm128<F32>(xf);
    if (valid && g == 0) a.inv[r] = inv;
    const elem* W = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.W) + (bh % a.H) * a.w_hs);
    for (int gi = 0; gi < a.G; ++gi) {
        const bool last = gi == a.G - 1;
        const int Lgi = last ? a.L - (a.G - 1) * a.Lg : a.Lg;
        const int MT = last ? a.MTl : a.MT;
        const int NPL = 16 * MT;
        ucache* u = reinterpret_cast<ucache*>(a.u + (size_t)gi * a.ustep);
        for (int t = 0; t < MT; ++t) {
            const int rr = 16 * t + ln;
            const int table = rr / a.Pp, plane = rr % a.Pp;
            const bool ok = table < Lgi && plane < a.P;
            const elem* wr = W + ((size_t)(gi * a.Lg + (ok ? table : 0)) * a.P + (ok ? plane : 0)) * D128 + 8 * g;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mma(ok ? ld_frag<F32>(wr + 32 * s) : zero_frag<F32>(), xf[s], acc);
            float hs[4], uu[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) hs[i] = acc[i];
            tanh4(hs, inv, uu);
            const uvec uq = round_u<F32>(uu);
            if (valid) *reinterpret_cast<uvec*>(u + r * NPL + 16 * t + 4 * g) = uq;
        }
    }
}

// ---------------------------------------------------------------------------
// e = -<dO, O> / D per token over the 128 columns
// ---------------------------------------------------------------------------
// 16 lanes per token, 8 columns each; 16 tokens per workgroup.
template <bool F32>
__global__ __launch_bounds__(256) void k_erow(const void* dO, const void* O, const float* __restrict__ D,
                                              float* __restrict__ E, int64_t rows) {
    using elem = typename Prec<F32>::elem;
    using frag = typename Prec<F32>::frag;
    const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    float acc = 0.f;
    if (r < rows) {
        const frag a = ld_frag<F32>(reinterpret_cast<const elem*>(dO) + (size_t)r * D128 + 8 * q);
        const frag b = ld_frag<F32>(reinterpret_cast<const elem*>(O) + (size_t)r * D128 + 8 * q);
        if constexpr (F32) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += a[j] * b[j];
        } else {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x2 pa = {a[2 * j], a[2 * j + 1]}, pb = {b[2 * j], b[2 * j + 1]};
                acc = __builtin_amdgcn_fdot2_f32_bf16(pa, pb, acc, false);
            }
        }
    }
    acc = sum_row16(acc);
    if (r < rows && q == 0) E[r] = -acc * rcp_(D[r]);
}

// ---------------------------------------------------------------------------
// back-projection and the normalisation's chain rule
// ---------------------------------------------------------------------------
struct BackArgs {
    const void* X;        // [BH][N][128] queries or keys
    const float* inv;     // their 1 / max(|x|, eps)
    const char* dh;       // group 0's per-plane gradients [rows][NPL] float32; group g at dh + g * dstep bytes
    size_t dstep;
    const void* WTp;      // back-projection operands of group 0 (k_prep, 8 column tiles); group g
    size_t wt_gs;         // at WTp + g * wt_gs bytes, head h of W at + h * wt_hs bytes
    int64_t wt_hs;
    int H;
    void* out;            // dQ or dK [BH][N][128]
    int64_t N;
    int G, MT, MTl;
    float beta;
};

// dx_hat = sum over the groups' projection rows of dh_r w_r (the matrix
// cores, 32 rows (two tiles) per step, eight 16-column output tiles), then
// dx = (dx_hat - x_hat <x_hat, dx_hat>) beta / max(|x|, eps) (below eps the
// normalisation is a plain scaling and the radial term is kept). Token
// layout as k_planes: lane (ln, g) holds columns 16 dt + 4 g .. +3 of token ln
// of its wave.
template <bool F32>
__global__ __launch_bounds__(NT) void k_backproject(BackArgs a) {
    using elem = typename Prec<F32>::elem;
    using frag = typename Prec<F32>::frag;
    const int lane = threadIdx.x & 63, ln = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.y;
    const int64_t n = ((int64_t)blockIdx.x * NW + w) * 16 + ln;
    const bool valid = n < a.N;
    const size_t r = (size_t)bh * a.N + (valid ? n : 0);
    f32x4 dX[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dX[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    for (int gi = 0; gi < a.G; ++gi) {
        const int MT = gi == a.G - 1 ? a.MTl : a.MT;
        const int NPL = 16 * MT;
        const float* dhr = reinterpret_cast<const float*>(a.dh + (size_t)gi * a.dstep) + r * NPL;
        const elem* WTp = reinterpret_cast<const elem*>(reinterpret_cast<const char*>(a.WTp) + gi * a.wt_gs +
                                                        (bh % a.H) * a.wt_hs);
        for (int m = 0; m < (MT + 1) / 2; ++m) {
            const f32x4 lo = valid ? *reinterpret_cast<const f32x4*>(dhr + 32 * m + 4 * g) : zero4;
            const f32x4 hi =
                (valid && 2 * m + 1 < MT) ? *reinterpret_cast<const f32x4*>(dhr + 32 * m + 16 + 4 * g) : zero4;
            const frag df = pack<F32>(lo, hi);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                dX[dt] = mma(ld_frag<F32>(WTp + ((size_t)(m * 8 + dt) * 64 + lane) * 8), df, dX[dt]);
        }
    }
    const float inv = valid ? a.inv[r] : 1.f;
    const elem* xrow = reinterpret_cast<const elem*>(a.X) + r * D128;
    float xv[8][4];
    float radial = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        typename Prec<F32>::half h;
        if (valid) {
            h = *reinterpret_cast<const typename Prec<F32>::half*>(xrow + 16 * dt + 4 * g);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = to_elem<F32>(0.f);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[dt][i] = (float)h[i];
            radial += xv[dt][i] * inv * dX[dt][i];
        }
    }
    radial = sum_groups(radial);
    const bool tangent = inv < rcp_(NORM_EPS);
    const float binv = a.beta * inv;   // the per-plane gradients carry dt/dh without beta
    if (!valid) return;
    elem* orow = reinterpret_cast<elem*>(a.out) + r * D128;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        typename Prec<F32>::half o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = to_elem<F32>((tangent ? dX[dt][i] - xv[dt][i] * inv * radial : dX[dt][i]) * binv);
        *reinterpret_cast<typename Prec<F32>::half*>(orow + 16 * dt + 4 * g) = o;
    }
}

// ---------------------------------------------------------------------------
// launch sequences
// ---------------------------------------------------------------------------
template <bool F32>
race_status_t run_planes(const Shape& s, const Derived& d, const void* X, const void* W, char* base,
                         const CacheLayout& cl, hipStream_t st) {
    PlanesArgs a;
    a.X = X; a.W = W; a.u = base + cl.u; a.ustep = cl.ustep; a.inv = reinterpret_cast<float*>(base + cl.inv);
    a.N = s.N; a.L = s.L; a.P = s.P; a.Pp = d.Pp; a.G = d.G; a.Lg = d.Lg; a.MT = d.MT; a.MTl = d.MTl;
    a.H = (int)s.H; a.w_hs = w_head_bytes(s, F32);
    profile_mark("planes", st);
    hipLaunchKernelGGL(k_planes<F32>, dim3((unsigned)((s.N + 63) / 64), (unsigned)d.BH), dim3(NT), 0, st, a);
    return launch_ok();
}

template <bool F32>
race_status_t run_backproject(const Shape& s, const Derived& d, const void* X, const char* cache,
                              const CacheLayout& cl, const char* dh, const void* WTp, void* out, float beta,
                              hipStream_t st) {
    BackArgs a;
    a.X = X; a.inv = reinterpret_cast<const float*>(cache + cl.inv); a.dh = dh + cl.u; a.dstep = cl.ustep;
    a.WTp = WTp; a.wt_gs = (s.w_per_head ? (size_t)s.H : 1) * wt_bytes(d);
    a.wt_hs = s.w_per_head ? (int64_t)wt_bytes(d) : 0; a.H = (int)s.H;
    a.out = out; a.N = s.N; a.G = d.G; a.MT = d.MT; a.MTl = d.MTl; a.beta = beta;
    profile_mark("backproject", st);
    hipLaunchKernelGGL(k_backproject<F32>, dim3((unsigned)((s.N + 63) / 64), (unsigned)d.BH), dim3(NT), 0, st, a);
    return launch_ok();
}

// Value half h of a [BH][N][128] tensor: columns 64 h .. 64 h + 63 (rows
// 128 elements apart).
template <bool F32>
inline const void* half_cols(const void* p, int h) {
    return reinterpret_cast<const char*>(p) + (size_t)h * 64 * (F32 ? 4 : 2);
}
template <bool F32>
inline void* half_cols(void* p, int h) {
    return reinterpret_cast<char*>(p) + (size_t)h * 64 * (F32 ? 4 : 2);
}

// Forward into O: plane values of queries and keys (into saved when given,
// else the workspace), then per value half the keys' chunk sketches, their
// scan (or total) and the read-out. D is written by the first half.
template <bool F32>
race_status_t run_forward_h2(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c, void* O,
                             void* saved) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = reinterpret_cast<char*>(saved);
    char* qbase = saved ? sv + sl.q : ws + wl.Qc;
    char* kbase = saved ? sv + sl.k : ws + wl.Kc;
    const float beta = c.hard ? HARD_BETA : c.beta;
    RACE_TRY(run_planes<F32>(s, d, c.Q, c.W, qbase, cl, st));
    RACE_TRY(run_planes<F32>(s, d, c.K, c.W, kbase, cl, st));
    for (int h = 0; h < 2; ++h) {
        float* Sb = ((s.causal && saved) ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.S)) +
                    half_states_floats(d, d.NC, h);
        float* St = (saved ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.St)) +
                    half_states_floats(d, 1, h);
        const void* Vh = half_cols<F32>(c.V, h);
        for (int g = 0; g < d.G; ++g) {
            const Group gr = group(d, g);
            float* Sg = Sb + group_states_floats(d, d.NC, g);
            RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
                using C = typename decltype(tag)::type;
                return run_totals<C, false, true>(s, d, gr, nullptr, Vh, nullptr, nullptr, plane_cache(kbase, cl, g),
                                                  nullptr, beta, Sg, st, D128, 64);
            })));
            if (s.causal) {
                RACE_TRY(run_scan<SCAN_EXCL>(s, d, gr.F65, gr.F, !F32, Sg, nullptr, 0,
                                             reinterpret_cast<float*>(ws + wl.scan), st));
            } else {
                RACE_TRY(run_scan<SCAN_TOTAL>(s, d, gr.F65, gr.F, !F32, Sg, St + group_states_floats(d, 1, g), gr.F65,
                                              nullptr, st));
            }
        }
        PassArgs a{};
        a.Zsrc = Vh; a.beta = beta; a.out0 = half_cols<F32>(O, h); a.hard = c.hard;
        a.Dv = (saved && h == 0) ? reinterpret_cast<float*>(sv + sl.D) : nullptr;
        RACE_TRY((run_pass_groups<F32, PASS_FWD, true>(s, d, wl, ws, a, st, [&](const Group& gr, PassArgs& ag) {
            ag.W = group_w(c.W, s, gr, F32);   // not read: the plane values are given
            ag.ca = plane_cache(qbase, cl, gr.g);
            ag.cb = plane_cache(kbase, cl, gr.g);
            ag.rs = D128; ag.dh = 64;
            if (s.causal) {
                ag.state = Sb + group_states_floats(d, d.NC, gr.g);
                ag.state_bh_stride = d.NC * gr.F65; ag.state_chunk_stride = gr.F65;
            } else {
                ag.state = St + group_states_floats(d, 1, gr.g);
                ag.state_bh_stride = gr.F65; ag.state_chunk_stride = 0;
            }
        })));
    }
    return RACE_OK;
}

template <bool F32>
race_status_t run_backward_h2(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    const void* O = c.O_in;
    const void* saved = c.saved_in;
    if (!saved) {
        RACE_TRY(run_forward_h2<F32>(s, d, wl, c, ws + wl.Ov, ws + wl.Sv));
        O = ws + wl.Ov;
        saved = ws + wl.Sv;
    }
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = const_cast<char*>(reinterpret_cast<const char*>(saved));
    char* qbase = sv + sl.q;
    char* kbase = sv + sl.k;
    const float* S = reinterpret_cast<const float*>(saved);
    float* Dv = reinterpret_cast<float*>(sv + sl.D);
    float* Ev = reinterpret_cast<float*>(ws + wl.E);
    char* dhQ = ws + wl.dhQ;
    char* dhK = ws + wl.dhK;
    const int64_t per_head = s.causal ? d.NC : 1;
    using elem = typename Prec<F32>::elem;
    const int64_t hw = s.w_per_head ? s.H : 1;
    auto wtp = [&](int g) { return reinterpret_cast<elem*>(ws + wl.wt + (size_t)g * hw * wt_bytes(d)); };
    for (int g = 0; g < d.G; ++g) {
        const Group gr = group(d, g);
        profile_mark("prep", st);
        RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
            using C = typename decltype(tag)::type;
            hipLaunchKernelGGL(k_prep<C>, dim3(8, (unsigned)hw), dim3(256), 0, st,
                               reinterpret_cast<const elem*>(group_w(c.W, s, gr, F32)), gr.L, wtp(g),
                               w_head_bytes(s, F32) / (int64_t)sizeof(elem),
                               s.w_per_head ? (int64_t)(wt_bytes(d) / sizeof(elem)) : 0, s.d, d.NDT);
            return launch_ok();
        })));
    }
    const int64_t rows = d.BH * s.N;
    if ((rows + 15) / 16 > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
    profile_mark("erow", st);
    hipLaunchKernelGGL(k_erow<F32>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, c.dO, O, Dv, Ev, rows);
    RACE_TRY(launch_ok());

    // query side: per-plane gradients of both halves, then dQ
    for (int h = 0; h < 2; ++h) {
        const float* Sh = S + half_states_floats(d, per_head, h);
        PassArgs q{};
        q.Zsrc = half_cols<F32>(c.V, h); q.Ysrc = half_cols<F32>(c.dO, h); q.beta = c.beta;
        q.Dv = Dv; q.Ev = Ev; q.half = h;
        RACE_TRY((run_pass_groups<F32, PASS_BWD_Q, true>(s, d, wl, ws, q, st, [&](const Group& gr, PassArgs& ag) {
            ag.ca = plane_cache(qbase, cl, gr.g);
            ag.cb = plane_cache(kbase, cl, gr.g);
            ag.rs = D128; ag.dh = 64; ag.gmode = 0;
            ag.dhb = reinterpret_cast<float*>(dhQ + cl.u_of(gr.g));
            ag.state = Sh + group_states_floats(d, per_head, gr.g);
            ag.state_bh_stride = s.causal ? d.NC * gr.F65 : gr.F65;
            ag.state_chunk_stride = s.causal ? gr.F65 : 0;
        })));
    }
    RACE_TRY(run_backproject<F32>(s, d, c.Q, qbase, cl, dhQ, wtp(0), c.dQ, c.beta, st));

    // gradient sketches of the queries per half (e only in the first)
    float* Tw = reinterpret_cast<float*>(ws + wl.T);
    float* Ttw = reinterpret_cast<float*>(ws + wl.Tt);
    for (int h = 0; h < 2; ++h) {
        for (int g = 0; g < d.G; ++g) {
            const Group gr = group(d, g);
            float* Tg = Tw + half_states_floats(d, d.NC, h) + group_states_floats(d, d.NC, g);
            RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
                using C = typename decltype(tag)::type;
                return run_totals<C, true>(s, d, gr, nullptr, half_cols<F32>(c.dO, h), Dv, Ev,
                                           plane_cache(qbase, cl, g), nullptr, c.beta, Tg, st, D128, 64, h);
            })));
            if (s.causal) {
                RACE_TRY(run_scan<SCAN_REV_EXCL>(s, d, gr.F65, gr.F, !F32, Tg, nullptr, 0,
                                                 reinterpret_cast<float*>(ws + wl.scan), st));
            } else {
                RACE_TRY(run_scan<SCAN_TOTAL>(s, d, gr.F65, gr.F, !F32, Tg,
                                              Ttw + half_states_floats(d, 1, h) + group_states_floats(d, 1, g),
                                              gr.F65, nullptr, st));
            }
        }
    }
    // key side: dV per half, then the keys' per-plane gradients and dK
    auto key_side = [&](int h) {
        return [&, h](const Group& gr, PassArgs& ag) {
            ag.ca = plane_cache(kbase, cl, gr.g);
            ag.cb = plane_cache(qbase, cl, gr.g);
            ag.rs = D128; ag.dh = 64;
            if (s.causal) {
                ag.state = Tw + half_states_floats(d, d.NC, h) + group_states_floats(d, d.NC, gr.g);
                ag.state_bh_stride = d.NC * gr.F65; ag.state_chunk_stride = gr.F65;
            } else {
                ag.state = Ttw + half_states_floats(d, 1, h) + group_states_floats(d, 1, gr.g);
                ag.state_bh_stride = gr.F65; ag.state_chunk_stride = 0;
            }
        };
    };
    for (int h = 0; h < 2; ++h) {
        PassArgs k{};
        k.Zsrc = half_cols<F32>(c.dO, h); k.Ysrc = half_cols<F32>(c.V, h); k.beta = c.beta;
        k.Dv = Dv; k.Ev = Ev; k.out1 = half_cols<F32>(c.dV, h); k.half = h;
        RACE_TRY((run_pass_groups<F32, PASS_BWD_V>(s, d, wl, ws, k, st, key_side(h))));
    }
    for (int h = 0; h < 2; ++h) {
        PassArgs k{};
        k.Zsrc = half_cols<F32>(c.dO, h); k.Ysrc = half_cols<F32>(c.V, h); k.beta = c.beta;
        k.Dv = Dv; k.Ev = Ev; k.half = h;
        auto ks = key_side(h);
        RACE_TRY((run_pass_groups<F32, PASS_BWD_K, true>(s, d, wl, ws, k, st, [&](const Group& gr, PassArgs& ag) {
            ks(gr, ag);
            ag.gmode = 0;
            ag.dhb = reinterpret_cast<float*>(dhK + cl.u_of(gr.g));
        })));
    }
    return run_backproject<F32>(s, d, c.K, kbase, cl, dhK, wtp(0), c.dK, c.beta, st);
}

// Prefill: the keys' plane values, then per value half the chunk sums of the
// keys' sketch (float32 form) and their total into that half's value sums of
// each group's part of the running state (the masses with the first half).
template <bool F32>
race_status_t run_prefill_h2(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    float* Sb = reinterpret_cast<float*>(ws + wl.S);
    const CacheLayout cl = cache_layout(s, d);
    char* kbase = ws + wl.Kc;
    const float beta = c.hard ? HARD_BETA : c.beta;
    RACE_TRY(run_planes<F32>(s, d, c.K, c.W, kbase, cl, st));
    for (int h = 0; h < 2; ++h) {
        for (int g = 0; g < d.G; ++g) {
            const Group gr = group(d, g);
            float* Sg = Sb + group_states_floats(d, d.NC, g);
            RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
                using C = typename decltype(tag)::type;
                return run_totals<C, false, true>(s, d, gr, nullptr, half_cols<F32>(c.V, h), nullptr, nullptr,
                                                  plane_cache(kbase, cl, g), nullptr, beta, Sg, st, D128, 64, 0, 1);
            })));
            profile_mark("state_total", st);
            float* vals = c.state + (size_t)g * d.F * d.RW + (size_t)h * gr.F * DH;
            hipLaunchKernelGGL(k_state_total<SCAN_TOTAL>, dim3((unsigned)((gr.F65 + 255) / 256), (unsigned)d.BH),
                               dim3(256), 0, st, Sg, vals, (int)d.NC, gr.F, d.RSall,
                               h == 0 ? (int64_t)2 * gr.F * DH : (int64_t)-1);
            RACE_TRY(launch_ok());
        }
    }
    return RACE_OK;
}

template <bool F32>
race_status_t dispatch_h2(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    if (c.op == OP_FWD) return run_forward_h2<F32>(s, d, wl, c, c.O, c.saved_out);
    if (c.op == OP_BWD) return run_backward_h2<F32>(s, d, wl, c);
    if (c.op == OP_PREFILL) return run_prefill_h2<F32>(s, d, wl, c);
    return RACE_ERR_UNSUPPORTED;
}

}  // namespace race
