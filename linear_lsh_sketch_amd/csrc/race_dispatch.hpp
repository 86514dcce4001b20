// Launch sequences for the forward, backward, hash, prefill and decode entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <functional>
#include <type_traits>

#include "race_decode.hpp"
#include "race_host.hpp"
#include "race_kernels.hpp"

namespace race {

enum { OP_FWD = 0, OP_BWD = 1, OP_HASH = 2, OP_PREFILL = 3, OP_DECODE = 4 };

// Temperature the sketch kernels use for the hard buckets: tanh(beta u)
// evaluates as 1 - 2 / (1 + 2^(2 log2(e) beta u)), and with this beta the
// exponent overflows (t = 1) or underflows (t = -1) for every |u| >= 1e-28,
// while u = 0 (a padded table's plane, or an exactly orthogonal row) still
// gives t = 0.
constexpr float HARD_BETA = 1e30f;

struct Call {
    int op;
    const void *Q, *K, *V, *W, *dO;
    const void* O_in;       // backward: the forward output (null: recompute the forward)
    const void* saved_in;   // backward: what the forward kept (null: recompute the forward)
    void* saved_out;        // forward: where to keep the states and D (may be null)
    float beta;
    void *O, *dQ, *dK, *dV;
    void* ws;
    hipStream_t stream;
    const void* X;                 // hash
    int32_t* ids;                  // hash
    unsigned long long* near_zero; // hash
    float* state;                  // prefill (out) / decode (in and out): running sketch [BH][RSall]
    int hard;                      // forward (float32), prefill, decode: one-hot buckets (temperature = +inf)
};

template <bool F32>
race_status_t dispatch(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c);

// Forward and backward at head dimension 128 (race_h2.hpp, built in
// translation units of their own).
template <bool F32>
race_status_t dispatch_h2(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c);

// Profiling aid (race_attn_profile_events): records a caller-owned event on the
// stream before each launch of the current call, when enabled on this thread.
void profile_mark(const char* stage, hipStream_t stream);

inline race_status_t launch_ok() {
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

#define RACE_TRY(x)                          \
    do {                                     \
        race_status_t rc_ = (x);             \
        if (rc_ != RACE_OK) return rc_;      \
    } while (0)

// Compile-time configuration of one table group's launches: fn(Tag<Cfg>{})
// for the (P, MT) pair (MT = projection tiles of the group).
template <class C>
struct Tag {
    using type = C;
};

template <bool F32, class Fn>
race_status_t with_cfg(int P, int MT, Fn&& fn) {
#define RACE_CFG(P_, MT_) \
    if (P == P_ && MT == MT_) return fn(Tag<Cfg<P_, MT_, F32>>{});
    RACE_CFG(1, 1) RACE_CFG(1, 2) RACE_CFG(1, 4) RACE_CFG(1, 8)
    RACE_CFG(2, 1) RACE_CFG(2, 2) RACE_CFG(2, 4) RACE_CFG(2, 8)
    RACE_CFG(3, 1) RACE_CFG(3, 2) RACE_CFG(3, 4) RACE_CFG(3, 8)
    RACE_CFG(4, 1) RACE_CFG(4, 2) RACE_CFG(4, 4) RACE_CFG(4, 8)
    RACE_CFG(5, 1) RACE_CFG(5, 2) RACE_CFG(5, 4)
    RACE_CFG(6, 1) RACE_CFG(6, 2)
#undef RACE_CFG
    return RACE_ERR_UNSUPPORTED;
}

// Bytes between the hyperplanes of consecutive heads (0: one W for all).
inline int64_t w_head_bytes(const Shape& s, bool f32) {
    return s.w_per_head ? (int64_t)s.L * s.P * s.d * (f32 ? 4 : 2) : 0;
}

// CACHED = false: sketch of K, [V | 1] (storing the keys' plane values in pc,
// or with PG reading them from pc); CACHED = true: gradient sketch of the
// queries from their plane values pc. Head dimension 128 passes one value
// half: rows rs = 128 apart, dh = 64 columns, e = 0 in the second (ezero).
template <class C, bool CACHED, bool PG = false>
race_status_t run_totals(const Shape& s, const Derived& d, const Group& gr, const void* Xb, const void* Z,
                         const float* Dv, const float* Ev, const PlaneCache& pc, const void* W, float beta,
                         float* out, hipStream_t st, int rs = 0, int dh = 0, int ezero = 0, int f32form = 0) {
    TotArgs a;
    a.Xb = Xb; a.Z = Z; a.Dv = Dv; a.Ev = Ev; a.W = W; a.pc = pc; a.out = out;
    a.N = s.N; a.chunk = s.chunk; a.nchunks = (int)d.NC; a.L = gr.L; a.beta = beta;
    a.H = (int)s.H; a.w_hs = w_head_bytes(s, C::F32); a.dh = dh ? dh : s.d; a.rs = rs ? rs : s.d;
    a.ezero = ezero;
    a.f32form = f32form;
    profile_mark(CACHED ? "totals_qg" : "totals_kv", st);
    // bf16 groups of eight feature chunks take them as one block (one
    // feature-tile write and two barriers per sub-block; the value operands
    // are read once); the LDS still fits three workgroups per CU
    using CT = Cfg<C::P, C::MT, C::F32, (!C::F32 && C::NKC == 8) ? 8 : 0>;
    hipLaunchKernelGGL((k_totals<CT, CACHED, PG>), dim3((unsigned)d.NC, (unsigned)d.BH), dim3(NT), 0, st, a);
    return launch_ok();
}

// One side's plane values (table group g) and inverse norms.
inline PlaneCache plane_cache(void* base, const CacheLayout& cl, int g) {
    char* b = reinterpret_cast<char*>(base);
    PlaneCache p;
    p.u = b + cl.u_of(g);
    p.inv = reinterpret_cast<float*>(b + cl.inv);
    return p;
}

// Scan of one group's chunk states [BH][NC][F65 floats] (F features; the
// compact form of bf16 inputs: 32 F words of bf16 pairs, then 33 F + 64 -
// 32 F float32 words); the total of head bh goes to total + bh * total_stride.
template <int KIND>
race_status_t run_scan(const Shape& s, const Derived& d, int64_t F65, int F, bool compact, float* states,
                       float* total, int64_t total_stride, float* segbuf, hipStream_t st) {
    ScanShape sh;
    sh.nchunks = (int)d.NC;
    sh.stride = (int)F65;
    sh.npair = compact ? 32 * F : 0;
    sh.nwords = compact ? 33 * F + DH : (int)F65;
    const unsigned gx = (unsigned)((sh.nwords + 255) / 256);
    profile_mark(KIND == SCAN_EXCL ? "scan_excl" : KIND == SCAN_REV_EXCL ? "scan_rev_excl" : "scan_total", st);
    const int segs = KIND == SCAN_TOTAL ? 1 : scan_segs(s, d, sh.nwords);
    if (segs == 1) {
        hipLaunchKernelGGL(k_scan<KIND>, dim3(gx, (unsigned)d.BH), dim3(256), 0, st, states, total, sh, total_stride);
        return launch_ok();
    }
    const dim3 grid(gx, (unsigned)(d.BH * segs));
    hipLaunchKernelGGL(k_scan_segsum<KIND>, grid, dim3(256), 0, st, states, segbuf, sh, segs);
    RACE_TRY(launch_ok());
    hipLaunchKernelGGL(k_scan_segapply<KIND>, grid, dim3(256), 0, st, states, segbuf, sh, segs);
    return launch_ok();
}

enum { PASS_FWD = 0, PASS_BWD_Q = 1, PASS_BWD_V = 2, PASS_BWD_K = 3 };

// The forward and the query-side backward use feature blocks of two chunks in
// bf16 (smaller LDS tiles and operand sets, so two workgroups fit on a CU).
// (P = 6 holds four chunks per tile: its blocks are whole tiles.)
template <class C>
using Blk2Cfg = Cfg<C::P, C::MT, C::F32, C::F32 ? 0 : (C::KB > 2 ? C::KB : 2)>;

// H2: the head-dimension-128 forms (the forward reads the queries' plane
// values, the query and key gradient passes leave per-plane gradients).
template <class C, int KIND, bool H2 = false>
race_status_t run_pass(const Shape& s, const Derived& d, PassArgs a, hipStream_t st) {
    a.N = s.N; a.chunk = s.chunk; a.causal = s.causal;
    const dim3 grid((unsigned)d.NC, (unsigned)d.BH), block(NT);
    using CB = Blk2Cfg<C>;
    // causal groups of P = 4 have at most four projection tiles (race_host.hpp),
    // so the eight-tile causal passes are never built
    if constexpr (C::P == 4 && C::MT == 8) {
        if (s.causal) return RACE_ERR_UNSUPPORTED;
    }
    constexpr bool CAUSAL_OK = !(C::P == 4 && C::MT == 8);
    if constexpr (KIND == PASS_FWD) {
        profile_mark("pass_fwd", st);
        // bf16 hard buckets run their own instantiation (the exact
        // denominator); float32 needs none
        auto fwd = [&](auto hard) {
            constexpr bool HD = decltype(hard)::value;
            if constexpr (CAUSAL_OK) {
                if (s.causal) hipLaunchKernelGGL((k_fwd<CB, true, H2, HD>), grid, block, 0, st, a);
                else hipLaunchKernelGGL((k_fwd<CB, false, H2, HD>), grid, block, 0, st, a);
            } else {
                hipLaunchKernelGGL((k_fwd<CB, false, H2, HD>), grid, block, 0, st, a);
            }
        };
        if constexpr (!C::F32) {
            if (a.hard) fwd(std::true_type{});
            else fwd(std::false_type{});
        } else {
            fwd(std::false_type{});
        }
    } else if constexpr (KIND == PASS_BWD_Q) {
        profile_mark("pass_bwd_q", st);
        if constexpr (CAUSAL_OK) {
            if (s.causal) hipLaunchKernelGGL((k_bwd_q<CB, true, H2>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_bwd_q<CB, false, H2>), grid, block, 0, st, a);
        } else {
            hipLaunchKernelGGL((k_bwd_q<CB, false, H2>), grid, block, 0, st, a);
        }
    } else if constexpr (KIND == PASS_BWD_V) {
        profile_mark("pass_bwd_v", st);
        if constexpr (CAUSAL_OK) {
            if (s.causal) hipLaunchKernelGGL((k_bwd_k<CB, true, KPART_DV>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_bwd_k<CB, false, KPART_DV>), grid, block, 0, st, a);
        } else {
            hipLaunchKernelGGL((k_bwd_k<CB, false, KPART_DV>), grid, block, 0, st, a);
        }
    } else {
        profile_mark("pass_bwd_k", st);
        if constexpr (CAUSAL_OK) {
            if (s.causal) hipLaunchKernelGGL((k_bwd_k<CB, true, KPART_DK, H2>), grid, block, 0, st, a);
            else hipLaunchKernelGGL((k_bwd_k<CB, false, KPART_DK, H2>), grid, block, 0, st, a);
        } else {
            hipLaunchKernelGGL((k_bwd_k<CB, false, KPART_DK, H2>), grid, block, 0, st, a);
        }
    }
    return launch_ok();
}

// Launch one pass of every table group in order: group g adds to the partial
// outputs of the groups before it, the last one finishes the outputs.
template <bool F32, int KIND, bool H2 = false>
race_status_t run_pass_groups(const Shape& s, const Derived& d, const WsLayout& wl, char* ws, PassArgs a,
                              hipStream_t st, const std::function<void(const Group&, PassArgs&)>& per_group) {
    for (int g = 0; g < d.G; ++g) {
        const Group gr = group(d, g);
        PassArgs ag = a;
        ag.L = gr.L;
        ag.H = (int)s.H;
        ag.w_hs = w_head_bytes(s, F32);
        ag.wt_hs = s.w_per_head ? (int64_t)wt_bytes(d) : 0;
        ag.dh = s.d;
        ag.rs = s.d;
        ag.gmode = (g > 0 ? ACC_IN : 0) | (g + 1 < d.G ? ACC_OUT : 0);
        ag.acc = d.G > 1 ? reinterpret_cast<float*>(ws + wl.acc) : nullptr;
        ag.accD = d.G > 1 ? reinterpret_cast<float*>(ws + wl.accD) : nullptr;
        per_group(gr, ag);
        RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
            using C = typename decltype(tag)::type;
            return run_pass<C, KIND, H2>(s, d, ag, st);
        })));
    }
    return RACE_OK;
}

// Hyperplanes of table group g (W is [L, P, d], or [H, L, P, d] with the
// heads w_head_bytes apart; groups are consecutive tables).
inline const void* group_w(const void* W, const Shape& s, const Group& gr, bool f32) {
    return reinterpret_cast<const char*>(W) + (size_t)gr.t0 * s.P * s.d * (f32 ? 4 : 2);
}

// Forward into O; when `saved` is set it receives the sketch states, D and
// the plane values of queries and keys (else the keys' go to the workspace).
template <bool F32>
race_status_t run_forward(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c, void* O, void* saved) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = reinterpret_cast<char*>(saved);
    char* kbase = saved ? sv + sl.k : ws + wl.Kc;
    // per-chunk states (causal: in saved when given) and, non-causal, the totals
    float* Sb = (s.causal && saved) ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.S);
    float* St = saved ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.St);
    const float beta = c.hard ? HARD_BETA : c.beta;
    for (int g = 0; g < d.G; ++g) {
        const Group gr = group(d, g);
        float* Sg = Sb + group_states_floats(d, d.NC, g);
        const PlaneCache kc = plane_cache(kbase, cl, g);
        const void* Wg = group_w(c.W, s, gr, F32);
        RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
            using C = typename decltype(tag)::type;
            return run_totals<C, false>(s, d, gr, c.K, c.V, nullptr, nullptr, kc, Wg, beta, Sg, st);
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
    a.Xa = c.Q; a.Zsrc = c.V; a.beta = beta; a.out0 = O; a.hard = c.hard;
    a.Dv = saved ? reinterpret_cast<float*>(sv + sl.D) : nullptr;
    return run_pass_groups<F32, PASS_FWD>(s, d, wl, ws, a, st, [&](const Group& gr, PassArgs& ag) {
        ag.W = group_w(c.W, s, gr, F32);
        ag.ca = saved ? plane_cache(sv + sl.q, cl, gr.g) : PlaneCache{};
        ag.cb = plane_cache(kbase, cl, gr.g);
        if (s.causal) {
            ag.state = Sb + group_states_floats(d, d.NC, gr.g);
            ag.state_bh_stride = d.NC * gr.F65; ag.state_chunk_stride = gr.F65;
        } else {
            ag.state = St + group_states_floats(d, 1, gr.g);
            ag.state_bh_stride = gr.F65; ag.state_chunk_stride = 0;
        }
    });
}

template <bool F32>
race_status_t run_backward(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    // O and what the forward kept, recomputed when not given
    const void* O = c.O_in;
    const void* saved = c.saved_in;
    if (!saved) {
        RACE_TRY(run_forward<F32>(s, d, wl, c, ws + wl.Ov, ws + wl.Sv));
        O = ws + wl.Ov;
        saved = ws + wl.Sv;
    }
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = const_cast<char*>(reinterpret_cast<const char*>(saved));
    const float* S = reinterpret_cast<const float*>(saved);
    float* Dv = reinterpret_cast<float*>(sv + sl.D);
    float* Ev = reinterpret_cast<float*>(ws + wl.E);
    using elem = typename Prec<F32>::elem;
    // back-projection tables: one per group and head of W
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

    PassArgs q{};
    q.Xa = c.Q; q.Zsrc = c.V; q.Ysrc = c.dO; q.Osrc = O; q.beta = c.beta;
    q.Dv = Dv; q.Ev = Ev; q.out0 = c.dQ;
    RACE_TRY((run_pass_groups<F32, PASS_BWD_Q>(s, d, wl, ws, q, st, [&](const Group& gr, PassArgs& ag) {
        ag.W = group_w(c.W, s, gr, F32);
        ag.WTp = wtp(gr.g);
        ag.ca = plane_cache(sv + sl.q, cl, gr.g);
        ag.cb = plane_cache(sv + sl.k, cl, gr.g);
        ag.state = S + group_states_floats(d, s.causal ? d.NC : 1, gr.g);
        ag.state_bh_stride = s.causal ? d.NC * gr.F65 : gr.F65;
        ag.state_chunk_stride = s.causal ? gr.F65 : 0;
    })));

    // gradient sketches of the queries, reverse-scanned (causal) or summed
    float* Tw = reinterpret_cast<float*>(ws + wl.T);
    float* Ttw = reinterpret_cast<float*>(ws + wl.Tt);
    for (int g = 0; g < d.G; ++g) {
        const Group gr = group(d, g);
        float* Tg = Tw + group_states_floats(d, d.NC, g);
        RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
            using C = typename decltype(tag)::type;
            return run_totals<C, true>(s, d, gr, c.Q, c.dO, Dv, Ev, plane_cache(sv + sl.q, cl, g),
                                       group_w(c.W, s, gr, F32), c.beta, Tg, st);
        })));
        if (s.causal) {
            RACE_TRY(run_scan<SCAN_REV_EXCL>(s, d, gr.F65, gr.F, !F32, Tg, nullptr, 0,
                                             reinterpret_cast<float*>(ws + wl.scan), st));
        } else {
            RACE_TRY(run_scan<SCAN_TOTAL>(s, d, gr.F65, gr.F, !F32, Tg, Ttw + group_states_floats(d, 1, g), gr.F65,
                                          nullptr, st));
        }
    }
    PassArgs k{};
    k.Xa = c.K; k.Zsrc = c.dO; k.Ysrc = c.V; k.beta = c.beta;
    k.Dv = Dv; k.Ev = Ev; k.out0 = c.dK; k.out1 = c.dV;
    auto key_side = [&](const Group& gr, PassArgs& ag) {
        ag.W = group_w(c.W, s, gr, F32);
        ag.WTp = wtp(gr.g);
        ag.ca = plane_cache(sv + sl.k, cl, gr.g);
        ag.cb = plane_cache(sv + sl.q, cl, gr.g);
        if (s.causal) {
            ag.state = Tw + group_states_floats(d, d.NC, gr.g);
            ag.state_bh_stride = d.NC * gr.F65; ag.state_chunk_stride = gr.F65;
        } else {
            ag.state = Ttw + group_states_floats(d, 1, gr.g);
            ag.state_bh_stride = gr.F65; ag.state_chunk_stride = 0;
        }
    };
    // dV of every group, then dK (each output's partials share one buffer)
    RACE_TRY((run_pass_groups<F32, PASS_BWD_V>(s, d, wl, ws, k, st, key_side)));
    return run_pass_groups<F32, PASS_BWD_K>(s, d, wl, ws, k, st, key_side);
}

template <bool F32>
race_status_t dispatch(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    hipStream_t st = c.stream;
    if (c.op == OP_HASH) {
        const int64_t blocks = (s.N + 63) / 64;   // per (batch, head) sequence
        if (blocks > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
        for (int g = 0; g < d.G; ++g) {
            const Group gr = group(d, g);
            profile_mark("hash", st);
            RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
                using C = typename decltype(tag)::type;
                hipLaunchKernelGGL(k_hash<C>, dim3((unsigned)blocks, (unsigned)d.BH), dim3(NT), 0, st, c.X,
                                   group_w(c.W, s, gr, F32), s.N, gr.L, s.L, (int)s.H, w_head_bytes(s, F32), s.d,
                                   c.ids + gr.t0, c.near_zero);
                return launch_ok();
            })));
        }
        return RACE_OK;
    }
    if (d.VH == 2 && c.op != OP_DECODE) return dispatch_h2<F32>(s, d, wl, c);
    if (c.op == OP_FWD) return run_forward<F32>(s, d, wl, c, c.O, c.saved_out);
    if (c.op == OP_BWD) return run_backward<F32>(s, d, wl, c);
    if (c.op == OP_PREFILL) {
        // chunk sums of the keys' sketch, then their total straight into each
        // group's part of the running state
        char* ws = reinterpret_cast<char*>(c.ws);
        float* Sb = reinterpret_cast<float*>(ws + wl.S);
        const CacheLayout cl = cache_layout(s, d);
        const float beta = c.hard ? HARD_BETA : c.beta;
        for (int g = 0; g < d.G; ++g) {
            const Group gr = group(d, g);
            float* Sg = Sb + group_states_floats(d, d.NC, g);
            RACE_TRY((with_cfg<F32>(s.P, gr.MT, [&](auto tag) {
                using C = typename decltype(tag)::type;
                return run_totals<C, false>(s, d, gr, c.K, c.V, nullptr, nullptr, plane_cache(ws + wl.Kc, cl, g),
                                            group_w(c.W, s, gr, F32), beta, Sg, st, 0, 0, 0, 1);
            })));
            profile_mark("state_total", st);
            hipLaunchKernelGGL(k_state_total<SCAN_TOTAL>, dim3((unsigned)((gr.F65 + 255) / 256), (unsigned)d.BH),
                               dim3(256), 0, st, Sg, c.state + (size_t)g * d.F * d.RW, (int)d.NC, gr.F, d.RSall,
                               (int64_t)gr.F * DH);
            RACE_TRY(launch_ok());
        }
        return RACE_OK;
    }
    if (c.op == OP_DECODE) {
        return with_cfg<F32>(s.P, d.MT, [&](auto tag) {
            using C = typename decltype(tag)::type;
            DecodeArgs a{};
            a.q = c.Q; a.k = c.K; a.v = c.V; a.W = c.W; a.state = c.state; a.o = c.O; a.T = (int)s.N;
            a.P = s.P; a.L = s.L; a.F = C::F; a.KB = C::KB; a.TPT = C::TPT; a.TPL = C::TPL;
            a.G = d.G; a.Lg = d.Lg; a.Fl = d.Fl;
            a.beta = c.beta; a.hard = c.hard;
            a.H = (int)s.H; a.w_hs = w_head_bytes(s, C::F32); a.dh = s.d; a.VH = d.VH;
            static_assert(C::F <= DEC_MAXF && C::F % DEC_RG == 0, "decode tiling");
            constexpr int NR = C::F / DEC_RG;   // state rows per thread
            // head dimension 128: the second value half first, without storing
            // the masses, then the first half
            auto launch = [&](auto xw, auto one) {
                constexpr int XW = decltype(xw)::value;
                for (int h = d.VH - 1; h >= 0; --h) {
                    a.half = h;
                    a.store_mass = h == 0;
                    profile_mark("decode", st);
                    if constexpr (decltype(one)::value) {
                        hipLaunchKernelGGL((k_decode_one<C::F32, NR, XW>), dim3((unsigned)d.BH), dim3(DEC_NT), 0, st,
                                           a);
                    } else {
                        hipLaunchKernelGGL((k_decode_multi<C::F32, NR, XW>), dim3((unsigned)d.BH), dim3(DEC_NT), 0,
                                           st, a);
                    }
                    RACE_TRY(launch_ok());
                }
                return RACE_OK;
            };
            using X64 = std::integral_constant<int, 64>;
            using X128 = std::integral_constant<int, 128>;
            if (d.G == 1) {
                return s.d == 128 ? launch(X128{}, std::false_type{}) : launch(X64{}, std::false_type{});
            }
            // one launch per token (and value half): every table group of each head in turn
            for (int tok = 0; tok < a.T; ++tok) {
                a.tok = tok;
                RACE_TRY(s.d == 128 ? launch(X128{}, std::true_type{}) : launch(X64{}, std::true_type{}));
            }
            return RACE_OK;
        });
    }
    return RACE_ERR_INVALID_ARG;
}

}  // namespace race
