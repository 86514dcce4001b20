// Launch sequences for the forward, backward, hash, prefill and decode entry points.
#pragma once

#include <hip/hip_runtime.h>

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
    float* state;                  // prefill (out) / decode (in and out): running sketch [BH][F * 65]
    int hard;                      // forward (float32), prefill, decode: one-hot buckets (temperature = +inf)
};

template <bool F32>
race_status_t dispatch(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c);

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

// CACHED = false: sketch of K, [V | 1] (storing the keys' plane values in pc);
// CACHED = true: gradient sketch of the queries from their plane values pc.
template <class C, bool CACHED>
race_status_t run_totals(const Shape& s, const Derived& d, const void* Xb, const void* Z, const float* Dv,
                         const float* Ev, const PlaneCache& pc, const void* W, float beta, float* out,
                         hipStream_t st) {
    TotArgs a;
    a.Xb = Xb; a.Z = Z; a.Dv = Dv; a.Ev = Ev; a.W = W; a.pc = pc; a.out = out;
    a.N = s.N; a.chunk = s.chunk; a.nchunks = (int)d.NC; a.L = s.L; a.beta = beta;
    profile_mark(CACHED ? "totals_qg" : "totals_kv", st);
    hipLaunchKernelGGL((k_totals<C, CACHED>), dim3((unsigned)d.NC, (unsigned)d.BH), dim3(NT), 0, st, a);
    return launch_ok();
}

inline PlaneCache plane_cache(void* base, const CacheLayout& cl) {
    char* b = reinterpret_cast<char*>(base);
    PlaneCache p;
    p.u = b + cl.u;
    p.inv = reinterpret_cast<float*>(b + cl.inv);
    return p;
}

template <int KIND>
race_status_t run_scan(const Shape& s, const Derived& d, float* states, float* total, float* segbuf,
                       hipStream_t st) {
    const int elems = (int)d.F65;
    const unsigned gx = (unsigned)((elems + 255) / 256);
    profile_mark(KIND == SCAN_EXCL ? "scan_excl" : KIND == SCAN_REV_EXCL ? "scan_rev_excl" : "scan_total", st);
    const int segs = KIND == SCAN_TOTAL ? 1 : scan_segs(s, d);
    if (segs == 1) {
        hipLaunchKernelGGL(k_scan<KIND>, dim3(gx, (unsigned)d.BH), dim3(256), 0, st, states, total, (int)d.NC,
                           elems);
        return launch_ok();
    }
    const dim3 grid(gx, (unsigned)(d.BH * segs));
    hipLaunchKernelGGL(k_scan_segsum<KIND>, grid, dim3(256), 0, st, states, segbuf, (int)d.NC, elems, segs);
    RACE_TRY(launch_ok());
    hipLaunchKernelGGL(k_scan_segapply<KIND>, grid, dim3(256), 0, st, states, segbuf, (int)d.NC, elems, segs);
    return launch_ok();
}

enum { PASS_FWD = 0, PASS_BWD_Q = 1, PASS_BWD_K = 2 };

// The forward and the query-side backward use feature blocks of two chunks in
// bf16 (smaller LDS tiles and operand sets, so two workgroups fit on a CU).
template <class C>
using Blk2Cfg = Cfg<C::P, C::MT, C::F32, C::F32 ? 0 : 2>;

template <class C, int KIND>
race_status_t run_pass(const Shape& s, const Derived& d, PassArgs a, hipStream_t st) {
    a.N = s.N; a.chunk = s.chunk; a.L = s.L; a.causal = s.causal;
    const dim3 grid((unsigned)d.NC, (unsigned)d.BH), block(NT);
    if constexpr (KIND == PASS_FWD) {
        profile_mark("pass_fwd", st);
        if (s.causal) hipLaunchKernelGGL((k_fwd<Blk2Cfg<C>, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_fwd<Blk2Cfg<C>, false>), grid, block, 0, st, a);
    } else if constexpr (KIND == PASS_BWD_Q) {
        profile_mark("pass_bwd_q", st);
        if (s.causal) hipLaunchKernelGGL((k_bwd_q<Blk2Cfg<C>, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_q<Blk2Cfg<C>, false>), grid, block, 0, st, a);
    } else {
        // key side: dV and dK in two passes of two workgroups per CU each
        using CK = Blk2Cfg<C>;
        profile_mark("pass_bwd_v", st);
        if (s.causal) hipLaunchKernelGGL((k_bwd_k<CK, true, KPART_DV>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_k<CK, false, KPART_DV>), grid, block, 0, st, a);
        RACE_TRY(launch_ok());
        profile_mark("pass_bwd_k", st);
        if (s.causal) hipLaunchKernelGGL((k_bwd_k<CK, true, KPART_DK>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_bwd_k<CK, false, KPART_DK>), grid, block, 0, st, a);
    }
    return launch_ok();
}

// Forward into O; when `saved` is set it receives the sketch states, D and
// the plane values of queries and keys (else the keys' go to the workspace).
template <class C>
race_status_t run_forward(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c, void* O, void* saved) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = reinterpret_cast<char*>(saved);
    const PlaneCache kc = plane_cache(saved ? sv + sl.k : ws + wl.Kc, cl);
    PlaneCache qc{};
    if (saved) qc = plane_cache(sv + sl.q, cl);
    float* Sb = (s.causal && saved) ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.S);
    const float beta = c.hard ? HARD_BETA : c.beta;
    RACE_TRY((run_totals<C, false>(s, d, c.K, c.V, nullptr, nullptr, kc, c.W, beta, Sb, st)));
    PassArgs a{};
    a.Xa = c.Q; a.ca = qc; a.cb = kc; a.Zsrc = c.V; a.W = c.W; a.beta = beta; a.out0 = O; a.hard = c.hard;
    a.Dv = saved ? reinterpret_cast<float*>(sv + sl.D) : nullptr;
    if (s.causal) {
        RACE_TRY(run_scan<SCAN_EXCL>(s, d, Sb, nullptr, reinterpret_cast<float*>(ws + wl.scan), st));
        a.state = Sb; a.state_bh_stride = d.NC * d.F65; a.state_chunk_stride = d.F65;
    } else {
        float* St = saved ? reinterpret_cast<float*>(saved) : reinterpret_cast<float*>(ws + wl.St);
        RACE_TRY(run_scan<SCAN_TOTAL>(s, d, Sb, St, nullptr, st));
        a.state = St; a.state_bh_stride = d.F65; a.state_chunk_stride = 0;
    }
    return run_pass<C, PASS_FWD>(s, d, a, st);
}

template <class C>
race_status_t run(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    char* ws = reinterpret_cast<char*>(c.ws);
    hipStream_t st = c.stream;
    if (c.op == OP_HASH) {
        const int64_t rows = d.BH * s.N;
        const int64_t blocks = (rows + 63) / 64;
        if (blocks > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
        profile_mark("hash", st);
        hipLaunchKernelGGL(k_hash<C>, dim3((unsigned)blocks), dim3(NT), 0, st, c.X, c.W, rows, s.L, c.ids,
                           c.near_zero);
        return launch_ok();
    }
    if (c.op == OP_FWD) return run_forward<C>(s, d, wl, c, c.O, c.saved_out);
    if (c.op == OP_PREFILL) {
        // chunk sums of the keys' sketch, then their total straight into the state
        float* Sb = reinterpret_cast<float*>(ws + wl.S);
        const PlaneCache kc = plane_cache(ws + wl.Kc, cache_layout(s, d));
        RACE_TRY((run_totals<C, false>(s, d, c.K, c.V, nullptr, nullptr, kc, c.W, c.hard ? HARD_BETA : c.beta,
                                       Sb, st)));
        return run_scan<SCAN_TOTAL>(s, d, Sb, c.state, nullptr, st);
    }
    if (c.op == OP_DECODE) {
        DecodeArgs a{};
        a.q = c.Q; a.k = c.K; a.v = c.V; a.W = c.W; a.state = c.state; a.o = c.O; a.T = (int)s.N;
        a.P = s.P; a.L = s.L; a.F = C::F; a.KB = C::KB; a.TPT = C::TPT; a.TPL = C::TPL;
        a.beta = c.beta; a.hard = c.hard;
        static_assert(C::F <= DEC_MAXF && C::F % DEC_RG == 0, "decode tiling");
        profile_mark("decode", st);
        constexpr int NR = C::F / DEC_RG;   // state rows per thread
        if (a.T == 1) hipLaunchKernelGGL((k_decode_one<C::F32, NR>), dim3((unsigned)d.BH), dim3(DEC_NT), 0, st, a);
        else hipLaunchKernelGGL((k_decode_multi<C::F32, NR>), dim3((unsigned)d.BH), dim3(DEC_NT), 0, st, a);
        return launch_ok();
    }

    // backward: O and what the forward kept, recomputed when not given
    const void* O = c.O_in;
    const void* saved = c.saved_in;
    if (!saved) {
        RACE_TRY(run_forward<C>(s, d, wl, c, ws + wl.Ov, ws + wl.Sv));
        O = ws + wl.Ov;
        saved = ws + wl.Sv;
    }
    const SavedLayout sl = saved_layout(s, d);
    const CacheLayout cl = cache_layout(s, d);
    char* sv = const_cast<char*>(reinterpret_cast<const char*>(saved));
    const PlaneCache qc = plane_cache(sv + sl.q, cl), kc = plane_cache(sv + sl.k, cl);
    const float* S = reinterpret_cast<const float*>(saved);
    float* Dv = reinterpret_cast<float*>(sv + sl.D);
    float* Ev = reinterpret_cast<float*>(ws + wl.E);
    using elem = typename Prec<C::F32>::elem;
    elem* WTp = reinterpret_cast<elem*>(ws + wl.wt);
    profile_mark("prep", st);
    hipLaunchKernelGGL(k_prep<C>, dim3(8), dim3(256), 0, st, reinterpret_cast<const elem*>(c.W), s.L, WTp);
    RACE_TRY(launch_ok());

    PassArgs q{};
    q.Xa = c.Q; q.ca = qc; q.cb = kc; q.Zsrc = c.V; q.Ysrc = c.dO; q.Osrc = O; q.W = c.W; q.WTp = WTp;
    q.beta = c.beta;
    q.Dv = Dv; q.Ev = Ev; q.out0 = c.dQ;
    q.state = S;
    q.state_bh_stride = s.causal ? d.NC * d.F65 : d.F65;
    q.state_chunk_stride = s.causal ? d.F65 : 0;
    RACE_TRY((run_pass<C, PASS_BWD_Q>(s, d, q, st)));

    float* Tw = reinterpret_cast<float*>(ws + wl.T);
    RACE_TRY((run_totals<C, true>(s, d, c.Q, c.dO, Dv, Ev, qc, c.W, c.beta, Tw, st)));
    PassArgs k{};
    k.Xa = c.K; k.ca = kc; k.cb = qc; k.Zsrc = c.dO; k.Ysrc = c.V; k.W = c.W; k.WTp = WTp; k.beta = c.beta;
    k.Dv = Dv; k.Ev = Ev; k.out0 = c.dK; k.out1 = c.dV;
    if (s.causal) {
        RACE_TRY(run_scan<SCAN_REV_EXCL>(s, d, Tw, nullptr, reinterpret_cast<float*>(ws + wl.scan), st));
        k.state = Tw; k.state_bh_stride = d.NC * d.F65; k.state_chunk_stride = d.F65;
    } else {
        float* Ttw = reinterpret_cast<float*>(ws + wl.Tt);
        RACE_TRY(run_scan<SCAN_TOTAL>(s, d, Tw, Ttw, nullptr, st));
        k.state = Ttw; k.state_bh_stride = d.F65; k.state_chunk_stride = 0;
    }
    return run_pass<C, PASS_BWD_K>(s, d, k, st);
}

#define RACE_CASE(P_, MT_)                                                   \
    if (s.P == P_ && d.MT == MT_) return run<Cfg<P_, MT_, F32>>(s, d, wl, c);

template <bool F32>
race_status_t dispatch(const Shape& s, const Derived& d, const WsLayout& wl, const Call& c) {
    RACE_CASE(1, 1) RACE_CASE(1, 2) RACE_CASE(1, 4) RACE_CASE(1, 8)
    RACE_CASE(2, 1) RACE_CASE(2, 2) RACE_CASE(2, 4) RACE_CASE(2, 8)
    RACE_CASE(3, 1) RACE_CASE(3, 2) RACE_CASE(3, 4) RACE_CASE(3, 8)
    RACE_CASE(4, 1) RACE_CASE(4, 2) RACE_CASE(4, 4) RACE_CASE(4, 8)
    return RACE_ERR_UNSUPPORTED;
}

}  // namespace race
