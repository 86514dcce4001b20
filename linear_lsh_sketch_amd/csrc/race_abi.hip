// C-ABI entry points of libraceattn: argument validation, workspace sizing and
// dispatch to the bf16 / float32 launch sequences. No C++ exception escapes.
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "race_attn.h"
#include "race_dispatch.hpp"

namespace race {
// the launch sequences are compiled once, in their own translation units
extern template race_status_t dispatch<true>(const Shape&, const Derived&, const WsLayout&, const Call&);
extern template race_status_t dispatch<false>(const Shape&, const Derived&, const WsLayout&, const Call&);
}  // namespace race

using namespace race;

// Device scratch of the allocation-free forward (race_attn_fwd_noalloc): a
// fixed array in the library's code object, one copy per GPU, held until the
// process ends. Host code never uses its name as an address: the device
// address of each GPU's copy comes from hipGetSymbolAddress (scratch_base).
static __device__ __align__(256) unsigned char scratch[RACE_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each GPU, looked up once per device with the
// device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

race_status_t scratch_base(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RACE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RACE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RACE_OK;
}

// Per-thread profiling state (race_attn_profile_events). Only the calling
// thread's own calls read or write it, so concurrent callers do not interact.
constexpr int kMaxStages = 256;
thread_local hipEvent_t* t_events = nullptr;
thread_local int t_capacity = 0;
thread_local int t_count = 0;
thread_local const char* t_names[kMaxStages + 1];
thread_local hipStream_t t_stream = nullptr;

race_status_t prepare(int64_t B, int64_t H, int64_t N, int d, int P, int L, int causal, int chunk,
                      Shape& s, Derived& dv) {
    s.B = B; s.H = H; s.N = N; s.d = d; s.P = P; s.L = L; s.causal = causal ? 1 : 0; s.chunk = chunk;
    s.w_per_head = 0;
    return derive(s, dv);
}

// The element type, and whether W holds one set of hyperplanes per head
// (RACE_W_PER_HEAD or'ed into the dtype argument).
bool dtype_ok(int t) {
    const int base = t & ~RACE_W_PER_HEAD;
    return base == RACE_F32 || base == RACE_BF16;
}
race_dtype_t base_dtype(int t) { return (race_dtype_t)(t & ~RACE_W_PER_HEAD); }
int per_head(int t) { return (t & RACE_W_PER_HEAD) ? 1 : 0; }

// Hard buckets: the denominator sums F (all groups) products of a mass, an
// integer of magnitude at most N, and a feature in {-1, 0, 1}, so every
// partial sum is an exact float32 integer while F * N < 2^24.
bool hard_exact(const Shape& s, const Derived& dv) { return (dv.F65all / 65) * s.N < (int64_t(1) << 24); }

// Vector loads and stores of 16 bytes need 16-byte aligned tensors.
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool all_aligned(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (!aligned(p)) return false;
    return true;
}

race_status_t guarded(race_status_t (*fn)(const Shape&, const Derived&, const WsLayout&, const Call&),
                      const Shape& s, const Derived& dv, const WsLayout& wl, const Call& c) {
    try {
        return fn(s, dv, wl, c);
    } catch (...) {
        return RACE_ERR_HIP;
    }
}

race_status_t go(race_dtype_t dtype_flags, const Shape& s, const Derived& dv, const WsLayout& wl, const Call& c) {
    const race_dtype_t dtype = base_dtype(dtype_flags);
    (void)hipGetLastError();  // clear a stale error so it is not reported as ours
    t_count = 0;
    t_stream = c.stream;
    race_status_t rc =
        dtype == RACE_F32 ? guarded(dispatch<true>, s, dv, wl, c) : guarded(dispatch<false>, s, dv, wl, c);
    profile_mark("end", c.stream);
    return rc;
}

}  // namespace

namespace race {
void profile_mark(const char* stage, hipStream_t stream) {
    if (!t_events || t_count >= t_capacity || t_count > kMaxStages) return;
    if (hipEventRecord(t_events[t_count], stream) == hipSuccess) t_names[t_count++] = stage;
}
}  // namespace race

extern "C" {

race_status_t race_attn_profile_events(void** events, int capacity) {
    if (events && capacity < 2) return RACE_ERR_INVALID_ARG;
    t_events = reinterpret_cast<hipEvent_t*>(events);
    t_capacity = events ? (capacity < kMaxStages + 1 ? capacity : kMaxStages + 1) : 0;
    t_count = 0;
    return RACE_OK;
}

int race_attn_profile_count(void) { return t_count; }

const char* race_attn_profile_stage(int i) { return (i >= 0 && i < t_count) ? t_names[i] : nullptr; }


race_status_t race_attn_workspace_bytes(int64_t B, int64_t H, int64_t N, int d, int P, int L, int causal,
                                        int chunk, int for_backward, size_t* bytes) {
    const int kind = for_backward & ~RACE_W_PER_HEAD;
    if (!bytes || kind < WS_FWD || kind > WS_FWD_SAVED) return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, causal, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(for_backward);
    *bytes = ws_layout(s, dv, kind).total;
    return RACE_OK;
}

race_status_t race_attn_saved_bytes(int64_t B, int64_t H, int64_t N, int d, int P, int L, int causal,
                                    int chunk, size_t* bytes) {
    if (!bytes) return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, causal, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    *bytes = saved_bytes(s, dv);
    return RACE_OK;
}

race_status_t race_attn_fwd(const void* Q, const void* K, const void* V, const void* W, int64_t B, int64_t H,
                            int64_t N, int d, int P, int L, float temperature, int causal, int chunk,
                            race_dtype_t dtype, void* O, void* saved, void* ws, size_t ws_bytes, void* stream) {
    if (!Q || !K || !V || !W || !O || !ws || !dtype_ok(dtype) || std::isnan(temperature) ||
        temperature == -INFINITY || !all_aligned({Q, K, V, W, O, ws, saved}))
        return RACE_ERR_INVALID_ARG;
    const bool hard = std::isinf(temperature);
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, causal, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    if (hard && !hard_exact(s, dv)) return RACE_ERR_UNSUPPORTED;
    const WsLayout wl = ws_layout(s, dv, saved ? WS_FWD_SAVED : WS_FWD);
    if (ws_bytes < wl.total) return RACE_ERR_WORKSPACE;
    Call c{};
    c.op = OP_FWD; c.Q = Q; c.K = K; c.V = V; c.W = W; c.saved_out = saved; c.beta = temperature; c.O = O;
    c.hard = hard;
    c.ws = ws; c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, wl, c);
}

race_status_t race_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const void* W, int64_t B,
                                    int64_t H, int64_t N, int d, int P, int L, float temperature, int causal,
                                    int chunk, race_dtype_t dtype, void* O, void* saved, void* stream) {
    if (!Q || !K || !V || !W || !O || !dtype_ok(dtype) || std::isnan(temperature) ||
        temperature == -INFINITY || !all_aligned({Q, K, V, W, O, saved}))
        return RACE_ERR_INVALID_ARG;
    const bool hard = std::isinf(temperature);
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, causal, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    if (hard && !hard_exact(s, dv)) return RACE_ERR_UNSUPPORTED;
    const WsLayout wl = ws_layout(s, dv, saved ? WS_FWD_SAVED : WS_FWD);
    if (wl.total > (size_t)RACE_NOALLOC_SCRATCH_BYTES) return RACE_ERR_WORKSPACE;
    void* ws = nullptr;
    rc = scratch_base(&ws);
    if (rc != RACE_OK) return rc;
    Call c{};
    c.op = OP_FWD; c.Q = Q; c.K = K; c.V = V; c.W = W; c.saved_out = saved; c.beta = temperature; c.O = O;
    c.hard = hard;
    c.ws = ws; c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, wl, c);
}

race_status_t race_attn_bwd(const void* Q, const void* K, const void* V, const void* W, const void* O,
                            const void* dO, const void* saved, int64_t B, int64_t H, int64_t N, int d, int P,
                            int L, float temperature, int causal, int chunk, race_dtype_t dtype, void* dQ, void* dK,
                            void* dV, void* ws, size_t ws_bytes, void* stream) {
    if (!Q || !K || !V || !W || !dO || !dQ || !dK || !dV || !ws || !dtype_ok(dtype) ||
        !std::isfinite(temperature) || (O == nullptr) != (saved == nullptr) ||
        !all_aligned({Q, K, V, W, O, dO, saved, dQ, dK, dV, ws}))
        return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, causal, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    const WsLayout wl = ws_layout(s, dv, saved ? WS_BWD : WS_BWD_RECOMPUTE);
    if (ws_bytes < wl.total) return RACE_ERR_WORKSPACE;
    Call c{};
    c.op = OP_BWD; c.Q = Q; c.K = K; c.V = V; c.W = W; c.dO = dO; c.O_in = O; c.saved_in = saved;
    c.beta = temperature; c.dQ = dQ; c.dK = dK; c.dV = dV; c.ws = ws;
    c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, wl, c);
}

race_status_t race_attn_hash(const void* X, const void* W, int64_t B, int64_t H, int64_t N, int d, int P, int L,
                             race_dtype_t dtype, int32_t* bucket_ids, unsigned long long* near_zero,
                             void* stream) {
    if (!X || !W || !bucket_ids || !near_zero || !dtype_ok(dtype) || !all_aligned({X, W}))
        return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, 0, 1, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    Call c{};
    c.op = OP_HASH; c.X = X; c.W = W; c.ids = bucket_ids; c.near_zero = near_zero;
    c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, WsLayout{}, c);
}

race_status_t race_attn_state_bytes(int64_t B, int64_t H, int d, int P, int L, size_t* bytes) {
    if (!bytes) return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, 1, d, P, L, 0, 1, s, dv);
    if (rc != RACE_OK) return rc;
    *bytes = (size_t)dv.BH * (size_t)dv.RSall * sizeof(float);
    return RACE_OK;
}

race_status_t race_attn_prefill(const void* K, const void* V, const void* W, int64_t B, int64_t H, int64_t N,
                                int d, int P, int L, float temperature, int chunk, race_dtype_t dtype,
                                float* state, void* ws, size_t ws_bytes, void* stream) {
    if (!K || !V || !W || !state || !ws || !dtype_ok(dtype) || std::isnan(temperature) ||
        temperature == -INFINITY || !all_aligned({K, V, W, state, ws}))
        return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, N, d, P, L, 0, chunk, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    const WsLayout wl = ws_layout(s, dv, WS_FWD);
    if (ws_bytes < wl.total) return RACE_ERR_WORKSPACE;
    Call c{};
    c.op = OP_PREFILL; c.K = K; c.V = V; c.W = W; c.beta = temperature; c.hard = std::isinf(temperature);
    c.state = state; c.ws = ws; c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, wl, c);
}

race_status_t race_attn_decode(const void* q, const void* k, const void* v, const void* W, int64_t B, int64_t H,
                               int64_t T, int d, int P, int L, float temperature, race_dtype_t dtype, float* state,
                               void* o, void* stream) {
    if (!q || !k || !v || !W || !state || !o || !dtype_ok(dtype) || std::isnan(temperature) ||
        temperature == -INFINITY || !all_aligned({W, state}))
        return RACE_ERR_INVALID_ARG;
    Shape s;
    Derived dv;
    race_status_t rc = prepare(B, H, T, d, P, L, 0, 1, s, dv);
    if (rc != RACE_OK) return rc;
    s.w_per_head = per_head(dtype);
    if (T > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
    Call c{};
    c.op = OP_DECODE; c.Q = q; c.K = k; c.V = v; c.W = W; c.O = o; c.beta = temperature;
    c.hard = std::isinf(temperature); c.state = state; c.stream = reinterpret_cast<hipStream_t>(stream);
    return go(dtype, s, dv, WsLayout{}, c);
}

const char* race_attn_status_string(race_status_t status) {
    switch (status) {
        case RACE_OK: return "RACE_OK";
        case RACE_ERR_INVALID_ARG: return "RACE_ERR_INVALID_ARG";
        case RACE_ERR_UNSUPPORTED: return "RACE_ERR_UNSUPPORTED";
        case RACE_ERR_WORKSPACE: return "RACE_ERR_WORKSPACE";
        case RACE_ERR_HIP: return "RACE_ERR_HIP";
    }
    return "RACE_ERR_UNKNOWN";
}

}  // extern "C"
