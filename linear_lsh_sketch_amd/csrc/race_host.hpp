// Host-side shape validation and workspace layout (no device code).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cmath>

#include "race_attn.h"

namespace race {

struct Shape {
    int64_t B, H, N;
    int d, P, L;
    int causal, chunk;
};

struct Derived {
    int Pp, MT, KB, F, NPAIR;
    int NPL;       // projection rows per token (MT * 16)
    int64_t BH, NC;
    int64_t F65;   // floats per sketch state: F * 64 value sums + F masses
};

struct WsLayout {
    size_t wt;     // backward: back-projection operand table
    size_t S;      // forward: per-chunk sketch states (or chunk totals, non-causal)
    size_t St;     // forward, non-causal: whole-sequence sketch
    size_t T;      // backward: per-chunk gradient sketch states
    size_t Tt;     // backward, non-causal: whole-sequence gradient sketch
    size_t E;      // backward: per-token e = -<dO, O>/D
    size_t Sv;     // backward without saved: the recomputed forward's saved buffer
    size_t Ov;     // backward without saved: the recomputed forward output
    size_t Kc;     // forward without saved: the keys' plane values
    size_t scan;   // segment sums of the segmented chunk scan (when used)
    size_t total;
};

// Plane values of one side (queries or keys): u = tanh of the normalised
// projection [rows][NPL] (float16 for bf16 inputs, float32 for float32; sized
// for float32, the upper bound), then 1 / max(|x|, eps) [rows] in float32.
struct CacheLayout {
    size_t u, inv, total;
};

// The saved buffer: float32 sketch states (per chunk, causal; the total,
// non-causal), the float32 per-token denominators D, then the plane values of
// the queries and of the keys.
struct SavedLayout {
    size_t D;
    size_t q;       // queries' plane values
    size_t k;       // keys' plane values
    size_t total;
};

// Workspace kinds (race_attn_workspace_bytes' for_backward argument).
enum { WS_FWD = 0, WS_BWD = 1, WS_BWD_RECOMPUTE = 2, WS_FWD_SAVED = 3 };

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Largest chunk (tokens per workgroup): the kernels address the rows of a
// chunk with 32-bit byte offsets, up to 512 bytes per row.
constexpr int MAX_CHUNK = 1 << 20;

inline bool mul_ok(int64_t a, int64_t b, int64_t& out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    out = a * b;
    return true;
}

inline race_status_t derive(const Shape& s, Derived& d) {
    if (s.B < 1 || s.H < 1 || s.N < 1 || s.d < 1 || s.P < 1 || s.L < 1 || s.chunk < 1)
        return RACE_ERR_INVALID_ARG;
    if (s.d != 64 || s.P > 4) return RACE_ERR_UNSUPPORTED;
    // in-chunk byte offsets (rows of up to 512 bytes) are 32-bit
    if (s.chunk > MAX_CHUNK) return RACE_ERR_UNSUPPORTED;
    d.Pp = (s.P == 3) ? 4 : s.P;
    const int64_t rows = (int64_t)s.L * d.Pp;
    if (rows > 128) return RACE_ERR_UNSUPPORTED;
    int mt = (int)((rows + 15) / 16);
    int p2 = 1;
    while (p2 < mt) p2 <<= 1;
    d.MT = p2;
    d.KB = (s.P == 4) ? 2 : 1;
    d.F = 32 * d.MT * d.KB;
    d.NPAIR = (d.MT + 1) / 2;
    d.NPL = d.MT * 16;
    int64_t bh, elems;
    if (!mul_ok(s.B, s.H, bh) || !mul_ok(bh, s.N, elems) || !mul_ok(elems, s.d, elems))
        return RACE_ERR_INVALID_ARG;
    if (elems > INT64_MAX / 8) return RACE_ERR_INVALID_ARG;
    d.BH = bh;
    d.NC = (s.N + s.chunk - 1) / s.chunk;
    d.F65 = (int64_t)d.F * 65;
    if (d.BH > 65535 || d.NC > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
    return RACE_OK;
}

inline CacheLayout cache_layout(const Shape& s, const Derived& d) {
    const size_t rows = (size_t)d.BH * (size_t)s.N;
    CacheLayout c;
    c.u = 0;
    c.inv = align256(rows * (size_t)d.NPL * sizeof(float));
    c.total = c.inv + align256(rows * sizeof(float));
    return c;
}

inline SavedLayout saved_layout(const Shape& s, const Derived& d) {
    const size_t per = (size_t)d.F65 * sizeof(float);
    const size_t states = s.causal ? (size_t)d.BH * (size_t)d.NC * per : (size_t)d.BH * per;
    const size_t cache = cache_layout(s, d).total;
    SavedLayout l;
    l.D = align256(states);
    l.q = l.D + align256((size_t)d.BH * (size_t)s.N * sizeof(float));
    l.k = l.q + cache;
    l.total = l.k + cache;
    return l;
}

inline size_t saved_bytes(const Shape& s, const Derived& d) { return saved_layout(s, d).total; }

// Segments of the chunk scan: one pass over the chunks when the grid of
// (state elements / 256) x heads already has enough workgroups to keep the
// memory busy; otherwise up to 16 segments of at least 64 chunks each,
// summed first and then scanned from their offsets (two launches).
inline int scan_segs(const Shape& s, const Derived& d) {
    if (!s.causal) return 1;
    const int64_t blocks = (d.F65 + 255) / 256 * d.BH;
    if (blocks >= 192) return 1;
    int64_t segs = (768 + blocks - 1) / blocks;
    if (segs > 16) segs = 16;
    if (segs > d.NC / 64) segs = d.NC / 64;
    return segs < 2 ? 1 : (int)segs;
}

inline WsLayout ws_layout(const Shape& s, const Derived& d, int kind) {
    WsLayout w{};
    const size_t per = (size_t)d.F65 * sizeof(float);
    const size_t chunks = (size_t)d.BH * (size_t)d.NC * per;
    const size_t totals = (size_t)d.BH * per;
    const size_t tokens = (size_t)d.BH * (size_t)s.N;
    size_t off = 0;
    if (kind != WS_BWD) {
        w.S = off;   off = align256(off + chunks);
        w.St = off;  off = align256(off + (s.causal ? 0 : totals));
    }
    if (kind == WS_FWD) {
        w.Kc = off;  off = align256(off + cache_layout(s, d).total);
    }
    if (kind == WS_BWD || kind == WS_BWD_RECOMPUTE) {
        w.wt = off;  off = align256(off + (size_t)d.NPAIR * 4 * 64 * 8 * sizeof(float));
        w.T = off;   off = align256(off + chunks);
        w.Tt = off;  off = align256(off + (s.causal ? 0 : totals));
        w.E = off;   off = align256(off + tokens * sizeof(float));
    }
    if (kind == WS_BWD_RECOMPUTE) {
        w.Sv = off;  off = align256(off + saved_bytes(s, d));
        w.Ov = off;  off = align256(off + tokens * (size_t)s.d * sizeof(float));
    }
    const int segs = scan_segs(s, d);
    w.scan = off;    off = align256(off + (segs > 1 ? (size_t)d.BH * (size_t)segs * per : 0));
    w.total = off;
    return w;
}

}  // namespace race
