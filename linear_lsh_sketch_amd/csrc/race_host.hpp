// Host-side shape validation and workspace layout (no device code).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cmath>
#include <initializer_list>

#include "race_attn.h"

namespace race {

struct Shape {
    int64_t B, H, N;
    int d, P, L;
    int causal, chunk;
    int w_per_head;   // W is [H, L, P, d] (head h of every batch uses W[h]) instead of [L, P, d]
};

// Tables are processed in groups of at most Lg (one launch per group and
// pass): every pass is linear in the features of the tables, so the groups'
// partial results add up, and only the forward's final division (and the
// normalisation's chain rule of the gradients) waits for the last group.
// Groups 0 .. G-2 hold Lg tables each; the last holds the rest. A group of
// n tables has MT = ceil(n P' / 16) rounded to a power of two projection
// tiles, F = 32 MT KB features and F * 65 floats per sketch state.
struct Derived {
    int Pp, KB;
    int G, Lg;     // number of table groups, tables per full group
    int MT, F, NPAIR;
    int NPL;       // projection rows per token (MT * 16)
    int64_t F65;   // floats per sketch state: F * 64 value sums + F masses
    int Ll, MTl, Fl, NPLl;   // the last group (equal to the full one when L % Lg == 0)
    int64_t F65l;
    int64_t F65all;          // all groups of one head (a chunk state's floats)
    int64_t RSall;           // the running state of one head, in floats: per group VH halves of
                             // F x 64 float32 value sums and F float64 masses (RW F floats)
    int RW;                  // 64 VH + 2
    int64_t BH, NC;
    // Head dimension 128: the sketch passes run once per half of the value
    // columns (64 each), on plane values computed beforehand from the whole
    // 128-dimensional rows; VH = 2 sets of sketch states. Otherwise VH = 1.
    int VH;
    int NDT;   // 16-column tiles of the back-projection operands: 8 at head dimension 128, else 4
};

// Largest number of table groups (launches per pass): L * 2^P <= 2^16 features.
constexpr int MAX_FEATURES = 1 << 16;

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
    size_t acc;    // more than one table group: partial outputs [rows][64], float32
    size_t accD;   // and the forward's partial denominators [rows]
    size_t Qc;     // head dimension 128, forward without saved: the queries' plane values
    size_t dhQ;    // head dimension 128, backward: gradients wrt the queries' and keys'
    size_t dhK;    // normalised projections, float32, laid out as the plane values
    size_t total;
};

// Plane values of one side (queries or keys): per table group g,
// u = tanh of the normalised projection [rows][NPL_g] (float16 for bf16
// inputs, float32 for float32; sized for float32, the upper bound), then
// 1 / max(|x|, eps) [rows] in float32 (shared by the groups).
struct CacheLayout {
    size_t u;       // group 0's plane values
    size_t ustep;   // bytes from one full group's plane values to the next
    size_t inv, total;
    size_t u_of(int g) const { return u + (size_t)g * ustep; }
};

// The saved buffer: sketch states in slots of F * 65 floats (float32, or the
// compact form for bf16 inputs; per chunk, causal; the total,
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
    if ((s.d != 64 && s.d != 32 && s.d != 128) || s.P > 6) return RACE_ERR_UNSUPPORTED;
    // in-chunk byte offsets (rows of up to 512 bytes) are 32-bit
    if (s.chunk > MAX_CHUNK) return RACE_ERR_UNSUPPORTED;
    // planes per table padded to 1, 2, 4 or 8 (P = 5, 6: two lane groups)
    d.Pp = s.P <= 2 ? s.P : (s.P <= 4 ? 4 : 8);
    if ((int64_t)s.L << s.P > MAX_FEATURES) return RACE_ERR_UNSUPPORTED;
    d.KB = s.P == 6 ? 4 : (s.P == 4 || s.P == 5) ? 2 : 1;
    // tables per group: P = 4, causal: up to 16 (four projection tiles, 256
    // features: the state fits two workgroups per CU, which pays more than the
    // partial outputs cost); P = 5, 6: 256 features (8 and 4 tables);
    // otherwise up to 128 projection rows (the non-causal passes have no
    // in-sub-block terms, so carrying partial outputs between groups costs
    // more than one workgroup per CU does)
    d.Lg = s.P == 6 ? 4 : s.P == 5 ? 8 : (s.P == 4 && s.causal) ? 16 : 128 / d.Pp;
    d.G = (s.L + d.Lg - 1) / d.Lg;
    const int Lfull = d.G > 1 ? d.Lg : s.L;
    d.Ll = s.L - (d.G - 1) * d.Lg;
    auto tiles = [&](int n) {
        const int mt = (n * d.Pp + 15) / 16;
        int p2 = 1;
        while (p2 < mt) p2 <<= 1;
        return p2;
    };
    d.MT = tiles(Lfull);
    d.F = 32 * d.MT * d.KB;
    d.NPAIR = (d.MT + 1) / 2;
    d.NPL = d.MT * 16;
    d.MTl = tiles(d.Ll);
    d.Fl = 32 * d.MTl * d.KB;
    d.NPLl = d.MTl * 16;
    int64_t bh, elems;
    if (!mul_ok(s.B, s.H, bh) || !mul_ok(bh, s.N, elems) || !mul_ok(elems, s.d, elems))
        return RACE_ERR_INVALID_ARG;
    if (elems > INT64_MAX / 8) return RACE_ERR_INVALID_ARG;
    d.BH = bh;
    d.NC = (s.N + s.chunk - 1) / s.chunk;
    d.F65 = (int64_t)d.F * 65;
    d.F65l = (int64_t)d.Fl * 65;
    d.F65all = (int64_t)(d.G - 1) * d.F65 + d.F65l;
    d.VH = s.d == 128 ? 2 : 1;
    d.RW = 64 * d.VH + 2;
    d.RSall = ((int64_t)(d.G - 1) * d.F + d.Fl) * d.RW;
    d.NDT = s.d == 128 ? 8 : 4;
    if (d.BH > 65535 || d.NC > 0x7fffffff) return RACE_ERR_UNSUPPORTED;
    return RACE_OK;
}

// Per-group view: tables [t0, t0 + L), MT projection tiles, F features.
struct Group {
    int g, t0, L, MT, F, NPL;
    int64_t F65;
};

inline Group group(const Derived& d, int g) {
    const bool last = g == d.G - 1;
    Group r;
    r.g = g;
    r.t0 = g * d.Lg;
    r.L = last ? d.Ll : d.Lg;
    r.MT = last ? d.MTl : d.MT;
    r.F = last ? d.Fl : d.F;
    r.NPL = last ? d.NPLl : d.NPL;
    r.F65 = last ? d.F65l : d.F65;
    return r;
}

inline CacheLayout cache_layout(const Shape& s, const Derived& d) {
    const size_t rows = (size_t)d.BH * (size_t)s.N;
    CacheLayout c;
    c.u = 0;
    c.ustep = align256(rows * (size_t)d.NPL * sizeof(float));
    c.inv = c.u_of(d.G - 1) + align256(rows * (size_t)d.NPLl * sizeof(float));
    c.total = c.inv + align256(rows * sizeof(float));
    return c;
}

// Sketch states of all groups, group-major: group g's array
// [BH][per_head][F65_g] starts after the full groups before it.
// per_head = chunks (per-chunk states) or 1 (whole-sequence totals).
inline size_t group_states_floats(const Derived& d, int64_t per_head, int g) {
    return (size_t)g * (size_t)d.BH * (size_t)per_head * (size_t)d.F65;
}
inline size_t all_states_bytes(const Derived& d, int64_t per_head) {
    return (group_states_floats(d, per_head, d.G - 1) + (size_t)d.BH * (size_t)per_head * (size_t)d.F65l) *
           sizeof(float);
}

// Sketch states of value half h (head dimension 128: two sets, one after the other).
inline size_t half_states_floats(const Derived& d, int64_t per_head, int h) {
    return (size_t)h * all_states_bytes(d, per_head) / sizeof(float);
}

inline SavedLayout saved_layout(const Shape& s, const Derived& d) {
    const size_t states = (size_t)d.VH * all_states_bytes(d, s.causal ? d.NC : 1);
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
// (state words / 256) x heads already has enough workgroups to keep the
// memory busy; otherwise up to 16 segments of at least 64 chunks each,
// summed first and then scanned from their offsets (two launches).
inline int scan_segs(const Shape& s, const Derived& d, int64_t nwords) {
    if (!s.causal) return 1;
    const int64_t blocks = (nwords + 255) / 256 * d.BH;
    if (blocks >= 192) return 1;
    int64_t segs = (768 + blocks - 1) / blocks;
    if (segs > 16) segs = 16;
    if (segs > d.NC / 64) segs = d.NC / 64;
    return segs < 2 ? 1 : (int)segs;
}

// Back-projection operand table of one group (k_prep), sized for float32.
inline size_t wt_bytes(const Derived& d) {
    return align256((size_t)d.NPAIR * (size_t)d.NDT * 64 * 8 * sizeof(float));
}

inline WsLayout ws_layout(const Shape& s, const Derived& d, int kind) {
    WsLayout w{};
    const size_t chunks = (size_t)d.VH * all_states_bytes(d, d.NC);
    const size_t totals = (size_t)d.VH * all_states_bytes(d, 1);
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
        w.wt = off;  off = align256(off + (size_t)d.G * (s.w_per_head ? (size_t)s.H : 1) * wt_bytes(d));
        w.T = off;   off = align256(off + chunks);
        w.Tt = off;  off = align256(off + (s.causal ? 0 : totals));
        w.E = off;   off = align256(off + tokens * sizeof(float));
    }
    if (kind == WS_BWD_RECOMPUTE) {
        w.Sv = off;  off = align256(off + saved_bytes(s, d));
        w.Ov = off;  off = align256(off + tokens * (size_t)s.d * sizeof(float));
    }
    // head dimension 128: the queries' plane values (the forward reads them
    // instead of projecting), and the per-plane gradients of both sides
    if (d.VH == 2) {
        if (kind == WS_FWD) {
            w.Qc = off;  off = align256(off + cache_layout(s, d).total);
        }
        if (kind == WS_BWD || kind == WS_BWD_RECOMPUTE) {
            w.dhQ = off; off = align256(off + cache_layout(s, d).total);
            w.dhK = off; off = align256(off + cache_layout(s, d).total);
        }
    }
    // partial outputs of the groups before the last: [rows][64] (the
    // kernels' working width, whatever the head dimension) and the forward's
    // partial denominators [rows], float32
    if (d.G > 1) {
        w.acc = off;  off = align256(off + tokens * (size_t)64 * sizeof(float));
        w.accD = off; off = align256(off + tokens * sizeof(float));
    }
    // segment sums of one group's scan at a time (the largest of the groups,
    // either state form: float32, F65 words, F65 floats per segment; compact,
    // 33 F + 64 words of which 32 F bf16 pairs, F65 + 64 floats per segment)
    size_t seg_bytes = 0;
    for (const int F : {d.F, d.Fl}) {
        const int64_t f65 = (int64_t)F * 65;
        const int64_t forms[2][2] = {{f65, f65}, {33 * (int64_t)F + 64, f65 + 64}};
        for (const auto& fm : forms) {
            const int segs = scan_segs(s, d, fm[0]);
            if (segs > 1) {
                const size_t b = (size_t)d.BH * (size_t)segs * (size_t)fm[1] * sizeof(float);
                if (b > seg_bytes) seg_bytes = b;
            }
        }
    }
    w.scan = off;
    off = align256(off + seg_bytes);
    w.total = off;
    return w;
}

}  // namespace race
