// Drives the host-side shape validation and buffer layouts of libraceattn
// (race_host.hpp: derive, group views, saved / cache / workspace layouts,
// scan segmentation) over valid, boundary and invalid shapes, for an
// AddressSanitizer / UndefinedBehaviorSanitizer build (tests/test_sanitizers.py).
// Exit status 0 when every layout is consistent.
#include <cstdio>

#include "race_host.hpp"

using namespace race;

static int check_shape(int64_t B, int64_t H, int64_t N, int d, int P, int L, int causal, int chunk, int& n_ok) {
    Shape s{B, H, N, d, P, L, causal, chunk};
    Derived dv{};
    const race_status_t rc = derive(s, dv);
    if (rc != RACE_OK) return 0;
    ++n_ok;
    int bad = 0;
    // groups tile the tables in order, each within the per-group limits
    int t = 0;
    int64_t f65 = 0;
    for (int g = 0; g < dv.G; ++g) {
        const Group gr = group(dv, g);
        bad |= gr.t0 != t || gr.L < 1 || gr.L > dv.Lg || gr.MT < 1 || gr.F != 32 * gr.MT * dv.KB;
        bad |= gr.F65 != (int64_t)gr.F * 65 || gr.F > 512;
        t += gr.L;
        f65 += gr.F65;
    }
    bad |= t != L || f65 != dv.F65all;
    const SavedLayout sl = saved_layout(s, dv);
    const CacheLayout cl = cache_layout(s, dv);
    bad |= !(sl.D <= sl.q && sl.q <= sl.k && sl.k + cl.total == sl.total);
    bad |= cl.u_of(dv.G - 1) >= cl.inv || cl.inv >= cl.total;
    for (int kind = WS_FWD; kind <= WS_FWD_SAVED; ++kind) {
        const WsLayout w = ws_layout(s, dv, kind);
        bad |= w.total < w.scan;
        if (kind == WS_BWD_RECOMPUTE) bad |= w.total < sl.total;
        // the group partials are addressed as [rows][64] float32 whatever d is
        if (dv.G > 1) bad |= w.accD < w.acc + (size_t)dv.BH * (size_t)N * 64 * sizeof(float);
        // head dimension 128: two sets of sketch states, the queries' plane
        // values (forward without saved) and the per-plane gradients of both sides
        if (dv.VH == 2 && kind == WS_FWD) bad |= w.Qc < w.Kc + cl.total || w.total < w.Qc + cl.total;
        if (dv.VH == 2 && (kind == WS_BWD || kind == WS_BWD_RECOMPUTE))
            bad |= w.dhQ < w.E || w.dhK < w.dhQ + cl.total || w.total < w.dhK + cl.total;
    }
    if (dv.VH == 2) bad |= sl.D < 2 * all_states_bytes(dv, causal ? dv.NC : 1);
    for (int g = 0; g < dv.G; ++g) {
        const int segs = scan_segs(s, dv, group(dv, g).F65);
        bad |= segs < 1 || segs > 16;
    }
    return bad;
}

int main() {
    int bad = 0, n_ok = 0, n_all = 0;
    const int64_t Ns[] = {1, 2, 63, 64, 65, 1000, 1 << 20, 12000000, 75000000};
    const int chunks[] = {1, 7, 64, 256, 1024, 2048, 1 << 20, (1 << 20) + 1, 0, -3};
    const int Ls[] = {1, 3, 4, 5, 8, 13, 16, 17, 31, 32, 33, 40, 64, 65, 100, 128, 129, 4096, 4097, 0, -1};
    for (int64_t N : Ns)
        for (int chunk : chunks)
            for (int P = -1; P <= 8; ++P)
                for (int L : Ls)
                    for (int causal = 0; causal < 2; ++causal) {
                        ++n_all;
                        bad |= check_shape(2, 3, N, 64, P, L, causal, chunk, n_ok);
                    }
    // sizes whose products overflow, and head dims other than 64
    const int64_t big[][3] = {{1ll << 40, 1ll << 20, 1ll << 20}, {1, 70000, 10}, {INT64_MAX, 1, 1}, {1, 1, INT64_MAX}};
    for (auto& b : big) bad |= check_shape(b[0], b[1], b[2], 64, 4, 8, 1, 16, n_ok);
    for (int d : {0, 32, 63, 65, 128}) bad |= check_shape(1, 1, 10, d, 4, 8, 1, 16, n_ok);
    for (int P : {4, 5}) bad |= check_shape(2, 2, 500, 32, P, 40, 1, 128, n_ok);   // d = 32 with table groups
    for (int P : {2, 4, 5})
        for (int causal = 0; causal < 2; ++causal)
            bad |= check_shape(2, 2, 500, 128, P, 40, causal, 128, n_ok);   // d = 128, table groups
    std::printf("host driver: %d of %d shapes valid, %s\n", n_ok, n_all, bad ? "FAILED" : "ok");
    return bad ? 1 : 0;
}
