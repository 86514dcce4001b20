"""Full-size GPU checks in the benchmark's launch configuration.

The 12M-token (B1 H4, L16 P4, chunk 1024) and 75M-token (B1 H1, L8 P4,
chunk 2048) causal workloads run at their real shapes through the C ABI.
Against the oracle, on outputs it can compute exactly:

* forward O on a sample of the first 65,536 tokens of every head (a causal
  output depends only on its prefix);
* backward with dO kept on those first 65,536 tokens and zero after them: then
  dQ, dK, dV of the prefix depend only on the prefix, and every later
  gradient row is exactly zero.

Properties that hold at any size: finiteness everywhere, bitwise run-to-run
determinism of the whole backward, agreement between two chunk sizes on late
tokens, and hard-hash ids on sampled rows.
"""
import json
import os

import numpy as np
import pytest

import synth
from helpers import from_torch, rel_l2, to_f64
from oracle import stream as oracle
from synth.workloads import BY_NAME

pytestmark = pytest.mark.gpu

PREFIX = 65536
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _checksum(t):
    import torch
    v = t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    return int(v.to(torch.int64).sum().item()), int((v.to(torch.int64) * 7919 % 65521).sum().item())


def _host_prefix(w, tid, n):
    """The first n tokens of every head, from the host generator (bit-identical
    to the device generator)."""
    out = np.empty((w.B, w.H, n, w.d), np.uint16)
    for b in range(w.B):
        for h in range(w.H):
            out[b, h] = synth.normal(w.seed, tid, (n, w.d), "bf16", start=((b * w.H + h) * w.N) * w.d)
    return out


@pytest.mark.parametrize("name", ["causal_long_n12M", "causal_extreme_n75M"])
def test_fullsize_causal(name):
    import torch
    import linear_lsh_sketch_amd as race

    w = BY_NAME[name]
    print(f"[fullsize] {name} B{w.B} H{w.H} N{w.N} L{w.L} P{w.P} chunk{w.chunk}", flush=True)
    dev = torch.device("cuda:0")
    shape = (w.B, w.H, w.N, w.d)
    T = {}
    for k, tid in (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO)):
        T[k] = synth.normal_device(w.seed, tid, torch.empty(shape, dtype=torch.bfloat16, device=dev))
    Wd = synth.normal_device(w.seed, synth.TID_W, torch.empty((w.L, w.P, w.d), dtype=torch.bfloat16, device=dev))
    # keep dO only on the prefix
    T["dO"][:, :, PREFIX:, :] = 0
    saved = race.alloc_saved(w.B, w.H, w.N, w.P, w.L, True, w.chunk, dev)
    O = race.forward(T["Q"], T["K"], T["V"], Wd, w.P, w.L, 1.0, True, w.chunk, saved=saved)
    dQ, dK, dV = race.backward(T["Q"], T["K"], T["V"], Wd, T["dO"], w.P, w.L, 1.0, True, w.chunk, O=O,
                               saved=saved)
    torch.cuda.synchronize()
    for t, nm in ((O, "O"), (dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        assert bool(torch.isfinite(t).all()), nm
    # later gradient rows are exactly zero
    for t, nm in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        assert int(torch.count_nonzero(t[:, :, PREFIX:, :]).item()) == 0, nm
    print(f"[fullsize] peak HBM {torch.cuda.max_memory_allocated() / 2**30:.1f} GiB", flush=True)

    # oracle on the prefix
    host = {k: _host_prefix(w, tid, PREFIX) for k, tid in
            (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO))}
    W64 = to_f64(synth.normal(w.seed, synth.TID_W, (w.L, w.P, w.d), "bf16"))
    sample = np.unique(np.concatenate([np.arange(0, PREFIX, 97), np.arange(PREFIX - 64, PREFIX)]))
    refO = oracle.forward(host["Q"], host["K"], host["V"], W64, 1.0, True, sample=sample)
    rdQ, rdK, rdV = oracle.backward(host["Q"], host["K"], host["V"], W64, host["dO"], 1.0, True, sample=sample)
    idx = torch.from_numpy(sample).to(dev)
    got = {k: from_torch(t.index_select(2, idx)) for k, t in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV))}
    errs = {"O": rel_l2(got["O"], refO), "dQ": rel_l2(got["dQ"], rdQ), "dK": rel_l2(got["dK"], rdK),
            "dV": rel_l2(got["dV"], rdV)}
    print("[fullsize] prefix rel_l2", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)

    # determinism of the whole backward (random dO everywhere)
    synth.normal_device(w.seed, synth.TID_DO, T["dO"])
    race.backward(T["Q"], T["K"], T["V"], Wd, T["dO"], w.P, w.L, 1.0, True, w.chunk, O=O, saved=saved,
                  grads=(dQ, dK, dV))
    torch.cuda.synchronize()
    c1 = [_checksum(t) for t in (dQ, dK, dV)]
    assert all(bool(torch.isfinite(t).all()) for t in (dQ, dK, dV))
    race.backward(T["Q"], T["K"], T["V"], Wd, T["dO"], w.P, w.L, 1.0, True, w.chunk, O=O, saved=saved,
                  grads=(dQ, dK, dV))
    torch.cuda.synchronize()
    assert c1 == [_checksum(t) for t in (dQ, dK, dV)]

    # a second chunk size agrees on late tokens (exercises the long scans)
    late = torch.arange(w.N - 4096, w.N, 37, device=dev)
    O1 = O.index_select(2, late).float()
    del saved
    O2 = race.forward(T["Q"], T["K"], T["V"], Wd, w.P, w.L, 1.0, True, 4 * w.chunk, out=O)
    torch.cuda.synchronize()
    d = rel_l2(O2.index_select(2, late).float().cpu().numpy(), O1.cpu().numpy())
    print(f"[fullsize] chunk {w.chunk} vs {4 * w.chunk} on late tokens: rel {d:.2e}", flush=True)
    assert d < 2e-2

    # late tokens against the oracle's full-sequence goldens: dO kept on the
    # last 4,096 tokens only (written by tests/golden/make_fullsize.py, which
    # streams the float64 oracle over the whole sequence of the heads it keeps)
    gold_path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if os.path.exists(gold_path):
        g = np.load(gold_path, allow_pickle=False)
        meta = json.loads(str(g["meta"]))
        win = int(meta["window"])
        synth.normal_device(w.seed, synth.TID_DO, T["dO"])
        T["dO"][:, :, : w.N - win, :] = 0
        saved = race.alloc_saved(w.B, w.H, w.N, w.P, w.L, True, w.chunk, dev)
        race.forward(T["Q"], T["K"], T["V"], Wd, w.P, w.L, 1.0, True, w.chunk, out=O, saved=saved)
        race.backward(T["Q"], T["K"], T["V"], Wd, T["dO"], w.P, w.L, 1.0, True, w.chunk, O=O, saved=saved,
                      grads=(dQ, dK, dV))
        torch.cuda.synchronize()
        del saved
        idx = torch.from_numpy(g["sample"]).to(dev)
        heads = [int(h) for h in g["heads"]]
        errs = {}
        for k, t in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
            got = from_torch(t[0].index_select(1, idx)[heads])   # B = 1: [heads, sample, d]
            errs[k] = rel_l2(got, g[k])
        print(f"[fullsize] late tokens (last {win}, heads {heads}) vs oracle goldens rel_l2",
              {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        for k, e in errs.items():
            assert e <= 2e-2, (k, e)
    else:
        print(f"[fullsize] no golden file {gold_path}", flush=True)

    # hard-hash ids on sampled rows
    ids, nz = race.hard_hash(T["Q"], Wd, w.P, w.L)
    torch.cuda.synchronize()
    rows = torch.arange(0, PREFIX, 101, device=dev)
    got_ids = ids.index_select(2, rows).cpu().numpy()
    ref_ids, _ = oracle.hard_hash(host["Q"][:, :, rows.cpu().numpy(), :], W64)
    mism = got_ids != ref_ids
    if mism.any():
        Xh = to_f64(host["Q"][:, :, rows.cpu().numpy(), :])
        Xh = Xh / np.linalg.norm(Xh, axis=-1, keepdims=True)
        h = np.einsum("bhnd,lpd->bhnlp", Xh, W64)
        assert np.all(np.min(np.abs(h), axis=-1)[mism] < 1e-5)
    print(f"[fullsize] hash near-zero projections over the whole tensor: {int(nz.item())}", flush=True)
    del T, O, dQ, dK, dV, ids
    torch.cuda.empty_cache()


def _host_heads(w, tid, heads):
    """Whole sequences of the given (flattened batch, head) indices from the
    host generator."""
    out = np.empty((len(heads), w.N, w.d), np.uint16)
    for i, bh in enumerate(heads):
        if w.qk_dist == "mixture" and tid in (synth.TID_Q, synth.TID_K):
            ids = synth.TID_QIDS if tid == synth.TID_Q else synth.TID_KIDS
            out[i] = synth.mixture(w.seed, tid, ids, w.N, w.d, "bf16", row0=bh * w.N)
        else:
            out[i] = synth.normal(w.seed, tid, (w.N, w.d), "bf16", start=bh * w.N * w.d)
    return out


@pytest.mark.parametrize("name", ["noncausal_encoder_n4096", "causal_lm_n32768_mixture"])
def test_fullsize_multihead(name):
    """The two multi-head workloads at their full B x H in the benchmark's
    launch configuration; the first, a middle and the last (batch, head)
    sequences against the oracle over every token."""
    import torch
    import linear_lsh_sketch_amd as race

    w = BY_NAME[name]
    print(f"[fullsize] {name} B{w.B} H{w.H} N{w.N} L{w.L} P{w.P} chunk{w.chunk} causal={w.causal}", flush=True)
    dev = torch.device("cuda:0")
    shape = (w.B, w.H, w.N, w.d)
    T = {}
    for k, tid in (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO)):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        if w.qk_dist == "mixture" and k in ("Q", "K"):
            synth.mixture_device(w.seed, tid, synth.TID_QIDS if k == "Q" else synth.TID_KIDS, t)
        else:
            synth.normal_device(w.seed, tid, t)
        T[k] = t
    Wd = synth.normal_device(w.seed, synth.TID_W, torch.empty((w.L, w.P, w.d), dtype=torch.bfloat16, device=dev))
    saved = race.alloc_saved(w.B, w.H, w.N, w.P, w.L, w.causal, w.chunk, dev)
    O = race.forward(T["Q"], T["K"], T["V"], Wd, w.P, w.L, w.beta, w.causal, w.chunk, saved=saved)
    dQ, dK, dV = race.backward(T["Q"], T["K"], T["V"], Wd, T["dO"], w.P, w.L, w.beta, w.causal, w.chunk, O=O,
                               saved=saved)
    torch.cuda.synchronize()
    for t, nm in ((O, "O"), (dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        assert bool(torch.isfinite(t).all()), nm
    BH = w.B * w.H
    heads = [0, BH // 2, BH - 1]
    host = {k: _host_heads(w, tid, heads) for k, tid in
            (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO))}
    W64 = to_f64(synth.normal(w.seed, synth.TID_W, (w.L, w.P, w.d), "bf16"))
    ref = {"O": oracle.forward(host["Q"], host["K"], host["V"], W64, w.beta, w.causal)}
    ref["dQ"], ref["dK"], ref["dV"] = oracle.backward(host["Q"], host["K"], host["V"], W64, host["dO"], w.beta,
                                                      w.causal)
    hidx = torch.tensor(heads, device=dev)
    errs = {}
    for k, t in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
        got = from_torch(t.reshape(BH, w.N, w.d).index_select(0, hidx))
        errs[k] = rel_l2(got, ref[k])
    print(f"[fullsize] heads {heads} of {BH} vs oracle rel_l2", {k: f"{v:.2e}" for k, v in errs.items()},
          flush=True)
    for k, e in errs.items():
        assert e <= 2e-2, (k, e)
