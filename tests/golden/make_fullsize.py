"""Write the full-size late-token goldens from the float64 CPU oracle.

For the two long causal workloads (12M tokens, B1 H4 L16 P4; 75M tokens,
B1 H1 L8 P4), this streams the oracle (``oracle/race_oracle.c``, a plain
per-token recurrence) over the whole sequence of the chosen heads and keeps:

* O at sampled late tokens (every 37th of the last 4,096, and the last token);
* dQ, dK, dV at the same tokens, for an upstream gradient dO that is the
  seeded normal draw on the last 4,096 tokens and zero before them (so the
  key-side gradients of late tokens depend only on that window, while their
  forward states and the query-side gradients depend on the whole prefix).

Inputs are the seeded synthetic tensors of ``synth`` (the same streams the GPU
tests generate on the device). Nothing here touches the GPU library: the only
arithmetic is the oracle's. The arrays are staged in memory-mapped files in a
scratch directory (deleted at the end) so that the 75M-token inputs (38 GB)
do not have to sit in anonymous memory.

Run from the repository root:  python tests/golden/make_fullsize.py [names...]
"""
from __future__ import annotations

import hashlib
import json
import os
import shutil
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import stream as oracle  # noqa: E402
from synth.workloads import BY_NAME  # noqa: E402

WINDOW = 4096
STRIDE = 37
HEADS = {"causal_long_n12M": (0, 3), "causal_extreme_n75M": (0,)}
PIECE = 1 << 24   # elements generated per call


def late_sample(N: int) -> np.ndarray:
    return np.unique(np.concatenate([np.arange(N - WINDOW, N, STRIDE), [N - 1]])).astype(np.int64)


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}.npz")


def _oracle_digest() -> str:
    with open(os.path.join(ROOT, "oracle", "race_oracle.c"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _fill(mm: np.ndarray, seed: int, tid: int, heads, w) -> None:
    """mm: [len(heads), N, d] uint16 memmap; head h of the workload tensor."""
    n = w.N * w.d
    for i, h in enumerate(heads):
        flat = mm[i].reshape(-1)
        start = h * n   # B = 1: flat index of head h
        for p0 in range(0, n, PIECE):
            p1 = min(n, p0 + PIECE)
            flat[p0:p1] = synth.normal(seed, tid, (p1 - p0,), "bf16", start=start + p0)


def make(name: str, scratch: str) -> str:
    w = BY_NAME[name]
    assert w.B == 1 and w.causal and w.dtype == "bf16"
    heads = HEADS[name]
    os.makedirs(scratch, exist_ok=True)
    shape = (len(heads), w.N, w.d)
    arrs = {}
    t0 = time.time()
    for k, tid in (("Q", synth.TID_Q), ("K", synth.TID_K), ("V", synth.TID_V), ("dO", synth.TID_DO)):
        arrs[k] = np.lib.format.open_memmap(os.path.join(scratch, f"{name}_{k}.npy"), mode="w+",
                                            dtype=np.uint16, shape=shape)
        _fill(arrs[k], w.seed, tid, heads, w)
    arrs["dO"][:, : w.N - WINDOW, :] = 0
    for a in arrs.values():
        a.flush()
    W64 = synth.bf16_bits_to_f64(synth.normal(w.seed, synth.TID_W, (w.L, w.P, w.d), "bf16"))
    print(f"[{name}] inputs ready in {time.time() - t0:.0f} s", flush=True)
    sample = late_sample(w.N)
    t1 = time.time()
    O = oracle.forward(arrs["Q"], arrs["K"], arrs["V"], W64, w.beta, True, sample=sample)
    print(f"[{name}] forward {time.time() - t1:.0f} s", flush=True)
    t2 = time.time()
    dQ, dK, dV = oracle.backward(arrs["Q"], arrs["K"], arrs["V"], W64, arrs["dO"], w.beta, True, sample=sample)
    print(f"[{name}] backward {time.time() - t2:.0f} s", flush=True)
    meta = {"workload": w.as_dict(), "heads": list(heads), "window": WINDOW, "stride": STRIDE,
            "oracle_sha256": _oracle_digest(), "oracle_seconds": round(time.time() - t1, 1)}
    out = golden_path(name)
    np.savez_compressed(out, O=O, dQ=dQ, dK=dK, dV=dV, sample=sample, heads=np.array(heads, np.int64),
                        meta=np.array(json.dumps(meta)))
    del arrs
    print(f"[{name}] wrote {out}", flush=True)
    return out


def main(argv) -> None:
    names = argv or list(HEADS)
    scratch = os.path.join(ROOT, "_work", "golden_tmp")
    oracle.build(force=False)
    for nm in names:
        try:
            make(nm, os.path.join(scratch, nm))
        finally:
            shutil.rmtree(os.path.join(scratch, nm), ignore_errors=True)


if __name__ == "__main__":
    main(sys.argv[1:])
