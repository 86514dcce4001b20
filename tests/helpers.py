"""Shared test helpers: seeded inputs (from synth) and error metrics."""
from __future__ import annotations

import numpy as np

import synth


def host_inputs(seed, B, H, N, d, P, L, dtype, dist="normal"):
    """Q, K, V, dO as host arrays in the library dtype (bf16 as uint16 bits)
    and W as the same dtype; returns a dict."""
    sh = (B, H, N, d)
    if dist == "mixture":
        Q = synth.mixture(seed, synth.TID_Q, synth.TID_QIDS, B * H * N, d, dtype).reshape(sh)
        K = synth.mixture(seed, synth.TID_K, synth.TID_KIDS, B * H * N, d, dtype).reshape(sh)
    else:
        Q = synth.normal(seed, synth.TID_Q, sh, dtype)
        K = synth.normal(seed, synth.TID_K, sh, dtype)
    V = synth.normal(seed, synth.TID_V, sh, dtype)
    dO = synth.normal(seed, synth.TID_DO, sh, dtype)
    W = synth.normal(seed, synth.TID_W, (L, P, d), dtype)
    return {"Q": Q, "K": K, "V": V, "dO": dO, "W": W}


def to_f64(a):
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def to_torch(a, device):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.copy()).to(device)


def from_torch(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))
