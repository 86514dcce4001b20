"""A multi-head attention block around the RACE core (PyTorch module).

The RACE Attention layer replaces softmax attention inside a standard
multi-head block: queries, keys and values are linear projections of the
input, every head attends with RACE, and an output projection mixes the
heads (the pages evaluate it in place of softmax attention in language
models, masked language models and classifiers: Japanese gist.science page,
section 4.1; Italian technical summary, section 4). The four projections are
plain dense GEMMs (torch.nn.Linear, i.e. the ROCm BLAS libraries); the
attention core, forward and backward, runs in libraceattn's kernels through
``RaceAttnFunction``. The hyperplanes W are a fixed random buffer, not
trained (randomised projections: fugumt.com page, English abstract).
"""
from __future__ import annotations

import torch

from . import (WS_BWD, WS_FWD_SAVED, alloc_saved, alloc_state, alloc_workspace, race_attn_bwd, race_attn_decode,
               race_attn_fwd, race_attn_prefill)

HEAD_DIM = 64          # default head dimension (32, 64 and 128 are supported)


class RaceAttnFunction(torch.autograd.Function):
    """O = RACE-attention(Q, K, V) with the exact gradient of the kernels'
    forward. Q, K, V: [B, H, N, d] contiguous (d = 32, 64 or 128), one dtype
    (bf16 or float32); W: [L, P, d]. The forward keeps the sketch states,
    denominators and plane values (`saved`) for the backward, which takes
    them with O."""

    @staticmethod
    def forward(ctx, Q, K, V, W, P, L, temperature, causal, chunk):
        Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
        B, H, N, d = Q.shape
        saved = alloc_saved(B, H, N, P, L, causal, chunk, Q.device, d)
        ws = alloc_workspace(B, H, N, P, L, causal, chunk, WS_FWD_SAVED, Q.device, d)
        O = race_attn_fwd(Q, K, V, W, P, L, temperature, causal, chunk, saved=saved, ws=ws)
        ctx.save_for_backward(Q, K, V, W, O)
        ctx.saved_buf = saved
        ctx.cfg = (P, L, temperature, causal, chunk)
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, W, O = ctx.saved_tensors
        P, L, temperature, causal, chunk = ctx.cfg
        B, H, N, d = Q.shape
        ws = alloc_workspace(B, H, N, P, L, causal, chunk, WS_BWD, Q.device, d)
        dQ, dK, dV = race_attn_bwd(Q, K, V, W, dO.contiguous(), P, L, temperature, causal, chunk, O=O,
                                   saved=ctx.saved_buf, ws=ws)
        ctx.saved_buf = None
        return dQ, dK, dV, None, None, None, None, None, None


def race_attention(Q, K, V, W, P, L, temperature=1.0, causal=True, chunk=1024):
    """Differentiable RACE attention of [B, H, N, d] tensors."""
    return RaceAttnFunction.apply(Q, K, V, W, P, L, temperature, causal, chunk)


class RaceMHA(torch.nn.Module):
    """Multi-head attention with the RACE core: x [B, N, d_model] ->
    [B, N, d_model], d_model = heads * head_dim (head_dim 32, 64 or 128),
    bias-free projections."""

    def __init__(self, d_model: int, P: int = 4, L: int = 16, temperature: float = 1.0, causal: bool = True,
                 chunk: int = 1024, seed: int = 0, device=None, dtype=None, head_dim: int = HEAD_DIM):
        super().__init__()
        if head_dim not in (32, 64, 128):
            raise ValueError("head_dim must be 32, 64 or 128")
        if d_model % head_dim:
            raise ValueError(f"d_model must be a multiple of {head_dim}")
        self.head_dim = head_dim
        self.heads = d_model // head_dim
        self.P, self.L, self.temperature, self.causal, self.chunk = P, L, temperature, causal, chunk
        kw = {"device": device, "dtype": dtype}
        self.wq = torch.nn.Linear(d_model, d_model, bias=False, **kw)
        self.wk = torch.nn.Linear(d_model, d_model, bias=False, **kw)
        self.wv = torch.nn.Linear(d_model, d_model, bias=False, **kw)
        self.wo = torch.nn.Linear(d_model, d_model, bias=False, **kw)
        gen = torch.Generator().manual_seed(seed)
        planes = torch.randn((L, P, head_dim), generator=gen, dtype=torch.float32)
        self.register_buffer("planes", planes.to(device=device, dtype=dtype or torch.float32))

    def split(self, t):
        B, N, _ = t.shape
        return t.view(B, N, self.heads, self.head_dim).transpose(1, 2).contiguous()

    def forward(self, x):
        B, N, D = x.shape
        q, k, v = self.split(self.wq(x)), self.split(self.wk(x)), self.split(self.wv(x))
        o = race_attention(q, k, v, self.planes, self.P, self.L, self.temperature, self.causal, self.chunk)
        return self.wo(o.transpose(1, 2).reshape(B, N, D))

    # --- incremental decoding (causal blocks, no autograd) -------------------
    # The running sketch of every head replaces the key-value cache: its size
    # does not grow with the sequence.

    @torch.no_grad()
    def prefill(self, x):
        """Causal outputs of a prompt x [B, N, d_model] and the running state
        after it (pass the state to ``step``)."""
        if not self.causal:
            raise ValueError("incremental decoding needs a causal block")
        B, N, D = x.shape
        q, k, v = self.split(self.wq(x)), self.split(self.wk(x)), self.split(self.wv(x))
        o = race_attn_fwd(q, k, v, self.planes, self.P, self.L, self.temperature, True, self.chunk)
        state = race_attn_prefill(k, v, self.planes, self.P, self.L, self.temperature, self.chunk)
        return self.wo(o.transpose(1, 2).reshape(B, N, D)), state

    @torch.no_grad()
    def empty_state(self, batch: int):
        """The running state of sequences with no tokens yet."""
        return alloc_state(batch, self.heads, self.P, self.L, self.planes.device, self.head_dim)

    @torch.no_grad()
    def step(self, x, state):
        """Outputs of T new tokens x [B, T, d_model] that continue the
        sequences of `state` (updated in place), each attending causally to
        everything before it and to itself."""
        if not self.causal:
            raise ValueError("incremental decoding needs a causal block")
        B, T, D = x.shape
        q, k, v = self.split(self.wq(x)), self.split(self.wk(x)), self.split(self.wv(x))
        o = race_attn_decode(q, k, v, self.planes, state, self.P, self.L, self.temperature)
        return self.wo(o.transpose(1, 2).reshape(B, T, D))
