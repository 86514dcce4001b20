"""The RACE multi-head attention block (linear_lsh_sketch_amd.mha) on the GPU:
its gradients against a float64 CPU reference whose attention core is the
oracle, a synthetic language-model loss that can only fall if attention
carries information from the first token to every later one, and
incremental decoding (prompt, then a few tokens at a time) against the full
forward.
"""
import math

import numpy as np
import pytest

from helpers import rel_l2
from oracle import dense

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mha():
    import torch
    import linear_lsh_sketch_amd as race
    from linear_lsh_sketch_amd import mha as mha_mod
    assert torch.cuda.is_available()
    race.lib()
    return mha_mod


def oracle_core():
    import torch

    class OracleCore(torch.autograd.Function):
        """RACE core in float64 on the CPU through the oracle (forward and its
        exact backward), [B, H, N, 64] tensors."""

        @staticmethod
        def forward(ctx, Q, K, V, W, beta, causal):
            ctx.save_for_backward(Q, K, V, W)
            ctx.beta, ctx.causal = beta, causal
            O = dense.forward_batched(Q.numpy(), K.numpy(), V.numpy(), W.numpy(), beta, causal)
            return torch.from_numpy(O)

        @staticmethod
        def backward(ctx, dO):
            Q, K, V, W = ctx.saved_tensors
            g = dense.backward_batched(Q.numpy(), K.numpy(), V.numpy(), W.numpy(), dO.numpy(), ctx.beta,
                                       ctx.causal)
            return tuple(torch.from_numpy(x) for x in g) + (None, None, None)

    return OracleCore


@pytest.mark.parametrize("causal,hd", [(True, 64), (False, 64), (True, 128), (False, 32)])
def test_mha_block_gradients_match_float64_reference(mha, causal, hd):
    """Float32 block on the GPU (projections in the BLAS library, core in the
    library's kernels) against the same block in float64 on the CPU with the
    oracle as its core: output, input gradient and the four projection
    weights' gradients; head dimensions 64, 128 and 32."""
    import torch
    B, N, D, P, L, chunk, beta = 2, 150, 2 * hd, 4, 8, 64, 1.3
    print(f"[case] mha grads causal={causal} B={B} N={N} D={D} head_dim={hd} P={P} L={L} chunk={chunk}",
          flush=True)
    torch.manual_seed(3)
    dev = torch.device("cuda:0")
    blk = mha.RaceMHA(D, P, L, beta, causal, chunk, seed=5, device=dev, dtype=torch.float32, head_dim=hd)
    x = torch.randn(B, N, D)
    g = torch.randn(B, N, D)
    xg = x.to(dev).requires_grad_(True)
    out = blk(xg)
    (out * g.to(dev)).sum().backward()
    torch.cuda.synchronize()

    # float64 reference with the same weights
    Core = oracle_core()
    ws = {n: getattr(blk, n).weight.detach().cpu().double().requires_grad_(True) for n in ("wq", "wk", "wv", "wo")}
    planes = blk.planes.detach().cpu().double()
    xr = x.double().requires_grad_(True)

    def split(t):
        return t.view(B, N, blk.heads, hd).transpose(1, 2).contiguous()

    q, k, v = (split(xr @ ws[n].T) for n in ("wq", "wk", "wv"))
    o = Core.apply(q, k, v, planes, beta, causal)
    ref = o.transpose(1, 2).reshape(B, N, D) @ ws["wo"].T
    (ref * g.double()).sum().backward()

    errs = {"out": rel_l2(out.detach().cpu().double().numpy(), ref.detach().numpy()),
            "dx": rel_l2(xg.grad.cpu().double().numpy(), xr.grad.numpy())}
    for n in ("wq", "wk", "wv", "wo"):
        errs[n] = rel_l2(getattr(blk, n).weight.grad.cpu().double().numpy(), ws[n].grad.numpy())
    print("   rel_l2", {k_: f"{v_:.1e}" for k_, v_ in errs.items()}, flush=True)
    for k_, v_ in errs.items():
        assert v_ <= 1e-4, (k_, v_)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mha_language_model_loss_falls(mha, dtype):
    """A one-layer causal language model (embedding, RACE attention block with
    a residual, linear head) on synthetic sequences: the first token is one of
    8 markers, the rest are random filler tokens, and every later position
    must predict the marker. Without attention the best loss is ln 8; after
    150 Adam steps it must be far below (the block has learned to route the
    first token's value to every query)."""
    import torch
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    vocab, markers, D, N, B, P, L, chunk = 40, 8, 128, 128, 8, 4, 16, 32
    print(f"[case] mha lm {dtype} N={N} B={B} D={D} chunk={chunk}", flush=True)
    torch.manual_seed(0)
    emb = torch.nn.Embedding(vocab, D).to(dev, dt)
    blk = mha.RaceMHA(D, P, L, 1.0, True, chunk, seed=1, device=dev, dtype=dt)
    head = torch.nn.Linear(D, markers).to(dev, dt)
    params = [*emb.parameters(), *blk.parameters(), *head.parameters()]
    opt = torch.optim.Adam(params, lr=3e-3)
    gen = torch.Generator().manual_seed(7)
    losses = []
    for step in range(150):
        x = torch.randint(markers, vocab, (B, N), generator=gen)
        m = torch.randint(0, markers, (B,), generator=gen)
        x[:, 0] = m
        x, y = x.to(dev), m.to(dev)[:, None].expand(B, N - 1)
        h = emb(x)
        logits = head(h + blk(h))
        loss = torch.nn.functional.cross_entropy(logits[:, 1:].float().reshape(-1, markers), y.reshape(-1))
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
        assert math.isfinite(losses[-1]), step
    first, last = np.mean(losses[:5]), np.mean(losses[-10:])
    print(f"   loss {first:.3f} -> {last:.3f} (ln 8 = {math.log(8):.3f})", flush=True)
    assert last < 0.3 * math.log(8), (first, last)


@pytest.mark.parametrize("dtype,hd", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_mha_incremental_decoding_matches_full_forward(mha, dtype, hd):
    """Generation with the block: a prompt through ``prefill``, then pieces of
    1, 3 and 1 tokens through ``step``, give the rows of the full causal
    forward of the whole sequence (the sketch stands in for the key-value
    cache)."""
    import torch
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    B, n0, D = 2, 300, 2 * hd
    torch.manual_seed(11)
    blk = mha.RaceMHA(D, 4, 16, 1.0, True, 64, seed=2, device=dev, dtype=dt, head_dim=hd)
    x = torch.randn(B, n0 + 5, D, device=dev).to(dt)
    with torch.no_grad():
        full = blk(x).float()
    out0, state = blk.prefill(x[:, :n0])
    pieces = [out0.float()]
    pos = n0
    for T in (1, 3, 1):
        pieces.append(blk.step(x[:, pos:pos + T].contiguous(), state).float())
        pos += T
    got = torch.cat(pieces, dim=1)
    torch.cuda.synchronize()
    err = float((got - full).norm() / full.norm())
    print(f"[case] mha incremental {dtype} head_dim={hd}: rel_l2 {err:.1e}", flush=True)
    assert err <= (1e-5 if dtype == "f32" else 1e-2), err
    assert torch.equal(blk.empty_state(B), torch.zeros_like(state))
