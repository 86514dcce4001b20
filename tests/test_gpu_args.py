"""Every entry point of the binding rejects mismatched outputs and short
buffers before the C call (the C ABI takes no sizes for O, dQ, dK, dV or
saved, so the binding checks them). No kernel runs in these tests."""
import pytest

import linear_lsh_sketch_amd as race

pytestmark = pytest.mark.gpu


def _inputs(dtype):
    import torch
    dev = torch.device("cuda:0")
    B, H, N, d, P, L = 1, 2, 70, 64, 4, 5
    Q, K, V, dO = (torch.zeros((B, H, N, d), dtype=dtype, device=dev) for _ in range(4))
    W = torch.zeros((L, P, d), dtype=dtype, device=dev)
    return dev, (B, H, N, d, P, L), Q, K, V, dO, W


@pytest.mark.parametrize("causal", [False, True])
def test_forward_rejects_bad_out_saved_ws(causal):
    import torch
    dev, (B, H, N, d, P, L), Q, K, V, dO, W = _inputs(torch.float32)
    chunk = 32
    with pytest.raises(ValueError, match="out"):
        race.forward(Q, K, V, W, P, L, 1.0, causal, chunk, out=torch.empty_like(Q, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        race.forward(Q, K, V, W, P, L, 1.0, causal, chunk, out=Q[:, :, :-1].contiguous())
    nsv = race.saved_bytes(B, H, N, d, P, L, causal, chunk)
    with pytest.raises(ValueError, match="saved"):
        race.forward(Q, K, V, W, P, L, 1.0, causal, chunk, saved=torch.empty(nsv - 1, dtype=torch.uint8, device=dev))
    nws = race.workspace_bytes(B, H, N, d, P, L, causal, chunk, race.WS_FWD)
    with pytest.raises(ValueError, match="ws"):
        race.forward(Q, K, V, W, P, L, 1.0, causal, chunk, ws=torch.empty(nws - 1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="ws"):
        race.forward(Q, K, V, W, P, L, 1.0, causal, chunk,
                     ws=torch.empty(nws, dtype=torch.uint8, device="cpu"))


def test_backward_rejects_bad_grads_and_buffers():
    import torch
    dev, (B, H, N, d, P, L), Q, K, V, dO, W = _inputs(torch.float32)
    chunk = 32
    good = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    for i in range(3):
        g = list(good)
        g[i] = torch.empty_like(Q, dtype=torch.bfloat16)
        with pytest.raises(ValueError):
            race.backward(Q, K, V, W, dO, P, L, 1.0, True, chunk, grads=tuple(g))
    nsv = race.saved_bytes(B, H, N, d, P, L, True, chunk)
    with pytest.raises(ValueError, match="saved"):
        race.backward(Q, K, V, W, dO, P, L, 1.0, True, chunk, O=torch.empty_like(Q),
                      saved=torch.empty(nsv - 1, dtype=torch.uint8, device=dev))
    nws = race.workspace_bytes(B, H, N, d, P, L, True, chunk, race.WS_BWD_RECOMPUTE)
    with pytest.raises(ValueError, match="ws"):
        race.backward(Q, K, V, W, dO, P, L, 1.0, True, chunk, ws=torch.empty(nws - 1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="dO"):
        race.backward(Q, K, V, W, dO[:, :, :-1].contiguous(), P, L, 1.0, True, chunk)


def test_hash_and_prefill_reject_bad_shapes():
    import torch
    dev, (B, H, N, d, P, L), Q, K, V, dO, W = _inputs(torch.bfloat16)
    with pytest.raises(ValueError, match="W"):
        race.hard_hash(Q, W[:, :-1].contiguous(), P, L)
    with pytest.raises(ValueError, match="W"):
        race.hard_hash(Q, W, P, L + 1)
    nws = race.workspace_bytes(B, H, N, d, P, L, False, 64, race.WS_FWD)
    with pytest.raises(ValueError, match="ws"):
        race.prefill(K, V, W, P, L, 1.0, 64, ws=torch.empty(nws - 1, dtype=torch.uint8, device=dev))
