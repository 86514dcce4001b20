"""The allocation-free forward (race_attn_fwd_noalloc) against race_attn_fwd
through the C ABI: the same kernels with the workspace in the library's fixed
per-GPU scratch array instead of a caller buffer. Two calls in a row, the
second on a smaller input (the array keeps the first call's contents), both
bit-identical to the workspace entry point; a shape whose workspace exceeds
the array is rejected before any device work."""
import pytest

import linear_lsh_sketch_amd as race

pytestmark = pytest.mark.gpu

CASES = [  # (dtype, causal, B, H, N, P, L, chunk, temperature, with saved, head dimension)
    ("bf16", True, 2, 3, 1500, 4, 16, 256, 1.0, True, 64),
    ("bf16", True, 1, 2, 333, 4, 16, 128, 1.0, False, 64),
    ("f32", False, 1, 2, 700, 2, 8, 512, 1.3, False, 64),
    ("f32", True, 1, 1, 129, 3, 5, 64, float("inf"), True, 64),
    # head dimension 128 (plane values in the workspace, two value halves)
    # and 32, with table groups
    ("bf16", True, 1, 2, 700, 4, 20, 128, 1.0, True, 128),
    ("f32", False, 1, 1, 300, 4, 5, 64, 1.0, False, 128),
    ("bf16", True, 1, 2, 400, 5, 9, 128, 1.0, True, 32),
    ("bf16", False, 1, 1, 200, 4, 40, 64, 1.0, False, 32),
]


def _inputs(dt, B, H, N, P, L, seed, d):
    import torch
    import synth
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    T = [synth.normal_device(seed, tid, torch.empty((B, H, N, d), dtype=tdt, device=dev))
         for tid in (synth.TID_Q, synth.TID_K, synth.TID_V)]
    W = synth.normal_device(seed, synth.TID_W, torch.empty((L, P, d), dtype=tdt, device=dev))
    return T, W


def _pair(big, small):
    import torch
    for case, seed in ((big, 11), (small, 12)):
        dt, causal, B, H, N, P, L, chunk, beta, with_saved, d = case
        print(f"[noalloc] {case}", flush=True)
        (Q, K, V), W = _inputs(dt, B, H, N, P, L, seed, d)
        # zero-filled: a bf16 run leaves the float32-sized tail of the plane
        # value regions unwritten, so both buffers start from the same bytes
        ref_saved = race.alloc_saved(B, H, N, P, L, causal, chunk, Q.device, d).zero_() if with_saved else None
        ref = race.forward(Q, K, V, W, P, L, beta, causal, chunk, saved=ref_saved)
        out = torch.full_like(Q, float("nan"))
        sv = (torch.zeros_like(ref_saved) if with_saved else None)
        got = race.forward_noalloc(Q, K, V, W, P, L, beta, causal, chunk, out=out, saved=sv)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16) if dt == "bf16" else got.view(torch.int32),
                           ref.view(torch.int16) if dt == "bf16" else ref.view(torch.int32))
        if with_saved:
            # the states, denominators and plane values the backward takes
            nb = race.saved_bytes(B, H, N, d, P, L, causal, chunk)
            assert torch.equal(sv[:nb], ref_saved[:nb])


def test_noalloc_forward_matches_workspace_forward():
    _pair(CASES[0], CASES[1])
    _pair(CASES[2], CASES[3])
    _pair(CASES[4], CASES[5])
    _pair(CASES[6], CASES[7])


def test_noalloc_rejects_workspace_beyond_the_scratch_array():
    import torch
    B, H, N, P, L, chunk = 1, 4, 1 << 17, 4, 16, 1024
    need = race.workspace_bytes(B, H, N, 64, P, L, True, chunk, race.WS_FWD)
    assert need > race.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    Q = torch.zeros((B, H, N, 64), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((L, P, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(race.RaceError) as e:
        race.forward_noalloc(Q, Q, Q, W, P, L, 1.0, True, chunk, out=torch.empty_like(Q))
    assert e.value.code == race.RACE_ERR_WORKSPACE
