"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any
device work."""
import ctypes
import os
import re

import pytest

import linear_lsh_sketch_amd as race

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "race_attn.h")
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation first


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(race_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = race.lib()
    names = declared_symbols()
    assert set(names) == set(race.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def test_profile_hook_without_gpu():
    L = race.lib()
    assert L.race_attn_profile_events(None, 0) == race.RACE_OK
    assert L.race_attn_profile_count() == 0
    assert L.race_attn_profile_stage(0) is None
    arr = (ctypes.c_void_p * 1)()
    assert L.race_attn_profile_events(arr, 1) == race.RACE_ERR_INVALID_ARG


def test_status_strings():
    assert race.status_string(0) == "RACE_OK"
    assert race.status_string(3) == "RACE_ERR_WORKSPACE"
    assert race.status_string(99) == "RACE_ERR_UNKNOWN"


def _a256(x):
    return -(-x // 256) * 256


def test_workspace_and_saved_sizes():
    # causal: per-chunk states of F * 65 floats (F = 32 * MT * KB), then one
    # float32 denominator per token, then for queries and keys the per-token
    # plane values (16 * MT soft values u, sized as float32, and one norm)
    N, rows = 12_000_000, 4 * 12_000_000
    fwd = race.workspace_bytes(1, 4, N, 64, 4, 16, True, 1024, race.WS_FWD)
    fwd_s = race.workspace_bytes(1, 4, N, 64, 4, 16, True, 1024, race.WS_FWD_SAVED)
    bwd = race.workspace_bytes(1, 4, N, 64, 4, 16, True, 1024, race.WS_BWD)
    rec = race.workspace_bytes(1, 4, N, 64, 4, 16, True, 1024, race.WS_BWD_RECOMPUTE)
    saved = race.saved_bytes(1, 4, N, 64, 4, 16, True, 1024)
    nchunks = -(-N // 1024)
    states = 4 * nchunks * 256 * 65 * 4
    cache = _a256(rows * 64 * 4) + _a256(rows * 4)
    assert saved == _a256(states) + _a256(rows * 4) + 2 * cache
    assert fwd_s >= states and fwd >= fwd_s + cache
    # gradient states and e per token
    assert bwd >= states + rows * 4
    # plus a saved buffer and the forward output (float32 bound); each kind
    # holds one buffer for the segment sums of the chunk scan (at most 16
    # segments of F * 65 + 64 floats per head), which the recompute kind
    # shares between its forward and backward
    seg_max = 4 * 16 * (256 * 65 + 64) * 4
    assert rec >= fwd_s + bwd + saved + rows * 64 * 4 - 2 * seg_max
    # non-causal: the total sketch (L8 P2: MT = 1, F = 32)
    rows_nc = 6 * 100
    cache_nc = _a256(rows_nc * 16 * 4) + _a256(rows_nc * 4)
    assert race.saved_bytes(2, 3, 100, 64, 2, 8, False, 64) == \
        _a256(6 * 32 * 65 * 4) + _a256(rows_nc * 4) + 2 * cache_nc


def test_table_group_sizes():
    # P4 L40 runs as table groups of 16, 16 and 8 (four, four and two
    # projection tiles: 256, 256 and 128 features per state)
    B, H, N, chunk = 2, 3, 1000, 128
    rows, nch = B * H * N, -(-N // chunk)
    f65 = (256 * 2 + 128) * 65 * 4
    f66 = (256 * 2 + 128) * 66 * 4     # running state: float64 masses
    states = B * H * nch * f65
    cache = 2 * _a256(rows * 64 * 4) + _a256(rows * 32 * 4) + _a256(rows * 4)
    saved = race.saved_bytes(B, H, N, 64, 4, 40, True, chunk)
    assert saved == _a256(states) + _a256(rows * 4) + 2 * cache
    # the running state holds the groups one after the other
    assert race.state_bytes(B, H, 4, 40) == B * H * f66
    # the workspace adds the partial outputs of the groups before the last
    # ([rows][64] and the denominators, float32)
    one = race.workspace_bytes(B, H, N, 64, 4, 16, True, chunk, race.WS_BWD)
    three = race.workspace_bytes(B, H, N, 64, 4, 40, True, chunk, race.WS_BWD)
    assert three >= one + _a256(rows * 64 * 4) + _a256(rows * 4)
    # P < 4: groups of 128 projection rows (P2: 64 tables)
    assert race.state_bytes(1, 1, 2, 64) == 8 * 32 * 66 * 4
    assert race.state_bytes(1, 1, 2, 65) == (8 + 1) * 32 * 66 * 4


def test_segmented_scan_workspace():
    # one causal head of 2^20 tokens, L8 P1 (F = 32, 65 F floats per state):
    # chunk 1024 gives 1024 chunks and 9 workgroups per pass, so the chunk
    # scans run in 16 segments whose sums take BH * 16 * (65 F + 64) floats
    # more (sized for the compact form of bf16 inputs: two floats per word of
    # bf16 value pairs, and the float32 row of the empty subset)
    per = 32 * 65 * 4
    seg = race.workspace_bytes(1, 1, 1 << 20, 64, 1, 8, True, 1024, race.WS_FWD_SAVED)
    assert seg == _a256(1024 * per) + _a256(16 * (per + 64 * 4))
    # four chunks: one pass, no segment sums
    one = race.workspace_bytes(1, 1, 4096, 64, 1, 8, True, 1024, race.WS_FWD_SAVED)
    assert one == _a256(4 * per)


def test_workspace_kind_rejected():
    out = ctypes.c_size_t(0)
    for kind in (-1, 4):
        assert race.lib().race_attn_workspace_bytes(1, 1, 10, 64, 4, 8, 1, 16, kind, ctypes.byref(out)) == \
            race.RACE_ERR_INVALID_ARG


@pytest.mark.parametrize("args,code", [
    ((0, 1, 10, 64, 4, 8, 1, 16, 0), race.RACE_ERR_INVALID_ARG),        # B = 0
    ((1, 1, 0, 64, 4, 8, 1, 16, 0), race.RACE_ERR_INVALID_ARG),         # N = 0
    ((1, 1, 10, 48, 4, 8, 1, 16, 0), race.RACE_ERR_UNSUPPORTED),        # d not 32 or 64
    ((1, 1, 10, 64, 7, 8, 1, 16, 0), race.RACE_ERR_UNSUPPORTED),        # P > 6
    ((1, 1, 10, 64, 0, 8, 1, 16, 0), race.RACE_ERR_INVALID_ARG),        # P = 0
    ((1, 1, 10, 64, 4, 4097, 1, 16, 0), race.RACE_ERR_UNSUPPORTED),     # L * 2^P > 2^16
    ((1, 1, 10, 64, 4, 8, 1, 0, 0), race.RACE_ERR_INVALID_ARG),         # chunk = 0
    ((1, 70000, 10, 64, 4, 8, 1, 16, 0), race.RACE_ERR_UNSUPPORTED),    # B*H > 65535
    ((1 << 40, 1 << 20, 1 << 20, 64, 4, 8, 1, 16, 0), race.RACE_ERR_INVALID_ARG),  # overflow
    ((1, 1, 10, 64, 4, 8, 1, (1 << 20) + 1, 0), race.RACE_ERR_UNSUPPORTED),  # chunk > 2^20
])
def test_workspace_bytes_rejects(args, code):
    out = ctypes.c_size_t(0)
    assert race.lib().race_attn_workspace_bytes(*args, ctypes.byref(out)) == code


def test_forward_argument_errors_before_device_work():
    L = race.lib()
    ok = (FAKE, FAKE, FAKE, FAKE, 1, 1, 100, 64, 4, 8, 1.0, 1, 64, race.RACE_BF16, FAKE, None, FAKE)
    need = race.workspace_bytes(1, 1, 100, 64, 4, 8, True, 64, race.WS_FWD)
    # null query
    assert L.race_attn_fwd(None, *ok[1:], need, None) == race.RACE_ERR_INVALID_ARG
    # bad dtype
    bad = list(ok); bad[13] = 7
    assert L.race_attn_fwd(*bad, need, None) == race.RACE_ERR_INVALID_ARG
    # non-finite temperature
    bad = list(ok); bad[10] = float("nan")
    assert L.race_attn_fwd(*bad, need, None) == race.RACE_ERR_INVALID_ARG
    bad = list(ok); bad[10] = float("-inf")
    assert L.race_attn_fwd(*bad, need, None) == race.RACE_ERR_INVALID_ARG
    # hard buckets (temperature = +inf), both dtypes: accepted up to the size
    # check while F * N < 2^24 (F = 128 features here), refused beyond
    bad = list(ok); bad[10] = float("inf")
    assert L.race_attn_fwd(*bad, need - 1, None) == race.RACE_ERR_WORKSPACE
    bad[13] = race.RACE_F32
    assert L.race_attn_fwd(*bad, need - 1, None) == race.RACE_ERR_WORKSPACE
    bad[6] = 200_000
    big = race.workspace_bytes(1, 1, 200_000, 64, 4, 8, True, 64, race.WS_FWD)
    assert L.race_attn_fwd(*bad, big, None) == race.RACE_ERR_UNSUPPORTED
    # workspace too small
    assert L.race_attn_fwd(*ok, need - 1, None) == race.RACE_ERR_WORKSPACE
    # unsupported head dim (32, 64 and 128 are supported)
    bad = list(ok); bad[7] = 96
    assert L.race_attn_fwd(*bad, need, None) == race.RACE_ERR_UNSUPPORTED


def test_p6_sizes_for_both_dtypes():
    # P = 6 is supported for both input types: the sizes are reported, and an
    # undersized workspace is still refused before any launch (the pointers
    # here are never dereferenced)
    L = race.lib()
    need = race.workspace_bytes(1, 1, 100, 64, 6, 4, True, 64, race.WS_FWD)
    assert need > 0 and race.saved_bytes(1, 1, 100, 64, 6, 4, True, 64) > 0
    for dt in (race.RACE_F32, race.RACE_BF16):
        args = (FAKE, FAKE, FAKE, FAKE, 1, 1, 100, 64, 6, 4, 1.0, 1, 64, dt, FAKE, None, FAKE, need - 1, None)
        assert L.race_attn_fwd(*args) == race.RACE_ERR_WORKSPACE
    assert race.state_bytes(1, 1, 6, 4) > 0


def test_backward_and_hash_argument_errors():
    L = race.lib()
    need = race.workspace_bytes(1, 1, 100, 64, 4, 8, False, 64, race.WS_BWD_RECOMPUTE)
    need_saved = race.workspace_bytes(1, 1, 100, 64, 4, 8, False, 64, race.WS_BWD)
    assert need_saved < need
    # Q K V W O dO saved
    args = [FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 100, 64, 4, 8, 1.0, 0, 64, race.RACE_F32,
            FAKE, FAKE, FAKE, FAKE]
    assert L.race_attn_bwd(*args, need - 1, None) == race.RACE_ERR_WORKSPACE
    a2 = list(args); a2[17] = None   # dQ
    assert L.race_attn_bwd(*a2, need, None) == race.RACE_ERR_INVALID_ARG
    # O without saved, saved without O
    a3 = list(args); a3[4] = FAKE
    assert L.race_attn_bwd(*a3, need, None) == race.RACE_ERR_INVALID_ARG
    a4 = list(args); a4[6] = FAKE
    assert L.race_attn_bwd(*a4, need, None) == race.RACE_ERR_INVALID_ARG
    a6 = list(args); a6[13] = float("inf")   # the hard limit has no gradient: rejected
    assert L.race_attn_bwd(*a6, need, None) == race.RACE_ERR_INVALID_ARG
    # both given: the smaller workspace is enough, one byte less is not
    a5 = list(args); a5[4] = FAKE; a5[6] = FAKE
    assert L.race_attn_bwd(*a5, need_saved - 1, None) == race.RACE_ERR_WORKSPACE
    assert L.race_attn_hash(FAKE, FAKE, 1, 1, 10, 64, 4, 8, race.RACE_F32, None, FAKE, None) == \
        race.RACE_ERR_INVALID_ARG
    assert L.race_attn_hash(FAKE, FAKE, 1, 1, 10, 64, 4, 8, race.RACE_F32, None, FAKE, None) == \
        race.RACE_ERR_INVALID_ARG
    assert L.race_attn_hash(FAKE, FAKE, 1, 1, 10, 64, 7, 8, race.RACE_F32, FAKE, FAKE, None) == \
        race.RACE_ERR_UNSUPPORTED


def test_state_bytes():
    # per head and feature 64 float32 value sums and a float64 mass (66 floats):
    # F = 32 * MT * KB (L16 P4: MT 4, KB 2 -> 256; L5 P3: 5 tables of 4 padded
    # planes -> MT 2, KB 1 -> 64; L8 P2: MT 1 -> 32)
    for (B, H, P, L, F) in [(1, 4, 4, 16, 256), (2, 3, 3, 5, 64), (1, 1, 2, 8, 32), (1, 1, 4, 32, 512)]:
        assert race.state_bytes(B, H, P, L) == B * H * F * 66 * 4
    out = ctypes.c_size_t(0)
    # head dimension 128: two halves of value sums per feature (F = 128 at L8 P4)
    assert race.lib().race_attn_state_bytes(1, 1, 128, 4, 8, ctypes.byref(out)) == race.RACE_OK
    assert out.value == 128 * 130 * 4 and race.state_bytes(2, 3, 4, 8, 128) == 6 * 128 * 130 * 4
    assert race.lib().race_attn_state_bytes(1, 1, 96, 4, 8, ctypes.byref(out)) == race.RACE_ERR_UNSUPPORTED
    assert race.lib().race_attn_state_bytes(1, 1, 64, 7, 8, ctypes.byref(out)) == race.RACE_ERR_UNSUPPORTED
    assert race.lib().race_attn_state_bytes(0, 1, 64, 4, 8, ctypes.byref(out)) == race.RACE_ERR_INVALID_ARG
    assert race.lib().race_attn_state_bytes(1, 1, 64, 4, 8, None) == race.RACE_ERR_INVALID_ARG


def test_prefill_and_decode_argument_errors():
    L = race.lib()
    need = race.workspace_bytes(1, 1, 100, 64, 4, 8, False, 64, race.WS_FWD)
    # K V W B H N d P L temperature chunk dtype state ws
    ok = [FAKE, FAKE, FAKE, 1, 1, 100, 64, 4, 8, 1.0, 64, race.RACE_BF16, FAKE, FAKE]
    assert L.race_attn_prefill(*ok, need - 1, None) == race.RACE_ERR_WORKSPACE
    for i, v in [(0, None), (12, None), (13, None), (11, 5), (9, float("nan")), (9, float("-inf"))]:
        bad = list(ok); bad[i] = v
        assert L.race_attn_prefill(*bad, need, None) == race.RACE_ERR_INVALID_ARG, i
    bad = list(ok); bad[5] = 0   # empty prompt: the zero state needs no call
    assert L.race_attn_prefill(*bad, need, None) == race.RACE_ERR_INVALID_ARG
    bad = list(ok); bad[10] = (1 << 20) + 1
    assert L.race_attn_prefill(*bad, need, None) == race.RACE_ERR_UNSUPPORTED
    # q k v W B H T d P L temperature dtype state o
    dec = [FAKE, FAKE, FAKE, FAKE, 2, 3, 1, 64, 4, 8, 1.0, race.RACE_F32, FAKE, FAKE]
    for i, v in [(0, None), (3, None), (12, None), (13, None), (11, 9), (10, float("nan")),
                 (10, float("-inf")), (4, 0), (6, 0), (6, -3)]:
        bad = list(dec); bad[i] = v
        assert L.race_attn_decode(*bad, None) == race.RACE_ERR_INVALID_ARG, i
    for i in (3, 12):   # W, state not 16-byte aligned
        bad = list(dec); bad[i] = ctypes.c_void_p(0x10004)
        assert L.race_attn_decode(*bad, None) == race.RACE_ERR_INVALID_ARG, i
    bad = list(dec); bad[6] = 1 << 31   # more tokens than a 32-bit count
    assert L.race_attn_decode(*bad, None) == race.RACE_ERR_UNSUPPORTED
    for i, v in [(7, 48), (8, 7), (9, 4097)]:
        bad = list(dec); bad[i] = v
        assert L.race_attn_decode(*bad, None) == race.RACE_ERR_UNSUPPORTED, i


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU fallback: without the built library every entry point raises
    monkeypatch.setattr(race, "_lib", None)
    monkeypatch.setattr(race, "LIB_PATH", str(tmp_path / "libraceattn.so"))
    with pytest.raises(RuntimeError, match="not built"):
        race.lib()
    with pytest.raises(RuntimeError, match="not built"):
        race.workspace_bytes(1, 1, 10, 64, 4, 8, True, 16, race.WS_FWD)


def test_binding_buffer_checks_on_host_tensors():
    """The binding's output and buffer checks (shape, dtype, device,
    contiguity, byte size) that every entry point runs before the C call."""
    import torch
    ref = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16)
    race._check_like(torch.zeros_like(ref), ref, "out")
    for bad in (torch.zeros((1, 2, 8, 64), dtype=torch.float32),     # twice the bytes per element
                torch.zeros((1, 2, 9, 64), dtype=torch.bfloat16),
                torch.zeros((1, 2, 64, 8), dtype=torch.bfloat16).transpose(2, 3)):
        with pytest.raises(ValueError):
            race._check_like(bad, ref, "out")
    buf = torch.zeros(100, dtype=torch.float32)          # 400 bytes
    race._check_buf(buf, 400, buf.device, "ws")
    with pytest.raises(ValueError):
        race._check_buf(buf, 401, buf.device, "ws")
    with pytest.raises(ValueError):
        race._check_buf(buf[::2], 10, buf.device, "ws")
    assert race._nbytes(buf) == 400
