"""Python binding of libraceattn (RACE Attention on MI355X).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of ``libraceattn.so``; PyTorch provides device memory and the stream.
The names mirror the C ABI in ``include/race_attn.h``.  There is no CPU
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libraceattn.so")

RACE_OK, RACE_ERR_INVALID_ARG, RACE_ERR_UNSUPPORTED, RACE_ERR_WORKSPACE, RACE_ERR_HIP = range(5)
RACE_F32, RACE_BF16 = 0, 1
RACE_W_PER_HEAD = 0x100      # or'ed into dtype: W is [H, L, P, d]

SYMBOLS = ("race_attn_workspace_bytes", "race_attn_saved_bytes", "race_attn_fwd",
           "race_attn_fwd_noalloc", "race_attn_bwd", "race_attn_hash", "race_attn_state_bytes", "race_attn_prefill",
           "race_attn_decode", "race_attn_profile_events", "race_attn_profile_count",
           "race_attn_profile_stage", "race_attn_status_string")


class RaceError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


_lib = None


def lib():
    """Load libraceattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libraceattn.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        fl = ctypes.c_float
        L.race_attn_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                                ctypes.POINTER(sz)]
        L.race_attn_saved_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.race_attn_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, fl, i32, i32, i32,
                                    vp, vp, vp, sz, vp]
        L.race_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, fl, i32, i32,
                                            i32, vp, vp, vp]
        L.race_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, fl, i32, i32,
                                    i32, vp, vp, vp, vp, sz, vp]
        L.race_attn_hash.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, i32, vp, vp, vp]
        L.race_attn_state_bytes.argtypes = [i64, i64, i32, i32, i32, ctypes.POINTER(sz)]
        L.race_attn_prefill.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, i32, fl, i32, i32, vp, vp,
                                        sz, vp]
        L.race_attn_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, fl, i32, vp, vp, vp]
        L.race_attn_profile_events.argtypes = [vp, i32]
        L.race_attn_profile_count.argtypes = []
        L.race_attn_profile_stage.argtypes = [i32]
        L.race_attn_profile_stage.restype = ctypes.c_char_p
        L.race_attn_status_string.argtypes = [i32]
        L.race_attn_status_string.restype = ctypes.c_char_p
        for name in ("race_attn_workspace_bytes", "race_attn_saved_bytes", "race_attn_fwd",
                     "race_attn_fwd_noalloc", "race_attn_bwd", "race_attn_hash", "race_attn_state_bytes", "race_attn_prefill",
                     "race_attn_decode", "race_attn_profile_events", "race_attn_profile_count"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().race_attn_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != RACE_OK:
        raise RaceError(code, where)


WS_FWD, WS_BWD, WS_BWD_RECOMPUTE, WS_FWD_SAVED = 0, 1, 2, 3


def workspace_bytes(B, H, N, d, P, L, causal, chunk, kind) -> int:
    """Workspace bytes (race_attn_workspace_bytes' for_backward): kind 0
    forward without saved, 3 forward with saved, 1 backward given O and saved,
    2 backward recomputing the forward."""
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_workspace_bytes(B, H, N, d, P, L, int(bool(causal)), chunk, int(kind),
                                           ctypes.byref(out)),
           "race_attn_workspace_bytes")
    return out.value


def saved_bytes(B, H, N, d, P, L, causal, chunk) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_saved_bytes(B, H, N, d, P, L, int(bool(causal)), chunk, ctypes.byref(out)),
           "race_attn_saved_bytes")
    return out.value


def _w_flag(W, H, L, P, d):
    """RACE_W_PER_HEAD for per-head hyperplanes W [H, L, P, d], 0 for shared
    W [L, P, d]; anything else raises."""
    if tuple(W.shape) == (L, P, d):
        return 0
    if tuple(W.shape) == (H, L, P, d):
        return RACE_W_PER_HEAD
    raise ValueError(f"W must be [L, P, d] = {(L, P, d)} or [H, L, P, d] = {(H, L, P, d)}, got {tuple(W.shape)}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return RACE_F32
    if t.dtype == torch.bfloat16:
        return RACE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_inputs(*ts):
    dt = ts[0].dtype
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if t.dtype != dt:
            raise ValueError("all tensors must share one dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_like(t, ref, name):
    """An output tensor must match its input in shape, dtype and device, and be contiguous."""
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ref.dtype} tensor of shape {tuple(ref.shape)} "
                         f"on {ref.device}")


def _check_buf(t, nbytes, device, name):
    """A byte buffer (workspace, saved): contiguous, on the inputs' GPU, at least nbytes long."""
    if not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous tensor on {device}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")


def _nbytes(t):
    return t.numel() * t.element_size()


def alloc_workspace(B, H, N, P, L, causal, chunk, kind, device, d=64):
    """kind: WS_* (or'ed with RACE_W_PER_HEAD for per-head hyperplanes)."""
    import torch
    n = workspace_bytes(B, H, N, d, P, L, causal, chunk, kind)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def alloc_saved(B, H, N, P, L, causal, chunk, device, d=64):
    import torch
    n = saved_bytes(B, H, N, d, P, L, causal, chunk)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def race_attn_fwd(Q, K, V, W, P, L, temperature=1.0, causal=False, chunk=1024, out=None,
                  saved=None, ws=None, stream=None):
    """O = RACE attention of Q, K, V ([B, H, N, d]) with hyperplanes W ([L, P, d])."""
    import torch
    _check_inputs(Q, K, V, W)
    B, H, N, d = Q.shape
    wf = _w_flag(W, H, L, P, d)
    if K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must share one shape")
    if out is not None:
        _check_like(out, Q, "out")
    O = out if out is not None else torch.empty_like(Q)
    kind = (WS_FWD_SAVED if saved is not None else WS_FWD) | wf
    if saved is not None:
        _check_buf(saved, saved_bytes(B, H, N, d, P, L, causal, chunk), Q.device, "saved")
    if ws is None:
        ws = alloc_workspace(B, H, N, P, L, causal, chunk, kind, Q.device, d)
    _check_buf(ws, workspace_bytes(B, H, N, d, P, L, causal, chunk, kind), Q.device, "ws")
    code = lib().race_attn_fwd(_p(Q), _p(K), _p(V), _p(W), B, H, N, d, P, L, float(temperature),
                               int(bool(causal)), chunk, _dtype_code(Q) | wf, _p(O), _p(saved), _p(ws),
                               _nbytes(ws), _stream(stream))
    _check(code, "race_attn_fwd")
    return O


NOALLOC_SCRATCH_BYTES = 64 << 20


def race_attn_fwd_noalloc(Q, K, V, W, P, L, temperature=1.0, causal=False, chunk=1024, *, out,
                          saved=None, stream=None):
    """race_attn_fwd without a workspace argument: the library's fixed
    per-GPU scratch array (NOALLOC_SCRATCH_BYTES) serves as the workspace, and
    the call allocates nothing, so `out` (and `saved`, if wanted) are given by
    the caller. Calls that overlap on one GPU share that array and race."""
    _check_inputs(Q, K, V, W)
    B, H, N, d = Q.shape
    wf = _w_flag(W, H, L, P, d)
    if K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K, V must share one shape")
    _check_like(out, Q, "out")
    if saved is not None:
        _check_buf(saved, saved_bytes(B, H, N, d, P, L, causal, chunk), Q.device, "saved")
    code = lib().race_attn_fwd_noalloc(_p(Q), _p(K), _p(V), _p(W), B, H, N, d, P, L, float(temperature),
                                       int(bool(causal)), chunk, _dtype_code(Q) | wf, _p(out), _p(saved),
                                       _stream(stream))
    _check(code, "race_attn_fwd_noalloc")
    return out


def race_attn_bwd(Q, K, V, W, dO, P, L, temperature=1.0, causal=False, chunk=1024, O=None, saved=None,
                  ws=None, grads=None, stream=None):
    """(dQ, dK, dV) of <dO, RACE-attention(Q, K, V)>. O and saved (from the
    forward call) are given together, or both omitted (the forward is then
    recomputed inside the call)."""
    import torch
    _check_inputs(Q, K, V, W, dO)
    if (O is None) != (saved is None):
        raise ValueError("O and saved are given together or not at all")
    B, H, N, d = Q.shape
    wf = _w_flag(W, H, L, P, d)
    if O is not None:
        _check_inputs(Q, O)
        if O.shape != Q.shape:
            raise ValueError("O must have the shape of Q")
    if dO.shape != Q.shape:
        raise ValueError("dO must have the shape of Q")
    if saved is not None:
        _check_buf(saved, saved_bytes(B, H, N, d, P, L, causal, chunk), Q.device, "saved")
    if grads is None:
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = grads
    for t, nm in ((dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _check_like(t, Q, nm)
    kind = (WS_BWD if saved is not None else WS_BWD_RECOMPUTE) | wf
    if ws is None:
        ws = alloc_workspace(B, H, N, P, L, causal, chunk, kind, Q.device, d)
    _check_buf(ws, workspace_bytes(B, H, N, d, P, L, causal, chunk, kind), Q.device, "ws")
    code = lib().race_attn_bwd(_p(Q), _p(K), _p(V), _p(W), _p(O), _p(dO), _p(saved), B, H, N, d, P, L,
                               float(temperature), int(bool(causal)), chunk, _dtype_code(Q) | wf, _p(dQ),
                               _p(dK), _p(dV), _p(ws), _nbytes(ws), _stream(stream))
    _check(code, "race_attn_bwd")
    return dQ, dK, dV


def race_attn_hash(X, W, P, L, stream=None):
    """Hard bucket ids [B, H, N, L] (int32) and the near-zero projection count."""
    import torch
    _check_inputs(X, W)
    B, H, N, d = X.shape
    wf = _w_flag(W, H, L, P, d)
    ids = torch.empty((B, H, N, L), dtype=torch.int32, device=X.device)
    nz = torch.zeros(1, dtype=torch.int64, device=X.device)
    code = lib().race_attn_hash(_p(X), _p(W), B, H, N, d, P, L, _dtype_code(X) | wf, _p(ids), _p(nz),
                                _stream(stream))
    _check(code, "race_attn_hash")
    return ids, nz


def state_bytes(B, H, P, L, d=64) -> int:
    """Bytes of the running sketch of B * H heads (race_attn_state_bytes): per
    feature float32 value sums and a float64 mass."""
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_state_bytes(B, H, d, P, L, ctypes.byref(out)), "race_attn_state_bytes")
    return out.value


def alloc_state(B, H, P, L, device, d=64):
    """A zeroed running sketch (the state of an empty sequence), held in a
    float32 tensor of race_attn_state_bytes bytes."""
    import torch
    return torch.zeros(state_bytes(B, H, P, L, d) // 4, dtype=torch.float32, device=device)


def race_attn_prefill(K, V, W, P, L, temperature=1.0, chunk=1024, state=None, ws=None, stream=None):
    """Running sketch of the prompt K, V ([B, H, N, d]); temperature = inf
    gives the hard buckets. Returns the state (float32, overwritten)."""
    _check_inputs(K, V, W)
    B, H, N, d = K.shape
    wf = _w_flag(W, H, L, P, d)
    if V.shape != K.shape:
        raise ValueError("K and V must share one shape")
    if state is None:
        state = alloc_state(B, H, P, L, K.device, d)
    _check_state(state, B, H, P, L, d, K.device)
    if ws is None:
        ws = alloc_workspace(B, H, N, P, L, False, chunk, WS_FWD, K.device, d)
    _check_buf(ws, workspace_bytes(B, H, N, d, P, L, False, chunk, WS_FWD), K.device, "ws")
    code = lib().race_attn_prefill(_p(K), _p(V), _p(W), B, H, N, d, P, L, float(temperature), chunk,
                                   _dtype_code(K) | wf, _p(state), _p(ws), _nbytes(ws), _stream(stream))
    _check(code, "race_attn_prefill")
    return state


def _check_state(state, B, H, P, L, d, device):
    import torch
    if state.dtype != torch.float32 or not state.is_contiguous() or state.device != device:
        raise ValueError("state must be a contiguous float32 tensor on the inputs' GPU")
    if state.numel() * 4 < state_bytes(B, H, P, L, d):
        raise ValueError("state is smaller than race_attn_state_bytes")


def race_attn_decode(q, k, v, W, state, P, L, temperature=1.0, out=None, stream=None):
    """Causal decode: q, k, v are [B, H, d] (one token per head) or
    [B, H, T, d] (T tokens per head, in order); each token's k, v join
    `state` (in place), then its q reads it. Returns o shaped like q."""
    import torch
    _check_inputs(q, k, v, W)
    if q.dim() == 3:
        (B, H, d), T = q.shape, 1
    elif q.dim() == 4:
        B, H, T, d = q.shape
    else:
        raise ValueError("q must be [B, H, d] or [B, H, T, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    wf = _w_flag(W, H, L, P, d)
    _check_state(state, B, H, P, L, d, q.device)
    o = out if out is not None else torch.empty_like(q)
    if out is not None and (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor shaped like q")
    code = lib().race_attn_decode(_p(q), _p(k), _p(v), _p(W), B, H, T, d, P, L, float(temperature),
                                  _dtype_code(q) | wf, _p(state), _p(o), _stream(stream))
    _check(code, "race_attn_decode")
    return o


class StageTimer:
    """Per-kernel timing of library calls with HIP events (the library records
    them on its own stream between its launches; see race_attn_profile_events)."""

    def __init__(self, capacity: int = 257):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.n = capacity
        self.events = (ctypes.c_void_p * capacity)()
        for i in range(capacity):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev

    def __enter__(self):
        _check(lib().race_attn_profile_events(self.events, self.n), "race_attn_profile_events")
        return self

    def __exit__(self, *exc):
        lib().race_attn_profile_events(None, 0)

    def stages(self):
        """[(kernel name, milliseconds)] of the last call on this thread (synchronises)."""
        n = lib().race_attn_profile_count()
        if n < 2:
            return []
        self.hip.hipEventSynchronize(self.events[n - 1])
        out = []
        for i in range(n - 1):
            ms = ctypes.c_float(0)
            self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[i], self.events[i + 1])
            out.append((lib().race_attn_profile_stage(i).decode(), float(ms.value)))
        return out

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.events[i])


# short aliases
forward = race_attn_fwd
forward_noalloc = race_attn_fwd_noalloc
backward = race_attn_bwd
hard_hash = race_attn_hash
prefill = race_attn_prefill
decode = race_attn_decode
