"""ctypes wrapper of the streaming float64 oracle (race_oracle.c).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libraceoracle.so")
SRC = os.path.join(HERE, "race_oracle.c")

_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB):
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", SRC,
                               "-o", LIB, "-lm"])
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_forward.argtypes = [vp, vp, vp, i32, vp, i64, i64, i32, i32, i32, dbl, i32,
                                       vp, i64, vp, vp]
        lib.oracle_backward.argtypes = [vp, vp, vp, vp, i32, vp, i64, i64, i32, i32, i32, dbl,
                                        i32, vp, i64, vp, vp, vp]
        lib.oracle_hash.argtypes = [vp, i32, vp, i64, i32, i32, i32, vp, vp]
        for f in (lib.oracle_forward, lib.oracle_backward, lib.oracle_hash):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:      # bf16 bit patterns
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(*arrs):
    out = [np.ascontiguousarray(a) for a in arrs]
    codes = {_dtype_code(a) for a in out}
    if len(codes) != 1:
        raise TypeError("Q, K, V (and dO) must share one dtype")
    return out, codes.pop()


def forward(Q, K, V, W, beta=1.0, causal=False, sample=None, return_den=False):
    """Q, K, V: [..., N, d] arrays (float32, float64 or bf16 bits as uint16).

    W: [L, P, d] float64.  Returns O as float64 [..., n_out, d] where n_out is
    len(sample) if given, else N.
    """
    (Q, K, V), code = _prep(Q, K, V)
    W = np.ascontiguousarray(W, dtype=np.float64)
    L, P, d = W.shape
    N = Q.shape[-2]
    BH = int(np.prod(Q.shape[:-2])) if Q.ndim > 2 else 1
    smp = None if sample is None else np.ascontiguousarray(sample, dtype=np.int64)
    n_out = N if smp is None else len(smp)
    O = np.empty(Q.shape[:-2] + (n_out, d))
    D = np.empty(Q.shape[:-2] + (n_out,))
    rc = _load().oracle_forward(_ptr(Q), _ptr(K), _ptr(V), code, _ptr(W), BH, N, d, P, L,
                                float(beta), int(bool(causal)), _ptr(smp),
                                0 if smp is None else len(smp), _ptr(O), _ptr(D))
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed: {rc}")
    return (O, D) if return_den else O


def backward(Q, K, V, W, dO, beta=1.0, causal=False, sample=None):
    (Q, K, V, dO), code = _prep(Q, K, V, dO)
    W = np.ascontiguousarray(W, dtype=np.float64)
    L, P, d = W.shape
    N = Q.shape[-2]
    BH = int(np.prod(Q.shape[:-2])) if Q.ndim > 2 else 1
    smp = None if sample is None else np.ascontiguousarray(sample, dtype=np.int64)
    n_out = N if smp is None else len(smp)
    shp = Q.shape[:-2] + (n_out, d)
    dQ, dK, dV = np.empty(shp), np.empty(shp), np.empty(shp)
    rc = _load().oracle_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), code, _ptr(W), BH, N, d,
                                 P, L, float(beta), int(bool(causal)), _ptr(smp),
                                 0 if smp is None else len(smp), _ptr(dQ), _ptr(dK), _ptr(dV))
    if rc != 0:
        raise RuntimeError(f"oracle_backward failed: {rc}")
    return dQ, dK, dV


def hard_hash(X, W):
    (X,), code = _prep(X)
    W = np.ascontiguousarray(W, dtype=np.float64)
    L, P, d = W.shape
    rows = X.size // d
    ids = np.empty(X.shape[:-1] + (L,), np.int32)
    nz = np.zeros(1, np.int64)
    rc = _load().oracle_hash(_ptr(X), code, _ptr(W), rows, d, P, L, _ptr(ids), _ptr(nz))
    if rc != 0:
        raise RuntimeError(f"oracle_hash failed: {rc}")
    return ids, int(nz[0])
