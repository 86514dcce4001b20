"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

Holds no attention arithmetic: it maps (seed, tensor id, flat index) to
numbers with Philox-4x32-10 (Salmon et al., SC'11) and a double-precision
Box-Muller transform.  The host generator lives in ``synth.c``; the device
generator (same stream definition, for filling HBM at the large sizes) lives
in ``synth_dev.hip``.

Tensor ids: W = 0, Q = 1, K = 2, V = 3, dO = 4, mixture centres = 5,
query cluster ids = 6, key cluster ids = 7.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

TID_W, TID_Q, TID_K, TID_V, TID_DO, TID_CENTRES, TID_QIDS, TID_KIDS = range(8)
DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2}


def build_host(force: bool = True) -> str:
    if force or not os.path.exists(HOST_LIB):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               os.path.join(HERE, "synth.c"), "-o", HOST_LIB, "-lm"])
    return HOST_LIB


def build_device(force: bool = True) -> str:
    if force or not os.path.exists(DEV_LIB):
        subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               os.path.join(HERE, "synth_dev.hip"), "-o", DEV_LIB])
    return DEV_LIB


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_philox.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.synth_mixture.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_uint32, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_int, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        _host = lib
    return _host


def philox(ctr, key):
    """Raw Philox-4x32-10 block (four uint32 words) for counter ``ctr`` and key ``key``."""
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _host_lib().synth_philox(c, k, o)
    return list(o)


def _alloc(n, dtype):
    return {"f32": np.empty(n, np.float32), "bf16": np.empty(n, np.uint16),
            "f64": np.empty(n, np.float64)}[dtype]


def normal(seed: int, tid: int, shape, dtype: str = "f64", scale: float = 1.0, start: int = 0):
    """Normal draws of the given shape; bf16 is returned as raw uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = _alloc(n, dtype)
    _host_lib().synth_normal(seed, tid, start, n, scale, DTYPE_CODE[dtype],
                             out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def mixture(seed: int, tid_noise: int, tid_ids: int, rows: int, d: int, dtype: str = "f64",
            row0: int = 0, n_centres: int = 64, centre_sd: float = 1.0, noise_sd: float = 0.3):
    """Unit-length rows drawn around ``n_centres`` shared Gaussian centres."""
    out = _alloc(rows * d, dtype)
    _host_lib().synth_mixture(seed, tid_noise, tid_ids, TID_CENTRES, n_centres, centre_sd,
                              noise_sd, d, row0, rows, DTYPE_CODE[dtype],
                              out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(rows, d)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64,
                                         ctypes.c_uint64, ctypes.c_double, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_dev_normal.restype = ctypes.c_int
        lib.synth_dev_mixture.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_int, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
        lib.synth_dev_mixture.restype = ctypes.c_int
        _dev = lib
    return _dev


def normal_device(seed: int, tid: int, tensor, scale: float = 1.0, start: int = 0, stream=None):
    """Fill a contiguous CUDA/HIP torch tensor (float32 or bfloat16) in place."""
    import torch
    assert tensor.is_cuda and tensor.is_contiguous()
    code = {torch.float32: 0, torch.bfloat16: 1}[tensor.dtype]
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = _dev_lib().synth_dev_normal(seed, tid, start, tensor.numel(), scale, code,
                                     ctypes.c_void_p(tensor.data_ptr()), ctypes.c_void_p(s))
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal failed: {rc}")
    return tensor


def mixture_device(seed: int, tid_noise: int, tid_ids: int, tensor, row0: int = 0,
                   n_centres: int = 64, centre_sd: float = 1.0, noise_sd: float = 0.3, stream=None):
    import torch
    assert tensor.is_cuda and tensor.is_contiguous()
    d = tensor.shape[-1]
    code = {torch.float32: 0, torch.bfloat16: 1}[tensor.dtype]
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = _dev_lib().synth_dev_mixture(seed, tid_noise, tid_ids, TID_CENTRES, n_centres, centre_sd,
                                      noise_sd, d, row0, tensor.numel() // d, code,
                                      ctypes.c_void_p(tensor.data_ptr()), ctypes.c_void_p(s))
    if rc != 0:
        raise RuntimeError(f"synth_dev_mixture failed: {rc}")
    return tensor
