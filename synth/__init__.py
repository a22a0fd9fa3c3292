"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Only input generation lives here: random weights, KV-cache contents, token ids,
coin flips and shuffles. Nothing in this package computes any part of the
decode/verify step. The heavy lifting is ``synth.c`` (SplitMix64 counters and
Marsaglia's polar method, multi-threaded); this module loads it with ctypes and
returns NumPy / PyTorch CPU tensors.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

F32, F16, BF16 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile synth.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            u64, i64, i32p = ctypes.c_uint64, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
            L.synth_key.restype = u64
            L.synth_key.argtypes = [u64, ctypes.POINTER(u64), ctypes.c_int]
            L.synth_raw.restype = u64
            L.synth_raw.argtypes = [u64, u64]
            L.synth_normal.restype = None
            L.synth_normal.argtypes = [u64, u64, i64, ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
            L.synth_uniform_int.restype = None
            L.synth_uniform_int.argtypes = [u64, u64, i64, i64, i64, i32p]
            L.synth_uniform.restype = None
            L.synth_uniform.argtypes = [u64, u64, i64, ctypes.POINTER(ctypes.c_double)]
            L.synth_raw_fill.restype = None
            L.synth_raw_fill.argtypes = [u64, u64, i64, ctypes.POINTER(u64)]
            _lib = L
    return _lib


def key(seed: int, *tags: int) -> int:
    """Stream key derived from a seed and integer tags (order matters)."""
    arr = (ctypes.c_uint64 * max(1, len(tags)))(*[t & 0xFFFFFFFFFFFFFFFF for t in tags])
    return int(lib().synth_key(seed & 0xFFFFFFFFFFFFFFFF, arr, len(tags)))


def raw(k: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_raw_fill(k, start, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    return out


def normal_into(out, k: int, start: int, mean: float, std: float) -> None:
    """Fill a contiguous NumPy array or CPU torch tensor (fp32 / fp16 / bf16) in place."""
    code, ptr, n = _describe(out)
    lib().synth_normal(k, start, n, float(mean), float(std), code, ctypes.c_void_p(ptr))


def normal(k: int, start: int, n: int, mean: float = 0.0, std: float = 1.0, dtype: str = "f32"):
    """Return a CPU torch tensor of n values mean + std * N(0,1), rounded to dtype."""
    import torch

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    t = torch.empty(n, dtype=tdt)
    normal_into(t, k, start, mean, std)
    return t


def uniform_int(k: int, start: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi)."""
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_int(k, start, n, lo, hi, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return out


def uniform(k: int, start: int, n: int) -> np.ndarray:
    """n doubles uniform in [0, 1)."""
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform(k, start, n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    """A seeded permutation of range(n): sort positions by their raw 64-bit draws."""
    r = raw(k, 0, n)
    return np.argsort(r, kind="stable").astype(np.int64)


def _describe(out):
    try:
        import torch

        if isinstance(out, torch.Tensor):
            assert out.device.type == "cpu" and out.is_contiguous()
            code = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[out.dtype]
            return code, out.data_ptr(), out.numel()
    except ImportError:  # pragma: no cover
        pass
    assert isinstance(out, np.ndarray) and out.flags["C_CONTIGUOUS"]
    code = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}[out.dtype]
    return code, out.ctypes.data, out.size
