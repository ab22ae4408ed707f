"""Seeded synthetic inputs for the MC2 per-rank operators.

This package only makes tensors.  It is shared by the oracle tests, the GPU
parity tests and the benchmark, and it contains none of the operators'
arithmetic.  The stream and distribution definitions are in ``gen.c``.

Storage conventions (numpy side): fp32 -> float32, fp16 -> float16,
bf16 -> uint16 bit patterns, int8 -> int8, FLOAT8_E4M3FN and FLOAT8_E8M0 ->
uint8 codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmc2gen.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "e4m3fn": 5, "e8m0": 7}
NP_STORAGE = {
    "f32": np.float32,
    "f16": np.float16,
    "bf16": np.uint16,
    "i8": np.int8,
    "e4m3fn": np.uint8,
    "e8m0": np.uint8,
}
DISTS = {"uniform": 0, "int": 1, "normal": 2}


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.mc2gen_fill.restype = ctypes.c_int
        lib.mc2gen_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p]
        lib.mc2gen_words.restype = None
        lib.mc2gen_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
        _lib = lib
    return _lib


def words(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().mc2gen_words(seed, tid, start, n, out.ctypes.data)
    return out


def fill(seed: int, tid: int, dist: str, a: float, b: float, dtype: str, shape,
         start: int = 0) -> np.ndarray:
    """Elements [start, start + prod(shape)) of tensor stream (seed, tid)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    rc = _load().mc2gen_fill(seed, tid, DISTS[dist], float(a), float(b), DTYPES[dtype], start, n,
                             out.ctypes.data)
    if rc != 0:
        raise ValueError(f"mc2gen_fill failed with code {rc}")
    return out


from .configs import CONFIGS, TensorSpec, make, make_tensor  # noqa: E402,F401


def to_torch(arr: np.ndarray, dtype: str, device="cuda"):
    """numpy storage (see module doc) -> torch tensor of the matching torch dtype."""
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    elif dtype == "e4m3fn":
        t = torch.from_numpy(arr).view(torch.float8_e4m3fn)
    elif dtype == "e5m2":
        t = torch.from_numpy(arr).view(torch.float8_e5m2)
    elif dtype == "e8m0":
        t = torch.from_numpy(arr).view(torch.float8_e8m0fnu)
    else:
        t = torch.from_numpy(arr)
    return t.to(device) if device is not None else t


def from_torch(t) -> np.ndarray:
    """torch tensor -> numpy storage (bf16 as uint16 bits, 8-bit floats as uint8 codes)."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2) or \
            (hasattr(torch, "float8_e8m0fnu") and t.dtype == torch.float8_e8m0fnu):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Storage of int4 inputs: codes (-8..7) along the last dimension (even length) two per
    byte, value 2i in the low nibble of byte i and value 2i + 1 in the high nibble."""
    c = np.asarray(codes).astype(np.int16)
    assert c.shape[-1] % 2 == 0 and c.min(initial=0) >= -8 and c.max(initial=0) <= 7
    u = (c & 0xF).astype(np.uint8)
    return np.ascontiguousarray(u[..., 0::2] | (u[..., 1::2] << 4))
