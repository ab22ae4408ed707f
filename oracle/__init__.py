"""Oracle for the MC2 per-rank operators -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper over ``mc2_oracle.c``, the plain CPU implementation of what
the operators compute.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the product path
(``comm_matmul_tensor_amd``) never does, and it shares no code with it.

All arrays are numpy arrays in the storage conventions of ``mc2_inputs``
(bf16 as uint16 bit patterns, fp8 and E8M0 as uint8 codes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mc2_oracle.c")
_LIB = os.path.join(_HERE, "libmc2_oracle.so")

DT = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "i32": 4, "e4m3fn": 5, "e5m2": 6, "e8m0": 7}
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i8": np.int8,
            "i32": np.int32, "e4m3fn": np.uint8, "e5m2": np.uint8, "e8m0": np.uint8}

P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no contraction, no fast-math."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        sig = {
            "orc_allgather": (None, [P, INT, I64, I64, P]),
            "orc_matmul": (None, [P, INT, P, INT, I64, I64, I64, INT, P]),
            "orc_allgather_matmul": (None, [P, INT, I64, I64, P, I64, INT, INT, P, P]),
            "orc_matmul_reduce_scatter": (None, [P, P, INT, INT, INT, I64, I64, I64, P, INT, P, P]),
            "orc_permute": (None, [P, INT, I64, I64, P]),
            "orc_add_bias": (None, [P, P, I64, I64, INT]),
            "orc_unpack_int4": (None, [P, I64, P]),
            "orc_bias_grad": (None, [P, I64, I64, INT, P]),
            "orc_smooth_quant": (None, [P, I64, I64, P, INT, P, P]),
            "orc_int8_matmul": (I64, [P, P, I64, I64, I64, P]),
            "orc_dequant": (None, [P, P, P, P, I64, I64, INT, P]),
            "orc_alltoall_quant_matmul": (I64, [P, INT, I64, I64, INT, P, I64, P, P, P, P, P, P, P, P]),
            "orc_permute_i8": (None, [P, INT, I64, I64, P]),
            "orc_alltoall_quant_matmul_static": (I64, [P, INT, I64, I64, P, P, I64, P, P, INT, P, P, P]),
            "orc_quant_all_reduce": (INT, [P, P, INT, I64, I64, INT, INT, P, INT]),
            "orc_quant_reduce_scatter": (INT, [P, P, INT, INT, I64, I64, INT, INT, P, INT]),
            "orc_decode_array": (INT, [INT, I64, P, P]),
            "orc_encode_array": (INT, [INT, I64, P, P]),
            "orc_num_threads": (INT, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _ptr_array(arrs: Sequence[np.ndarray]):
    arr = (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])
    return arr


def num_threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------- formats
def decode(dtype: str, codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    st = np.dtype(_STORAGE[dtype])
    codes = codes.view(st) if codes.dtype.itemsize == st.itemsize else codes.astype(st)
    out = np.empty(codes.shape, dtype=np.float64)
    if _load().orc_decode_array(DT[dtype], codes.size, _ptr(codes), _ptr(out)) != 0:
        raise ValueError(dtype)
    return out


def encode(dtype: str, values: np.ndarray) -> np.ndarray:
    values = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(values.shape, dtype=_STORAGE[dtype])
    if _load().orc_encode_array(DT[dtype], values.size, _ptr(values), _ptr(out)) != 0:
        raise ValueError(dtype)
    return out


# ---------------------------------------------------------------- AllGatherMatmul
def allgather(shards: Sequence[np.ndarray]) -> np.ndarray:
    shards = [np.ascontiguousarray(s) for s in shards]
    m_local, k = shards[0].shape
    out = np.empty((len(shards) * m_local, k), dtype=shards[0].dtype)
    _load().orc_allgather(_ptr_array(shards), len(shards), m_local, k * shards[0].itemsize, _ptr(out))
    return out


def matmul(a: np.ndarray, b: np.ndarray, dtype: str, a_trans: bool = False,
           b_trans: bool = False) -> np.ndarray:
    """round(A @ B); a_trans: a holds A^T as (k, m); b_trans: b holds B^T as (n, k)."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a_trans:
        k, m = a.shape
    else:
        m, k = a.shape
    n = b.shape[0] if b_trans else b.shape[1]
    assert (b.shape[1] if b_trans else b.shape[0]) == k
    out = np.empty((m, n), dtype=_STORAGE[dtype])
    _load().orc_matmul(_ptr(a), int(a_trans), _ptr(b), int(b_trans), m, n, k, DT[dtype], _ptr(out))
    return out


def allgather_matmul(shards: Sequence[np.ndarray], x2: np.ndarray, dtype: str,
                     x2_trans: bool = False, gather_output: bool = True):
    shards = [np.ascontiguousarray(s) for s in shards]
    x2 = np.ascontiguousarray(x2)
    r = len(shards)
    m_local, k = shards[0].shape
    n = x2.shape[0] if x2_trans else x2.shape[1]
    out = np.empty((r * m_local, n), dtype=_STORAGE[dtype])
    g = np.empty((r * m_local, k), dtype=_STORAGE[dtype]) if gather_output else None
    _load().orc_allgather_matmul(_ptr_array(shards), r, m_local, k, _ptr(x2), n, int(x2_trans),
                                 DT[dtype], _ptr(out), _ptr(g))
    return out, g


def matmul_grad_input(dy: np.ndarray, w: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """dX_partial = dY @ W with W in nn.Linear (out, in) layout, i.e. (n_local, k)."""
    return matmul(dy, w, dtype)


def matmul_grad_weight(dy: np.ndarray, ag_x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """dW = dY^T @ AG(X)."""
    return matmul(dy, ag_x, dtype, a_trans=True)


# ---------------------------------------------------------------- AlltoAllQuantMatmul
def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """(..., c) bytes holding two int4 codes each -> (..., 2c) int8 codes (low nibble first)."""
    packed = np.ascontiguousarray(packed).view(np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int8)
    _load().orc_unpack_int4(_ptr(packed), out.size, _ptr(out))
    return out


def alltoall_quant_matmul_a16w4(x1, r: int, x2_packed, x2_scale, smooth=None, bias=None,
                                dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """A16W4: the dynamic per-token chain of alltoall_quant_matmul with the int4 weight
    (rank_size h, n / 2 bytes) unpacked to its codes."""
    return alltoall_quant_matmul(x1, r, unpack_int4(x2_packed), x2_scale, smooth, bias, dtype)


def alltoall_quant_matmul_a4w4(x1_packed, r: int, x1_scale, x2_packed, x2_scale, bias=None,
                               dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """A4W4: the full-quantisation chain of alltoall_quant_matmul_static with the int4
    activations (bs, h / 2 bytes) and weight (rank_size h, n / 2 bytes) unpacked."""
    return alltoall_quant_matmul_static(unpack_int4(x1_packed), r, x1_scale, unpack_int4(x2_packed), x2_scale, bias,
                                        dtype)


def add_bias(y: np.ndarray, bias: np.ndarray, dtype: str) -> np.ndarray:
    """round(y + bias) per row: the listing's `out = out + bias` after the fused op."""
    out = np.array(y, dtype=_STORAGE[dtype], copy=True, order="C")
    bias = np.ascontiguousarray(bias, dtype=_STORAGE[dtype])
    m, n = out.shape
    assert bias.shape == (n,)
    _load().orc_add_bias(_ptr(out), _ptr(bias), m, n, DT[dtype])
    return out


def bias_grad(dy: np.ndarray, dtype: str) -> np.ndarray:
    """grad_bias = dy.sum(dim=0), rounded once to the dtype."""
    dy = np.ascontiguousarray(dy, dtype=_STORAGE[dtype])
    m, n = dy.shape
    out = np.empty((n,), dtype=_STORAGE[dtype])
    _load().orc_bias_grad(_ptr(dy), m, n, DT[dtype], _ptr(out))
    return out


def matmul_reduce_scatter(x: np.ndarray, x2: np.ndarray, recv: Sequence[Optional[np.ndarray]], rank: int,
                          dtype: str, x2_trans: bool = False) -> Dict[str, np.ndarray]:
    """One rank's share of Y = ReduceScatter_m(x @ x2): "partial" = round(x @ x2) (m, n)
    and "out" = round(sum over ranks j in order of block `rank` of rank j's partial),
    (m / r, n); recv[j] is rank j's block for this rank (recv[rank] unused)."""
    x = np.ascontiguousarray(x)
    x2 = np.ascontiguousarray(x2)
    r = len(recv)
    m, k = x.shape
    n = x2.shape[0] if x2_trans else x2.shape[1]
    assert (x2.shape[1] if x2_trans else x2.shape[0]) == k and m % r == 0
    rows = m // r
    dummy = np.zeros((rows, n), dtype=_STORAGE[dtype])
    blocks = [dummy if (j == rank or recv[j] is None) else np.ascontiguousarray(recv[j]) for j in range(r)]
    for b in blocks:
        assert b.shape == (rows, n)
    partial = np.empty((m, n), dtype=_STORAGE[dtype])
    out = np.empty((rows, n), dtype=_STORAGE[dtype])
    _load().orc_matmul_reduce_scatter(_ptr(x), _ptr(x2), int(x2_trans), r, rank, m, k, n, _ptr_array(blocks),
                                      DT[dtype], _ptr(partial), _ptr(out))
    return {"partial": partial, "out": out}


def permute(x1: np.ndarray, r: int) -> np.ndarray:
    x1 = np.ascontiguousarray(x1)
    bs, h = x1.shape
    out = np.empty((bs // r, r * h), dtype=x1.dtype)
    _load().orc_permute(_ptr(x1), r, bs, h, _ptr(out))
    return out


def smooth_quant(p: np.ndarray, smooth: Optional[np.ndarray], dtype: str = "bf16"):
    p = np.ascontiguousarray(p)
    rows, cols = p.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s1 = np.empty(rows, dtype=np.float32)
    sm = None if smooth is None else np.ascontiguousarray(smooth)
    _load().orc_smooth_quant(_ptr(p), rows, cols, _ptr(sm), DT[dtype], _ptr(q), _ptr(s1))
    return q, s1


def int8_matmul(q: np.ndarray, x2: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    x2 = np.ascontiguousarray(x2, dtype=np.int8)
    m, k = q.shape
    n = x2.shape[1]
    acc = np.empty((m, n), dtype=np.int32)
    ovf = _load().orc_int8_matmul(_ptr(q), _ptr(x2), m, n, k, _ptr(acc))
    if ovf:
        raise OverflowError(f"{ovf} int32 overflows")
    return acc


def dequant(acc, s1, s2, bias, out_dtype: str = "bf16") -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s1 = np.ascontiguousarray(s1, dtype=np.float32)
    s2 = np.ascontiguousarray(s2, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias)
    m, n = acc.shape
    out = np.empty((m, n), dtype=_STORAGE[out_dtype])
    _load().orc_dequant(_ptr(acc), _ptr(s1), _ptr(s2), _ptr(b), m, n, DT[out_dtype], _ptr(out))
    return out


def alltoall_quant_matmul(x1, r: int, x2, x2_scale, smooth=None, bias=None,
                          dtype: str = "bf16") -> Dict[str, np.ndarray]:
    x1 = np.ascontiguousarray(x1)
    x2 = np.ascontiguousarray(x2, dtype=np.int8)
    x2_scale = np.ascontiguousarray(x2_scale, dtype=np.float32)
    bs, h = x1.shape
    n = x2.shape[1]
    rows, cols = bs // r, r * h
    out = np.empty((rows, n), dtype=_STORAGE[dtype])
    perm = np.empty((rows, cols), dtype=x1.dtype)
    q = np.empty((rows, cols), dtype=np.int8)
    s1 = np.empty(rows, dtype=np.float32)
    acc = np.empty((rows, n), dtype=np.int32)
    sm = None if smooth is None else np.ascontiguousarray(smooth)
    b = None if bias is None else np.ascontiguousarray(bias)
    ovf = _load().orc_alltoall_quant_matmul(_ptr(x1), r, bs, h, DT[dtype], _ptr(x2), n,
                                            _ptr(x2_scale), _ptr(sm), _ptr(b), _ptr(out), _ptr(perm),
                                            _ptr(q), _ptr(s1), _ptr(acc))
    if ovf:
        raise OverflowError(f"{ovf} int32 overflows")
    return {"out": out, "permuted": perm, "q": q, "s1": s1, "acc": acc}


def permute_i8(x1: np.ndarray, r: int) -> np.ndarray:
    """AlltoAll + permute of an int8 (bs, h) x1 into (bs / r, r h)."""
    x1 = np.ascontiguousarray(x1, dtype=np.int8)
    bs, h = x1.shape
    out = np.empty((bs // r, r * h), dtype=np.int8)
    _load().orc_permute_i8(_ptr(x1), r, bs, h, _ptr(out))
    return out


def alltoall_quant_matmul_static(x1, r: int, x1_scale, x2, x2_scale, bias=None,
                                 dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """Full-quant AlltoAllQuantMatmul: x1 int8 (bs, h) with one fp32 scale per
    permuted token (bs / r); out = (P @ x2) * x1_scale * x2_scale + bias."""
    x1 = np.ascontiguousarray(x1, dtype=np.int8)
    x1_scale = np.ascontiguousarray(x1_scale, dtype=np.float32)
    x2 = np.ascontiguousarray(x2, dtype=np.int8)
    x2_scale = np.ascontiguousarray(x2_scale, dtype=np.float32)
    bs, h = x1.shape
    n = x2.shape[1]
    rows, cols = bs // r, r * h
    out = np.empty((rows, n), dtype=_STORAGE[dtype])
    perm = np.empty((rows, cols), dtype=np.int8)
    acc = np.empty((rows, n), dtype=np.int32)
    b = None if bias is None else np.ascontiguousarray(bias)
    ovf = _load().orc_alltoall_quant_matmul_static(_ptr(x1), r, bs, h, _ptr(x1_scale), _ptr(x2), n,
                                                   _ptr(x2_scale), _ptr(b), DT[dtype], _ptr(out), _ptr(perm),
                                                   _ptr(acc))
    if ovf:
        raise OverflowError(f"{ovf} int32 overflows")
    return {"out": out, "permuted": perm, "acc": acc}


# ---------------------------------------------------------------- QuantAllReduce
def quant_all_reduce(xs: Sequence[np.ndarray], scales: Sequence[np.ndarray], x_dtype: str,
                     scale_dtype: str, out_dtype: str) -> np.ndarray:
    xs = [np.ascontiguousarray(x) for x in xs]
    scales = [np.ascontiguousarray(s) for s in scales]
    shape = xs[0].shape
    h = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty(shape, dtype=_STORAGE[out_dtype])
    rc = _load().orc_quant_all_reduce(_ptr_array(xs), _ptr_array(scales), len(xs), rows, h,
                                      DT[x_dtype], DT[scale_dtype], _ptr(out), DT[out_dtype])
    if rc != 0:
        raise ValueError("unsupported dtype combination")
    return out


def quant_reduce_scatter(xs: Sequence[np.ndarray], scales: Sequence[np.ndarray], rank: int, x_dtype: str,
                         scale_dtype: str, out_dtype: str) -> np.ndarray:
    """Rows [rank rows / r, (rank + 1) rows / r) of the QuantAllReduce sum, as (rows / r, h)."""
    xs = [np.ascontiguousarray(x) for x in xs]
    scales = [np.ascontiguousarray(s) for s in scales]
    shape = xs[0].shape
    h = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty((rows // len(xs), h), dtype=_STORAGE[out_dtype])
    rc = _load().orc_quant_reduce_scatter(_ptr_array(xs), _ptr_array(scales), len(xs), rank, rows, h,
                                          DT[x_dtype], DT[scale_dtype], _ptr(out), DT[out_dtype])
    if rc != 0:
        raise ValueError("unsupported dtype combination or rows not divisible by the ranks")
    return out
