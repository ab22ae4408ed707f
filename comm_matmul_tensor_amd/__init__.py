"""comm_matmul_tensor_amd -- Python binding of libmc2 (MC2 per-rank compute on MI355X).

A thin ctypes layer over the C ABI declared in ``include/mc2.h``.  It only
marshals arguments: torch supplies device memory and the current HIP stream,
and every step of every operator runs in libmc2's HIP kernels.  There is no
CPU or PyTorch fallback: if ``libmc2.so`` is missing, importing this package
raises.

Functions carry the C names:
  mc2_allgather_matmul, mc2_allgather_arrival_fallbacks, mc2_matmul_grad_input, mc2_matmul_grad_weight,
  mc2_matmul_reduce_scatter,
  mc2_alltoall_quant_matmul_workspace_size, mc2_alltoall_quant_matmul, mc2_alltoall_quant_matmul_static,
  mc2_quant_all_reduce, mc2_quant_reduce_scatter, mc2_status_string, mc2_last_error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmc2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python comm_matmul_tensor_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

# status codes and dtype codes of include/mc2.h
MC2_OK = 0
STATUS_NAMES = {0: "MC2_OK", 1: "MC2_ERR_NULL", 2: "MC2_ERR_SHAPE", 3: "MC2_ERR_DTYPE",
                4: "MC2_ERR_UNSUPPORTED", 5: "MC2_ERR_WORKSPACE", 6: "MC2_ERR_NO_DEVICE",
                7: "MC2_ERR_HIP", 8: "MC2_ERR_ALIGN"}
MC2_F32, MC2_F16, MC2_BF16, MC2_I8, MC2_I32, MC2_F8E4M3FN, MC2_F8E5M2, MC2_E8M0 = range(8)
MC2_AG_FUSED_WRITE, MC2_AG_ARRIVAL = 0, 1

_TORCH_DT = {
    torch.float32: MC2_F32, torch.float16: MC2_F16, torch.bfloat16: MC2_BF16, torch.int8: MC2_I8,
    torch.int32: MC2_I32, torch.float8_e4m3fn: MC2_F8E4M3FN, torch.float8_e5m2: MC2_F8E5M2,
}
if hasattr(torch, "float8_e8m0fnu"):
    _TORCH_DT[torch.float8_e8m0fnu] = MC2_E8M0

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGS = {
    "mc2_allgather_matmul": [_P, _INT, _I64, _I64, _P, _I64, _INT, _INT, _P, _P, _INT, _INT, _P],
    "mc2_matmul_grad_input": [_P, _P, _I64, _I64, _I64, _INT, _P, _P],
    "mc2_matmul_grad_weight": [_P, _P, _I64, _I64, _I64, _INT, _P, _P],
    "mc2_alltoall_quant_matmul_workspace_size": [_INT, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "mc2_alltoall_quant_matmul": [_P, _INT, _I64, _I64, _INT, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, ctypes.c_size_t, _P],
    "mc2_quant_all_reduce": [_P, _P, _INT, _I64, _I64, _INT, _INT, _P, _INT, _P],
    "mc2_quant_reduce_scatter": [_P, _P, _INT, _INT, _I64, _I64, _INT, _INT, _P, _INT, _P],
    "mc2_allgather_arrival_fallbacks": [_INT, ctypes.POINTER(ctypes.c_uint)],
    "mc2_matmul_reduce_scatter": [_P, _P, _INT, _INT, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P],
    "mc2_alltoall_quant_matmul_static": [_P, _INT, _I64, _I64, _P, _P, _I64, _P, _P, _P, _INT, _P, _P, _P],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.mc2_status_string.argtypes = [ctypes.c_int]
_lib.mc2_status_string.restype = ctypes.c_char_p
_lib.mc2_last_error.argtypes = []
_lib.mc2_last_error.restype = ctypes.c_char_p


class Mc2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def mc2_status_string(status: int) -> str:
    return _lib.mc2_status_string(status).decode()


def mc2_last_error() -> str:
    return _lib.mc2_last_error().decode()


def _check(status: int):
    if status != MC2_OK:
        raise Mc2Error(status, mc2_last_error() or mc2_status_string(status))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], name: str):
    return None if t is None else _dev(t, name)


def _ptrs(ts: Sequence[torch.Tensor], name: str):
    return (ctypes.c_void_p * len(ts))(*[_dev(t, f"{name}[{i}]") for i, t in enumerate(ts)])


def _dt(t: torch.Tensor) -> int:
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


# ------------------------------------------------------------------ AllGatherMatmul
def mc2_allgather_matmul(shards: Sequence[torch.Tensor], x2: torch.Tensor, *, x2_trans: bool = False,
                         out: Optional[torch.Tensor] = None, gather_out: Optional[torch.Tensor] = None,
                         gather_output: bool = True, mode: int = MC2_AG_FUSED_WRITE, rank_id: int = 0,
                         stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """out = AllGather_m(shards) @ x2 and gather_out = AllGather_m(shards).

    x2 is (k, n), or with x2_trans=True a (n, k) buffer holding x2^T.
    """
    r = len(shards)
    m_local, k = shards[0].shape
    n = x2.shape[0] if x2_trans else x2.shape[1]
    dev = shards[0].device
    if out is None:
        out = torch.empty((r * m_local, n), dtype=shards[0].dtype, device=dev)
    if gather_out is None and (gather_output or mode == MC2_AG_ARRIVAL):
        gather_out = torch.empty((r * m_local, k), dtype=shards[0].dtype, device=dev)
    for i, s in enumerate(shards):
        if s.shape != (m_local, k) or s.dtype != shards[0].dtype:
            raise ValueError(f"shard {i} has shape {tuple(s.shape)} / {s.dtype}")
    _check(_lib.mc2_allgather_matmul(_ptrs(shards, "shards"), r, m_local, k, _dev(x2, "x2"), n,
                                     int(x2_trans), _dt(shards[0]), _dev(out, "out"),
                                     _opt(gather_out, "gather_out"), mode, rank_id, _stream(stream)))
    return out, gather_out


def mc2_allgather_arrival_fallbacks(reset: bool = False) -> int:
    """GEMM workgroups of MC2_AG_ARRIVAL calls whose wait for a row block timed
    out (they read the shard directly); waits for the device to be idle."""
    n = ctypes.c_uint(0)
    _check(_lib.mc2_allgather_arrival_fallbacks(int(reset), ctypes.byref(n)))
    return n.value


def mc2_matmul_grad_input(dy: torch.Tensor, w: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """dX_partial = dY @ W, W in nn.Linear (out, in) = (n_local, k) layout."""
    m, n_local = dy.shape
    k = w.shape[1]
    if out is None:
        out = torch.empty((m, k), dtype=dy.dtype, device=dy.device)
    _check(_lib.mc2_matmul_grad_input(_dev(dy, "dy"), _dev(w, "w"), m, n_local, k, _dt(dy),
                                      _dev(out, "dx_partial"), _stream(stream)))
    return out


def mc2_matmul_reduce_scatter(x: torch.Tensor, x2: torch.Tensor, recv: Sequence[Optional[torch.Tensor]],
                              rank_id: int, *, x2_trans: bool = False, out: Optional[torch.Tensor] = None,
                              partial_out: Optional[torch.Tensor] = None,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rank rank_id's share of ReduceScatter_m(x @ x2): returns (out, partial_out).
    recv[j] (j != rank_id) is the (m / len(recv), n) block rank j sends; x2 is (k, n), or
    (n, k) with x2_trans (the row-parallel forward passes the nn.Linear weight that way)."""
    ws = len(recv)
    m, k = x.shape
    n = x2.shape[0] if x2_trans else x2.shape[1]
    if (x2.shape[1] if x2_trans else x2.shape[0]) != k:
        raise ValueError("x2 does not match x's contraction size")
    if ws < 1 or m % ws != 0:
        raise ValueError("m must be divisible by the number of ranks")
    for j, b in enumerate(recv):
        if j != rank_id and (b is None or tuple(b.shape) != (m // ws, n) or b.dtype != x.dtype):
            raise ValueError(f"recv[{j}] must be a ({m // ws}, {n}) tensor of x's dtype")
    if out is None:
        out = torch.empty((m // ws, n), dtype=x.dtype, device=x.device)
    if partial_out is None:
        partial_out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    ptrs = (ctypes.c_void_p * ws)(*[None if j == rank_id else _dev(b, f"recv[{j}]") for j, b in enumerate(recv)])
    _check(_lib.mc2_matmul_reduce_scatter(_dev(x, "x"), _dev(x2, "x2"), ws, rank_id, m, k, n, int(bool(x2_trans)),
                                          _dt(x), ptrs, _dev(out, "out"), _dev(partial_out, "partial_out"),
                                          _stream(stream)))
    return out, partial_out


def mc2_matmul_grad_weight(dy: torch.Tensor, ag_x: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """dW = dY^T @ AllGather_m(X)."""
    m, n_local = dy.shape
    k = ag_x.shape[1]
    if out is None:
        out = torch.empty((n_local, k), dtype=dy.dtype, device=dy.device)
    _check(_lib.mc2_matmul_grad_weight(_dev(dy, "dy"), _dev(ag_x, "ag_x"), m, n_local, k, _dt(dy),
                                       _dev(out, "dw"), _stream(stream)))
    return out


# ------------------------------------------------------------------ AlltoAllQuantMatmul
def mc2_alltoall_quant_matmul_workspace_size(rank_size: int, bs: int, h: int, n: int) -> int:
    size = ctypes.c_size_t(0)
    _check(_lib.mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n, ctypes.byref(size)))
    return size.value


def mc2_alltoall_quant_matmul(x1: torch.Tensor, rank_size: int, x2: torch.Tensor, x2_scale: torch.Tensor,
                              x1_smooth: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                              *, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              permuted_out: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                              x1_scale_out: Optional[torch.Tensor] = None, acc_out: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """A16W8 dynamic per-token AlltoAllQuantMatmul; returns out (bs / rank_size, n)."""
    bs, h = x1.shape
    n = x2.shape[1]
    if out is None:
        out = torch.empty((bs // rank_size, n), dtype=x1.dtype, device=x1.device)
    need = mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x1.device)
    _check(_lib.mc2_alltoall_quant_matmul(
        _dev(x1, "x1"), rank_size, bs, h, _dt(x1), _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
        _opt(x1_smooth, "x1_smooth"), _opt(bias, "bias"), _dev(out, "out"), _opt(permuted_out, "permuted_out"),
        _opt(q_out, "q_out"), _opt(x1_scale_out, "x1_scale_out"), _opt(acc_out, "acc_out"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def mc2_alltoall_quant_matmul_static(x1: torch.Tensor, rank_size: int, x1_scale: torch.Tensor, x2: torch.Tensor,
                                     x2_scale: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                                     permuted_out: Optional[torch.Tensor] = None,
                                     acc_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Full-quant AlltoAllQuantMatmul: x1 int8 (bs, h), x1_scale fp32 (bs / rank_size);
    out = (P @ x2) * x1_scale * x2_scale + bias with P the permuted x1."""
    bs, h = x1.shape
    n = x2.shape[1]
    rows = bs // rank_size
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype, device=x1.device)
    if x1.dtype != torch.int8 or x2.dtype != torch.int8:
        raise TypeError("x1 and x2 must be int8")
    if x1_scale.numel() != rows or x2_scale.numel() != n:
        raise ValueError("x1_scale must hold bs / rank_size scales and x2_scale n")
    _check(_lib.mc2_alltoall_quant_matmul_static(_dev(x1, "x1"), rank_size, bs, h, _dev(x1_scale, "x1_scale"),
                                                 _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
                                                 _opt(bias, "bias"), _dev(out, "out"), _dt(out),
                                                 _opt(permuted_out, "permuted_out"), _opt(acc_out, "acc_out"),
                                                 _stream(stream)))
    return out


# ------------------------------------------------------------------ QuantAllReduce
def mc2_quant_all_reduce(x: Sequence[torch.Tensor], scales: Sequence[torch.Tensor], *,
                         out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """out = sum_i x[i] * scales[i] (pergroup fp32 scales, or E8M0 mx scales)."""
    r = len(x)
    shape = tuple(x[0].shape)
    h = shape[-1]
    rows = 1
    for s in shape[:-1]:
        rows *= s
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=x[0].device)
    if tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    per_scale = 128 if _dt(scales[0]) == MC2_F32 else 32
    for i in range(r):
        if tuple(x[i].shape) != shape or x[i].dtype != x[0].dtype or scales[i].dtype != scales[0].dtype:
            raise ValueError(f"rank {i} tensors differ from rank 0")
        if scales[i].numel() * per_scale != rows * h:
            raise ValueError(f"scales[{i}] holds {scales[i].numel()} scales, expected {rows * h // per_scale}")
    _check(_lib.mc2_quant_all_reduce(_ptrs(x, "x"), _ptrs(scales, "scales"), r, rows, h, _dt(x[0]),
                                     _dt(scales[0]), _dev(out, "out"), _dt(out), _stream(stream)))
    return out


def mc2_quant_reduce_scatter(x: Sequence[torch.Tensor], scales: Sequence[torch.Tensor], rank_id: int, *,
                             out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """Rows [rank_id rows / r, (rank_id + 1) rows / r) of mc2_quant_all_reduce's sum, as a
    (rows / r, h) tensor (rows = the product of x's leading dimensions)."""
    r = len(x)
    shape = tuple(x[0].shape)
    h = shape[-1]
    rows = 1
    for s in shape[:-1]:
        rows *= s
    if rows % r != 0:
        raise ValueError("rows must be divisible by the number of ranks")
    if out is None:
        out = torch.empty((rows // r, h), dtype=out_dtype, device=x[0].device)
    if out.numel() != rows // r * h:
        raise ValueError(f"out holds {out.numel()} elements, expected {rows // r * h}")
    per_scale = 128 if _dt(scales[0]) == MC2_F32 else 32
    for i in range(r):
        if tuple(x[i].shape) != shape or x[i].dtype != x[0].dtype or scales[i].dtype != scales[0].dtype:
            raise ValueError(f"rank {i} tensors differ from rank 0")
        if scales[i].numel() * per_scale != rows * h:
            raise ValueError(f"scales[{i}] holds {scales[i].numel()} scales, expected {rows * h // per_scale}")
    _check(_lib.mc2_quant_reduce_scatter(_ptrs(x, "x"), _ptrs(scales, "scales"), r, rank_id, rows, h, _dt(x[0]),
                                         _dt(scales[0]), _dev(out, "out"), _dt(out), _stream(stream)))
    return out


__all__ = [
    "mc2_allgather_matmul", "mc2_allgather_arrival_fallbacks", "mc2_matmul_grad_input", "mc2_matmul_grad_weight",
    "mc2_matmul_reduce_scatter",
    "mc2_alltoall_quant_matmul_workspace_size", "mc2_alltoall_quant_matmul", "mc2_alltoall_quant_matmul_static",
    "mc2_quant_all_reduce", "mc2_quant_reduce_scatter",
    "mc2_status_string", "mc2_last_error", "Mc2Error", "LIB_PATH",
]
