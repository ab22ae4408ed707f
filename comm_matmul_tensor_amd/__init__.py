"""comm_matmul_tensor_amd -- Python binding of libmc2 (MC2 per-rank compute on MI355X).

A thin ctypes layer over the C ABI declared in ``include/mc2.h``.  It only
marshals arguments: torch supplies device memory and the current HIP stream,
and every step of every operator runs in libmc2's HIP kernels.  There is no
CPU or PyTorch fallback: if ``libmc2.so`` is missing, importing this package
raises.

Functions carry the C names:
  mc2_allgather_matmul, mc2_allgather_matmul_bias, mc2_allgather_arrival_fallbacks, mc2_matmul_grad_input,
  mc2_matmul_grad_weight, mc2_matmul_reduce_scatter, mc2_matmul_reduce_scatter_bias, mc2_bias_grad,
  mc2_alltoall_quant_matmul_workspace_size, mc2_alltoall_quant_matmul, mc2_alltoall_quant_matmul_static,
  mc2_alltoall_quant_matmul_noalloc, mc2_alltoall_quant_matmul_a16w4, mc2_alltoall_quant_matmul_a4w4,
  mc2_quant_all_reduce, mc2_quant_reduce_scatter, mc2_status_string, mc2_last_error;
and the test hook mc2_testing_arrival (csrc/testing.h, outside the public header).

Every call checks each tensor's shape, dtype and device against the sizes it
passes to the library before anything runs on the device (the C ABI sees only
pointers and sizes), and allocates its outputs and workspace on the stream the
kernels run on.
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
    "mc2_testing_arrival": [ctypes.c_uint64, _INT],
    "mc2_alltoall_quant_matmul_noalloc": [_P, _INT, _I64, _I64, _INT, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P],
    "mc2_allgather_matmul_bias": [_P, _INT, _I64, _I64, _P, _I64, _INT, _INT, _P, _P, _P, _INT, _INT, _P],
    "mc2_matmul_reduce_scatter_bias": [_P, _P, _INT, _INT, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P, _P],
    "mc2_bias_grad": [_P, _I64, _I64, _INT, _P, _P],
    "mc2_alltoall_quant_matmul_a16w4": [_P, _INT, _I64, _I64, _INT, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, ctypes.c_size_t, _P],
    "mc2_alltoall_quant_matmul_a4w4": [_P, _INT, _I64, _I64, _P, _P, _I64, _P, _P, _P, _INT, _P, _P,
                                       ctypes.c_size_t, _P],
    "mc2_alltoall_quant_matmul_a16w4_workspace_size": [_INT, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
    "mc2_alltoall_quant_matmul_a4w4_workspace_size": [_INT, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
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


def _stream_obj(stream):
    """The torch stream the call runs on: the current one, a torch stream, or a raw
    hipStream_t handle (wrapped so that allocations are made on it too)."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _want(t, name: str, shape, dtype=None, optional: bool = False):
    """Shape and dtype of one argument, checked before anything touches the device: the
    C ABI sees only pointers and the sizes passed beside them, so a tensor smaller than
    those sizes would be read or written out of bounds."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _same_device(named):
    """Every tensor contiguous and on one device, the current one."""
    named = [(name, t) for name, t in named if t is not None]
    for name, t in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = None
    for name, t in named:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    if dev is not None and dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {dev} but the current device is cuda:{torch.cuda.current_device()}")
    return dev


def _2d(t, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _16bit(t, name: str):
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")


# ------------------------------------------------------------------ AllGatherMatmul
def mc2_allgather_matmul(shards: Sequence[torch.Tensor], x2: torch.Tensor, *, x2_trans: bool = False,
                         out: Optional[torch.Tensor] = None, gather_out: Optional[torch.Tensor] = None,
                         gather_output: bool = True, mode: int = MC2_AG_FUSED_WRITE, rank_id: int = 0,
                         stream=None, _bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """out = AllGather_m(shards) @ x2 and gather_out = AllGather_m(shards).

    x2 is (k, n), or with x2_trans=True a (n, k) buffer holding x2^T.
    """
    r = len(shards)
    if r < 1:
        raise ValueError("no shards")
    m_local, k = _2d(shards[0], "shards[0]")
    _16bit(shards[0], "shards[0]")
    dt = shards[0].dtype
    for i, s in enumerate(shards):
        _want(s, f"shards[{i}]", (m_local, k), dt)
    xs = _2d(x2, "x2")
    n = xs[0] if x2_trans else xs[1]
    _want(x2, "x2", (n, k) if x2_trans else (k, n), dt)
    _want(out, "out", (r * m_local, n), dt, optional=True)
    _want(gather_out, "gather_out", (r * m_local, k), dt, optional=True)
    _want(_bias, "bias", (n,), dt, optional=True)
    dev = _same_device([(f"shards[{i}]", s) for i, s in enumerate(shards)] +
                       [("x2", x2), ("out", out), ("gather_out", gather_out), ("bias", _bias)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((r * m_local, n), dtype=dt, device=dev)
        if gather_out is None and (gather_output or mode == MC2_AG_ARRIVAL):
            gather_out = torch.empty((r * m_local, k), dtype=dt, device=dev)
        if _bias is None:
            _check(_lib.mc2_allgather_matmul(_ptrs(shards, "shards"), r, m_local, k, _dev(x2, "x2"), n,
                                             int(x2_trans), _dt(shards[0]), _dev(out, "out"),
                                             _opt(gather_out, "gather_out"), mode, rank_id, st.cuda_stream))
        else:
            _check(_lib.mc2_allgather_matmul_bias(_ptrs(shards, "shards"), r, m_local, k, _dev(x2, "x2"), n,
                                                  int(x2_trans), _dt(shards[0]), _dev(_bias, "bias"),
                                                  _dev(out, "out"), _opt(gather_out, "gather_out"), mode, rank_id,
                                                  st.cuda_stream))
    return out, gather_out


def mc2_allgather_matmul_bias(shards: Sequence[torch.Tensor], x2: torch.Tensor, bias: torch.Tensor, *,
                              x2_trans: bool = False, out: Optional[torch.Tensor] = None,
                              gather_out: Optional[torch.Tensor] = None, gather_output: bool = True,
                              mode: int = MC2_AG_FUSED_WRITE, rank_id: int = 0,
                              stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The column-parallel layer's forward: out = AllGather_m(shards) @ x2 + bias (bias (n,))."""
    if bias is None:
        raise ValueError("bias is required")
    return mc2_allgather_matmul(shards, x2, x2_trans=x2_trans, out=out, gather_out=gather_out,
                                gather_output=gather_output, mode=mode, rank_id=rank_id, stream=stream, _bias=bias)


def mc2_allgather_arrival_fallbacks(reset: bool = False) -> int:
    """GEMM wavefronts (workgroups on the checked path) of MC2_AG_ARRIVAL calls whose wait
    for a piece of the gathered matrix timed out (they read the shards directly); waits for
    the device to be idle."""
    n = ctypes.c_uint(0)
    _check(_lib.mc2_allgather_arrival_fallbacks(int(reset), ctypes.byref(n)))
    return n.value


def mc2_testing_arrival(wait_ticks: int = 0, raised_slabs: int = -1) -> None:
    """Test hook (csrc/testing.h, not part of include/mc2.h): later arrival-mode calls wait at
    most wait_ticks ticks of the 100 MHz GPU counter per piece (0: the 200 ms default) and the
    copy raises the ready flags of the first raised_slabs slabs of K only (negative: all)."""
    _check(_lib.mc2_testing_arrival(int(wait_ticks), int(raised_slabs)))


def mc2_matmul_grad_input(dy: torch.Tensor, w: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """dX_partial = dY @ W, W in nn.Linear (out, in) = (n_local, k) layout."""
    m, n_local = _2d(dy, "dy")
    _16bit(dy, "dy")
    k = _2d(w, "w")[1]
    _want(w, "w", (n_local, k), dy.dtype)
    _want(out, "out", (m, k), dy.dtype, optional=True)
    dev = _same_device([("dy", dy), ("w", w), ("out", out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((m, k), dtype=dy.dtype, device=dev)
        _check(_lib.mc2_matmul_grad_input(_dev(dy, "dy"), _dev(w, "w"), m, n_local, k, _dt(dy),
                                          _dev(out, "dx_partial"), st.cuda_stream))
    return out


def mc2_matmul_reduce_scatter(x: torch.Tensor, x2: torch.Tensor, recv: Sequence[Optional[torch.Tensor]],
                              rank_id: int, *, x2_trans: bool = False, out: Optional[torch.Tensor] = None,
                              partial_out: Optional[torch.Tensor] = None, stream=None,
                              _bias: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rank rank_id's share of ReduceScatter_m(x @ x2): returns (out, partial_out).
    recv[j] (j != rank_id) is the (m / len(recv), n) block rank j sends; x2 is (k, n), or
    (n, k) with x2_trans (the row-parallel forward passes the nn.Linear weight that way)."""
    ws = len(recv)
    m, k = _2d(x, "x")
    _16bit(x, "x")
    xs = _2d(x2, "x2")
    n = xs[0] if x2_trans else xs[1]
    _want(x2, "x2", (n, k) if x2_trans else (k, n), x.dtype)
    if ws < 1 or m % ws != 0:
        raise ValueError("m must be divisible by the number of ranks")
    if not 0 <= rank_id < ws:
        raise ValueError(f"rank_id {rank_id} outside [0, {ws})")
    for j, b in enumerate(recv):
        if j != rank_id:
            _want(b, f"recv[{j}]", (m // ws, n), x.dtype)
    _want(out, "out", (m // ws, n), x.dtype, optional=True)
    _want(partial_out, "partial_out", (m, n), x.dtype, optional=True)
    _want(_bias, "bias", (n,), x.dtype, optional=True)
    dev = _same_device([("x", x), ("x2", x2), ("out", out), ("partial_out", partial_out), ("bias", _bias)] +
                       [(f"recv[{j}]", b) for j, b in enumerate(recv) if j != rank_id])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((m // ws, n), dtype=x.dtype, device=dev)
        if partial_out is None:
            partial_out = torch.empty((m, n), dtype=x.dtype, device=dev)
        ptrs = (ctypes.c_void_p * ws)(*[None if j == rank_id else _dev(b, f"recv[{j}]")
                                        for j, b in enumerate(recv)])
        if _bias is None:
            _check(_lib.mc2_matmul_reduce_scatter(_dev(x, "x"), _dev(x2, "x2"), ws, rank_id, m, k, n,
                                                  int(bool(x2_trans)), _dt(x), ptrs, _dev(out, "out"),
                                                  _dev(partial_out, "partial_out"), st.cuda_stream))
        else:
            _check(_lib.mc2_matmul_reduce_scatter_bias(_dev(x, "x"), _dev(x2, "x2"), ws, rank_id, m, k, n,
                                                       int(bool(x2_trans)), _dt(x), ptrs, _dev(_bias, "bias"),
                                                       _dev(out, "out"), _dev(partial_out, "partial_out"),
                                                       st.cuda_stream))
    return out, partial_out


def mc2_matmul_reduce_scatter_bias(x: torch.Tensor, x2: torch.Tensor, recv: Sequence[Optional[torch.Tensor]],
                                   rank_id: int, bias: torch.Tensor, *, x2_trans: bool = False,
                                   out: Optional[torch.Tensor] = None, partial_out: Optional[torch.Tensor] = None,
                                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The row-parallel layer's forward share: out = ReduceScatter_m(x @ x2) block + bias (bias (n,))."""
    if bias is None:
        raise ValueError("bias is required")
    return mc2_matmul_reduce_scatter(x, x2, recv, rank_id, x2_trans=x2_trans, out=out, partial_out=partial_out,
                                     stream=stream, _bias=bias)


def mc2_bias_grad(dy: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """grad_bias = dy.sum(dim=0) for dy (m, n), rounded once to dy's dtype."""
    m, n = _2d(dy, "dy")
    _16bit(dy, "dy")
    _want(out, "out", (n,), dy.dtype, optional=True)
    dev = _same_device([("dy", dy), ("out", out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((n,), dtype=dy.dtype, device=dev)
        _check(_lib.mc2_bias_grad(_dev(dy, "dy"), m, n, _dt(dy), _dev(out, "grad_bias"), st.cuda_stream))
    return out


def mc2_matmul_grad_weight(dy: torch.Tensor, ag_x: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """dW = dY^T @ AllGather_m(X)."""
    m, n_local = _2d(dy, "dy")
    _16bit(dy, "dy")
    k = _2d(ag_x, "ag_x")[1]
    _want(ag_x, "ag_x", (m, k), dy.dtype)
    _want(out, "out", (n_local, k), dy.dtype, optional=True)
    dev = _same_device([("dy", dy), ("ag_x", ag_x), ("out", out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((n_local, k), dtype=dy.dtype, device=dev)
        _check(_lib.mc2_matmul_grad_weight(_dev(dy, "dy"), _dev(ag_x, "ag_x"), m, n_local, k, _dt(dy),
                                           _dev(out, "dw"), st.cuda_stream))
    return out


# ------------------------------------------------------------------ AlltoAllQuantMatmul
def mc2_alltoall_quant_matmul_workspace_size(rank_size: int, bs: int, h: int, n: int) -> int:
    size = ctypes.c_size_t(0)
    _check(_lib.mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n, ctypes.byref(size)))
    return size.value


def mc2_alltoall_quant_matmul_a16w4_workspace_size(rank_size: int, bs: int, h: int, n: int) -> int:
    size = ctypes.c_size_t(0)
    _check(_lib.mc2_alltoall_quant_matmul_a16w4_workspace_size(rank_size, bs, h, n, ctypes.byref(size)))
    return size.value


def mc2_alltoall_quant_matmul_a4w4_workspace_size(rank_size: int, bs: int, h: int, n: int) -> int:
    size = ctypes.c_size_t(0)
    _check(_lib.mc2_alltoall_quant_matmul_a4w4_workspace_size(rank_size, bs, h, n, ctypes.byref(size)))
    return size.value


def _a2a_sizes(x1, rank_size, x2):
    bs, h = _2d(x1, "x1")
    if rank_size < 1 or bs % rank_size != 0:
        raise ValueError(f"bs = {bs} must be a multiple of rank_size = {rank_size}")
    n = _2d(x2, "x2")[1]
    _want(x2, "x2", (rank_size * h, n), torch.int8)
    return bs, h, n, bs // rank_size, rank_size * h


def mc2_alltoall_quant_matmul(x1: torch.Tensor, rank_size: int, x2: torch.Tensor, x2_scale: torch.Tensor,
                              x1_smooth: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                              *, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              permuted_out: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                              x1_scale_out: Optional[torch.Tensor] = None, acc_out: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """A16W8 dynamic per-token AlltoAllQuantMatmul; returns out (bs / rank_size, n)."""
    bs, h, n, rows, cols = _a2a_sizes(x1, rank_size, x2)
    _16bit(x1, "x1")
    _want(x2_scale, "x2_scale", (n,), torch.float32)
    _want(x1_smooth, "x1_smooth", (cols,), x1.dtype, optional=True)
    _want(bias, "bias", (n,), x1.dtype, optional=True)
    _want(out, "out", (rows, n), x1.dtype, optional=True)
    _want(permuted_out, "permuted_out", (rows, cols), x1.dtype, optional=True)
    _want(q_out, "q_out", (rows, cols), torch.int8, optional=True)
    _want(x1_scale_out, "x1_scale_out", (rows,), torch.float32, optional=True)
    _want(acc_out, "acc_out", (rows, n), torch.int32, optional=True)
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.dim() != 1):
        raise ValueError("workspace must be a 1-D tensor")
    dev = _same_device([("x1", x1), ("x2", x2), ("x2_scale", x2_scale), ("x1_smooth", x1_smooth),
                        ("bias", bias), ("out", out), ("permuted_out", permuted_out), ("q_out", q_out),
                        ("x1_scale_out", x1_scale_out), ("acc_out", acc_out), ("workspace", workspace)])
    need = mc2_alltoall_quant_matmul_workspace_size(rank_size, bs, h, n)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((rows, n), dtype=x1.dtype, device=dev)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(_lib.mc2_alltoall_quant_matmul(
            _dev(x1, "x1"), rank_size, bs, h, _dt(x1), _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
            _opt(x1_smooth, "x1_smooth"), _opt(bias, "bias"), _dev(out, "out"), _opt(permuted_out, "permuted_out"),
            _opt(q_out, "q_out"), _opt(x1_scale_out, "x1_scale_out"), _opt(acc_out, "acc_out"),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), st.cuda_stream))
    return out


def mc2_alltoall_quant_matmul_a16w4(x1: torch.Tensor, rank_size: int, x2: torch.Tensor, x2_scale: torch.Tensor,
                                    x1_smooth: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                                    *, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                    permuted_out: Optional[torch.Tensor] = None, q_out: Optional[torch.Tensor] = None,
                                    x1_scale_out: Optional[torch.Tensor] = None,
                                    acc_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A16W4: mc2_alltoall_quant_matmul with x2 a uint8 (rank_size h, n / 2) tensor of int4 codes
    (two per byte, low nibble first)."""
    bs, h = _2d(x1, "x1")
    if rank_size < 1 or bs % rank_size != 0:
        raise ValueError(f"bs = {bs} must be a multiple of rank_size = {rank_size}")
    n = 2 * _2d(x2, "x2")[1]
    rows, cols = bs // rank_size, rank_size * h
    _16bit(x1, "x1")
    _want(x2, "x2", (cols, n // 2), torch.uint8)
    _want(x2_scale, "x2_scale", (n,), torch.float32)
    _want(x1_smooth, "x1_smooth", (cols,), x1.dtype, optional=True)
    _want(bias, "bias", (n,), x1.dtype, optional=True)
    _want(out, "out", (rows, n), x1.dtype, optional=True)
    _want(permuted_out, "permuted_out", (rows, cols), x1.dtype, optional=True)
    _want(q_out, "q_out", (rows, cols), torch.int8, optional=True)
    _want(x1_scale_out, "x1_scale_out", (rows,), torch.float32, optional=True)
    _want(acc_out, "acc_out", (rows, n), torch.int32, optional=True)
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.dim() != 1):
        raise ValueError("workspace must be a 1-D tensor")
    dev = _same_device([("x1", x1), ("x2", x2), ("x2_scale", x2_scale), ("x1_smooth", x1_smooth),
                        ("bias", bias), ("out", out), ("permuted_out", permuted_out), ("q_out", q_out),
                        ("x1_scale_out", x1_scale_out), ("acc_out", acc_out), ("workspace", workspace)])
    need = mc2_alltoall_quant_matmul_a16w4_workspace_size(rank_size, bs, h, n)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((rows, n), dtype=x1.dtype, device=dev)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(_lib.mc2_alltoall_quant_matmul_a16w4(
            _dev(x1, "x1"), rank_size, bs, h, _dt(x1), _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
            _opt(x1_smooth, "x1_smooth"), _opt(bias, "bias"), _dev(out, "out"), _opt(permuted_out, "permuted_out"),
            _opt(q_out, "q_out"), _opt(x1_scale_out, "x1_scale_out"), _opt(acc_out, "acc_out"),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), st.cuda_stream))
    return out


def mc2_alltoall_quant_matmul_a4w4(x1: torch.Tensor, rank_size: int, x1_scale: torch.Tensor, x2: torch.Tensor,
                                   x2_scale: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                                   acc_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                   stream=None) -> torch.Tensor:
    """A4W4 full quantisation: x1 uint8 (bs, h / 2) and x2 uint8 (rank_size h, n / 2) tensors of int4
    codes (two per byte, low nibble first), x1_scale fp32 (bs / rank_size)."""
    bs, hb = _2d(x1, "x1")
    h = 2 * hb
    if rank_size < 1 or bs % rank_size != 0:
        raise ValueError(f"bs = {bs} must be a multiple of rank_size = {rank_size}")
    n = 2 * _2d(x2, "x2")[1]
    rows, cols = bs // rank_size, rank_size * h
    if x1.dtype != torch.uint8:
        raise TypeError("x1 must be uint8 (packed int4 codes)")
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"out must be float16 or bfloat16, got {out_dtype}")
    _want(x1_scale, "x1_scale", (rows,), torch.float32)
    _want(x2, "x2", (cols, n // 2), torch.uint8)
    _want(x2_scale, "x2_scale", (n,), torch.float32)
    _want(bias, "bias", (n,), out_dtype, optional=True)
    _want(out, "out", (rows, n), out_dtype, optional=True)
    _want(acc_out, "acc_out", (rows, n), torch.int32, optional=True)
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or workspace.dim() != 1):
        raise ValueError("workspace must be a 1-D tensor")
    dev = _same_device([("x1", x1), ("x1_scale", x1_scale), ("x2", x2), ("x2_scale", x2_scale), ("bias", bias),
                        ("out", out), ("acc_out", acc_out), ("workspace", workspace)])
    need = mc2_alltoall_quant_matmul_a4w4_workspace_size(rank_size, bs, h, n)
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((rows, n), dtype=out_dtype, device=dev)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check(_lib.mc2_alltoall_quant_matmul_a4w4(_dev(x1, "x1"), rank_size, bs, h, _dev(x1_scale, "x1_scale"),
                                                   _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"), _opt(bias, "bias"),
                                                   _dev(out, "out"), _dt(out), _opt(acc_out, "acc_out"),
                                                   _dev(workspace, "workspace"),
                                                   workspace.numel() * workspace.element_size(), st.cuda_stream))
    return out


# bytes of the library's own scratch array (include/mc2.h, MC2_NOALLOC_SCRATCH_BYTES)
MC2_NOALLOC_SCRATCH_BYTES = 48 << 20


def mc2_alltoall_quant_matmul_noalloc(x1: torch.Tensor, rank_size: int, x2: torch.Tensor, x2_scale: torch.Tensor,
                                      x1_smooth: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                                      *, out: torch.Tensor, permuted_out: Optional[torch.Tensor] = None,
                                      q_out: Optional[torch.Tensor] = None,
                                      x1_scale_out: Optional[torch.Tensor] = None,
                                      acc_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mc2_alltoall_quant_matmul for callers that cannot allocate: `out` must be given, and the
    workspace is the library's own per-GPU array (calls overlapping on one GPU race on it)."""
    bs, h, n, rows, cols = _a2a_sizes(x1, rank_size, x2)
    _16bit(x1, "x1")
    _want(x2_scale, "x2_scale", (n,), torch.float32)
    _want(x1_smooth, "x1_smooth", (cols,), x1.dtype, optional=True)
    _want(bias, "bias", (n,), x1.dtype, optional=True)
    _want(out, "out", (rows, n), x1.dtype)
    _want(permuted_out, "permuted_out", (rows, cols), x1.dtype, optional=True)
    _want(q_out, "q_out", (rows, cols), torch.int8, optional=True)
    _want(x1_scale_out, "x1_scale_out", (rows,), torch.float32, optional=True)
    _want(acc_out, "acc_out", (rows, n), torch.int32, optional=True)
    _same_device([("x1", x1), ("x2", x2), ("x2_scale", x2_scale), ("x1_smooth", x1_smooth), ("bias", bias),
                  ("out", out), ("permuted_out", permuted_out), ("q_out", q_out), ("x1_scale_out", x1_scale_out),
                  ("acc_out", acc_out)])
    st = _stream_obj(stream)
    _check(_lib.mc2_alltoall_quant_matmul_noalloc(
        _dev(x1, "x1"), rank_size, bs, h, _dt(x1), _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
        _opt(x1_smooth, "x1_smooth"), _opt(bias, "bias"), _dev(out, "out"), _opt(permuted_out, "permuted_out"),
        _opt(q_out, "q_out"), _opt(x1_scale_out, "x1_scale_out"), _opt(acc_out, "acc_out"), st.cuda_stream))
    return out


def mc2_alltoall_quant_matmul_static(x1: torch.Tensor, rank_size: int, x1_scale: torch.Tensor, x2: torch.Tensor,
                                     x2_scale: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
                                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                                     permuted_out: Optional[torch.Tensor] = None,
                                     acc_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Full-quant AlltoAllQuantMatmul: x1 int8 (bs, h), x1_scale fp32 (bs / rank_size);
    out = (P @ x2) * x1_scale * x2_scale + bias with P the permuted x1."""
    bs, h, n, rows, cols = _a2a_sizes(x1, rank_size, x2)
    if x1.dtype != torch.int8:
        raise TypeError("x1 must be int8")
    if out is not None:
        out_dtype = out.dtype
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"out must be float16 or bfloat16, got {out_dtype}")
    _want(x1_scale, "x1_scale", (rows,), torch.float32)
    _want(x2_scale, "x2_scale", (n,), torch.float32)
    _want(bias, "bias", (n,), out_dtype, optional=True)
    _want(out, "out", (rows, n), out_dtype, optional=True)
    _want(permuted_out, "permuted_out", (rows, cols), torch.int8, optional=True)
    _want(acc_out, "acc_out", (rows, n), torch.int32, optional=True)
    dev = _same_device([("x1", x1), ("x1_scale", x1_scale), ("x2", x2), ("x2_scale", x2_scale), ("bias", bias),
                        ("out", out), ("permuted_out", permuted_out), ("acc_out", acc_out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((rows, n), dtype=out_dtype, device=dev)
        _check(_lib.mc2_alltoall_quant_matmul_static(_dev(x1, "x1"), rank_size, bs, h, _dev(x1_scale, "x1_scale"),
                                                     _dev(x2, "x2"), n, _dev(x2_scale, "x2_scale"),
                                                     _opt(bias, "bias"), _dev(out, "out"), _dt(out),
                                                     _opt(permuted_out, "permuted_out"), _opt(acc_out, "acc_out"),
                                                     st.cuda_stream))
    return out


# ------------------------------------------------------------------ QuantAllReduce
def _qar_sizes(x, scales):
    r = len(x)
    if r < 1 or len(scales) != r:
        raise ValueError("x and scales need one tensor per rank")
    if not isinstance(x[0], torch.Tensor) or x[0].dim() < 2:
        raise ValueError("x[0] must be a tensor of 2 or more dimensions")
    shape = tuple(x[0].shape)
    h = shape[-1]
    rows = 1
    for s in shape[:-1]:
        rows *= s
    if not isinstance(scales[0], torch.Tensor):
        raise TypeError("scales[0] must be a torch.Tensor")
    per_scale = 128 if _dt(scales[0]) == MC2_F32 else 32
    for i in range(r):
        _want(x[i], f"x[{i}]", shape, x[0].dtype)
        if not isinstance(scales[i], torch.Tensor) or scales[i].dtype != scales[0].dtype:
            raise TypeError(f"scales[{i}] must be a tensor of scales[0]'s dtype")
        if scales[i].numel() * per_scale != rows * h:
            raise ValueError(f"scales[{i}] holds {scales[i].numel()} scales, expected {rows * h // per_scale}")
    return r, shape, rows, h


def mc2_quant_all_reduce(x: Sequence[torch.Tensor], scales: Sequence[torch.Tensor], *,
                         out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """out = sum_i x[i] * scales[i] (pergroup fp32 scales, or E8M0 mx scales)."""
    r, shape, rows, h = _qar_sizes(x, scales)
    if out is not None:
        out_dtype = out.dtype
    _want(out, "out", shape, out_dtype, optional=True)
    dev = _same_device([(f"x[{i}]", t) for i, t in enumerate(x)] + [(f"scales[{i}]", t) for i, t in enumerate(scales)]
                       + [("out", out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty(shape, dtype=out_dtype, device=dev)
        _check(_lib.mc2_quant_all_reduce(_ptrs(x, "x"), _ptrs(scales, "scales"), r, rows, h, _dt(x[0]),
                                         _dt(scales[0]), _dev(out, "out"), _dt(out), st.cuda_stream))
    return out


def mc2_quant_reduce_scatter(x: Sequence[torch.Tensor], scales: Sequence[torch.Tensor], rank_id: int, *,
                             out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """Rows [rank_id rows / r, (rank_id + 1) rows / r) of mc2_quant_all_reduce's sum, as a
    (rows / r, h) tensor (rows = the product of x's leading dimensions)."""
    r, shape, rows, h = _qar_sizes(x, scales)
    if rows % r != 0:
        raise ValueError("rows must be divisible by the number of ranks")
    if out is not None:
        out_dtype = out.dtype
    _want(out, "out", (rows // r, h), out_dtype, optional=True)
    dev = _same_device([(f"x[{i}]", t) for i, t in enumerate(x)] + [(f"scales[{i}]", t) for i, t in enumerate(scales)]
                       + [("out", out)])
    st = _stream_obj(stream)
    with torch.cuda.stream(st):
        if out is None:
            out = torch.empty((rows // r, h), dtype=out_dtype, device=dev)
        _check(_lib.mc2_quant_reduce_scatter(_ptrs(x, "x"), _ptrs(scales, "scales"), r, rank_id, rows, h,
                                             _dt(x[0]), _dt(scales[0]), _dev(out, "out"), _dt(out), st.cuda_stream))
    return out


__all__ = [
    "mc2_allgather_matmul", "mc2_allgather_matmul_bias", "mc2_allgather_arrival_fallbacks",
    "mc2_matmul_grad_input", "mc2_matmul_grad_weight", "mc2_matmul_reduce_scatter", "mc2_matmul_reduce_scatter_bias",
    "mc2_bias_grad",
    "mc2_alltoall_quant_matmul_workspace_size", "mc2_alltoall_quant_matmul", "mc2_alltoall_quant_matmul_static",
    "mc2_alltoall_quant_matmul_noalloc", "MC2_NOALLOC_SCRATCH_BYTES", "mc2_alltoall_quant_matmul_a16w4",
    "mc2_alltoall_quant_matmul_a4w4", "mc2_alltoall_quant_matmul_a16w4_workspace_size",
    "mc2_alltoall_quant_matmul_a4w4_workspace_size",
    "mc2_quant_all_reduce", "mc2_quant_reduce_scatter",
    "mc2_status_string", "mc2_last_error", "Mc2Error", "LIB_PATH",
]
