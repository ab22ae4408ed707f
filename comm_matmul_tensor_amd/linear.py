"""Tensor-parallel linear layers over libmc2 on one GPU.

The hyper_parallel ``tensor_parallel/mc2.py`` listing pairs each fused
operator with a custom backward and wraps both in ``MC2Linear``:

* ``AllGatherMatmulFunction`` (column-parallel): forward
  ``out = AllGather_m(x) @ w^T + bias``; backward ``grad_x =
  ReduceScatter_m(grad_out @ w)``, ``grad_w = grad_out^T @ AllGather_m(x)``,
  ``grad_bias = grad_out.sum(0)``.
* ``MatmulReduceScatterFunction`` (row-parallel): forward ``out =
  ReduceScatter_m(x @ w^T) + bias``; backward ``grad_x, grad_out_full =
  AllGather_m(grad_out) @ w``, ``grad_w = grad_out_full^T @ x``,
  ``grad_bias = grad_out_full.sum(0)``.
* ``MC2Linear._mc2_forward``: the fused ops gather and scatter along the
  first dimension of a 2-D activation, so the sequence dimension is moved
  to the front, the leading dimensions are flattened, and the result is
  reshaped and moved back.

On one GPU the r ranks of a tensor-parallel group are r sets of buffers on
the same device, so these functions take and return one tensor per rank and
run every rank's share: each step is a libmc2 call (the GEMMs, the gathers,
the reduce-scatter sums, the bias and its gradient all run in its HIP
kernels).  The only torch operations are allocations, views and, for a
sequence dimension other than 0, the permute-and-copy of the dimension move
(data movement, as in the listing).
"""
from __future__ import annotations

from typing import List, Sequence

import torch

from . import (mc2_allgather_matmul, mc2_bias_grad, mc2_matmul_grad_input, mc2_matmul_grad_weight,
               mc2_matmul_reduce_scatter)

__all__ = ["AllGatherMatmulFunction", "MatmulReduceScatterFunction", "MC2Linear", "move_dim_to_front",
           "move_front_to_dim", "normalize_sequence_dim"]


def normalize_sequence_dim(sequence_dim: int, ndim_leading: int) -> int:
    """A possibly negative sequence dimension resolved against the leading dimensions."""
    d = sequence_dim + ndim_leading if sequence_dim < 0 else sequence_dim
    if not 0 <= d < ndim_leading:
        raise ValueError(f"sequence_dim={sequence_dim} is out of range for {ndim_leading} leading dimensions")
    return d


def move_dim_to_front(t: torch.Tensor, dim: int) -> torch.Tensor:
    if dim == 0:
        return t
    order = (dim,) + tuple(i for i in range(t.dim()) if i != dim)
    return t.permute(*order).contiguous()


def move_front_to_dim(t: torch.Tensor, dim: int) -> torch.Tensor:
    """Inverse of move_dim_to_front."""
    if dim == 0:
        return t
    order = tuple(range(1, dim + 1)) + (0,) + tuple(range(dim + 1, t.dim()))
    return t.permute(*order).contiguous()


class AllGatherMatmulFunction(torch.autograd.Function):
    """Column-parallel fused AllGather + matmul of a whole group on one GPU.

    Inputs: r, has_bias, then x_0..x_{r-1} (m_local, k) (rank i's rows),
    w_0..w_{r-1} (n_local, k) (rank j's rows of the nn.Linear weight) and,
    with has_bias, b_0..b_{r-1} (n_local,).  Returns out_0..out_{r-1}, each
    (r m_local, n_local): rank j's columns of the layer output.
    """

    @staticmethod
    def forward(ctx, r: int, has_bias: bool, *ts):  # noqa: D401
        xs, ws = list(ts[:r]), list(ts[r:2 * r])
        bs = list(ts[2 * r:3 * r]) if has_bias else [None] * r
        outs, gathered = [], None
        for j in range(r):
            # x2 = w_j^T: the (n_local, k) weight passed as a transposed view
            out, g = mc2_allgather_matmul(xs, ws[j], x2_trans=True, gather_output=(j == 0), _bias=bs[j])
            if j == 0:
                gathered = g
            outs.append(out)
        ctx.r, ctx.has_bias = r, has_bias
        ctx.save_for_backward(gathered, *ws)
        return tuple(outs)

    @staticmethod
    def backward(ctx, *grad_outs):
        r = ctx.r
        gathered, *ws = ctx.saved_tensors
        gos = [g.contiguous() for g in grad_outs]
        m_local = gathered.shape[0] // r
        # each rank's dY_j @ W_j; rank i keeps the sum over j of block i
        partial = [mc2_matmul_grad_input(gos[j], ws[j]) for j in range(r)]
        grad_x = []
        for i in range(r):
            recv = [None if j == i else partial[j][i * m_local:(i + 1) * m_local] for j in range(r)]
            out, _ = mc2_matmul_reduce_scatter(gos[i], ws[i], recv, i)
            grad_x.append(out)
        grad_w = [mc2_matmul_grad_weight(gos[j], gathered) for j in range(r)]
        grads = [None, None] + grad_x + grad_w
        if ctx.has_bias:
            grads += [mc2_bias_grad(gos[j]) for j in range(r)]
        return tuple(grads)


class MatmulReduceScatterFunction(torch.autograd.Function):
    """Row-parallel fused matmul + ReduceScatter of a whole group on one GPU.

    Inputs: r, has_bias, then x_0..x_{r-1} (m, k_local) (rank j's columns of
    the activation), w_0..w_{r-1} (n, k_local) (rank j's columns of the
    nn.Linear weight) and, with has_bias, the replicated bias (n,).  Returns
    out_0..out_{r-1}, each (m / r, n): rank i's rows of the layer output.

    Rank i's sum needs block i of every other rank's partial product before
    its own call runs, so each rank first produces the blocks it sends (a
    call with zero blocks received, whose partial_out holds them) and then
    runs its reduce-scatter share with the blocks of the others: on one GPU
    every rank's GEMM runs twice (on r GPUs, once).
    """

    @staticmethod
    def forward(ctx, r: int, has_bias: bool, *ts):
        xs, ws = list(ts[:r]), list(ts[r:2 * r])
        bias = ts[2 * r] if has_bias else None
        m, n = xs[0].shape[0], ws[0].shape[0]
        rows = m // r
        zero = torch.zeros((rows, n), dtype=xs[0].dtype, device=xs[0].device)
        sent = []
        for j in range(r):
            _, part = mc2_matmul_reduce_scatter(xs[j], ws[j], [None if i == j else zero for i in range(r)], j,
                                                x2_trans=True)
            sent.append(part)
        outs = []
        for i in range(r):
            recv = [None if j == i else sent[j][i * rows:(i + 1) * rows] for j in range(r)]
            out, _ = mc2_matmul_reduce_scatter(xs[i], ws[i], recv, i, x2_trans=True, _bias=bias)
            outs.append(out)
        ctx.r, ctx.has_bias = r, has_bias
        ctx.save_for_backward(*xs, *ws)
        return tuple(outs)

    @staticmethod
    def backward(ctx, *grad_outs):
        r = ctx.r
        saved = ctx.saved_tensors
        xs, ws = saved[:r], saved[r:2 * r]
        gos = [g.contiguous() for g in grad_outs]
        grad_x, grad_w, full = [], [], None
        for j in range(r):
            # AllGather_m(dY) @ W_j with W_j (n, k_local) as x2 (k = n); the gathered dY once
            gx, g = mc2_allgather_matmul(gos, ws[j], gather_output=(j == 0))
            if j == 0:
                full = g
            grad_x.append(gx)
        for j in range(r):
            grad_w.append(mc2_matmul_grad_weight(full, xs[j]))
        grads = [None, None] + grad_x + grad_w
        if ctx.has_bias:
            grads.append(mc2_bias_grad(full))
        return tuple(grads)


class MC2Linear(torch.nn.Module):
    """The listing's MC2Linear for a whole tensor-parallel group on one GPU.

    mode "allgather" (column-parallel): weight rows split over the r ranks,
    each rank's input holds its slice of the sequence dimension, and each
    rank's output holds the whole sequence and its n / r output features.
    mode "reduce_scatter" (row-parallel): weight columns split over the
    ranks, each rank's input holds the whole sequence and its in / r
    features, and each rank's output holds its slice of the sequence and all
    n features.  forward takes and returns one tensor per rank, of shape
    (..., features) with the sequence along `sequence_dim`.
    """

    def __init__(self, in_features: int, out_features: int, world_size: int, mode: str, bias: bool = True,
                 sequence_dim: int = 0, dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        if mode not in ("allgather", "reduce_scatter"):
            raise ValueError(f"unknown mode {mode!r}")
        r = world_size
        self.mode, self.r, self.sequence_dim = mode, r, sequence_dim
        self.in_features, self.out_features = in_features, out_features
        if mode == "allgather":
            if out_features % r:
                raise ValueError("out_features must be divisible by world_size")
            shape_w, shape_b = (out_features // r, in_features), (out_features // r,)
            nb = r
        else:
            if in_features % r:
                raise ValueError("in_features must be divisible by world_size")
            shape_w, shape_b = (out_features, in_features // r), (out_features,)
            nb = 1
        kw = dict(dtype=dtype, device=device)
        self.weights = torch.nn.ParameterList([torch.nn.Parameter(torch.empty(shape_w, **kw)) for _ in range(r)])
        self.biases = torch.nn.ParameterList([torch.nn.Parameter(torch.empty(shape_b, **kw)) for _ in range(nb)]
                                             if bias else [])

    def forward(self, inputs: Sequence[torch.Tensor]) -> List[torch.Tensor]:
        r = self.r
        if len(inputs) != r:
            raise ValueError(f"expected {r} per-rank inputs, got {len(inputs)}")
        lead = tuple(inputs[0].shape[:-1])
        seq = normalize_sequence_dim(self.sequence_dim, len(lead))
        flat = []
        for x in inputs:
            xf = move_dim_to_front(x, seq)
            flat.append(xf.reshape(-1, xf.shape[-1]))
        other = tuple(d for i, d in enumerate(lead) if i != seq)
        has_bias = len(self.biases) > 0
        fn = AllGatherMatmulFunction if self.mode == "allgather" else MatmulReduceScatterFunction
        outs = fn.apply(r, has_bias, *flat, *self.weights, *self.biases)
        if self.mode == "allgather":
            seq_out = lead[seq] * r       # the gather expands the sequence dimension
        else:
            if lead[seq] % r:
                raise ValueError(f"sequence dimension {seq} (size {lead[seq]}) must be divisible by {r}")
            seq_out = lead[seq] // r      # the reduce-scatter splits it
        res = []
        for o in outs:
            o = o.reshape(seq_out, *other, o.shape[-1])
            res.append(move_front_to_dim(o, seq))
        return res
