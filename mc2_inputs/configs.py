"""The synthetic workloads, as tensor specifications.

Each workload lists its tensors in a fixed order; the position in that list is
the tensor id of its random stream, and the seed is the workload number.  The
shapes and value distributions follow the operators' example and production
shapes:

1 ``ag_tiny``     AllGatherMatmul with the torch_npu example's shapes:
                  8 ranks, gathered input (128, 512), x2 (512, 64), fp16.
2 ``ag_bf16_tp``  AllGatherMatmul for one tensor-parallel layer: 8 shards of
                  bf16 (512, 4096), x2 bf16 (4096, 1792) with std 0.02.
3 ``a16w8``       AlltoAllQuantMatmul, A16W8 dynamic per-token: x1 bf16
                  (8192, 4096) seen as (8, 1024, 4096), smooth scale bf16
                  (32768) in U(0.5, 2), x2 int8 (32768, 7168) in U{-127..127},
                  per-channel fp32 x2 scale (7168) in U(1e-3, 1e-2), bf16 bias.
4 ``colpar_bwd``  column-parallel backward: dY bf16 (8192, 1792), W bf16
                  (1792, 4096) in nn.Linear (out, in) layout with std 0.02,
                  AG(X) bf16 (8192, 4096).
5 ``qar_int8``    QuantAllReduce over 8 ranks, x int8 (4, 2048, 7168) with fp32
                  per-128-group scales (4, 2048, 56) in U(1e-3, 1e-2).
5 ``qar_mx``      QuantAllReduce over 8 ranks, x FLOAT8_E4M3FN from N(0, 1)
                  with saturation, E8M0 scales (4, 2048, 112, 2) with
                  exponents U{-8..0}.
6 ``a8w8``        AlltoAllQuantMatmul, full quantisation: x1 int8 (8192, 4096)
                  in U{-127..127} seen as (8, 1024, 4096), one fp32 scale per
                  permuted token (1024) in U(0.02, 0.04) (absmax / 127 of a
                  unit-normal row of 32768 values is about 0.034), x2 int8
                  (32768, 7168), x2 scale and bias as in ``a16w8``.
7 ``rs_fwd``      MatmulReduceScatter, row-parallel forward of the same TP layer,
                  one rank of 8: x bf16 (4096, 1792), w bf16 (4096, 1792) in
                  nn.Linear (out, in) layout with std 0.02 (x2 = w^T), and the
                  7 partial blocks (512, 4096) the other ranks send, bf16 with
                  the partials' std 0.02 sqrt(1792) = 0.85 (recv0 unused: rank 0).
8 ``rs_dx``       MatmulReduceScatter completing the column-parallel dX: dY bf16
                  (8192, 1792), W bf16 (1792, 4096) with std 0.02, blocks
                  (1024, 4096) with std 0.85 (rank 0).
9 ``a16w4``       AlltoAllQuantMatmul A16W4: ``a16w8``'s tensors with int4 weight
                  codes U{-8..7} (32768, 7168), stored two per byte (pack_int4).
10 ``a4w4``       AlltoAllQuantMatmul A4W4 (full quantisation): x1 int4 codes
                  U{-8..7} (8192, 4096), one fp32 scale per permuted token in
                  U(0.5, 0.7) (absmax / 7 of a unit-normal row is about 0.64),
                  int4 weight codes as in ``a16w4``, scales and bias as ``a8w8``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

import numpy as np


@dataclass(frozen=True)
class TensorSpec:
    tid: int
    shape: Tuple[int, ...]
    dist: str  # "normal" (a = mean, b = std), "uniform" [a, b), "int" a..b
    a: float
    b: float
    dtype: str


def _ag(r, m_local, k, n, dtype, x2_std):
    specs = {f"shard{i}": TensorSpec(i, (m_local, k), "normal", 0.0, 1.0, dtype) for i in range(r)}
    specs["x2"] = TensorSpec(r, (k, n), "normal", 0.0, x2_std, dtype)
    return specs


def _a16w8(r, bs, h, n):
    return {
        "x1": TensorSpec(0, (bs, h), "normal", 0.0, 1.0, "bf16"),
        "x1_smooth": TensorSpec(1, (r * h,), "uniform", 0.5, 2.0, "bf16"),
        "x2": TensorSpec(2, (r * h, n), "int", -127, 127, "i8"),
        "x2_scale": TensorSpec(3, (n,), "uniform", 1e-3, 1e-2, "f32"),
        "bias": TensorSpec(4, (n,), "normal", 0.0, 1.0, "bf16"),
    }


def _a8w8(r, bs, h, n):
    return {
        "x1": TensorSpec(0, (bs, h), "int", -127, 127, "i8"),
        "x1_scale": TensorSpec(1, (bs // r,), "uniform", 0.02, 0.04, "f32"),
        "x2": TensorSpec(2, (r * h, n), "int", -127, 127, "i8"),
        "x2_scale": TensorSpec(3, (n,), "uniform", 1e-3, 1e-2, "f32"),
        "bias": TensorSpec(4, (n,), "normal", 0.0, 1.0, "bf16"),
    }


def _a16w4(r, bs, h, n):
    """A16W8's tensors with int4 weight codes (-8..7); pack_int4 stores them two per byte."""
    specs = _a16w8(r, bs, h, n)
    specs["x2"] = TensorSpec(2, (r * h, n), "int", -8, 7, "i8")
    return specs


def _a4w4(r, bs, h, n):
    """Full-quantisation tensors with int4 activation and weight codes (-8..7) and
    per-token activation scales of about absmax / 7 of a unit-normal row."""
    specs = _a8w8(r, bs, h, n)
    specs["x1"] = TensorSpec(0, (bs, h), "int", -8, 7, "i8")
    specs["x1_scale"] = TensorSpec(1, (bs // r,), "uniform", 0.5, 0.7, "f32")
    specs["x2"] = TensorSpec(2, (r * h, n), "int", -8, 7, "i8")
    return specs


def _rs(r, m, k, n, x2_trans, w_std=0.02):
    specs = {
        "x": TensorSpec(0, (m, k), "normal", 0.0, 1.0, "bf16"),
        "x2": TensorSpec(1, (n, k) if x2_trans else (k, n), "normal", 0.0, w_std, "bf16"),
    }
    for j in range(r):
        specs[f"recv{j}"] = TensorSpec(2 + j, (m // r, n), "normal", 0.0, w_std * float(np.sqrt(k)), "bf16")
    return specs


def _bwd(m, n_local, k):
    return {
        "dy": TensorSpec(0, (m, n_local), "normal", 0.0, 1.0, "bf16"),
        "w": TensorSpec(1, (n_local, k), "normal", 0.0, 0.02, "bf16"),
        "ag_x": TensorSpec(2, (m, k), "normal", 0.0, 1.0, "bf16"),
    }


def _qar_int8(r, shape):
    *lead, h = shape
    specs = {f"x{i}": TensorSpec(i, tuple(shape), "int", -127, 127, "i8") for i in range(r)}
    for i in range(r):
        specs[f"scale{i}"] = TensorSpec(8 + i, tuple(lead) + (h // 128,), "uniform", 1e-3, 1e-2, "f32")
    return specs


def _qar_mx(r, shape):
    *lead, h = shape
    specs = {f"x{i}": TensorSpec(16 + i, tuple(shape), "normal", 0.0, 1.0, "e4m3fn") for i in range(r)}
    for i in range(r):
        specs[f"scale{i}"] = TensorSpec(24 + i, tuple(lead) + (h // 64, 2), "int", -8, 0, "e8m0")
    return specs


# name -> (seed, {"r": ranks, other scalars}, tensor specs)
CONFIGS: Dict[str, tuple] = {
    "ag_tiny": (1, {"r": 8, "m_local": 16, "k": 512, "n": 64, "dtype": "f16"},
                _ag(8, 16, 512, 64, "f16", 1.0)),
    "ag_bf16_tp": (2, {"r": 8, "m_local": 512, "k": 4096, "n": 1792, "dtype": "bf16"},
                   _ag(8, 512, 4096, 1792, "bf16", 0.02)),
    "a16w8": (3, {"r": 8, "bs": 8192, "h": 4096, "n": 7168}, _a16w8(8, 8192, 4096, 7168)),
    "colpar_bwd": (4, {"m": 8192, "n_local": 1792, "k": 4096}, _bwd(8192, 1792, 4096)),
    "qar_int8": (5, {"r": 8, "shape": (4, 2048, 7168)}, _qar_int8(8, (4, 2048, 7168))),
    "qar_mx": (5, {"r": 8, "shape": (4, 2048, 7168)}, _qar_mx(8, (4, 2048, 7168))),
    "a8w8": (6, {"r": 8, "bs": 8192, "h": 4096, "n": 7168}, _a8w8(8, 8192, 4096, 7168)),
    "rs_fwd": (7, {"r": 8, "rank": 0, "m": 4096, "k": 1792, "n": 4096, "x2_trans": True},
               _rs(8, 4096, 1792, 4096, True)),
    "rs_dx": (8, {"r": 8, "rank": 0, "m": 8192, "k": 1792, "n": 4096, "x2_trans": False},
              _rs(8, 8192, 1792, 4096, False)),
    "a16w4": (9, {"r": 8, "bs": 8192, "h": 4096, "n": 7168}, _a16w4(8, 8192, 4096, 7168)),
    "a4w4": (10, {"r": 8, "bs": 8192, "h": 4096, "n": 7168}, _a4w4(8, 8192, 4096, 7168)),
}


def scaled(kind: str, **dims):
    """Specs of a workload family at other sizes (for parity at small shapes)."""
    if kind == "ag":
        return _ag(dims["r"], dims["m_local"], dims["k"], dims["n"], dims["dtype"],
                   dims.get("x2_std", 1.0))
    if kind == "a16w8":
        return _a16w8(dims["r"], dims["bs"], dims["h"], dims["n"])
    if kind == "a8w8":
        return _a8w8(dims["r"], dims["bs"], dims["h"], dims["n"])
    if kind == "a16w4":
        return _a16w4(dims["r"], dims["bs"], dims["h"], dims["n"])
    if kind == "a4w4":
        return _a4w4(dims["r"], dims["bs"], dims["h"], dims["n"])
    if kind == "rs":
        return _rs(dims["r"], dims["m"], dims["k"], dims["n"], dims["x2_trans"], dims.get("w_std", 0.02))
    if kind == "bwd":
        return _bwd(dims["m"], dims["n_local"], dims["k"])
    if kind == "qar_int8":
        return _qar_int8(dims["r"], dims["shape"])
    if kind == "qar_mx":
        return _qar_mx(dims["r"], dims["shape"])
    raise KeyError(kind)


def make_tensor(seed: int, spec: TensorSpec) -> np.ndarray:
    from . import fill
    return fill(seed, spec.tid, spec.dist, spec.a, spec.b, spec.dtype, spec.shape)


def make(name_or_specs, seed: int = None) -> Dict[str, np.ndarray]:
    """All tensors of a named workload (or of a spec dict with an explicit seed)."""
    if isinstance(name_or_specs, str):
        cfg_seed, _, specs = CONFIGS[name_or_specs]
        seed = cfg_seed if seed is None else seed
    else:
        specs = name_or_specs
        if seed is None:
            raise ValueError("seed required with explicit specs")
    return {k: make_tensor(seed, s) for k, s in specs.items()}
