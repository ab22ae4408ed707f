"""MatmulReduceScatter (one rank's share) on the GPU vs the oracle.

Small shapes run the whole system: every rank's operands are generated, the
blocks rank `rank` receives are the oracle's partials of the other ranks, and
the GPU output is compared with the oracle's share.  partial_out rows of the
own block must stay untouched.  Tolerance for 16-bit outputs:
|gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref); integer-valued operands must
match bit for bit (every partial and every sum is exact).
"""
import numpy as np
import pytest

import mc2_inputs
import oracle
from parity import assert_bits_equal, assert_close16

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1  # a NaN pattern in both 16-bit formats


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available()
    import comm_matmul_tensor_amd as m
    return m


def _system(r, m, k, n, x2_trans, dtype, seed):
    """Operands of every rank (rank j: seed + j)."""
    xs, x2s = [], []
    for j in range(r):
        specs = mc2_inputs.configs.scaled("rs", r=r, m=m, k=k, n=n, x2_trans=x2_trans, w_std=0.05)
        for key in ("x", "x2"):
            s = specs[key]
            specs[key] = mc2_inputs.TensorSpec(s.tid, s.shape, s.dist, s.a, s.b, dtype)
        t = mc2_inputs.make({"x": specs["x"], "x2": specs["x2"]}, seed=seed + j)
        xs.append(t["x"])
        x2s.append(t["x2"])
    return xs, x2s


def _recv_for(rank, xs, x2s, dtype, x2_trans):
    r = len(xs)
    rows = xs[0].shape[0] // r
    return [None if j == rank else
            oracle.matmul(np.ascontiguousarray(xs[j][rank * rows:(rank + 1) * rows]), x2s[j], dtype, b_trans=x2_trans)
            for j in range(r)]


def _gpu(mc2, x, x2, recv, rank, x2_trans, dtype):
    import torch
    T = mc2_inputs.to_torch
    m = x.shape[0]
    n = x2.shape[0] if x2_trans else x2.shape[1]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    part = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda").view(tdt)
    out, part = mc2.mc2_matmul_reduce_scatter(T(x, dtype), T(x2, dtype), [None if b is None else T(b, dtype)
                                              for b in recv], rank, x2_trans=x2_trans, partial_out=part)
    torch.cuda.synchronize()
    return mc2_inputs.from_torch(out), mc2_inputs.from_torch(part)


def _check_partial(part, ref_part, rank, r, dtype):
    rows = part.shape[0] // r
    own = np.zeros(part.shape[0], dtype=bool)
    own[rank * rows:(rank + 1) * rows] = True
    assert np.all(part[own].view(np.uint16) == SENTINEL), "own-block rows of partial_out were written"
    assert_close16(part[~own], ref_part[~own], dtype, "partial_out")


# (r, m, k, n, x2_trans, dtype, rank): tile-aligned blocks, blocks that straddle
# tiles (m / r = 37), ragged n, k off the 8-element vector path, n = 1, a
# GEMM large enough for the 128 x 256 tile, and two with 4096 x 4096 partials
# (x2 given as (n, k): the 256 x 256 tile; x2 as (k, n): 256 x 128)
@pytest.mark.parametrize("r,m,k,n,x2_trans,dtype,rank", [
    (2, 256, 256, 128, False, "bf16", 1), (4, 512, 512, 256, True, "bf16", 2), (8, 1024, 320, 200, False, "f16", 5),
    (8, 296, 256, 72, True, "bf16", 7), (4, 100, 300, 33, False, "bf16", 0), (2, 64, 1000, 1, False, "f16", 0),
    (8, 1024, 512, 448, True, "f16", 3), (4, 1536, 768, 512, False, "bf16", 1),
    (8, 4096, 256, 2048, True, "bf16", 6), (2, 4096, 256, 4096, True, "bf16", 1),
    (2, 4096, 320, 4096, False, "f16", 0)])
def test_rs_shapes(mc2, r, m, k, n, x2_trans, dtype, rank):
    print(f"rs r={r} m={m} k={k} n={n} trans={x2_trans} {dtype} rank={rank}", flush=True)
    xs, x2s = _system(r, m, k, n, x2_trans, dtype, seed=300 + r + m + k)
    recv = _recv_for(rank, xs, x2s, dtype, x2_trans)
    ref = oracle.matmul_reduce_scatter(xs[rank], x2s[rank], recv, rank, dtype, x2_trans)
    out, part = _gpu(mc2, xs[rank], x2s[rank], recv, rank, x2_trans, dtype)
    _check_partial(part, ref["partial"], rank, r, dtype)
    assert_close16(out, ref["out"], dtype, "out")


@pytest.mark.parametrize("dtype,x2_trans", [("bf16", False), ("f16", True)])
def test_rs_exact_integer_system(mc2, dtype, x2_trans):
    """Operands in {-1, 0, 1}: partials and sums are exact integers, so every rank's
    output is bit-exact and the stacked outputs equal the unsharded int64 product."""
    rng = np.random.default_rng(31)
    r, m, k, n = 4, 256, 256, 64
    xi = [rng.integers(-1, 2, (m, k)) for _ in range(r)]
    wi = [rng.integers(-1, 2, (k, n)) for _ in range(r)]
    enc = (lambda a: a.astype(np.float16)) if dtype == "f16" else \
        (lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    xs = [enc(a) for a in xi]
    x2s = [enc(np.ascontiguousarray(w.T) if x2_trans else w) for w in wi]
    full = np.hstack(xi).astype(np.int64) @ np.vstack(wi).astype(np.int64)
    outs = []
    for rank in range(r):
        recv = _recv_for(rank, xs, x2s, dtype, x2_trans)
        out, part = _gpu(mc2, xs[rank], x2s[rank], recv, rank, x2_trans, dtype)
        ref = oracle.matmul_reduce_scatter(xs[rank], x2s[rank], recv, rank, dtype, x2_trans)
        assert_bits_equal(out, ref["out"], f"out rank {rank}")
        rows = m // r
        keep = np.ones(m, dtype=bool)
        keep[rank * rows:(rank + 1) * rows] = False
        assert_bits_equal(part[keep], ref["partial"][keep], f"partial rank {rank}")
        outs.append(out)
    got = np.concatenate(outs)
    if dtype == "f16":
        want = full.astype(np.float16)
    else:  # round-to-nearest-even by the library conversion (exact integers in fp32)
        import torch
        want = mc2_inputs.from_torch(torch.from_numpy(full.astype(np.float32)).to(torch.bfloat16))
    assert_bits_equal(got, want, "stacked outputs vs unsharded product")


def test_rs_largest_contraction(mc2):
    """k = 65534, the largest contraction the fused kernel accepts."""
    r, m, k, n, rank = 2, 32, 65534, 24, 1
    xs, x2s = _system(r, m, k, n, False, "bf16", seed=91)
    recv = _recv_for(rank, xs, x2s, "bf16", False)
    ref = oracle.matmul_reduce_scatter(xs[rank], x2s[rank], recv, rank, "bf16", False)
    out, part = _gpu(mc2, xs[rank], x2s[rank], recv, rank, False, "bf16")
    _check_partial(part, ref["partial"], rank, r, "bf16")
    assert_close16(out, ref["out"], "bf16", "out")


def test_rs_repeated_calls_and_ranks(mc2):
    """Same operands, every rank id in turn, twice: each call writes only its own block."""
    r, m, k, n = 4, 512, 256, 128
    xs, x2s = _system(r, m, k, n, True, "bf16", seed=77)
    for _ in range(2):
        for rank in range(r):
            recv = _recv_for(rank, xs, x2s, "bf16", True)
            ref = oracle.matmul_reduce_scatter(xs[rank], x2s[rank], recv, rank, "bf16", True)
            out, part = _gpu(mc2, xs[rank], x2s[rank], recv, rank, True, "bf16")
            _check_partial(part, ref["partial"], rank, r, "bf16")
            assert_close16(out, ref["out"], "bf16", "out")


@pytest.mark.parametrize("name", ["rs_fwd", "rs_dx"])
def test_rs_full_config(mc2, name):
    """Full workload with the received blocks as generated inputs: every element of
    partial_out (the own block untouched) and of out against the oracle; two runs
    bit-identical."""
    seed, d, specs = mc2_inputs.CONFIGS[name]
    t = mc2_inputs.make(name)
    r, rank, m, k, n, tr = d["r"], d["rank"], d["m"], d["k"], d["n"], d["x2_trans"]
    recv = [None if j == rank else t[f"recv{j}"] for j in range(r)]
    out, part = _gpu(mc2, t["x"], t["x2"], recv, rank, tr, "bf16")
    out2, _ = _gpu(mc2, t["x"], t["x2"], recv, rank, tr, "bf16")
    assert_bits_equal(out, out2, "run-to-run")
    ref = oracle.matmul_reduce_scatter(t["x"], t["x2"], recv, rank, "bf16", tr)
    _check_partial(part, ref["partial"], rank, r, "bf16")
    assert_close16(out, ref["out"], "bf16", "out")
