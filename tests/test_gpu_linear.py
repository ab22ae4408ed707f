"""The tensor-parallel layer's bias, its gradient and the autograd layers on the GPU.

- mc2_allgather_matmul_bias / mc2_matmul_reduce_scatter_bias against the oracle's
  fused op followed by its bias add (hyper_parallel mc2.py, the two forward
  functions), gather_out bit for bit;
- mc2_bias_grad bit for bit against the oracle (both sum exactly in fp64 and round
  once at these inputs);
- AllGatherMatmulFunction, MatmulReduceScatterFunction and MC2Linear (a whole
  group of r ranks on one GPU): every output and gradient against the oracle
  steps composed in the listing's order, and against the unsharded layer
  x W^T + b computed in fp64 (the same bound).
Float bound: |gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref).
"""
import numpy as np
import pytest

import mc2_inputs
import oracle
from parity import assert_bits_equal, assert_close16, decode16

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FC1


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available()
    import comm_matmul_tensor_amd as m
    return m


def gen(seed, tid, shape, std=1.0, dtype="bf16"):
    return mc2_inputs.fill(seed, tid, "normal", 0.0, std, dtype, shape)


T = mc2_inputs.to_torch
F = mc2_inputs.from_torch


# ---------------------------------------------------------------- bias entry points
@pytest.mark.parametrize("r,m_l,k,n,x2_trans,mode", [
    (4, 16, 512, 64, False, "fused"), (8, 5, 1000, 130, True, "fused"), (2, 129, 256, 129, False, "nogather"),
    (4, 64, 512, 200, True, "arrival"), (8, 128, 512, 224, False, "arrival"), (8, 512, 256, 4096, True, "nogather")])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_allgather_matmul_bias(mc2, r, m_l, k, n, x2_trans, mode, dtype):
    import torch
    print(f"ag+bias r={r} m_l={m_l} k={k} n={n} trans={x2_trans} {mode} {dtype}", flush=True)
    seed = 300 + r + m_l + k + n
    shards = [gen(seed, i, (m_l, k), 1.0, dtype) for i in range(r)]
    x2 = gen(seed, 20, (n, k) if x2_trans else (k, n), 0.05, dtype)
    bias = gen(seed, 21, (n,), 1.0, dtype)
    md = mc2.MC2_AG_ARRIVAL if mode == "arrival" else mc2.MC2_AG_FUSED_WRITE
    mc2.mc2_allgather_arrival_fallbacks(reset=True)
    out, g = mc2.mc2_allgather_matmul_bias([T(s, dtype) for s in shards], T(x2, dtype), T(bias, dtype),
                                           x2_trans=x2_trans, gather_output=(mode != "nogather"), mode=md,
                                           rank_id=r - 1)
    torch.cuda.synchronize()
    want, want_g = oracle.allgather_matmul(shards, x2, dtype, x2_trans=x2_trans)
    assert_close16(F(out), oracle.add_bias(want, bias, dtype), dtype, "out")
    if mode != "nogather":
        assert_bits_equal(F(g), want_g, "gather_out")
    else:
        assert g is None
    assert mc2.mc2_allgather_arrival_fallbacks() == 0


def test_allgather_matmul_bias_full_config(mc2):
    """8 x bf16 (512, 4096) @ (4096, 1792) + a (1792,) bias: every element."""
    import torch
    seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
    t = mc2_inputs.make("ag_bf16_tp")
    shards = [t[f"shard{i}"] for i in range(d["r"])]
    bias = gen(seed, 99, (d["n"],), 1.0)
    out, g = mc2.mc2_allgather_matmul_bias([T(s, "bf16") for s in shards], T(t["x2"], "bf16"), T(bias, "bf16"))
    torch.cuda.synchronize()
    want, want_g = oracle.allgather_matmul(shards, t["x2"], "bf16")
    assert_bits_equal(F(g), want_g, "gather_out")
    assert_close16(F(out), oracle.add_bias(want, bias, "bf16"), "bf16", "out")


@pytest.mark.parametrize("r,m,k,n,x2_trans,rank", [
    (4, 256, 256, 64, False, 1), (2, 74, 300, 33, True, 0), (8, 4096, 1792, 4096, True, 0),
    (8, 8192, 1792, 4096, False, 5)])
def test_matmul_reduce_scatter_bias(mc2, r, m, k, n, x2_trans, rank):
    import torch
    print(f"rs+bias r={r} m={m} k={k} n={n} trans={x2_trans} rank={rank}", flush=True)
    seed = 400 + r + m + n
    x = gen(seed, 0, (m, k))
    x2 = gen(seed, 1, (n, k) if x2_trans else (k, n), 0.02)
    rows = m // r
    recv = [None if j == rank else gen(seed, 10 + j, (rows, n), 0.85) for j in range(r)]
    bias = gen(seed, 2, (n,))
    part = torch.full((m, n), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out, part = mc2.mc2_matmul_reduce_scatter_bias(T(x, "bf16"), T(x2, "bf16"),
                                                   [None if b is None else T(b, "bf16") for b in recv], rank,
                                                   T(bias, "bf16"), x2_trans=x2_trans, partial_out=part)
    torch.cuda.synchronize()
    ref = oracle.matmul_reduce_scatter(x, x2, recv, rank, "bf16", x2_trans)
    p = F(part)
    own = np.zeros(m, dtype=bool)
    own[rank * rows:(rank + 1) * rows] = True
    assert np.all(p[own].view(np.uint16) == SENTINEL), "own-block rows of partial_out were written"
    assert_close16(p[~own], ref["partial"][~own], "bf16", "partial_out (no bias)")
    assert_close16(F(out), oracle.add_bias(ref["out"], bias, "bf16"), "bf16", "out")


@pytest.mark.parametrize("m,n", [(1, 8), (37, 5), (1000, 264), (3000, 1001), (8192, 1792), (4096, 4096)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bias_grad(mc2, m, n, dtype):
    """Both sides sum exactly in fp64 (the values span few binades) and round once:
    bit for bit, on the vector path (n % 8 == 0) and the per-column one."""
    import torch
    print(f"bias_grad m={m} n={n} {dtype}", flush=True)
    dy = gen(500 + m + n, 0, (m, n), 1.0, dtype)
    gb = mc2.mc2_bias_grad(T(dy, dtype))
    torch.cuda.synchronize()
    assert_bits_equal(F(gb), oracle.bias_grad(dy, dtype), "grad_bias")


def test_bias_grad_full_config(mc2):
    """dY of the column-parallel backward workload, (8192, 1792)."""
    import torch
    t = mc2_inputs.make("colpar_bwd")
    gb = mc2.mc2_bias_grad(T(t["dy"], "bf16"))
    torch.cuda.synchronize()
    assert_bits_equal(F(gb), oracle.bias_grad(t["dy"], "bf16"), "grad_bias")


# ---------------------------------------------------------------- the autograd layers
def _leaf(a, dtype="bf16"):
    return T(a, dtype).requires_grad_(True)


def test_column_parallel_function(mc2):
    """AllGatherMatmulFunction for r = 4 ranks: outputs and all gradients."""
    import torch
    from comm_matmul_tensor_amd.linear import AllGatherMatmulFunction
    r, m_l, k, n_l, seed = 4, 64, 256, 256, 600
    xs = [gen(seed, i, (m_l, k)) for i in range(r)]
    ws = [gen(seed, 10 + j, (n_l, k), 0.05) for j in range(r)]
    bs = [gen(seed, 20 + j, (n_l,)) for j in range(r)]
    gs = [gen(seed, 30 + j, (r * m_l, n_l)) for j in range(r)]
    X, W, B = [_leaf(a) for a in xs], [_leaf(a) for a in ws], [_leaf(a) for a in bs]
    outs = AllGatherMatmulFunction.apply(r, True, *X, *W, *B)
    torch.autograd.backward(outs, [T(g, "bf16") for g in gs])
    torch.cuda.synchronize()
    # the oracle steps in the listing's order
    gathered = oracle.allgather(xs)
    for j in range(r):
        o, _ = oracle.allgather_matmul(xs, ws[j], "bf16", x2_trans=True)
        assert_close16(F(outs[j].detach()), oracle.add_bias(o, bs[j], "bf16"), "bf16", f"out[{j}]")
    partial = [oracle.matmul_grad_input(gs[j], ws[j]) for j in range(r)]
    for i in range(r):
        recv = [None if j == i else partial[j][i * m_l:(i + 1) * m_l] for j in range(r)]
        ref = oracle.matmul_reduce_scatter(gs[i], ws[i], recv, i, "bf16")
        assert_close16(F(X[i].grad), ref["out"], "bf16", f"grad_x[{i}]")
    for j in range(r):
        assert_close16(F(W[j].grad), oracle.matmul_grad_weight(gs[j], gathered), "bf16", f"grad_w[{j}]")
        assert_bits_equal(F(B[j].grad), oracle.bias_grad(gs[j], "bf16"), f"grad_bias[{j}]")
    # the unsharded layer y = X W^T + b in fp64
    d = lambda a: decode16(a, "bf16")
    Xf, Wf, bf, Gf = d(gathered), d(np.concatenate(ws)), d(np.concatenate(bs)), d(np.concatenate(gs, axis=1))
    enc = lambda a: oracle.encode("bf16", a)
    y = np.concatenate([F(o.detach()) for o in outs], axis=1)
    assert_close16(y, enc(Xf @ Wf.T + bf), "bf16", "layer output vs x W^T + b")
    gx = np.concatenate([F(x.grad) for x in X])
    assert_close16(gx, enc(Gf @ Wf), "bf16", "grad_x vs dY W")
    gw = np.concatenate([F(w.grad) for w in W])
    assert_close16(gw, enc(Gf.T @ Xf), "bf16", "grad_w vs dY^T X")


def test_row_parallel_function(mc2):
    """MatmulReduceScatterFunction for r = 4 ranks: outputs and all gradients."""
    import torch
    from comm_matmul_tensor_amd.linear import MatmulReduceScatterFunction
    r, m, k_l, n, seed = 4, 256, 256, 256, 700
    rows = m // r
    xs = [gen(seed, j, (m, k_l)) for j in range(r)]
    ws = [gen(seed, 10 + j, (n, k_l), 0.05) for j in range(r)]
    b = gen(seed, 20, (n,))
    gs = [gen(seed, 30 + i, (rows, n)) for i in range(r)]
    X, W, B = [_leaf(a) for a in xs], [_leaf(a) for a in ws], _leaf(b)
    outs = MatmulReduceScatterFunction.apply(r, True, *X, *W, B)
    torch.autograd.backward(outs, [T(g, "bf16") for g in gs])
    torch.cuda.synchronize()
    # oracle: each rank's partial, the blocks it sends, the reduce and the bias
    partial = [oracle.matmul(xs[j], ws[j], "bf16", b_trans=True) for j in range(r)]
    for i in range(r):
        recv = [None if j == i else partial[j][i * rows:(i + 1) * rows] for j in range(r)]
        ref = oracle.matmul_reduce_scatter(xs[i], ws[i], recv, i, "bf16", True)
        assert_close16(F(outs[i].detach()), oracle.add_bias(ref["out"], b, "bf16"), "bf16", f"out[{i}]")
    full = oracle.allgather(gs)
    for j in range(r):
        gx, _ = oracle.allgather_matmul(gs, ws[j], "bf16")
        assert_close16(F(X[j].grad), gx, "bf16", f"grad_x[{j}]")
        assert_close16(F(W[j].grad), oracle.matmul_grad_weight(full, xs[j]), "bf16", f"grad_w[{j}]")
    assert_bits_equal(F(B.grad), oracle.bias_grad(full, "bf16"), "grad_bias")
    d = lambda a: decode16(a, "bf16")
    Xf, Wf = d(np.concatenate(xs, axis=1)), d(np.concatenate(ws, axis=1))
    y = np.concatenate([F(o.detach()) for o in outs])
    assert_close16(y, oracle.encode("bf16", Xf @ Wf.T + d(b)), "bf16", "layer output vs x W^T + b")


@pytest.mark.parametrize("mode", ["allgather", "reduce_scatter"])
@pytest.mark.parametrize("seq_dim", [0, 1, -2])
def test_mc2linear_sequence_dim(mc2, mode, seq_dim):
    """MC2Linear on (batch, seq, hidden) inputs with the sequence along seq_dim: the
    per-rank outputs equal the unsharded layer applied to the concatenated sequence,
    sliced as the mode distributes it."""
    import torch
    from comm_matmul_tensor_amd.linear import MC2Linear
    r, bsz, s, hin, hout, seed = 4, 2, 64, 1024, 256 * 4, 800
    lin = MC2Linear(hin, hout, r, mode, bias=True, sequence_dim=seq_dim)
    with torch.no_grad():
        for j, w in enumerate(lin.weights):
            w.copy_(T(gen(seed, 10 + j, tuple(w.shape), 0.05), "bf16"))
        for j, b in enumerate(lin.biases):
            b.copy_(T(gen(seed, 20 + j, tuple(b.shape)), "bf16"))
    sd = seq_dim % 2
    if mode == "allgather":   # each rank holds s / r of the sequence and all features
        shape = (bsz, s // r, hin) if sd == 1 else (s // r, bsz, hin)
        xs = [gen(seed, i, shape) for i in range(r)]
    else:                     # each rank holds the whole sequence and hin / r features
        shape = (bsz, s, hin // r) if sd == 1 else (s, bsz, hin // r)
        xs = [gen(seed, i, shape) for i in range(r)]
    outs = lin([T(x, "bf16") for x in xs])
    torch.cuda.synchronize()
    d = lambda a: decode16(a, "bf16")
    W = [d(F(w.detach())) for w in lin.weights]
    Bs = [d(F(b.detach())) for b in lin.biases]
    if mode == "allgather":
        xfull = np.concatenate([d(x) for x in xs], axis=sd)                 # the whole sequence
        for j in range(r):
            want = xfull @ W[j].T + Bs[j]
            assert outs[j].shape == want.shape
            assert_close16(F(outs[j].detach()), oracle.encode("bf16", want), "bf16", f"rank {j}")
    else:
        y = sum(d(xs[j]) @ W[j].T for j in range(r)) + Bs[0]                # all features, whole sequence
        for i in range(r):
            sl = [slice(None)] * 3
            sl[sd] = slice(i * s // r, (i + 1) * s // r)
            want = y[tuple(sl)]
            assert outs[i].shape == want.shape
            assert_close16(F(outs[i].detach()), oracle.encode("bf16", want), "bf16", f"rank {i}")
