"""Pins for the oracle's operators (CPU).

Every check compares the oracle with something that is not the oracle: hand
worked fixtures from the pages' formulas (tests/golden), exact rational brute
force on tiny inputs, integer special cases that any correct implementation
must reproduce exactly, library routines (numpy int64 / float64 matmul,
reshape / transpose), and invariants the pages state (the fused result equals
gather-then-multiply, dX / dW adjointness, the per-token quant error bound).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import mc2_inputs
import oracle
from brute import decode16, exact_matmul, near_tie, round_rne

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def enc(vals, fmt):
    """Brute-force encode of exact values (test-side, not the oracle's encoder)."""
    arr = np.array([round_rne(v, fmt) for v in np.asarray(vals, dtype=np.float64).ravel()],
                   dtype=np.uint16).reshape(np.shape(vals))
    return arr.view(np.float16) if fmt == "f16" else arr


def bits(a):
    return np.asarray(a).view(np.uint16)


# ----------------------------------------------------------------- AllGatherMatmul
def test_ag_worked_example():
    g = gold("worked_examples.json")["allgather_matmul"]
    shards = [enc(s, "bf16") for s in g["shards"]]
    out, gat = oracle.allgather_matmul(shards, enc(g["x2"], "bf16"), "bf16")
    assert np.array_equal(bits(out), bits(enc(g["out"], "bf16")))
    assert np.array_equal(bits(gat), bits(enc(g["gather_out"], "bf16")))


def test_ag_example_shapes_and_gather_is_concat():
    ex = gold("ag_example.json")
    seed, dims, specs = mc2_inputs.CONFIGS["ag_tiny"]
    assert dims["r"] == ex["world_size"]
    assert (dims["r"] * dims["m_local"], dims["k"]) == tuple(ex["x1_shape"])
    assert (dims["k"], dims["n"]) == tuple(ex["x2_shape"])
    assert [dims["m_local"], dims["k"]] == ex["single_shape"]
    assert ex["k_min"] <= dims["k"] < ex["k_max_exclusive"]
    t = mc2_inputs.make("ag_tiny")
    shards = [t[f"shard{i}"] for i in range(dims["r"])]
    out, gat = oracle.allgather_matmul(shards, t["x2"], "f16")
    assert out.shape == tuple(ex["out_shape"]) and gat.shape == tuple(ex["gather_out_shape"])
    assert np.array_equal(bits(gat), bits(np.concatenate(shards, axis=0)))


@pytest.mark.parametrize("r,m_l,k,n,dtype", [
    (2, 1, 256, 1, "bf16"), (2, 3, 300, 7, "f16"), (4, 1, 256, 7, "bf16"), (8, 1, 257, 2, "f16"),
])
def test_ag_matches_exact_rational_brute_force(r, m_l, k, n, dtype):
    specs = mc2_inputs.configs.scaled("ag", r=r, m_local=m_l, k=k, n=n, dtype=dtype)
    t = mc2_inputs.make(specs, seed=100 + r + k)
    shards = [t[f"shard{i}"] for i in range(r)]
    out, _ = oracle.allgather_matmul(shards, t["x2"], dtype)
    a = decode16(np.concatenate(shards), dtype)
    b = decode16(t["x2"], dtype)
    exact = exact_matmul(a, b)
    for i in range(r * m_l):
        for j in range(n):
            want = round_rne(exact[i][j], dtype)
            if near_tie(exact[i][j], dtype):
                continue  # fp64 summation may legitimately land on either side
            assert int(bits(out)[i, j]) == want, (i, j)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ag_exact_integer_case(dtype):
    """Small integers: every partial sum is an exact integer, so the result is the integer matmul."""
    rng = np.random.default_rng(7)
    r, m_l, k, n = 4, 5, 256, 9
    ints = [rng.integers(-2, 3, (m_l, k)) for _ in range(r)]
    x2i = rng.integers(-1, 2, (k, n))
    shards = [enc(s, dtype) for s in ints]
    out, _ = oracle.allgather_matmul(shards, enc(x2i, dtype), dtype)
    want = np.concatenate(ints) @ x2i  # exact integers; rounded to the format by brute force
    assert np.array_equal(bits(out), bits(enc(want, dtype)))


def test_ag_fused_equals_unfused_and_block_invariance():
    specs = mc2_inputs.configs.scaled("ag", r=4, m_local=6, k=320, n=40, dtype="bf16")
    t = mc2_inputs.make(specs, seed=11)
    shards = [t[f"shard{i}"] for i in range(4)]
    out, gat = oracle.allgather_matmul(shards, t["x2"], "bf16")
    assert np.array_equal(out, oracle.matmul(np.concatenate(shards), t["x2"], "bf16"))
    perm = [2, 0, 3, 1]
    out_p, _ = oracle.allgather_matmul([shards[i] for i in perm], t["x2"], "bf16")
    for pos, src in enumerate(perm):
        assert np.array_equal(out_p[pos * 6:(pos + 1) * 6], out[src * 6:(src + 1) * 6])


def test_ag_x2_transposed_view():
    specs = mc2_inputs.configs.scaled("ag", r=2, m_local=4, k=256, n=24, dtype="f16")
    t = mc2_inputs.make(specs, seed=12)
    shards = [t["shard0"], t["shard1"]]
    out, _ = oracle.allgather_matmul(shards, t["x2"], "f16")
    out_t, _ = oracle.allgather_matmul(shards, np.ascontiguousarray(t["x2"].T), "f16", x2_trans=True)
    assert np.array_equal(bits(out), bits(out_t))


def test_ag_against_float64_library_matmul():
    """numpy float64 matmul, then brute-force rounding; near-ties excused."""
    specs = mc2_inputs.configs.scaled("ag", r=8, m_local=2, k=512, n=33, dtype="bf16", x2_std=0.02)
    t = mc2_inputs.make(specs, seed=13)
    shards = [t[f"shard{i}"] for i in range(8)]
    out, _ = oracle.allgather_matmul(shards, t["x2"], "bf16")
    ref = decode16(np.concatenate(shards), "bf16") @ decode16(t["x2"], "bf16")
    want = enc(ref, "bf16")
    diff = np.nonzero(bits(out) != want)
    for i, j in zip(*diff):
        assert abs(int(bits(out)[i, j]) - int(want[i, j])) == 1 and near_tie(Fraction(ref[i, j]), "bf16", 1e-9)


# ----------------------------------------------------------------- MatmulReduceScatter
def _rs_system(xs, x2s, dtype, x2_trans=False):
    """Every rank's share, each fed the blocks the other ranks' partials hold for it."""
    r = len(xs)
    rows = xs[0].shape[0] // r
    shares = [oracle.matmul_reduce_scatter(xs[i], x2s[i], [None] * r, i, dtype, x2_trans) for i in range(r)]
    outs = []
    for i in range(r):
        recv = [None if j == i else np.ascontiguousarray(shares[j]["partial"][i * rows:(i + 1) * rows])
                for j in range(r)]
        outs.append(oracle.matmul_reduce_scatter(xs[i], x2s[i], recv, i, dtype, x2_trans)["out"])
    return [s_["partial"] for s_ in shares], outs


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("x2_trans", [False, True])
def test_rs_exact_integer_system_is_the_unsharded_product(dtype, x2_trans):
    """Row-parallel layer with small-integer operands: every partial and every sum is an
    exact integer, so the ranks' outputs stacked in rank order are X @ W with X = [x_0 | ... |
    x_{r-1}] (K split across the ranks) and W = [w_0; ...; w_{r-1}], here in int64."""
    rng = np.random.default_rng(21)
    r, m, k, n = 4, 12, 32, 5
    xi = [rng.integers(-1, 2, (m, k)) for _ in range(r)]
    wi = [rng.integers(-1, 2, (k, n)) for _ in range(r)]
    xs = [enc(a, dtype) for a in xi]
    x2s = [enc(w.T if x2_trans else w, dtype) for w in wi]
    partials, outs = _rs_system(xs, x2s, dtype, x2_trans)
    for a, w, p in zip(xi, wi, partials):
        assert np.array_equal(bits(p), bits(enc(a @ w, dtype)))
    full = np.hstack(xi).astype(np.int64) @ np.vstack(wi).astype(np.int64)
    assert np.array_equal(bits(np.concatenate(outs)), bits(enc(full, dtype)))


@pytest.mark.parametrize("r,rank,dtype,x2_trans", [(2, 1, "bf16", False), (4, 2, "bf16", True), (4, 0, "f16", False),
                                                   (1, 0, "bf16", False)])
def test_rs_matches_exact_rational_brute_force(r, rank, dtype, x2_trans):
    """partial = RNE of the exact product; out = RNE of the exact sum of the decoded blocks."""
    m, k, n = 2 * r, 6, 3
    x = mc2_inputs.fill(40 + r, 0, "normal", 0.0, 1.0, dtype, (m, k))
    x2 = mc2_inputs.fill(40 + r, 1, "normal", 0.0, 1.0, dtype, (n, k) if x2_trans else (k, n))
    recv = [None if j == rank else mc2_inputs.fill(40 + r, 2 + j, "normal", 0.0, 4.0, dtype, (2, n))
            for j in range(r)]
    res = oracle.matmul_reduce_scatter(x, x2, recv, rank, dtype, x2_trans)
    b = decode16(x2, dtype)
    exact = exact_matmul(decode16(x, dtype), b.T if x2_trans else b)
    for i in range(m):
        for j in range(n):
            if not near_tie(exact[i][j], dtype):
                assert int(bits(res["partial"])[i, j]) == round_rne(exact[i][j], dtype), (i, j)
    for t in range(2):
        for c in range(n):
            terms = [Fraction(float(decode16(res["partial"], dtype)[rank * 2 + t, c])) if j == rank else
                     Fraction(float(decode16(recv[j], dtype)[t, c])) for j in range(r)]
            assert int(bits(res["out"])[t, c]) == round_rne(sum(terms), dtype), (t, c)


def test_rs_is_the_adjoint_of_allgather():
    """The pages call the two operators duals: for exact data, sum_i <RS(P)_i, Z_i> equals
    <P_0 + ... + P_{r-1}, AllGather(Z)>, with the gather taken from the AllGather oracle."""
    rng = np.random.default_rng(22)
    r, m, k, n = 4, 8, 16, 6
    xs = [enc(rng.integers(-1, 2, (m, k)), "bf16") for _ in range(r)]
    x2s = [enc(rng.integers(-1, 2, (k, n)), "bf16") for _ in range(r)]
    partials, outs = _rs_system(xs, x2s, "bf16")
    zs = [enc(rng.integers(-3, 4, (m // r, n)), "bf16") for _ in range(r)]
    lhs = sum(float(np.sum(decode16(o, "bf16") * decode16(z, "bf16"))) for o, z in zip(outs, zs))
    g = oracle.allgather(zs)
    rhs = float(np.sum(sum(decode16(p, "bf16") for p in partials) * decode16(g, "bf16")))
    assert lhs == rhs


# ----------------------------------------------------------------- column-parallel backward
def test_bwd_worked_example():
    g = gold("worked_examples.json")["column_parallel_backward"]
    dy, w, x = (enc(g[k], "bf16") for k in ("dy", "w", "ag_x"))
    assert np.array_equal(bits(oracle.matmul_grad_input(dy, w)), bits(enc(g["dx"], "bf16")))
    assert np.array_equal(bits(oracle.matmul_grad_weight(dy, x)), bits(enc(g["dw"], "bf16")))


def test_bwd_adjoint_identity_exact():
    """<dY, G W^T> = <dY W, G> = <dY^T G, W> with small integers, all exact."""
    rng = np.random.default_rng(3)
    m, n_l, k = 24, 16, 40
    G = rng.integers(-3, 4, (m, k))
    W = rng.integers(-3, 4, (n_l, k))
    dY = rng.integers(-3, 4, (m, n_l))
    Gb, Wb, dYb = enc(G, "bf16"), enc(W, "bf16"), enc(dY, "bf16")
    Y = decode16(oracle.matmul(Gb, Wb, "bf16", b_trans=True), "bf16")       # forward G @ W^T
    dX = decode16(oracle.matmul_grad_input(dYb, Wb), "bf16")
    dW = decode16(oracle.matmul_grad_weight(dYb, Gb), "bf16")
    assert np.array_equal(Y, G @ W.T) and np.array_equal(dX, dY @ W) and np.array_equal(dW, dY.T @ G)
    lhs = np.sum(dY * Y)
    assert lhs == np.sum(dX * G) == np.sum(dW * W)


def test_bwd_dw_is_sum_over_gathered_blocks():
    """dW = dY^T AG(X) = sum_i dY[block i]^T X_i (the gather / dW duality)."""
    rng = np.random.default_rng(4)
    r, m_l, n_l, k = 4, 6, 8, 12
    X = [rng.integers(-3, 4, (m_l, k)) for _ in range(r)]
    dY = rng.integers(-3, 4, (r * m_l, n_l))
    dW = decode16(oracle.matmul_grad_weight(enc(dY, "bf16"), enc(np.concatenate(X), "bf16")), "bf16")
    blocks = sum(dY[i * m_l:(i + 1) * m_l].T @ X[i] for i in range(r))
    assert np.array_equal(dW, blocks)


def test_bwd_against_float64_library_matmul():
    specs = mc2_inputs.configs.scaled("bwd", m=64, n_local=96, k=80)
    t = mc2_inputs.make(specs, seed=14)
    dx = oracle.matmul_grad_input(t["dy"], t["w"])
    dw = oracle.matmul_grad_weight(t["dy"], t["ag_x"])
    for got, ref in ((dx, decode16(t["dy"], "bf16") @ decode16(t["w"], "bf16")),
                     (dw, decode16(t["dy"], "bf16").T @ decode16(t["ag_x"], "bf16"))):
        want = enc(ref, "bf16")
        for i, j in zip(*np.nonzero(got != want)):
            assert near_tie(Fraction(ref[i, j]), "bf16", 1e-9)


# ----------------------------------------------------------------- AlltoAllQuantMatmul
def test_permute_worked_example_and_library_form():
    g = gold("worked_examples.json")["permute"]
    x1 = np.array(g["x1"], dtype=np.uint16)
    assert np.array_equal(oracle.permute(x1, g["rank_size"]), np.array(g["permuted"], dtype=np.uint16))
    rng = np.random.default_rng(5)
    for r, bs, h in ((2, 6, 5), (4, 8, 16), (8, 16, 3), (1, 5, 7)):
        x = rng.integers(0, 65535, (bs, h)).astype(np.uint16)
        p = oracle.permute(x, r)
        assert np.array_equal(p, x.reshape(r, bs // r, h).transpose(1, 0, 2).reshape(bs // r, r * h))
        back = p.reshape(bs // r, r, h).transpose(1, 0, 2).reshape(bs, h)  # inverse permute
        assert np.array_equal(back, x)
        if r == 1:
            assert np.array_equal(p, x)


def test_smooth_quant_worked_example():
    g = gold("worked_examples.json")["smooth_quant"]
    for row, sm, q_want, s_want in zip(g["p"], g["smooth_rows"], g["q"], g["s1"]):
        q, s1 = oracle.smooth_quant(enc([row], "bf16"), enc(sm, "bf16"))
        assert q.tolist() == [q_want] and float(s1[0]) == s_want


def test_smooth_quant_bounds_and_closed_forms():
    specs = mc2_inputs.configs.scaled("a16w8", r=4, bs=64, h=96, n=8)
    t = mc2_inputs.make(specs, seed=15)
    p = oracle.permute(t["x1"], 4)
    q, s1 = oracle.smooth_quant(p, t["x1_smooth"])
    y = decode16(p, "bf16") * decode16(t["x1_smooth"], "bf16")   # exact in fp64
    amax = np.abs(y).max(axis=1)
    assert np.all(s1 > 0)
    # scale is the row absmax over 127, correctly rounded to fp32
    for i in range(len(s1)):
        assert Fraction(float(s1[i])) == Fraction(float(np.float32(Fraction(float(amax[i])) / 127)))
    assert np.all(np.abs(q).max(axis=1) == 127)
    # |q - y/s| <= 1/2 plus the fp32 division error of y/s (|y/s| <= 127: at most 2^-17)
    err = np.abs(q * s1[:, None].astype(np.float64) - y)
    assert np.all(err <= s1[:, None] * (0.5 + 2.0 ** -17))
    # closed form: integer rows whose absmax is 127 with unit smoothing give scale 1, q = y
    rng = np.random.default_rng(6)
    ints = rng.integers(-127, 128, (5, 64))
    ints[:, 3] = 127
    q2, s2 = oracle.smooth_quant(enc(ints, "bf16"), None)
    assert np.all(s2 == 1.0) and np.array_equal(q2, ints)
    # zero row
    q3, s3 = oracle.smooth_quant(np.zeros((2, 32), np.uint16), None)
    assert np.all(q3 == 0) and np.all(s3 == 0)


def test_int8_matmul_and_dequant_worked_example():
    g = gold("worked_examples.json")["int8_matmul_dequant"]
    acc = oracle.int8_matmul(np.array(g["q"], np.int8), np.array(g["x2"], np.int8))
    assert acc.tolist() == g["acc"]
    out = oracle.dequant(acc, np.array(g["s1"], np.float32), np.array(g["s2"], np.float32),
                         enc(g["bias"], "bf16"))
    assert np.array_equal(out, enc(g["out_bf16"], "bf16"))


def test_int8_matmul_vs_int64_library_and_selection():
    rng = np.random.default_rng(8)
    q = rng.integers(-127, 128, (9, 300)).astype(np.int8)
    x2 = rng.integers(-127, 128, (300, 17)).astype(np.int8)
    assert np.array_equal(oracle.int8_matmul(q, x2), q.astype(np.int64) @ x2.astype(np.int64))
    sel = np.zeros((300, 4), np.int8)
    cols = [0, 299, 17, 150]
    for j, c in enumerate(cols):
        sel[c, j] = 1
    assert np.array_equal(oracle.int8_matmul(q, sel), q[:, cols].astype(np.int32))
    # the extreme that the rank_size * H <= 35000 constraint keeps inside int32
    big = oracle.int8_matmul(np.full((1, 35000), -128, np.int8), np.full((35000, 1), -128, np.int8))
    assert int(big[0, 0]) == 35000 * 128 * 128


def test_dequant_unit_and_power_of_two_scales():
    rng = np.random.default_rng(9)
    acc = rng.integers(-2 ** 20, 2 ** 20, (6, 10)).astype(np.int32)
    ones = np.ones(6, np.float32), np.ones(10, np.float32)
    assert np.array_equal(oracle.dequant(acc, *ones, None), enc(acc.astype(np.float64), "bf16"))
    s1 = np.exp2(rng.integers(-10, 3, 6)).astype(np.float32)
    s2 = np.exp2(rng.integers(-12, 0, 10)).astype(np.float32)
    want = enc(acc * s1[:, None].astype(np.float64) * s2[None, :], "bf16")
    assert np.array_equal(oracle.dequant(acc, s1, s2, None), want)


def _exact_dequant_codes(acc, s1, s2, bias_bits, fmt):
    """round(acc x s1 x s2 + bias) from exact rationals, element by element."""
    b = decode16(bias_bits, fmt) if bias_bits is not None else np.zeros(acc.shape[1])
    return np.array([[round_rne(Fraction(int(acc[i, j])) * Fraction(float(s1[i])) * Fraction(float(s2[j]))
                                + Fraction(float(b[j])), fmt) for j in range(acc.shape[1])]
                     for i in range(acc.shape[0])], dtype=np.uint16)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_dequant_exact_rational_non_power_of_two_scales(fmt):
    """acc x s1 x s2 + bias with scales that are not powers of two (up to 79 significant
    bits in the product) equals the exact rational value rounded once, for int32
    accumulators across their whole range and biases of both signs."""
    rng = np.random.default_rng(19)
    m, n = 12, 16
    acc = np.concatenate([rng.integers(-2 ** 31, 2 ** 31, (m // 2, n)),
                          rng.integers(-3000, 3000, (m // 2, n))]).astype(np.int32)
    acc[0, :4] = [2 ** 31 - 1, -2 ** 31, 0, 1]
    s1 = rng.uniform(1e-3, 1e-2, m).astype(np.float32)
    s2 = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    if fmt == "f16":  # keep the products inside fp16's range
        s1 = (s1 * np.float32(2.0 ** -12)).astype(np.float32)
    bias = enc(rng.normal(0.0, 1.0, n) * (100.0 if fmt == "bf16" else 1.0), fmt)
    got = oracle.dequant(acc, s1, s2, bias, fmt)
    want = _exact_dequant_codes(acc, s1, s2, bias, fmt)
    assert np.array_equal(bits(got), want)
    got0 = oracle.dequant(acc, s1, s2, None, fmt)
    assert np.array_equal(bits(got0), _exact_dequant_codes(acc, s1, s2, None, fmt))


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_dequant_far_apart_terms(fmt):
    """Product and bias many binades apart (the smaller term only decides the rounding
    direction), both signs, against exact rationals."""
    rng = np.random.default_rng(23)
    n = 16
    acc = rng.integers(-2 ** 31, 2 ** 31, (4, n)).astype(np.int32)
    lo, hi = (1e-38, 1.0) if fmt == "bf16" else (1e-20, 2.0 ** -22)
    s1 = np.array([lo, lo, hi, hi], np.float32)               # rows 0-1: tiny products
    s2 = rng.uniform(0.3, 0.9, n).astype(np.float32)
    if fmt == "f16":
        s2 = (s2 * np.float32(2.0 ** -8)).astype(np.float32)
    big, small = (3.0e4, 1e-30) if fmt == "bf16" else (1000.0, 2.0 ** -20)
    signs = np.where(rng.integers(0, 2, n) == 1, 1.0, -1.0)
    for b in (big * signs, small * signs):
        bias = enc(b, fmt)
        got = oracle.dequant(acc, s1, s2, bias, fmt)
        assert np.array_equal(bits(got), _exact_dequant_codes(acc, s1, s2, bias, fmt))


def test_dequant_rounds_once_across_a_tie():
    """A product that needs 55 significant bits: acc x s1 x s2 = (2^54 + 1) 2^-80, with
    2^54 + 1 = 1417 x 10325701 x 1231205 (5 13 37 109 246241 279073).  Adding the bias
    2^-34 puts the exact value 2^-80 above the midpoint between the bf16 values 2^-26
    and 2^-26 + 2^-33, so it rounds up; fp64 evaluation would first round the product
    to 2^-26, land exactly on the midpoint and round to even (down)."""
    acc = np.array([[1417]], np.int32)
    s1 = np.array([10325701 * 2.0 ** -40], np.float32)
    s2 = np.array([1231205 * 2.0 ** -40], np.float32)
    assert float(s1[0]) == 10325701 * 2.0 ** -40 and float(s2[0]) == 1231205 * 2.0 ** -40
    assert 1417 * 10325701 * 1231205 == 2 ** 54 + 1
    bias = enc([2.0 ** -34], "bf16")
    got = oracle.dequant(acc, s1, s2, bias, "bf16")
    assert got[0, 0] == round_rne(Fraction(2 ** 54 + 1, 2 ** 80) + Fraction(1, 2 ** 34), "bf16")
    assert decode16(got, "bf16")[0, 0] == 2.0 ** -26 + 2.0 ** -33
    # the same with the opposite sign of the product lands below the midpoint of -2^-26
    got = oracle.dequant(-acc, s1, s2, enc([-2.0 ** -34], "bf16"), "bf16")
    assert decode16(got, "bf16")[0, 0] == -(2.0 ** -26 + 2.0 ** -33)


def test_alltoall_chain_is_composition_of_steps():
    specs = mc2_inputs.configs.scaled("a16w8", r=4, bs=32, h=64, n=24)
    t = mc2_inputs.make(specs, seed=16)
    res = oracle.alltoall_quant_matmul(t["x1"], 4, t["x2"], t["x2_scale"], t["x1_smooth"], t["bias"])
    p = oracle.permute(t["x1"], 4)
    q, s1 = oracle.smooth_quant(p, t["x1_smooth"])
    acc = oracle.int8_matmul(q, t["x2"])
    assert np.array_equal(res["permuted"], p) and np.array_equal(res["q"], q)
    assert np.array_equal(res["s1"], s1) and np.array_equal(res["acc"], acc)
    assert np.array_equal(res["out"], oracle.dequant(acc, s1, t["x2_scale"], t["bias"]))
    # and the float result is close to the unquantised smooth matmul (quantisation error only)
    y = decode16(p, "bf16") * decode16(t["x1_smooth"], "bf16")
    ref = (y @ t["x2"].astype(np.float64)) * t["x2_scale"].astype(np.float64) + decode16(t["bias"], "bf16")
    got = decode16(res["out"], "bf16")
    assert np.max(np.abs(got - ref)) <= 0.02 * np.sqrt(np.mean(ref ** 2)) + 0.01 * np.max(np.abs(ref))


def test_permute_i8_is_the_library_transpose():
    """The byte permute of the full-quant case: the library's reshape/transpose, inverse, r = 1 identity."""
    rng = np.random.default_rng(17)
    for r, bs, h in ((2, 6, 5), (4, 8, 16), (8, 16, 3), (1, 5, 7), (8, 8, 128)):
        x = rng.integers(-128, 128, (bs, h)).astype(np.int8)
        p = oracle.permute_i8(x, r)
        assert np.array_equal(p, x.reshape(r, bs // r, h).transpose(1, 0, 2).reshape(bs // r, r * h))
        assert np.array_equal(p.reshape(bs // r, r, h).transpose(1, 0, 2).reshape(bs, h), x)
        if r == 1:
            assert np.array_equal(p, x)


def test_static_quant_equals_dynamic_on_its_own_codes():
    """Full-quant mode fed with the dynamic path's own int8 codes (permuted back to the
    pre-AlltoAll layout) and its per-token scales reproduces the dynamic output bit for bit:
    both are permute -> exact int8 matmul -> the same dequant."""
    r, bs, h, n = 4, 32, 64, 24
    specs = mc2_inputs.configs.scaled("a16w8", r=r, bs=bs, h=h, n=n)
    t = mc2_inputs.make(specs, seed=18)
    dyn = oracle.alltoall_quant_matmul(t["x1"], r, t["x2"], t["x2_scale"], t["x1_smooth"], t["bias"])
    x1_i8 = dyn["q"].reshape(bs // r, r, h).transpose(1, 0, 2).reshape(bs, h)  # inverse permute (library form)
    st = oracle.alltoall_quant_matmul_static(x1_i8, r, dyn["s1"], t["x2"], t["x2_scale"], t["bias"])
    assert np.array_equal(st["permuted"], dyn["q"])
    assert np.array_equal(st["acc"], dyn["acc"])
    assert np.array_equal(st["out"].view(np.uint16), dyn["out"].view(np.uint16))


def test_static_quant_brute_force_tiny():
    """Python triple loop over the full-quant formulas: acc exact in Python integers, the
    dequant rounded once to bf16 from the exact rational value."""
    rng = np.random.default_rng(19)
    r, bs, h, n = 2, 4, 3, 5
    x1 = rng.integers(-127, 128, (bs, h)).astype(np.int8)
    x2 = rng.integers(-127, 128, (r * h, n)).astype(np.int8)
    s1 = np.array([0.5, 0.0078125], dtype=np.float32)           # per permuted token
    s2 = np.array([0.25, 1.0, 2.0, 0.125, 0.0625], dtype=np.float32)
    bias = enc([1.0, -2.0, 0.5, 0.0, 3.0], "bf16")
    st = oracle.alltoall_quant_matmul_static(x1, r, s1, x2, s2, bias)
    T = bs // r
    for t_ in range(T):
        for c in range(n):
            acc = sum(int(x1[j * T + t_, e]) * int(x2[j * h + e, c]) for j in range(r) for e in range(h))
            assert st["acc"][t_, c] == acc
            exact = Fraction(acc) * Fraction(float(s1[t_])) * Fraction(float(s2[c])) + \
                Fraction(float(decode16(bias[c:c + 1], "bf16")[0]))
            assert int(bits(st["out"])[t_, c]) == round_rne(exact, "bf16")


# ----------------------------------------------------------------- QuantAllReduce
def test_qar_worked_examples():
    w = gold("worked_examples.json")
    g = w["quant_all_reduce_pergroup"]
    h = g["h"]
    xs = [np.repeat(np.array(v, np.int8), 128)[None, :] for v in g["x_group_values"]]
    sc = [np.array([s], np.float32) for s in g["scales"]]
    out = oracle.quant_all_reduce(xs, sc, "i8", "f32", "f32")
    assert out.shape == (1, h)
    assert np.array_equal(out[0], np.repeat(np.array(g["out_group_values"], np.float32), 128))
    g = w["quant_all_reduce_mx"]
    xs = [np.repeat(np.array(v, np.uint8), 32)[None, :] for v in g["x_block_codes"]]
    sc = [np.array(s, np.uint8).reshape(1, g["h"] // 64, 2) for s in g["scale_codes"]]
    out = oracle.quant_all_reduce(xs, sc, "e4m3fn", "e8m0", "bf16")
    assert np.array_equal(out[0], enc(np.repeat(g["out_block_values"], 32), "bf16"))


def test_qar_scale_sizes_match_pages():
    for c in gold("qar_sizes.json")["cases"]:
        specs = mc2_inputs.configs.scaled("qar_int8", r=2, shape=(c["b"], c["s"], c["H"]))
        assert tuple(specs["scale0"].shape) == tuple(c["pergroup_scale_shape"])
        assert np.prod(specs["x0"].shape) == c["x_bytes"]
        assert np.prod(specs["scale0"].shape) * 4 == c["pergroup_scale_bytes"]
        specs = mc2_inputs.configs.scaled("qar_mx", r=2, shape=(c["b"], c["s"], c["H"]))
        assert tuple(specs["scale0"].shape) == tuple(c["mx_scale_shape"])
        assert np.prod(specs["scale0"].shape) == c["mx_scale_bytes"]


@pytest.mark.parametrize("r", [2, 4, 8])
def test_qar_unit_scales_integer_sum(r):
    rng = np.random.default_rng(r)
    xs = [rng.integers(-127, 128, (3, 1024)).astype(np.int8) for _ in range(r)]
    ones = [np.ones((3, 8), np.float32) for _ in range(r)]
    out = oracle.quant_all_reduce(xs, ones, "i8", "f32", "f32")
    assert np.array_equal(out, np.sum([x.astype(np.int64) for x in xs], axis=0).astype(np.float32))
    # mx: E8M0 127 is 1.0; small integers are exact E4M3FN codes
    vals = np.arange(-8, 9)
    codes = {v: int(np.where(oracle.decode("e4m3fn", np.arange(256, dtype=np.uint8)) == v)[0][0]) for v in vals}
    xi = [rng.integers(-8, 9, (2, 1024)) for _ in range(r)]
    xc = [np.vectorize(codes.get)(x).astype(np.uint8) for x in xi]
    s127 = [np.full((2, 16, 2), 127, np.uint8) for _ in range(r)]
    out = oracle.quant_all_reduce(xc, s127, "e4m3fn", "e8m0", "bf16")
    assert np.array_equal(out, enc(np.sum(xi, axis=0).astype(np.float64), "bf16"))


@pytest.mark.parametrize("r", [2, 4, 8])
def test_qrs_blocks_against_library_sum(r):
    """QuantReduceScatter: rank k's output is rows [k rows/r, (k+1) rows/r) of the rank sum.
    Scales are powers of two that differ per row and group, so every product and the fp64
    sum are exact and a wrong row block or scale offset changes the result."""
    rng = np.random.default_rng(60 + r)
    rows, h = 2 * r, 1024
    xs = [rng.integers(-127, 128, (rows, h)).astype(np.int8) for _ in range(r)]
    sc = [np.ldexp(1.0, rng.integers(-12, -2, (rows, h // 128))).astype(np.float32) for _ in range(r)]
    full = sum(x.astype(np.float64) * np.repeat(s_.astype(np.float64), 128, axis=1) for x, s_ in zip(xs, sc))
    for k in range(r):
        out = oracle.quant_reduce_scatter(xs, sc, k, "i8", "f32", "f32")
        assert np.array_equal(out, full[2 * k:2 * k + 2].astype(np.float32))
    # mx: E4M3FN codes of small integers, E8M0 exponents per row and 32-element block
    vals = np.arange(-8, 9)
    codes = {v: int(np.where(oracle.decode("e4m3fn", np.arange(256, dtype=np.uint8)) == v)[0][0]) for v in vals}
    xi = [rng.integers(-8, 9, (rows, h)) for _ in range(r)]
    xc = [np.vectorize(codes.get)(x).astype(np.uint8) for x in xi]
    ex = [rng.integers(120, 128, (rows, h // 64, 2)).astype(np.uint8) for _ in range(r)]
    full = sum(x.astype(np.float64) * np.repeat(np.ldexp(1.0, e.reshape(rows, h // 32).astype(int) - 127), 32, axis=1)
               for x, e in zip(xi, ex))
    for k in range(r):
        out = oracle.quant_reduce_scatter(xc, ex, k, "e4m3fn", "e8m0", "f32")
        assert np.array_equal(out, full[2 * k:2 * k + 2].astype(np.float32))


def test_qar_group_mapping_against_library_repeat():
    """Scales that differ per group reveal the element -> scale mapping."""
    rng = np.random.default_rng(10)
    rows, h, r = 3, 1024, 2
    xs = [np.ones((rows, h), np.int8) for _ in range(r)]
    sc = [np.exp2(rng.integers(-6, 6, (rows, h // 128))).astype(np.float32) for _ in range(r)]
    out = oracle.quant_all_reduce(xs, sc, "i8", "f32", "f32")
    assert np.array_equal(out, np.repeat(sc[0] + sc[1], 128, axis=1))
    one = np.full((rows, h), 0x38, np.uint8)  # E4M3FN 1.0
    e = [rng.integers(120, 135, (rows, h // 64, 2)).astype(np.uint8) for _ in range(r)]
    out = oracle.quant_all_reduce([one, one], e, "e4m3fn", "e8m0", "f32")
    per_block = np.exp2(e[0].reshape(rows, h // 32).astype(np.float64) - 127) + \
        np.exp2(e[1].reshape(rows, h // 32).astype(np.float64) - 127)
    assert np.array_equal(out, np.repeat(per_block, 32, axis=1).astype(np.float32))


def test_qar_exact_rational_on_generated_inputs():
    """Rounded once from the exact sum: compare with Fractions on a slice of the real workload."""
    specs = mc2_inputs.configs.scaled("qar_int8", r=8, shape=(1, 2, 1024))
    t = mc2_inputs.make(specs, seed=5)
    xs = [t[f"x{i}"] for i in range(8)]
    sc = [t[f"scale{i}"] for i in range(8)]
    out = oracle.quant_all_reduce(xs, sc, "i8", "f32", "f32").reshape(2, 1024)
    for tok in range(2):
        for c in range(0, 1024, 37):
            exact = sum(Fraction(int(xs[i].reshape(2, 1024)[tok, c])) *
                        Fraction(float(sc[i].reshape(2, 8)[tok, c // 128])) for i in range(8))
            assert float(out[tok, c]) == float(np.float32(float(exact))) or \
                Fraction(float(out[tok, c])) == Fraction(float(np.float32(exact)))
    specs = mc2_inputs.configs.scaled("qar_mx", r=8, shape=(1, 2, 1024))
    t = mc2_inputs.make(specs, seed=5)
    xs = [t[f"x{i}"] for i in range(8)]
    sc = [t[f"scale{i}"] for i in range(8)]
    out = oracle.quant_all_reduce(xs, sc, "e4m3fn", "e8m0", "bf16").reshape(2, 1024)
    dx = [oracle.decode("e4m3fn", x).reshape(2, 1024) for x in xs]
    for tok in range(2):
        for c in range(0, 1024, 41):
            exact = sum(Fraction(float(dx[i][tok, c])) *
                        Fraction(2) ** (int(sc[i].reshape(2, 32)[tok, c // 32]) - 127) for i in range(8))
            assert int(out[tok, c]) == round_rne(exact, "bf16")


# ----------------------------------------------------------------- layer bias and grad_bias (mc2.py listing)
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_add_bias_exact_rational(fmt):
    """out + bias on 16-bit values equals the exact sum rounded once, including exact
    cancellation, terms many binades apart and (fp16) overflow to infinity."""
    rng = np.random.default_rng(41)
    m, n = 6, 9
    y = enc(rng.normal(0, 1, (m, n)) * np.exp2(rng.integers(-12, 12, (m, n))), fmt)
    b = enc(rng.normal(0, 1, n) * np.exp2(rng.integers(-12, 12, n)), fmt)
    if fmt == "f16":
        y[1, 0], b[0] = enc([65504.0], fmt)[0], enc([32.0], fmt)[0]   # 65536 -> inf
    y[0] = enc(-decode16(b, fmt), fmt)                       # row 0: y = -bias exactly
    got = oracle.add_bias(y, b, fmt)
    yv, bv = decode16(y, fmt), decode16(b, fmt)
    want = np.array([[round_rne(Fraction(float(yv[i, j])) + Fraction(float(bv[j])), fmt) for j in range(n)]
                     for i in range(m)], dtype=np.uint16)
    assert np.array_equal(bits(got), want)
    assert np.all(bits(got)[0] == 0)                          # x + (-x) = +0
    if fmt == "f16":
        assert bits(got)[1, 0] == 0x7C00


def test_add_bias_zero_is_identity():
    rng = np.random.default_rng(42)
    y = enc(np.abs(rng.normal(0, 3, (5, 7))) + 0.5, "bf16")
    assert np.array_equal(oracle.add_bias(y, np.zeros(7, np.uint16), "bf16"), y)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_bias_grad_exact_rational_and_numpy(fmt):
    """grad_bias = dy.sum(dim=0): the exact column sum rounded once (exact rationals on a
    small case; numpy's float64 column sum, exact here, on a larger one)."""
    rng = np.random.default_rng(43)
    dy = enc(rng.normal(0, 1, (37, 5)), fmt)
    got = oracle.bias_grad(dy, fmt)
    v = decode16(dy, fmt)
    want = [round_rne(sum(Fraction(float(v[i, j])) for i in range(37)), fmt) for j in range(5)]
    assert bits(got).tolist() == want
    dy = enc(rng.normal(0, 1, (4096, 64)), fmt)
    s = decode16(dy, fmt).sum(axis=0)          # float64, exact: 8 + 13 bits of range + 12 of count
    assert np.array_equal(bits(oracle.bias_grad(dy, fmt)), enc(s, fmt).view(np.uint16))


def test_bias_grad_integer_columns():
    """Small-integer gradients: every column sum is an exact integer (numpy int64)."""
    rng = np.random.default_rng(44)
    ints = rng.integers(-3, 4, (1000, 33))
    got = oracle.bias_grad(enc(ints.astype(np.float64), "bf16"), "bf16")
    assert np.array_equal(got, enc(ints.sum(axis=0).astype(np.float64), "bf16"))


def test_column_parallel_layer_with_bias_equals_unsharded_linear():
    """r ranks' column shards of W and bias, each rank's AllGatherMatmul + bias, stacked
    along the output columns, equal the unsharded layer x W^T + b; with small-integer
    operands every value is exact, so bit for bit (numpy int64 reference)."""
    rng = np.random.default_rng(45)
    r, m_l, k, n_l = 4, 8, 256, 16
    xs = [rng.integers(-2, 3, (m_l, k)) for _ in range(r)]
    W = rng.integers(-2, 3, (r * n_l, k))
    b = rng.integers(-4, 5, r * n_l)
    e = lambda a: enc(np.asarray(a, np.float64), "bf16")
    outs = []
    for j in range(r):
        wj = np.ascontiguousarray(W[j * n_l:(j + 1) * n_l])
        o, _ = oracle.allgather_matmul([e(x) for x in xs], e(wj), "bf16", x2_trans=True)
        outs.append(oracle.add_bias(o, e(b[j * n_l:(j + 1) * n_l]), "bf16"))
    full = np.concatenate(xs) @ W.T + b
    assert np.array_equal(np.concatenate(outs, axis=1), e(full))


# ----------------------------------------------------------------- int4 operands (A16W4 / A4W4)
def test_unpack_int4_every_byte():
    """Each byte splits into the unique pair of int4 codes lo, hi in [-8, 7] with
    lo = byte (mod 16) and hi = byte / 16 (mod 16): its two's-complement nibbles."""
    b = np.arange(256, dtype=np.uint8)
    u = oracle.unpack_int4(b.reshape(1, 256)).reshape(256, 2).astype(np.int64)
    lo, hi = u[:, 0], u[:, 1]
    assert lo.min() == -8 and lo.max() == 7 and hi.min() == -8 and hi.max() == 7
    assert np.array_equal(lo % 16, b.astype(np.int64) % 16) and np.array_equal(hi % 16, b.astype(np.int64) // 16)
    assert len({(int(x), int(y)) for x, y in u}) == 256


def test_unpack_int4_order_and_generator_round_trip():
    """The reading's order (value 2i in the low nibble, 2i + 1 in the high one) on
    hand-written bytes, and the generator's packing inverts the oracle's unpacking."""
    got = oracle.unpack_int4(np.array([[0x21, 0xF8, 0x7F, 0x80]], np.uint8))
    assert got.tolist() == [[1, 2, -8, -1, -1, 7, 0, -8]]
    codes = mc2_inputs.fill(7, 3, "int", -8, 7, "i8", (37, 64))
    assert np.array_equal(oracle.unpack_int4(mc2_inputs.pack_int4(codes)), codes)


def test_a16w4_and_a4w4_chains_vs_numpy_int64():
    """The int4 chains: accumulators equal numpy's int64 product of the permuted codes
    (A4W4) or the quantised tokens (A16W4) with the unpacked weight."""
    r, bs, h, n = 4, 32, 64, 24
    t = mc2_inputs.make(mc2_inputs.configs.scaled("a16w4", r=r, bs=bs, h=h, n=n), seed=61)
    w_packed = mc2_inputs.pack_int4(t["x2"])
    res = oracle.alltoall_quant_matmul_a16w4(t["x1"], r, w_packed, t["x2_scale"], t["x1_smooth"], t["bias"])
    q, s1 = oracle.smooth_quant(oracle.permute(t["x1"], r), t["x1_smooth"])
    assert np.array_equal(res["q"], q) and np.array_equal(res["s1"], s1)
    assert np.array_equal(res["acc"], q.astype(np.int64) @ t["x2"].astype(np.int64))
    t = mc2_inputs.make(mc2_inputs.configs.scaled("a4w4", r=r, bs=bs, h=h, n=n), seed=62)
    res = oracle.alltoall_quant_matmul_a4w4(mc2_inputs.pack_int4(t["x1"]), r, t["x1_scale"],
                                            mc2_inputs.pack_int4(t["x2"]), t["x2_scale"], t["bias"])
    p = t["x1"].reshape(r, bs // r, h).transpose(1, 0, 2).reshape(bs // r, r * h).astype(np.int64)
    assert np.array_equal(res["acc"], p @ t["x2"].astype(np.int64))
    assert np.array_equal(res["out"], oracle.dequant(res["acc"], t["x1_scale"], t["x2_scale"], t["bias"]))
