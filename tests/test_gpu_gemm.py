"""AllGatherMatmul and the column-parallel backward GEMMs on the GPU vs the oracle.

Float outputs: |gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref) per element (fp32
accumulation on the GPU vs fp64 in the oracle, both rounded to 16 bits).
gather_out and the exact-integer cases: bit for bit.
"""
import numpy as np
import pytest

import mc2_inputs
import oracle
from parity import assert_bits_equal, assert_close16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available()
    import comm_matmul_tensor_amd as m
    return m


def _ag(mc2, r, m_l, k, n, dtype, x2_trans=False, seed=0, gather=True, x2_std=1.0):
    import torch
    specs = mc2_inputs.configs.scaled("ag", r=r, m_local=m_l, k=k, n=n, dtype=dtype, x2_std=x2_std)
    t = mc2_inputs.make(specs, seed=seed)
    shards = [t[f"shard{i}"] for i in range(r)]
    x2 = np.ascontiguousarray(t["x2"].T) if x2_trans else t["x2"]
    T = mc2_inputs.to_torch
    out, g = mc2.mc2_allgather_matmul([T(s, dtype) for s in shards], T(x2, dtype), x2_trans=x2_trans,
                                      gather_output=gather)
    torch.cuda.synchronize()
    want, want_g = oracle.allgather_matmul(shards, x2, dtype, x2_trans=x2_trans, gather_output=gather)
    return mc2_inputs.from_torch(out), (mc2_inputs.from_torch(g) if g is not None else None), want, want_g


def test_ag_tiny_example(mc2):
    """The API page's example: 8 ranks, gathered (128, 512) fp16 @ (512, 64)."""
    seed, d, specs = mc2_inputs.CONFIGS["ag_tiny"]
    out, g, want, want_g = _ag(mc2, d["r"], d["m_local"], d["k"], d["n"], "f16", seed=seed)
    assert_bits_equal(g, want_g, "gather_out")
    assert_close16(out, want, "f16", "out")


# The shapes with k % 64 == 0 and 16-byte rows run the gather-wavefront kernel (loads and
# gather copy in wavefronts 4-7): (4, 16, 512, 64) a single partial tile row; (8, 40, 512, 96)
# two whole tile rows and a partial one, 8 steps; (4, 96, 1536, 448) whole rows, two tile
# columns (each copies every other step), 24 steps; (2, 72, 640, 224) 10 steps; (4, 32, 256, 64)
# and (2, 64, 320, 128) the shortest loops the API allows, 4 and 5 steps.
@pytest.mark.parametrize("r,m_l,k,n", [
    (2, 1, 256, 1), (2, 3, 300, 7), (4, 16, 512, 64), (8, 5, 1000, 130), (4, 100, 264, 200),
    (8, 33, 768, 257), (2, 129, 256, 129), (8, 40, 512, 96), (4, 96, 1536, 448), (2, 72, 640, 224),
    (4, 32, 256, 64), (2, 64, 320, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("x2_trans", [False, True])
def test_ag_shapes(mc2, r, m_l, k, n, dtype, x2_trans):
    print(f"ag r={r} m_l={m_l} k={k} n={n} {dtype} trans={x2_trans}", flush=True)
    out, g, want, want_g = _ag(mc2, r, m_l, k, n, dtype, x2_trans, seed=r * 1000 + k + n)
    assert_bits_equal(g, want_g, "gather_out")
    assert_close16(out, want, dtype, "out")


def test_ag_without_gather_output(mc2):
    out, g, want, _ = _ag(mc2, 4, 8, 256, 48, "bf16", gather=False, seed=5)
    assert g is None
    assert_close16(out, want, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ag_exact_integer_bit_exact(mc2, dtype):
    """Small integers: fp32 accumulation is exact, so the GPU must equal the oracle bit for bit."""
    import torch
    rng = np.random.default_rng(11)
    r, m_l, k, n = 4, 40, 512, 96
    enc = lambda a: oracle.encode(dtype, a.astype(np.float64))
    shards = [enc(rng.integers(-3, 4, (m_l, k))) for _ in range(r)]
    x2 = enc(rng.integers(-2, 3, (k, n)))
    T = mc2_inputs.to_torch
    out, _ = mc2.mc2_allgather_matmul([T(s, dtype) for s in shards], T(x2, dtype))
    want, _ = oracle.allgather_matmul(shards, x2, dtype)
    assert_bits_equal(mc2_inputs.from_torch(out), want, "exact-integer out")


def test_ag_max_k(mc2):
    """k = 65534, the largest the op accepts."""
    out, g, want, want_g = _ag(mc2, 2, 2, 65534, 16, "bf16", seed=7, x2_std=0.05)
    assert_bits_equal(g, want_g, "gather_out")
    assert_close16(out, want, "bf16")


def test_ag_full_config(mc2):
    """8 x bf16 (512, 4096) @ (4096, 1792): gather_out bit for bit and every element of out
    against the oracle, at the launch configuration the benchmark times; two runs bit-identical."""
    import torch
    seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
    t = mc2_inputs.make("ag_bf16_tp")
    T = mc2_inputs.to_torch
    shards = [T(t[f"shard{i}"], "bf16") for i in range(d["r"])]
    x2 = T(t["x2"], "bf16")
    out, g = mc2.mc2_allgather_matmul(shards, x2)
    out2, _ = mc2.mc2_allgather_matmul(shards, x2)
    torch.cuda.synchronize()
    want, want_g = oracle.allgather_matmul([t[f"shard{i}"] for i in range(d["r"])], t["x2"], "bf16")
    assert_bits_equal(mc2_inputs.from_torch(g), want_g, "gather_out")
    o = mc2_inputs.from_torch(out)
    assert_bits_equal(o, mc2_inputs.from_torch(out2), "run-to-run")
    assert_close16(o, want, "bf16", "out")


# the last three take the 256 x 128 tile for dX (whole, and ragged in both
# dimensions) and the 128 x 256 tile for dW
@pytest.mark.parametrize("m,n_l,k", [(64, 256, 32), (200, 300, 130), (1024, 256, 520), (33, 1000, 7),
                                     (4096, 256, 2048), (8190, 264, 2040), (256, 4096, 2048)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_backward_shapes(mc2, m, n_l, k, dtype):
    import torch
    print(f"bwd m={m} n_l={n_l} k={k} {dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("bwd", m=m, n_local=n_l, k=k)
    for s in specs:
        specs[s] = mc2_inputs.TensorSpec(specs[s].tid, specs[s].shape, specs[s].dist, specs[s].a, specs[s].b, dtype)
    t = mc2_inputs.make(specs, seed=m + n_l + k)
    T = mc2_inputs.to_torch
    dx = mc2.mc2_matmul_grad_input(T(t["dy"], dtype), T(t["w"], dtype))
    dw = mc2.mc2_matmul_grad_weight(T(t["dy"], dtype), T(t["ag_x"], dtype))
    torch.cuda.synchronize()
    assert_close16(mc2_inputs.from_torch(dx), oracle.matmul_grad_input(t["dy"], t["w"], dtype), dtype, "dX")
    assert_close16(mc2_inputs.from_torch(dw), oracle.matmul_grad_weight(t["dy"], t["ag_x"], dtype), dtype, "dW")


# Outputs of 4096 x 4096 and ragged 4059 x 4083, with a contraction that is a
# whole number of K steps (fast path; 256 is the smallest allowed, 4 steps,
# and 320 an odd number of steps) or not (300: checked path).  dW (A
# M-contiguous) takes the two-stage 256 x 256 tile there; dX (A K-, B
# N-contiguous) the 256 x 128 one.
@pytest.mark.parametrize("m,n_l,k", [(4096, 256, 4096), (4059, 320, 4083), (4059, 300, 4083)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_big_tile_grad_input(mc2, m, n_l, k, dtype):
    import torch
    print(f"big-tile dX m={m} n_l={n_l} k={k} {dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("bwd", m=m, n_local=n_l, k=k)
    specs = {s: mc2_inputs.TensorSpec(v.tid, v.shape, v.dist, v.a, v.b, dtype) for s, v in specs.items()
             if s in ("dy", "w")}
    t = mc2_inputs.make(specs, seed=m + n_l + k)
    dx = mc2.mc2_matmul_grad_input(mc2_inputs.to_torch(t["dy"], dtype), mc2_inputs.to_torch(t["w"], dtype))
    torch.cuda.synchronize()
    assert_close16(mc2_inputs.from_torch(dx), oracle.matmul_grad_input(t["dy"], t["w"], dtype), dtype, "dX")


@pytest.mark.parametrize("m,n_l,k", [(256, 4096, 4096), (264, 4059, 4083)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_big_tile_grad_weight(mc2, m, n_l, k, dtype):
    import torch
    print(f"big-tile dW m={m} n_l={n_l} k={k} {dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("bwd", m=m, n_local=n_l, k=k)
    specs = {s: mc2_inputs.TensorSpec(v.tid, v.shape, v.dist, v.a, v.b, dtype) for s, v in specs.items()
             if s in ("dy", "ag_x")}
    t = mc2_inputs.make(specs, seed=m + n_l + k)
    dw = mc2.mc2_matmul_grad_weight(mc2_inputs.to_torch(t["dy"], dtype), mc2_inputs.to_torch(t["ag_x"], dtype))
    torch.cuda.synchronize()
    assert_close16(mc2_inputs.from_torch(dw), oracle.matmul_grad_weight(t["dy"], t["ag_x"], dtype), dtype, "dW")


@pytest.mark.parametrize("x2_trans", [False, True])
def test_big_tile_allgather_without_gather_output(mc2, x2_trans):
    """AllGatherMatmul of a 4096 x 4096 output with gather_output off: with x2 given
    as (n, k) the 256 x 256 tile (with gather_out only the three-stage tiles are used)."""
    out, g, want, _ = _ag(mc2, 8, 512, 256, 4096, "bf16", x2_trans=x2_trans, seed=21, gather=False)
    assert g is None
    assert_close16(out, want, "bf16", "out")


def test_backward_full_config(mc2):
    """dY (8192, 1792), W (1792, 4096), AG(X) (8192, 4096): every element of dX and of dW."""
    import torch
    t = mc2_inputs.make("colpar_bwd")
    T = mc2_inputs.to_torch
    dy, w, x = T(t["dy"], "bf16"), T(t["w"], "bf16"), T(t["ag_x"], "bf16")
    dx = mc2_inputs.from_torch(mc2.mc2_matmul_grad_input(dy, w))
    dw = mc2_inputs.from_torch(mc2.mc2_matmul_grad_weight(dy, x))
    torch.cuda.synchronize()
    assert_close16(dx, oracle.matmul_grad_input(t["dy"], t["w"]), "bf16", "dX")
    assert_close16(dw, oracle.matmul_grad_weight(t["dy"], t["ag_x"]), "bf16", "dW")


# ---------------------------------------------------------------- arrival emulation (MC2_AG_ARRIVAL)
def _arrival_case(mc2, r, m_l, k, n, dtype, rank_id, seed, x2_trans=False):
    import torch
    specs = mc2_inputs.configs.scaled("ag", r=r, m_local=m_l, k=k, n=n, dtype=dtype, x2_std=0.05)
    t = mc2_inputs.make(specs, seed=seed)
    T = mc2_inputs.to_torch
    shards_np = [t[f"shard{i}"] for i in range(r)]
    x2_np = np.ascontiguousarray(t["x2"].T) if x2_trans else t["x2"]
    shards = [T(s, dtype) for s in shards_np]
    x2 = T(x2_np, dtype)
    fused, _ = mc2.mc2_allgather_matmul(shards, x2, x2_trans=x2_trans)
    g = torch.full((r * m_l, k), float("nan"), dtype=shards[0].dtype, device="cuda")
    out, _ = mc2.mc2_allgather_matmul(shards, x2, x2_trans=x2_trans, gather_out=g, mode=mc2.MC2_AG_ARRIVAL,
                                      rank_id=rank_id)
    torch.cuda.synchronize()
    return shards_np, x2_np, mc2_inputs.from_torch(fused), mc2_inputs.from_torch(out), mc2_inputs.from_torch(g)


def _arrival_out(mc2, shards_np, x2_np, dtype, rank_id, x2_trans=False):
    """One more arrival-mode call on the same inputs (output only)."""
    import torch
    T = mc2_inputs.to_torch
    out, _ = mc2.mc2_allgather_matmul([T(s, dtype) for s in shards_np], T(x2_np, dtype), x2_trans=x2_trans,
                                      mode=mc2.MC2_AG_ARRIVAL, rank_id=rank_id)
    torch.cuda.synchronize()
    return mc2_inputs.from_torch(out)


@pytest.mark.parametrize("r,m_l,k,n,rank_id", [
    (2, 1, 256, 1, 1), (4, 16, 512, 64, 2), (8, 5, 1000, 130, 7), (4, 100, 264, 200, 0),
    (8, 33, 768, 257, 3), (2, 129, 256, 129, 1), (8, 128, 512, 224, 5)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ag_arrival_shapes(mc2, r, m_l, k, n, rank_id, dtype):
    """Arrival mode reads the copied gather_out: out within the oracle's bound, gather_out exact.
    (Its K walk is in order, the fused loops' is rotated, so the two differ in rounding.)"""
    print(f"arrival r={r} m_l={m_l} k={k} n={n} rank={rank_id} {dtype}", flush=True)
    mc2.mc2_allgather_arrival_fallbacks(reset=True)
    shards, x2, fused, out, g = _arrival_case(mc2, r, m_l, k, n, dtype, rank_id, seed=7000 + r * 100 + m_l)
    want, want_g = oracle.allgather_matmul(shards, x2, dtype)
    assert_bits_equal(g, want_g, "gather_out")
    assert_close16(out, want, dtype, "out")
    assert_close16(fused, want, dtype, "fused out")
    assert mc2.mc2_allgather_arrival_fallbacks() == 0


def test_ag_arrival_repeated_calls(mc2):
    """Consecutive arrival calls on new data: every call waits for its own copies."""
    import torch
    mc2.mc2_allgather_arrival_fallbacks(reset=True)
    for it in range(3):
        shards, x2, fused, out, g = _arrival_case(mc2, 4, 64, 512, 96, "bf16", rank_id=it % 4, seed=7500 + it,
                                                  x2_trans=bool(it % 2))
        want, want_g = oracle.allgather_matmul(shards, x2, "bf16", x2_trans=bool(it % 2))
        assert_bits_equal(g, want_g, f"gather_out call {it}")
        assert_close16(out, want, "bf16", f"arrival call {it}")
    assert mc2.mc2_allgather_arrival_fallbacks() == 0


def test_ag_arrival_full_config(mc2):
    """8 x bf16 (512, 4096) @ (4096, 1792) in arrival mode: every element within the oracle's bound."""
    import torch
    seed, d, specs = mc2_inputs.CONFIGS["ag_bf16_tp"]
    t = mc2_inputs.make("ag_bf16_tp")
    T = mc2_inputs.to_torch
    shards = [T(t[f"shard{i}"], "bf16") for i in range(d["r"])]
    x2 = T(t["x2"], "bf16")
    mc2.mc2_allgather_arrival_fallbacks(reset=True)
    fused, _ = mc2.mc2_allgather_matmul(shards, x2)
    out, g = mc2.mc2_allgather_matmul(shards, x2, mode=mc2.MC2_AG_ARRIVAL, rank_id=3)
    torch.cuda.synchronize()
    G = np.concatenate([t[f"shard{i}"] for i in range(d["r"])])
    assert_bits_equal(mc2_inputs.from_torch(g), G, "gather_out")
    want, _ = oracle.allgather_matmul([t[f"shard{i}"] for i in range(d["r"])], t["x2"], "bf16")
    assert_close16(mc2_inputs.from_torch(out), want, "bf16", "arrival out")
    assert mc2.mc2_allgather_arrival_fallbacks() == 0


# Time-out path: the copy still lands every piece but raises the flags of the
# first `raised` slabs of K only, with a short wait limit, so every wait on a
# withheld slab runs out and that wavefront (fast path) or workgroup (checked
# path) reads the rest of A from the shards.  raised = 0: the first wait runs
# out; raised = 1: the switch happens inside the main loop, after slab 0 came
# through the arrived buffer.  The output must equal a normal arrival-mode call on
# the same inputs bit for bit (both walk K in order; the shards hold the same
# values as the arrived buffer).
@pytest.mark.parametrize("r,m_l,k,n,raised,path", [
    (8, 128, 512, 224, 1, "fast"), (8, 128, 512, 224, 0, "fast"), (4, 64, 1024, 128, 3, "fast"),
    (8, 33, 768, 257, 2, "checked"), (2, 129, 256, 129, 0, "checked")])
def test_ag_arrival_timeout_fallback(mc2, r, m_l, k, n, raised, path):
    print(f"arrival time-out r={r} m_l={m_l} k={k} n={n} raised={raised} ({path})", flush=True)
    mc2.mc2_allgather_arrival_fallbacks(reset=True)
    # 2 ms: far longer than any raised piece takes to arrive, short enough for the test
    mc2.mc2_testing_arrival(wait_ticks=200000, raised_slabs=raised)
    try:
        shards, x2, fused, out, g = _arrival_case(mc2, r, m_l, k, n, "bf16", rank_id=1, seed=7700 + k + raised)
        fallbacks = mc2.mc2_allgather_arrival_fallbacks(reset=True)
    finally:
        mc2.mc2_testing_arrival(0, -1)
    want, want_g = oracle.allgather_matmul(shards, x2, "bf16")
    assert fallbacks > 0
    assert_bits_equal(g, want_g, "gather_out")
    assert_close16(out, want, "bf16", "out")
    # the default settings are back: the same inputs without a time-out give the same bits
    ref = _arrival_out(mc2, shards, x2, "bf16", rank_id=1)
    assert mc2.mc2_allgather_arrival_fallbacks() == 0
    assert_bits_equal(out, ref, "fallback vs arrival without time-outs")
    # and new data: no fallback
    shards, x2, fused, out, g = _arrival_case(mc2, r, m_l, k, n, "bf16", rank_id=0, seed=7800 + k)
    want, _ = oracle.allgather_matmul(shards, x2, "bf16")
    assert_close16(out, want, "bf16", "arrival after the hook")
    assert mc2.mc2_allgather_arrival_fallbacks() == 0
