"""QuantAllReduce dequant-sum on the GPU against the oracle (bit-exact).

Both sides compute the exact fp64 sum of the rank products in rank order and
round it once, so every output must match bit for bit.
"""
import numpy as np
import pytest

import mc2_inputs
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a device"
    import comm_matmul_tensor_amd as m
    return m


def _run(mc2, specs, seed, x_dtype, s_dtype, out_dtype, r):
    import torch
    t = mc2_inputs.make(specs, seed=seed)
    xs = [t[f"x{i}"] for i in range(r)]
    sc = [t[f"scale{i}"] for i in range(r)]
    want = oracle.quant_all_reduce(xs, sc, x_dtype, "f32" if s_dtype == "f32" else "e8m0", out_dtype)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    got = mc2.mc2_quant_all_reduce([mc2_inputs.to_torch(x, x_dtype) for x in xs],
                                   [mc2_inputs.to_torch(s, s_dtype) for s in sc], out_dtype=tdt)
    torch.cuda.synchronize()
    return mc2_inputs.from_torch(got), want, got


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


@pytest.mark.parametrize("r", [2, 4, 8])
@pytest.mark.parametrize("shape", [(1, 1024), (3, 1152), (2, 5, 8192)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_qar_int8_pergroup(mc2, r, shape, out_dtype):
    print(f"qar int8 r={r} shape={shape} out={out_dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("qar_int8", r=r, shape=shape)
    got, want, _ = _run(mc2, specs, 50 + r, "i8", "f32", out_dtype, r)
    assert np.array_equal(_bits(got), _bits(want))


@pytest.mark.parametrize("r", [2, 8])
@pytest.mark.parametrize("shape", [(1, 1024), (4, 3, 2048)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32", "f16"])
def test_qar_mx(mc2, r, shape, out_dtype):
    print(f"qar mx r={r} shape={shape} out={out_dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("qar_mx", r=r, shape=shape)
    got, want, _ = _run(mc2, specs, 60 + r, "e4m3fn", "e8m0", out_dtype, r)
    assert np.array_equal(_bits(got), _bits(want))


def test_qar_fp8_with_fp32_group_scales(mc2):
    """FLOAT scales with FLOAT8_E4M3FN x (pertoken-pergroup)."""
    specs = mc2_inputs.configs.scaled("qar_mx", r=4, shape=(2, 2048))
    for i in range(4):
        specs[f"scale{i}"] = mc2_inputs.TensorSpec(40 + i, (2, 16), "uniform", 1e-3, 1e-2, "f32")
    got, want, _ = _run(mc2, specs, 70, "e4m3fn", "f32", "f32", 4)
    assert np.array_equal(_bits(got), _bits(want))


def test_qar_all_codes_decode(mc2):
    """Every E4M3FN code and every E8M0 code through the kernel (unit scales / unit x)."""
    import torch
    codes = np.tile(np.arange(256, dtype=np.uint8), 4)[None, :]  # h = 1024
    zeros = np.zeros_like(codes)
    ones_e8 = np.full((1, 16, 2), 127, np.uint8)
    got = mc2.mc2_quant_all_reduce([mc2_inputs.to_torch(codes, "e4m3fn"), mc2_inputs.to_torch(zeros, "e4m3fn")],
                                   [mc2_inputs.to_torch(ones_e8, "e8m0")] * 2, out_dtype=torch.float32)
    want = oracle.quant_all_reduce([codes, zeros], [ones_e8] * 2, "e4m3fn", "e8m0", "f32")
    g = mc2_inputs.from_torch(got)
    assert np.array_equal(np.isnan(g), np.isnan(want)) and np.array_equal(g[~np.isnan(g)], want[~np.isnan(want)])
    one = np.full((1, 1024), 0x38, np.uint8)  # E4M3FN 1.0
    e8 = np.tile(np.arange(256, dtype=np.uint8), 1)[:32].reshape(1, 16, 2)
    for base in range(0, 256, 32):
        e8 = np.arange(base, base + 32, dtype=np.uint8).reshape(1, 16, 2)
        got = mc2.mc2_quant_all_reduce([mc2_inputs.to_torch(one, "e4m3fn"), mc2_inputs.to_torch(zeros, "e4m3fn")],
                                       [mc2_inputs.to_torch(e8, "e8m0")] * 2, out_dtype=torch.float32)
        want = oracle.quant_all_reduce([one, zeros], [e8, e8], "e4m3fn", "e8m0", "f32")
        g = mc2_inputs.from_torch(got)
        assert np.array_equal(np.isnan(g), np.isnan(want)) and np.array_equal(g[~np.isnan(g)], want[~np.isnan(want)])


@pytest.mark.parametrize("name,x_dtype,s_dtype,out_dtype", [
    ("qar_int8", "i8", "f32", "f32"), ("qar_mx", "e4m3fn", "e8m0", "bf16")])
def test_qar_full_config(mc2, name, x_dtype, s_dtype, out_dtype):
    """The full workload (8 ranks x (4, 2048, 7168)), every output, and run-to-run identity."""
    print(f"qar full {name}", flush=True)
    seed, dims, specs = mc2_inputs.CONFIGS[name]
    got, want, dev_out = _run(mc2, specs, seed, x_dtype, s_dtype, out_dtype, dims["r"])
    assert np.array_equal(_bits(got), _bits(want))


# ---------------------------------------------------------------- QuantReduceScatter
def _run_rs(mc2, specs, seed, x_dtype, s_dtype, out_dtype, r, rank):
    import torch
    t = mc2_inputs.make(specs, seed=seed)
    xs = [t[f"x{i}"] for i in range(r)]
    sc = [t[f"scale{i}"] for i in range(r)]
    sdt = "f32" if s_dtype == "f32" else "e8m0"
    want = oracle.quant_reduce_scatter(xs, sc, rank, x_dtype, sdt, out_dtype)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    got = mc2.mc2_quant_reduce_scatter([mc2_inputs.to_torch(x, x_dtype) for x in xs],
                                       [mc2_inputs.to_torch(s, s_dtype) for s in sc], rank, out_dtype=tdt)
    torch.cuda.synchronize()
    return mc2_inputs.from_torch(got), want


@pytest.mark.parametrize("r,shape,rank", [(2, (2, 1024), 1), (4, (4, 3, 1152), 2), (8, (2, 8, 8192), 7),
                                          (8, (16, 2048), 0), (8, (8, 1024), 6)])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_qrs_int8_pergroup(mc2, r, shape, rank, out_dtype):
    print(f"qrs int8 r={r} shape={shape} rank={rank} out={out_dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("qar_int8", r=r, shape=shape)
    got, want = _run_rs(mc2, specs, 70 + r, "i8", "f32", out_dtype, r, rank)
    assert np.array_equal(_bits(got), _bits(want))


@pytest.mark.parametrize("r,shape,rank", [(2, (2, 1024), 0), (8, (4, 2, 2048), 5)])
def test_qrs_mx(mc2, r, shape, rank):
    print(f"qrs mx r={r} shape={shape} rank={rank}", flush=True)
    specs = mc2_inputs.configs.scaled("qar_mx", r=r, shape=shape)
    got, want = _run_rs(mc2, specs, 80 + r, "e4m3fn", "e8m0", "bf16", r, rank)
    assert np.array_equal(_bits(got), _bits(want))


def test_qrs_every_rank_tiles_the_all_reduce(mc2):
    """The r outputs stacked in rank order are the QuantAllReduce output, bit for bit."""
    r, shape = 4, (8, 2048)
    specs = mc2_inputs.configs.scaled("qar_int8", r=r, shape=shape)
    full, _, _ = _run(mc2, specs, 90, "i8", "f32", "bf16", r)
    parts = [_run_rs(mc2, specs, 90, "i8", "f32", "bf16", r, k)[0] for k in range(r)]
    assert np.array_equal(_bits(np.concatenate(parts)), _bits(full.reshape(-1, shape[-1])))


@pytest.mark.parametrize("name,x_dtype,s_dtype,out_dtype", [
    ("qar_int8", "i8", "f32", "f32"), ("qar_mx", "e4m3fn", "e8m0", "bf16")])
def test_qrs_full_config(mc2, name, x_dtype, s_dtype, out_dtype):
    """The full workload's rank-3 share (1024 of 8192 rows), every output."""
    print(f"qrs full {name}", flush=True)
    seed, dims, specs = mc2_inputs.CONFIGS[name]
    got, want = _run_rs(mc2, specs, seed, x_dtype, s_dtype, out_dtype, dims["r"], 3)
    assert np.array_equal(_bits(got), _bits(want))


# ---------------------------------------------------------------- FLOAT8_E5M2 x
def _e5m2_codes(rng, shape):
    """Random finite E5M2 codes (exponent field 31 holds inf / NaN)."""
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7C) == 0x7C, c & 0x83, c).astype(np.uint8)


@pytest.mark.parametrize("r", [2, 8])
@pytest.mark.parametrize("s_dtype,out_dtype", [("e8m0", "bf16"), ("e8m0", "f32"), ("f32", "f32"), ("f32", "f16")])
def test_qar_e5m2(mc2, r, s_dtype, out_dtype):
    """FLOAT8_E5M2 x with E8M0 mx scales or fp32 group scales; also the reduce-scatter share."""
    import torch
    print(f"qar e5m2 r={r} scales={s_dtype} out={out_dtype}", flush=True)
    rng = np.random.default_rng(100 + r)
    rows, h = 8, 2048
    xs = [_e5m2_codes(rng, (rows, h)) for _ in range(r)]
    if s_dtype == "e8m0":
        sc = [rng.integers(119, 128, (rows, h // 64, 2)).astype(np.uint8) for _ in range(r)]
    else:
        sc = [rng.uniform(1e-3, 1e-2, (rows, h // 128)).astype(np.float32) for _ in range(r)]
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    tx = [mc2_inputs.to_torch(x, "e5m2") for x in xs]
    ts = [mc2_inputs.to_torch(s, s_dtype) for s in sc]
    got = mc2_inputs.from_torch(mc2.mc2_quant_all_reduce(tx, ts, out_dtype=tdt))
    want = oracle.quant_all_reduce(xs, sc, "e5m2", s_dtype, out_dtype)
    assert np.array_equal(_bits(got), _bits(want))
    rank = r - 1
    got = mc2_inputs.from_torch(mc2.mc2_quant_reduce_scatter(tx, ts, rank, out_dtype=tdt))
    want = oracle.quant_reduce_scatter(xs, sc, rank, "e5m2", s_dtype, out_dtype)
    assert np.array_equal(_bits(got), _bits(want))


def test_qar_e5m2_all_codes_decode(mc2):
    """Every E5M2 code through the kernel with unit scales: values, infinities and NaNs."""
    import torch
    codes = np.tile(np.arange(256, dtype=np.uint8), 4)[None, :]
    zeros = np.zeros_like(codes)
    ones_e8 = np.full((1, 16, 2), 127, np.uint8)
    got = mc2.mc2_quant_all_reduce([mc2_inputs.to_torch(codes, "e5m2"), mc2_inputs.to_torch(zeros, "e5m2")],
                                   [mc2_inputs.to_torch(ones_e8, "e8m0")] * 2, out_dtype=torch.float32)
    want = oracle.quant_all_reduce([codes, zeros], [ones_e8] * 2, "e5m2", "e8m0", "f32")
    g = mc2_inputs.from_torch(got)
    assert np.array_equal(np.isnan(g), np.isnan(want))
    assert np.array_equal(g[~np.isnan(g)], want[~np.isnan(want)])
