"""AlltoAllQuantMatmul with int4 operands on the GPU vs the oracle: A16W4 (int4
weight, the dynamic per-token chain) and A4W4 (int4 activations and weight,
full quantisation).  int4 codes are stored two per byte along the last
dimension, low nibble first (the reading of the page's constraints, taken in
the oracle).  Bit-exact: codes, per-token scales, int32 accumulators; the
16-bit output within |gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref)."""
import numpy as np
import pytest

import mc2_inputs
import oracle
from parity import assert_bits_equal, assert_close16

pytestmark = pytest.mark.gpu

T = mc2_inputs.to_torch
F = mc2_inputs.from_torch


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available()
    import comm_matmul_tensor_amd as m
    return m


def _u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8)).cuda()


def _a16w4(mc2, t, r, bs, h, n, dtype, debug=True):
    import torch
    rows, cols = bs // r, r * h
    dbg = {}
    if debug:
        dbg = dict(q_out=torch.empty((rows, cols), dtype=torch.int8, device="cuda"),
                   x1_scale_out=torch.empty((rows,), dtype=torch.float32, device="cuda"),
                   acc_out=torch.empty((rows, n), dtype=torch.int32, device="cuda"))
    out = mc2.mc2_alltoall_quant_matmul_a16w4(T(t["x1"], dtype), r, _u8(mc2_inputs.pack_int4(t["x2"])),
                                              T(t["x2_scale"], "f32"), T(t["x1_smooth"], dtype), T(t["bias"], dtype),
                                              **dbg)
    torch.cuda.synchronize()
    got = {"out": F(out)}
    got.update({k: F(v) for k, v in dbg.items()})
    return got


@pytest.mark.parametrize("r,bs,h,n,dtype", [
    (2, 2, 256, 16, "bf16"), (4, 64, 256, 96, "f16"), (8, 256, 512, 300, "bf16"), (8, 64, 2, 40, "bf16"),
    (2, 6, 136, 34, "f16"), (4, 520, 1024, 130, "bf16"), (8, 16, 4096, 64, "bf16"), (2, 40, 64, 2, "bf16")])
def test_a16w4_shapes(mc2, r, bs, h, n, dtype):
    print(f"a16w4 r={r} bs={bs} h={h} n={n} {dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("a16w4", r=r, bs=bs, h=h, n=n)
    for key in ("x1", "x1_smooth", "bias"):
        s = specs[key]
        specs[key] = mc2_inputs.TensorSpec(s.tid, s.shape, s.dist, s.a, s.b, dtype)
    t = mc2_inputs.make(specs, seed=1100 + r + bs + h + n)
    got = _a16w4(mc2, t, r, bs, h, n, dtype)
    ref = oracle.alltoall_quant_matmul_a16w4(t["x1"], r, mc2_inputs.pack_int4(t["x2"]), t["x2_scale"],
                                             t["x1_smooth"], t["bias"], dtype)
    assert_bits_equal(got["q_out"], ref["q"], "q")
    assert_bits_equal(got["x1_scale_out"], ref["s1"], "x1_scale")
    assert_bits_equal(got["acc_out"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], dtype, "out")


def test_a16w4_full_config(mc2):
    """bf16 (8192, 4096) on 8 ranks, int4 weight (32768, 7168): every element."""
    seed, d, specs = mc2_inputs.CONFIGS["a16w4"]
    t = mc2_inputs.make("a16w4")
    got = _a16w4(mc2, t, d["r"], d["bs"], d["h"], d["n"], "bf16")
    ref = oracle.alltoall_quant_matmul_a16w4(t["x1"], d["r"], mc2_inputs.pack_int4(t["x2"]), t["x2_scale"],
                                             t["x1_smooth"], t["bias"])
    assert_bits_equal(got["q_out"], ref["q"], "q")
    assert_bits_equal(got["acc_out"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], "bf16", "out")
    got2 = _a16w4(mc2, t, d["r"], d["bs"], d["h"], d["n"], "bf16", debug=False)
    assert_bits_equal(got2["out"], got["out"], "without the debug outputs")


def _a4w4(mc2, t, r, bs, h, n, dtype="bf16"):
    import torch
    acc = torch.empty((bs // r, n), dtype=torch.int32, device="cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    out = mc2.mc2_alltoall_quant_matmul_a4w4(_u8(mc2_inputs.pack_int4(t["x1"])), r, T(t["x1_scale"], "f32"),
                                             _u8(mc2_inputs.pack_int4(t["x2"])), T(t["x2_scale"], "f32"),
                                             T(t["bias"], dtype), out_dtype=tdt, acc_out=acc)
    torch.cuda.synchronize()
    return F(out), F(acc)


# h a multiple of 16 (16-code chunks inside one rank segment: vector loads) or
# not (chunks across a segment edge: code by code); n even, ragged or not
@pytest.mark.parametrize("r,bs,h,n,dtype", [
    (2, 2, 256, 16, "bf16"), (4, 64, 256, 96, "f16"), (8, 256, 512, 300, "bf16"), (8, 64, 2, 40, "bf16"),
    (2, 6, 22, 34, "f16"), (4, 520, 1000, 130, "bf16"), (8, 16, 4096, 64, "bf16"), (4, 12, 6, 2, "bf16")])
def test_a4w4_shapes(mc2, r, bs, h, n, dtype):
    print(f"a4w4 r={r} bs={bs} h={h} n={n} {dtype}", flush=True)
    specs = mc2_inputs.configs.scaled("a4w4", r=r, bs=bs, h=h, n=n)
    s = specs["bias"]
    specs["bias"] = mc2_inputs.TensorSpec(s.tid, s.shape, s.dist, s.a, s.b, dtype)
    t = mc2_inputs.make(specs, seed=1200 + r + bs + h + n)
    out, acc = _a4w4(mc2, t, r, bs, h, n, dtype)
    ref = oracle.alltoall_quant_matmul_a4w4(mc2_inputs.pack_int4(t["x1"]), r, t["x1_scale"],
                                            mc2_inputs.pack_int4(t["x2"]), t["x2_scale"], t["bias"], dtype)
    assert_bits_equal(acc, ref["acc"], "acc")
    assert_close16(out, ref["out"], dtype, "out")


def test_a4w4_full_config(mc2):
    """int4 (8192, 4096) on 8 ranks, int4 weight (32768, 7168): every element."""
    seed, d, specs = mc2_inputs.CONFIGS["a4w4"]
    t = mc2_inputs.make("a4w4")
    out, acc = _a4w4(mc2, t, d["r"], d["bs"], d["h"], d["n"])
    ref = oracle.alltoall_quant_matmul_a4w4(mc2_inputs.pack_int4(t["x1"]), d["r"], t["x1_scale"],
                                            mc2_inputs.pack_int4(t["x2"]), t["x2_scale"], t["bias"])
    assert_bits_equal(acc, ref["acc"], "acc")
    assert_close16(out, ref["out"], "bf16", "out")
