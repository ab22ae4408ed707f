"""AlltoAllQuantMatmul with full quantisation (int8 x1, one fp32 scale per
permuted token) on the GPU vs the oracle.

Bit-exact: the permuted int8 layout and the int32 accumulators.  The bf16 /
fp16 output: both sides dequantise the same exact accumulators, the GPU in
fp32 (a few roundings of 2^-24 relative) and the oracle in fp64, then round
once to 16 bits, so they differ by at most one unit in the last place:
|gpu - ref| <= 2^-7 |ref| + 1e-5 rms(ref).
"""
import numpy as np
import pytest

import mc2_inputs
import oracle
from parity import assert_bits_equal, assert_close16

pytestmark = pytest.mark.gpu

REL, RMS_REL = 2.0 ** -7, 1e-5


@pytest.fixture(scope="module")
def mc2():
    import torch
    assert torch.cuda.is_available()
    import comm_matmul_tensor_amd as m
    return m


def _run(mc2, r, bs, h, n, dtype="bf16", bias=True, seed=0, debug=True):
    import torch
    specs = mc2_inputs.configs.scaled("a8w8", r=r, bs=bs, h=h, n=n)
    s = specs["bias"]
    specs["bias"] = mc2_inputs.TensorSpec(s.tid, s.shape, s.dist, s.a, s.b, dtype)
    t = mc2_inputs.make(specs, seed=seed)
    T = mc2_inputs.to_torch
    rows, cols = bs // r, r * h
    dbg = {}
    if debug:
        dbg = dict(permuted_out=torch.empty((rows, cols), dtype=torch.int8, device="cuda"),
                   acc_out=torch.empty((rows, n), dtype=torch.int32, device="cuda"))
    b = T(t["bias"], dtype) if bias else None
    out = mc2.mc2_alltoall_quant_matmul_static(
        T(t["x1"], "i8"), r, T(t["x1_scale"], "f32"), T(t["x2"], "i8"), T(t["x2_scale"], "f32"), b,
        out_dtype=torch.bfloat16 if dtype == "bf16" else torch.float16, **dbg)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul_static(t["x1"], r, t["x1_scale"], t["x2"], t["x2_scale"],
                                              t["bias"] if bias else None, dtype)
    got = {"out": mc2_inputs.from_torch(out)}
    got.update({k.replace("_out", ""): mc2_inputs.from_torch(v) for k, v in dbg.items()})
    return got, ref


# h % 128 == 0 with n % 16 == 0 takes the direct-to-LDS path with the
# permute in its addressing; the other shapes take the checked loader.
@pytest.mark.parametrize("r,bs,h,n", [
    (2, 2, 256, 16), (4, 64, 256, 96), (4, 300, 384, 256), (2, 512, 640, 160), (8, 2048, 128, 256),
    (8, 16, 4096, 64), (8, 256, 512, 300), (8, 64, 2, 40), (2, 6, 136, 33), (4, 520, 1024, 129),
    (4, 128, 64, 48)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_a8w8_shapes(mc2, r, bs, h, n, dtype):
    print(f"a8w8 r={r} bs={bs} h={h} n={n} {dtype}", flush=True)
    got, ref = _run(mc2, r, bs, h, n, dtype, seed=r + bs + h + n)
    assert_bits_equal(got["permuted"], ref["permuted"], "permuted")
    assert_bits_equal(got["acc"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], dtype, "out", REL, RMS_REL)


def test_a8w8_without_optional_outputs(mc2):
    """No bias and no debug copies: the same output as with them."""
    got, ref = _run(mc2, 4, 256, 512, 160, bias=False, seed=5, debug=False)
    assert_close16(got["out"], ref["out"], "bf16", "out", REL, RMS_REL)
    got2, _ = _run(mc2, 4, 256, 512, 160, bias=False, seed=5, debug=True)
    assert_bits_equal(got["out"], got2["out"], "with / without debug outputs")


def test_a8w8_extreme_codes(mc2):
    """Every code at +-127 on both sides: the largest products the int8 path accumulates."""
    import torch
    r, bs, h, n = 8, 64, 512, 32
    rows, cols = bs // r, r * h
    rng = np.random.default_rng(7)
    x1 = np.where(rng.random((bs, h)) < 0.5, -127, 127).astype(np.int8)
    x2 = np.full((cols, n), 127, dtype=np.int8)
    x2[:, ::2] = -127
    s1 = np.full(rows, 2.0 ** -20, dtype=np.float32)
    s2 = np.full(n, 2.0 ** -6, dtype=np.float32)
    T = mc2_inputs.to_torch
    acc = torch.empty((rows, n), dtype=torch.int32, device="cuda")
    out = mc2.mc2_alltoall_quant_matmul_static(T(x1, "i8"), r, T(s1, "f32"), T(x2, "i8"), T(s2, "f32"),
                                               acc_out=acc)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul_static(x1, r, s1, x2, s2)
    assert_bits_equal(mc2_inputs.from_torch(acc), ref["acc"], "acc")
    assert_close16(mc2_inputs.from_torch(out), ref["out"], "bf16", "out", REL, RMS_REL)


@pytest.mark.parametrize("h", [4368, 4352])
def test_a8w8_largest_rank_h(mc2, h):
    """r*H near the top of the allowed range: segments of 4368 bytes (not whole 128-byte
    steps: checked loader) and of 4352 = 34 * 128 (direct-to-LDS path)."""
    print(f"a8w8 r=8 h={h}", flush=True)
    got, ref = _run(mc2, 8, 64, h, 96, seed=h)
    assert_bits_equal(got["permuted"], ref["permuted"], "permuted")
    assert_bits_equal(got["acc"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], "bf16", "out", REL, RMS_REL)


def test_a8w8_full_config(mc2):
    """int8 (8192, 4096) on 8 ranks -> (1024, 32768) @ int8 (32768, 7168): every permuted
    byte, every int32 accumulator and every output element; two runs bit-identical."""
    import torch
    seed, d, specs = mc2_inputs.CONFIGS["a8w8"]
    t = mc2_inputs.make("a8w8")
    r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
    rows, cols = bs // r, r * h
    T = mc2_inputs.to_torch
    perm = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    acc = torch.empty((rows, n), dtype=torch.int32, device="cuda")
    args = (T(t["x1"], "i8"), r, T(t["x1_scale"], "f32"), T(t["x2"], "i8"), T(t["x2_scale"], "f32"),
            T(t["bias"], "bf16"))
    out = mc2.mc2_alltoall_quant_matmul_static(*args, permuted_out=perm, acc_out=acc)
    out2 = mc2.mc2_alltoall_quant_matmul_static(*args)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul_static(t["x1"], r, t["x1_scale"], t["x2"], t["x2_scale"], t["bias"])
    assert_bits_equal(mc2_inputs.from_torch(perm), oracle.permute_i8(t["x1"], r), "permuted")
    assert_bits_equal(mc2_inputs.from_torch(acc), ref["acc"], "acc")
    o = mc2_inputs.from_torch(out)
    assert_bits_equal(o, mc2_inputs.from_torch(out2), "run-to-run")
    assert_close16(o, ref["out"], "bf16", "out", REL, RMS_REL)
