"""AlltoAllQuantMatmul A16W8 (dynamic per-token) on the GPU vs the oracle.

Bit-exact: the permuted layout, the int8 codes, the per-token fp32 scales
and the int32 accumulators.  The bf16 / fp16 output: |gpu - ref| <=
1e-2 |ref| + 1e-2 rms(ref) (fp32 dequant on the GPU vs fp64 in the oracle).
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


def _run(mc2, r, bs, h, n, dtype="bf16", smooth=True, bias=True, seed=0, debug=True, permuted=True):
    import torch
    specs = mc2_inputs.configs.scaled("a16w8", r=r, bs=bs, h=h, n=n)
    for key in ("x1", "x1_smooth", "bias"):
        s = specs[key]
        specs[key] = mc2_inputs.TensorSpec(s.tid, s.shape, s.dist, s.a, s.b, dtype)
    t = mc2_inputs.make(specs, seed=seed)
    T = mc2_inputs.to_torch
    rows, cols = bs // r, r * h
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    dbg = {}
    if debug:
        dbg = dict(q_out=torch.empty((rows, cols), dtype=torch.int8, device="cuda"),
                   x1_scale_out=torch.empty((rows,), dtype=torch.float32, device="cuda"),
                   acc_out=torch.empty((rows, n), dtype=torch.int32, device="cuda"))
        if permuted:
            dbg["permuted_out"] = torch.empty((rows, cols), dtype=tdt, device="cuda")
    sm = T(t["x1_smooth"], dtype) if smooth else None
    b = T(t["bias"], dtype) if bias else None
    out = mc2.mc2_alltoall_quant_matmul(T(t["x1"], dtype), r, T(t["x2"], "i8"), T(t["x2_scale"], "f32"), sm, b,
                                        **dbg)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul(t["x1"], r, t["x2"], t["x2_scale"], t["x1_smooth"] if smooth else None,
                                       t["bias"] if bias else None, dtype)
    got = {"out": mc2_inputs.from_torch(out)}
    got.update({k.replace("_out", "").replace("x1_scale", "s1"): mc2_inputs.from_torch(v) for k, v in dbg.items()})
    return got, ref


@pytest.mark.parametrize("r,bs,h,n", [
    (2, 2, 256, 16), (4, 64, 256, 96), (8, 256, 512, 300), (8, 64, 2, 40), (2, 6, 136, 33),
    (4, 520, 1024, 129), (8, 16, 4096, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_a16w8_shapes(mc2, r, bs, h, n, dtype):
    print(f"a16w8 r={r} bs={bs} h={h} n={n} {dtype}", flush=True)
    got, ref = _run(mc2, r, bs, h, n, dtype, seed=r + bs + h + n)
    assert_bits_equal(got["permuted"], ref["permuted"], "permuted")
    assert_bits_equal(got["s1"], ref["s1"], "x1_scale")
    assert_bits_equal(got["q"], ref["q"], "q")
    assert_bits_equal(got["acc"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], dtype, "out")


# Without the permuted copy the quantisation runs on the pipelined path (a
# persistent grid of at most 256 workgroups walking the tokens, C 16-byte
# chunks per thread).  Cases: C = 1..5, every thread's chunks whole (r h a
# multiple of 8192) or not, fewer tokens than workgroups, and tokens that do
# not divide evenly over 256 workgroups (1 to 3 per workgroup).
@pytest.mark.parametrize("r,bs,h,n,dtype", [
    (2, 2, 256, 16, "bf16"), (2, 20, 8, 24, "f16"), (8, 8 * 300, 512, 64, "bf16"), (4, 4 * 700, 2048, 32, "bf16"),
    (8, 8 * 40, 3072, 48, "f16"), (8, 8 * 600, 2560, 16, "bf16"), (4, 4 * 513, 4096, 16, "bf16"),
    (8, 8 * 520, 4104, 16, "bf16"), (8, 8 * 9, 4104, 40, "f16")])
def test_a16w8_pipelined_quant(mc2, r, bs, h, n, dtype):
    print(f"a16w8 pipelined r={r} bs={bs} h={h} n={n} {dtype}", flush=True)
    got, ref = _run(mc2, r, bs, h, n, dtype, seed=11 + r + bs + h, permuted=False)
    assert_bits_equal(got["s1"], ref["s1"], "x1_scale")
    assert_bits_equal(got["q"], ref["q"], "q")
    assert_bits_equal(got["acc"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], dtype, "out")


@pytest.mark.parametrize("smooth,bias", [(False, True), (True, False), (False, False)])
def test_a16w8_optional_inputs(mc2, smooth, bias):
    got, ref = _run(mc2, 4, 128, 512, 160, smooth=smooth, bias=bias, seed=3)
    assert_bits_equal(got["q"], ref["q"], "q")
    assert_bits_equal(got["s1"], ref["s1"], "x1_scale")
    assert_close16(got["out"], ref["out"], "bf16", "out")


def test_a16w8_zero_rows_and_ties(mc2):
    """All-zero tokens quantise to 0 with scale 0; rows built so y / s hits .5 exactly round to even."""
    import torch
    r, h, n = 2, 64, 32
    rows = np.zeros((4, r * h))
    rows[1, :] = np.tile([127, -2.5, 3.5, 0.5, -0.5, 1.5, 126.5, -126.5], r * h // 8)
    rows[2, ::3] = 1.0
    x1_p = oracle.encode("bf16", rows)                         # the permuted layout (4, 128)
    x1 = x1_p.reshape(4, r, h).transpose(1, 0, 2).reshape(4 * r, h).copy()  # inverse permute
    x2 = np.random.default_rng(0).integers(-127, 128, (r * h, n)).astype(np.int8)
    s2 = np.full(n, 0.01, np.float32)
    T = mc2_inputs.to_torch
    q = torch.empty((4, r * h), dtype=torch.int8, device="cuda")
    s1 = torch.empty((4,), dtype=torch.float32, device="cuda")
    out = mc2.mc2_alltoall_quant_matmul(T(x1, "bf16"), r, T(x2, "i8"), T(s2, "f32"), q_out=q, x1_scale_out=s1)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul(x1, r, x2, s2)
    assert_bits_equal(mc2_inputs.from_torch(q), ref["q"], "q")
    assert_bits_equal(mc2_inputs.from_torch(s1), ref["s1"], "s1")
    assert float(ref["s1"][0]) == 0.0 and not ref["q"][0].any()
    assert ref["q"][1, :8].tolist() == [127, -2, 4, 0, 0, 2, 126, -126]
    assert_close16(mc2_inputs.from_torch(out), ref["out"], "bf16", "out")


@pytest.mark.parametrize("permuted", [False, True])
@pytest.mark.parametrize("h", [64, 4096])
def test_a16w8_subnormal_scales(mc2, permuted, h):
    """Tokens whose scale amax / 127 is subnormal (every code through the division),
    tokens of subnormal inputs (y rounds in fp32), a token with one huge value and
    an ordinary one; pipelined path (no permuted copy) and one token per workgroup."""
    import torch
    r, n = 2, 16
    rng = np.random.default_rng(h + permuted)
    rows = rng.uniform(-1.0, 1.0, (4, r * h))
    rows[0] *= 1e-37          # normal bf16 values, s about 6e-40 (subnormal)
    rows[1] *= 3e-39          # subnormal bf16 values
    rows[2, 5] = 3e38         # one huge value, the rest of the row tiny relative to it
    rows[3] = rng.standard_normal(r * h)
    x1_p = oracle.encode("bf16", rows)
    x1 = x1_p.reshape(4, r, h).transpose(1, 0, 2).reshape(4 * r, h).copy()
    sm = oracle.encode("bf16", rng.uniform(0.5, 2.0, r * h))
    x2 = rng.integers(-127, 128, (r * h, n)).astype(np.int8)
    s2 = np.full(n, 0.01, np.float32)
    T = mc2_inputs.to_torch
    q = torch.empty((4, r * h), dtype=torch.int8, device="cuda")
    s1 = torch.empty((4,), dtype=torch.float32, device="cuda")
    extra = {"permuted_out": torch.empty((4, r * h), dtype=torch.bfloat16, device="cuda")} if permuted else {}
    print(f"a16w8 subnormal scales h={h} permuted={permuted}", flush=True)
    mc2.mc2_alltoall_quant_matmul(T(x1, "bf16"), r, T(x2, "i8"), T(s2, "f32"), T(sm, "bf16"),
                                  q_out=q, x1_scale_out=s1, **extra)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul(x1, r, x2, s2, sm)
    assert 0.0 < float(ref["s1"][0]) < 1.1754944e-38 and 0.0 < float(ref["s1"][1]) < 1.1754944e-38
    assert np.abs(ref["q"][0]).max() == 127 and np.abs(ref["q"][1]).max() == 127
    assert_bits_equal(mc2_inputs.from_torch(s1), ref["s1"], "s1")
    assert_bits_equal(mc2_inputs.from_torch(q), ref["q"], "q")


@pytest.mark.parametrize("permuted", [False, True])
def test_a16w8_tiny_f16_values(mc2, permuted):
    """fp16 tokens of small (1e-4) and subnormal (3e-6) values, one with a value near the
    fp16 maximum and an ordinary one: the fp16 decode of subnormal codes and the scales
    (normal in fp32 here) through both kernels."""
    import torch
    r, h, n = 2, 64, 16
    rng = np.random.default_rng(5 + permuted)
    rows = rng.uniform(-1.0, 1.0, (4, r * h))
    rows[0] *= 1e-4
    rows[1] *= 3e-6          # fp16 subnormal codes
    rows[2, 5] = 6e4
    rows[3] = rng.standard_normal(r * h)
    x1_p = oracle.encode("f16", rows)
    x1 = x1_p.reshape(4, r, h).transpose(1, 0, 2).reshape(4 * r, h).copy()
    sm = oracle.encode("f16", rng.uniform(0.5, 2.0, r * h))
    x2 = rng.integers(-127, 128, (r * h, n)).astype(np.int8)
    s2 = np.full(n, 0.01, np.float32)
    T = mc2_inputs.to_torch
    q = torch.empty((4, r * h), dtype=torch.int8, device="cuda")
    s1 = torch.empty((4,), dtype=torch.float32, device="cuda")
    extra = {"permuted_out": torch.empty((4, r * h), dtype=torch.float16, device="cuda")} if permuted else {}
    print(f"a16w8 tiny f16 values permuted={permuted}", flush=True)
    mc2.mc2_alltoall_quant_matmul(T(x1, "f16"), r, T(x2, "i8"), T(s2, "f32"), T(sm, "f16"),
                                  q_out=q, x1_scale_out=s1, **extra)
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul(x1, r, x2, s2, sm, None, "f16")
    assert np.abs(ref["q"][1]).max() == 127
    assert_bits_equal(mc2_inputs.from_torch(s1), ref["s1"], "s1")
    assert_bits_equal(mc2_inputs.from_torch(q), ref["q"], "q")


@pytest.mark.parametrize("h", [4374, 4368])
def test_a16w8_largest_rank_h(mc2, h):
    """r*H at the top of the allowed range: 34992 (H not a multiple of 16, element path)
    and 34944 (vector path with three 16-element units per thread)."""
    print(f"a16w8 r=8 h={h}", flush=True)
    got, ref = _run(mc2, 8, 16, h, 48, seed=h)
    assert_bits_equal(got["q"], ref["q"], "q")
    assert_bits_equal(got["s1"], ref["s1"], "x1_scale")
    assert_bits_equal(got["acc"], ref["acc"], "acc")
    assert_close16(got["out"], ref["out"], "bf16", "out")


def test_a16w8_full_config(mc2):
    """bf16 (8192, 4096) on 8 ranks -> (1024, 32768) @ int8 (32768, 7168): every code and
    scale, every int32 accumulator (bit for bit) and every output element."""
    import torch
    seed, d, specs = mc2_inputs.CONFIGS["a16w8"]
    t = mc2_inputs.make("a16w8")
    r, bs, h, n = d["r"], d["bs"], d["h"], d["n"]
    rows, cols = bs // r, r * h
    T = mc2_inputs.to_torch
    q = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    s1 = torch.empty((rows,), dtype=torch.float32, device="cuda")
    acc = torch.empty((rows, n), dtype=torch.int32, device="cuda")
    out = mc2.mc2_alltoall_quant_matmul(T(t["x1"], "bf16"), r, T(t["x2"], "i8"), T(t["x2_scale"], "f32"),
                                        T(t["x1_smooth"], "bf16"), T(t["bias"], "bf16"),
                                        q_out=q, x1_scale_out=s1, acc_out=acc)
    out2 = mc2.mc2_alltoall_quant_matmul(T(t["x1"], "bf16"), r, T(t["x2"], "i8"), T(t["x2_scale"], "f32"),
                                         T(t["x1_smooth"], "bf16"), T(t["bias"], "bf16"))
    torch.cuda.synchronize()
    ref = oracle.alltoall_quant_matmul(t["x1"], r, t["x2"], t["x2_scale"], t["x1_smooth"], t["bias"])
    assert_bits_equal(mc2_inputs.from_torch(q), ref["q"], "q")
    assert_bits_equal(mc2_inputs.from_torch(s1), ref["s1"], "s1")
    assert_bits_equal(mc2_inputs.from_torch(acc), ref["acc"], "acc")
    o = mc2_inputs.from_torch(out)
    assert_bits_equal(o, mc2_inputs.from_torch(out2), "run-to-run")
    assert_close16(o, ref["out"], "bf16", "out")
