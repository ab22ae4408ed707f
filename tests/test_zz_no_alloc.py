"""mc2_alltoall_quant_matmul_noalloc (the entry point for callers that cannot
allocate) against mc2_alltoall_quant_matmul on the same inputs, through the C
ABI: q, x1_scale, acc and out bit for bit (same kernels, same arithmetic),
plus the oracle on the codes.  Two calls in a row, the second smaller, so the
shared scratch array holds the first call's bytes when the second starts."""
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


def _both(mc2, name, r, bs, h, n, seed):
    import torch
    if name is None:
        t = mc2_inputs.make(mc2_inputs.configs.scaled("a16w8", r=r, bs=bs, h=h, n=n), seed=seed)
    else:
        t = mc2_inputs.make(name)
    T = mc2_inputs.to_torch
    x1, x2, s2 = T(t["x1"], "bf16"), T(t["x2"], "i8"), T(t["x2_scale"], "f32")
    sm, bias = T(t["x1_smooth"], "bf16"), T(t["bias"], "bf16")
    rows, cols = bs // r, r * h
    res = {}
    for which in ("workspace", "noalloc"):
        q = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
        s1 = torch.empty((rows,), dtype=torch.float32, device="cuda")
        acc = torch.empty((rows, n), dtype=torch.int32, device="cuda")
        out = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
        if which == "workspace":
            mc2.mc2_alltoall_quant_matmul(x1, r, x2, s2, sm, bias, out=out, q_out=q, x1_scale_out=s1, acc_out=acc)
        else:
            mc2.mc2_alltoall_quant_matmul_noalloc(x1, r, x2, s2, sm, bias, out=out, q_out=q, x1_scale_out=s1,
                                                  acc_out=acc)
        # and once more without the debug outputs: q and s1 then live in the scratch array
        out2 = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
        if which == "workspace":
            mc2.mc2_alltoall_quant_matmul(x1, r, x2, s2, sm, bias, out=out2)
        else:
            mc2.mc2_alltoall_quant_matmul_noalloc(x1, r, x2, s2, sm, bias, out=out2)
        torch.cuda.synchronize()
        F = mc2_inputs.from_torch
        res[which] = dict(q=F(q), s1=F(s1), acc=F(acc), out=F(out), out2=F(out2))
    return t, res


@pytest.mark.parametrize("calls", [[("a16w8", 8, 8192, 4096, 7168), (None, 4, 256, 512, 96)]])
def test_noalloc_matches_workspace_entry_point(mc2, calls):
    for i, (name, r, bs, h, n) in enumerate(calls):
        print(f"no-alloc call {i}: {name or 'scaled'} r={r} bs={bs} h={h} n={n}", flush=True)
        t, res = _both(mc2, name, r, bs, h, n, seed=950 + i)
        a, b = res["workspace"], res["noalloc"]
        for key in ("q", "s1", "acc", "out", "out2"):
            assert_bits_equal(b[key], a[key], f"call {i} {key}")
        assert_bits_equal(b["out2"], b["out"], f"call {i} scratch-held q vs q_out")
        p = oracle.permute(t["x1"], r)
        q_ref, s1_ref = oracle.smooth_quant(p, t["x1_smooth"])
        assert_bits_equal(b["q"], q_ref, f"call {i} q vs oracle")
        assert_bits_equal(b["s1"], s1_ref, f"call {i} s1 vs oracle")
        if name is None:  # the small call: the whole chain against the oracle
            ref = oracle.alltoall_quant_matmul(t["x1"], r, t["x2"], t["x2_scale"], t["x1_smooth"], t["bias"])
            assert_bits_equal(b["acc"], ref["acc"], f"call {i} acc vs oracle")
            assert_close16(b["out"], ref["out"], "bf16", f"call {i} out vs oracle")


def test_noalloc_rejects_sizes_beyond_the_array(mc2):
    import torch
    r, h, n = 8, 4096, 16
    rows = 1536  # rows * r * h = 48 MiB exactly, plus the scales: one token too many
    x1 = torch.zeros((rows * r, h), dtype=torch.bfloat16, device="cuda")
    x2 = torch.zeros((r * h, n), dtype=torch.int8, device="cuda")
    s2 = torch.ones((n,), dtype=torch.float32, device="cuda")
    out = torch.empty((rows, n), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mc2.Mc2Error, match="MC2_ERR_WORKSPACE"):
        mc2.mc2_alltoall_quant_matmul_noalloc(x1, r, x2, s2, out=out)
    # one token fewer fits
    x1 = torch.zeros(((rows - 1) * r, h), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((rows - 1, n), dtype=torch.bfloat16, device="cuda")
    mc2.mc2_alltoall_quant_matmul_noalloc(x1, r, x2, s2, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
