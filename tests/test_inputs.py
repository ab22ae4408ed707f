"""The seeded input generator: stream definition, distributions, storage encoders (CPU)."""
import numpy as np
import torch

import mc2_inputs

M64 = (1 << 64) - 1


def _mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_stream_matches_splitmix64_definition():
    """Pure-Python SplitMix64 (Steele, Lea, Flood 2014) against the C generator."""
    for seed, tid in ((1, 0), (5, 31), (123456, 7)):
        key = _mix64(((seed << 32) ^ tid ^ 0xD1B54A32D192ED03) & M64)
        want = [_mix64((key + (i + 1) * 0x9E3779B97F4A7C15) & M64) for i in range(64)]
        assert mc2_inputs.words(seed, tid, 64).tolist() == want
        assert mc2_inputs.words(seed, tid, 16, start=48).tolist() == want[48:]


def test_deterministic_and_sliceable():
    a = mc2_inputs.fill(3, 0, "normal", 0, 1, "bf16", (1000,))
    b = mc2_inputs.fill(3, 0, "normal", 0, 1, "bf16", (1000,))
    c = mc2_inputs.fill(3, 0, "normal", 0, 1, "bf16", (400,), start=600)
    assert np.array_equal(a, b) and np.array_equal(a[600:], c)
    assert not np.array_equal(a, mc2_inputs.fill(3, 1, "normal", 0, 1, "bf16", (1000,)))


def test_distributions():
    n = 1 << 20
    z = mc2_inputs.fill(2, 9, "normal", 0.0, 1.0, "f32", (n,))
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    u = mc2_inputs.fill(2, 10, "uniform", 1e-3, 1e-2, "f32", (n,))
    assert u.min() >= 1e-3 and u.max() < 1e-2 and abs(u.mean() - 5.5e-3) < 2e-5
    i = mc2_inputs.fill(2, 11, "int", -127, 127, "i8", (n,))
    assert i.min() == -127 and i.max() == 127 and abs(i.mean()) < 0.2
    e = mc2_inputs.fill(2, 12, "int", -8, 0, "e8m0", (n,))
    assert set(np.unique(e).tolist()) == set(range(119, 128))


def test_storage_encoders_match_torch():
    f = mc2_inputs.fill(4, 1, "normal", 0.0, 3.0, "f32", (200000,))
    bf = mc2_inputs.fill(4, 1, "normal", 0.0, 3.0, "bf16", (200000,))
    assert np.array_equal(bf, torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    h = mc2_inputs.fill(4, 1, "normal", 0.0, 3.0, "f16", (200000,))
    assert np.array_equal(h.view(np.uint16), f.astype(np.float16).view(np.uint16))
    f8 = mc2_inputs.fill(4, 1, "normal", 0.0, 3.0, "e4m3fn", (200000,))
    lib = torch.from_numpy(np.clip(f, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f8, lib)
    big = mc2_inputs.fill(4, 2, "normal", 0.0, 1000.0, "e4m3fn", (10000,))
    assert not np.any((big & 0x7F) == 0x7F) and np.any((big & 0x7F) == 0x7E)  # saturated, no NaN


def test_config_shapes():
    seed, dims, specs = mc2_inputs.CONFIGS["a16w8"]
    assert specs["x1"].shape == (8192, 4096) and specs["x1_smooth"].shape == (32768,)
    assert specs["x2"].shape == (32768, 7168) and specs["x2_scale"].shape == (7168,)
    seed, dims, specs = mc2_inputs.CONFIGS["qar_mx"]
    assert specs["scale3"].shape == (4, 2048, 112, 2) and specs["x7"].dtype == "e4m3fn"
    tids = [s.tid for name in mc2_inputs.CONFIGS for s in mc2_inputs.CONFIGS[name][2].values()
            if mc2_inputs.CONFIGS[name][0] == 5]
    assert len(tids) == len(set(tids))  # the two QuantAllReduce workloads share seed 5, not streams
