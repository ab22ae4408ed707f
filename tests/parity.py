"""Parity checks shared by the GPU tests (test infrastructure)."""
import numpy as np


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(bits).view(np.float16).astype(np.float64)


def assert_close16(got, want, dtype, what="", rel=1e-2, rms_rel=1e-2):
    """|gpu - ref| <= rel |ref| + rms_rel rms(ref), element by element."""
    g, w = decode16(got, dtype), decode16(want, dtype)
    assert g.shape == w.shape, (g.shape, w.shape)
    rms = np.sqrt(np.mean(w ** 2)) if w.size else 0.0
    err = np.abs(g - w)
    bound = rel * np.abs(w) + rms_rel * rms
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; first at {tuple(i)}: "
                             f"gpu {g[tuple(i)]!r} ref {w[tuple(i)]!r}")


def assert_bits_equal(got, want, what=""):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    eq = got.view(np.uint8).reshape(got.shape + (-1,)) == want.view(np.uint8).reshape(want.shape + (-1,))
    bad = ~np.all(eq, axis=-1)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} differ; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} ref {want[tuple(i)]!r}")
