"""CPU emulation of the rotated K walk of the GEMM main loops (gemm_mfma.hpp).

The int8 GEMM and the AllGatherMatmul loops start each workgroup's walk over
the nk steps of K at step rot = (tile row) mod nk and wrap around; step kt of
the loop handles physical step phys(kt) = (kt + rot) mod nk.  These tests
replay the loop's bookkeeping on the host and check that:

- the A offsets of the segmented K-contiguous operand (the AlltoAll permute's
  addressing: K split into segments stored kseg_stride bytes apart), advanced
  step by step with the wrap, are those of the physical steps, each once;
- in arrival mode every step's slab flag has been waited for before the loads
  of that step are issued (prologue: steps 0 and 1; step kt: step kt + 2);
- the gather copy, spread over the workgroups of a row of tiles (column tile
  tn copies the loop steps kt with kt % tiles_n == tn), writes every physical
  step of the row exactly once.
No GPU is involved.
"""
import pytest


def phys(kt, rot, nk):
    return kt + rot - nk if kt + rot >= nk else kt + rot


def a_offsets(nk, seg_steps, kseg_stride, step_bytes, rot):
    """The loop's A offsets: start at step rot, advance once per issued step."""
    seg_base = (rot // seg_steps) * kseg_stride
    a_next = seg_base + (rot % seg_steps) * step_bytes
    seg_left = seg_steps - rot % seg_steps
    a_phys = rot
    out = []
    for _ in range(nk):
        out.append(a_next)
        a_phys += 1
        if a_phys == nk:  # past the last step: back to step 0
            a_phys, seg_base, a_next, seg_left = 0, 0, 0, seg_steps
            continue
        seg_left -= 1
        if seg_left == 0:
            seg_base += kseg_stride
            a_next, seg_left = seg_base, seg_steps
        else:
            a_next += step_bytes
    return out


@pytest.mark.parametrize("nk,seg_steps", [(256, 32), (256, 256), (64, 64), (8, 4), (6, 3), (5, 5), (1, 1), (2, 1)])
def test_a_offsets_follow_the_physical_steps(nk, seg_steps):
    kseg_stride, step_bytes = 4 << 20, 128
    for rot in range(nk):
        got = a_offsets(nk, seg_steps, kseg_stride, step_bytes, rot)
        want = []
        for kt in range(nk):
            p = phys(kt, rot, nk)
            want.append((p // seg_steps) * kseg_stride + (p % seg_steps) * step_bytes)
        assert got == want, (nk, seg_steps, rot)
        assert sorted(got) == sorted(set(got)) and len(got) == nk


def arrival_waits_cover_loads(nk, sps, rot):
    """Replays the arrival loop's waits with polls that never report a slab early."""
    waited = set()
    slab = lambda kt: phys(kt, rot, nk) // sps

    def load(kt):
        assert slab(kt) in waited, f"step {kt} (physical {phys(kt, rot, nk)}) loaded before its slab arrived"

    waited.add(slab(0))
    if nk > 1 and phys(1, rot, nk) % sps == 0:
        waited.add(slab(1))
    load(0)
    if nk > 1:
        load(1)
    for kt in range(nk):
        if kt + 2 < nk:
            if phys(kt + 2, rot, nk) % sps == 0:
                waited.add(slab(kt + 2))
            load(kt + 2)
    return waited


@pytest.mark.parametrize("nk,sps", [(64, 16), (64, 64), (64, 1), (64, 5), (7, 3), (2, 1), (1, 1), (128, 8)])
def test_arrival_waits_before_every_load(nk, sps):
    slabs = (nk + sps - 1) // sps
    for rot in range(nk):
        waited = arrival_waits_cover_loads(nk, sps, rot)
        assert waited == set(range(slabs))


@pytest.mark.parametrize("nk,tiles_n", [(64, 8), (64, 1), (64, 3), (28, 32), (5, 2), (1, 4)])
def test_gather_copy_covers_each_step_once(nk, tiles_n):
    for rot in range(nk):
        copied = [phys(kt, rot, nk) for tn in range(tiles_n) for kt in range(tn, nk, tiles_n)]
        assert sorted(copied) == list(range(nk)), (nk, tiles_n, rot)
