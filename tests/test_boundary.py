"""The C-ABI library on the CPU: it loads, exports what include/mc2.h declares,
and rejects bad arguments on the host before touching any device."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mc2.h")
LIB = os.path.join(ROOT, "comm_matmul_tensor_amd", "libmc2.so")

# fake, 16-byte aligned addresses: only ever passed to calls that fail validation
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mc2_status|const char\*)\s+(mc2_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmc2.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    lib.mc2_status_string.restype = ctypes.c_char_p
    for s in range(9):
        assert lib.mc2_status_string(s).decode().startswith("MC2_")


def test_quant_mode_enum_matches_pages():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "quant_modes.json")))
    src = open(HEADER).read()
    for name, val in gold["modes"].items():
        m = re.search(rf"MC2_QUANT_{name.upper()}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == val, name


def _ptrs(*ps):
    return (ctypes.c_void_p * len(ps))(*[p.value if isinstance(p, ctypes.c_void_p) else p for p in ps])


def _err(lib):
    lib.mc2_last_error.restype = ctypes.c_char_p
    return lib.mc2_last_error().decode()


def test_allgather_matmul_validation(lib):
    f = lib.mc2_allgather_matmul
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    sh = _ptrs(A, A, A, A, A, A, A, A)
    BF16, F32 = 2, 0
    assert f(sh, 3, 16, 512, B, 64, 0, BF16, C, None, 0, 0, None) == 2            # world_size 3
    assert "world_size" in _err(lib)
    assert f(sh, 8, 16, 255, B, 64, 0, BF16, C, None, 0, 0, None) == 2            # k below 256
    assert f(sh, 8, 16, 65535, B, 64, 0, BF16, C, None, 0, 0, None) == 2          # k at 65535
    assert f(sh, 8, 0, 512, B, 64, 0, BF16, C, None, 0, 0, None) == 2             # empty
    assert f(sh, 8, 16, 512, B, 64, 0, F32, C, None, 0, 0, None) == 3             # fp32 input
    assert f(sh, 8, 16, 512, None, 64, 0, BF16, C, None, 0, 0, None) == 1         # x2 NULL
    assert f(_ptrs(A, None), 2, 16, 512, B, 64, 0, BF16, C, None, 0, 0, None) == 1
    assert f(sh, 8, 16, 512, B, 64, 0, BF16, C, None, 1, 0, None) == 1            # arrival w/o gather_out
    assert f(sh, 8, 16, 512, B, 64, 0, BF16, C, A, 1, 9, None) == 2               # bad rank_id
    assert f(sh, 8, 16, 512, B, 64, 0, BF16, C, None, 7, 0, None) == 4            # unknown mode
    assert f(sh, 8, 16, 512, ctypes.c_void_p(0x20008), 64, 0, BF16, C, None, 0, 0, None) == 8  # misaligned


def test_backward_validation(lib):
    gi, gw = lib.mc2_matmul_grad_input, lib.mc2_matmul_grad_weight
    for f in (gi, gw):
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert gi(A, B, 8192, 255, 4096, 2, C, None) == 2     # contraction n_local below 256
    assert gi(A, B, 8192, 65535, 4096, 2, C, None) == 2
    assert gi(A, B, 8192, 1792, 4096, 3, C, None) == 3    # int8 dtype
    assert gi(A, None, 8192, 1792, 4096, 2, C, None) == 1
    assert gw(A, B, 0, 1792, 4096, 2, C, None) == 2
    assert gw(A, B, 8192, 1792, 4096, 0, C, None) == 3


def test_alltoall_validation(lib):
    ws = lib.mc2_alltoall_quant_matmul_workspace_size
    ws.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    n = ctypes.c_size_t(0)
    assert ws(8, 8192, 4096, 7168, ctypes.byref(n)) == 0 and n.value >= 1024 * 32768
    assert ws(8, 8190, 4096, 7168, ctypes.byref(n)) == 2   # bs not divisible by rank_size
    assert ws(8, 8192, 4376, 7168, ctypes.byref(n)) == 2   # rank_size*h above 35000
    assert ws(4, 8192, 1002, 7168, ctypes.byref(n)) == 2   # rank_size*h not a multiple of 16
    assert ws(3, 8192, 4096, 7168, ctypes.byref(n)) == 2
    assert ws(8, 8192, 4096, 0, ctypes.byref(n)) == 2      # empty
    assert ws(8, 8192, 4096, 2 ** 31, ctypes.byref(n)) == 2  # n above INT32_MAX
    f = lib.mc2_alltoall_quant_matmul
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    assert ws(8, 64, 256, 32, ctypes.byref(n)) == 0
    need = n.value
    args = [A, 8, 64, 256, 2, B, 32, C, None, None, C, None, None, None, None, A, need, None]
    bad = list(args); bad[0] = None
    assert f(*bad) == 1                                    # x1 NULL
    bad = list(args); bad[16] = need - 1
    assert f(*bad) == 5                                    # workspace too small
    bad = list(args); bad[4] = 0
    assert f(*bad) == 3                                    # fp32 activations


def test_alltoall_static_validation(lib):
    f = lib.mc2_alltoall_quant_matmul_static
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    args = [A, 8, 64, 256, B, C, 32, B, None, A, 2, None, None, None]
    for i in (0, 4, 5, 7, 9):                              # x1, x1_scale, x2, x2_scale, out
        bad = list(args); bad[i] = None
        assert f(*bad) == 1
    bad = list(args); bad[1] = 3
    assert f(*bad) == 2                                    # rank_size 3
    bad = list(args); bad[2] = 60
    assert f(*bad) == 2                                    # bs not divisible by rank_size
    bad = list(args); bad[3] = 4376
    assert f(*bad) == 2                                    # rank_size*h above 35000
    bad = list(args); bad[6] = 0
    assert f(*bad) == 2                                    # empty
    bad = list(args); bad[10] = 0
    assert f(*bad) == 3                                    # fp32 out
    bad = list(args); bad[11] = ctypes.c_void_p(0x10008)
    assert f(*bad) == 8                                    # permuted_out misaligned


def test_int4_validation(lib):
    """A16W4 / A4W4: int4 codes two per byte (n even; A4W4 also h even); the
    workspace holds the widened int8 operands."""
    P4 = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    w16 = lib.mc2_alltoall_quant_matmul_a16w4_workspace_size
    w44 = lib.mc2_alltoall_quant_matmul_a4w4_workspace_size
    w8 = lib.mc2_alltoall_quant_matmul_workspace_size
    for f in (w16, w44, w8):
        f.argtypes = P4
    n, m = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert w8(8, 8192, 4096, 7168, ctypes.byref(m)) == 0
    assert w16(8, 8192, 4096, 7168, ctypes.byref(n)) == 0 and n.value == m.value + 32768 * 7168
    assert w16(8, 8192, 4096, 7167, ctypes.byref(n)) == 2     # n odd
    assert w16(4, 8192, 1002, 7168, ctypes.byref(n)) == 2     # rank_size*h not a multiple of 16
    assert w44(8, 8192, 4096, 7168, ctypes.byref(n)) == 0 and n.value == 8192 * 4096 + 32768 * 7168
    assert w44(4, 12, 6, 2, ctypes.byref(n)) == 0 and n.value == 256 + 24 * 2   # x1 part rounded up to 256
    assert w44(8, 8192, 4095, 7168, ctypes.byref(n)) == 2     # h odd
    assert w44(8, 8192, 4096, 7167, ctypes.byref(n)) == 2     # n odd
    assert w44(8, 8192, 4376, 7168, ctypes.byref(n)) == 2     # rank_size*h above 35000
    assert w44(8, 8192, 4096, 7168, None) == 1
    f = lib.mc2_alltoall_quant_matmul_a4w4
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert w44(8, 64, 256, 32, ctypes.byref(n)) == 0
    args = [A, 8, 64, 256, B, C, 32, B, None, A, 2, None, C, n.value, None]
    for i in (0, 4, 5, 7, 9):                                 # x1, x1_scale, x2, x2_scale, out
        bad = list(args); bad[i] = None
        assert f(*bad) == 1
    bad = list(args); bad[13] = n.value - 1
    assert f(*bad) == 5                                       # workspace too small
    bad = list(args); bad[12] = None
    assert f(*bad) == 5                                       # no workspace
    bad = list(args); bad[12] = ctypes.c_void_p(0x30008)
    assert f(*bad) == 8                                       # workspace misaligned
    bad = list(args); bad[3] = 255
    assert f(*bad) == 2                                       # h odd
    bad = list(args); bad[10] = 0
    assert f(*bad) == 3                                       # fp32 out
    g = lib.mc2_alltoall_quant_matmul_a16w4
    g.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    assert w16(8, 64, 256, 32, ctypes.byref(n)) == 0
    args = [A, 8, 64, 256, 2, B, 32, C, None, None, C, None, None, None, None, A, n.value, None]
    bad = list(args); bad[16] = n.value - 1
    assert g(*bad) == 5                                       # workspace without room for the widened weight
    bad = list(args); bad[6] = 31
    assert g(*bad) == 2                                       # n odd
    bad = list(args); bad[5] = None
    assert g(*bad) == 1                                       # x2 NULL


def test_matmul_reduce_scatter_validation(lib):
    f = lib.mc2_matmul_reduce_scatter
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    recv = _ptrs(A, None, B, C)                            # rank 1's own slot NULL
    args = [A, B, 4, 1, 64, 256, 32, 0, 2, recv, C, A, None]
    for i in (0, 1, 9, 10, 11):                            # x, x2, recv, out, partial_out
        bad = list(args); bad[i] = None
        assert f(*bad) == 1
    bad = list(args); bad[9] = _ptrs(A, B, None, C)
    assert f(*bad) == 1                                    # a peer's block NULL
    bad = list(args); bad[2] = 3
    assert f(*bad) == 2                                    # world size 3
    bad = list(args); bad[3] = 4
    assert f(*bad) == 2                                    # rank out of range
    bad = list(args); bad[4] = 62
    assert f(*bad) == 2                                    # m not divisible by world size
    bad = list(args); bad[5] = 255
    assert f(*bad) == 2                                    # contraction below 256
    bad = list(args); bad[5] = 65535
    assert f(*bad) == 2
    bad = list(args); bad[8] = 0
    assert f(*bad) == 3                                    # fp32
    bad = list(args); bad[10] = ctypes.c_void_p(0x30002)
    assert f(*bad) == 8                                    # out misaligned


def test_quant_all_reduce_validation(lib):
    f = lib.mc2_quant_all_reduce
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    xs, ss = _ptrs(A, A), _ptrs(B, B)
    I8, E4M3, E5M2, E8M0, F32, BF16, I32 = 3, 5, 6, 7, 0, 2, 4
    assert f(xs, ss, 2, 8, 1000, I8, F32, C, F32, None) == 2      # h not 128-aligned / below 1024
    assert f(xs, ss, 2, 8, 8320, I8, F32, C, F32, None) == 2      # h above 8192
    assert f(xs, ss, 2, 0, 1024, I8, F32, C, F32, None) == 2      # empty
    assert f(xs, ss, 6, 8, 1024, I8, F32, C, F32, None) == 2      # world size 6
    assert f(xs, ss, 2, 8, 1024, I8, E8M0, C, F32, None) == 3     # E8M0 needs fp8 x
    assert f(xs, ss, 2, 8, 1024, E4M3, I32, C, F32, None) == 3    # bad scale dtype
    assert f(xs, ss, 2, 8, 1024, E5M2, E8M0, C, I32, None) == 3   # bad out dtype
    assert f(xs, _ptrs(B, None), 2, 8, 1024, I8, F32, C, F32, None) == 1


def test_quant_reduce_scatter_validation(lib):
    f = lib.mc2_quant_reduce_scatter
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    xs, ss = _ptrs(A, A), _ptrs(B, B)
    I8, F32, BF16 = 3, 0, 2
    assert f(xs, ss, 2, 2, 8, 1024, I8, F32, C, F32, None) == 2     # rank out of range
    assert f(xs, ss, 2, 0, 7, 1024, I8, F32, C, F32, None) == 2     # rows not divisible by world size
    assert f(xs, ss, 2, 0, 8, 1000, I8, F32, C, F32, None) == 2     # h not 128-aligned
    assert f(xs, ss, 2, -1, 8, 1024, I8, F32, C, BF16, None) == 2
    assert f(xs, _ptrs(B, None), 2, 0, 8, 1024, I8, F32, C, F32, None) == 1
    assert f(xs, ss, 2, 0, 8, 1024, I8, 7, C, F32, None) == 3       # E8M0 scales with int8 x


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_no_device(lib):
    f = lib.mc2_quant_all_reduce
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert f(_ptrs(A, A), _ptrs(B, B), 2, 8, 1024, 3, 0, C, 0, None) == 6


def test_noalloc_rejects_sizes_beyond_its_array_on_the_host(lib):
    """The no-allocation A16W8 call refuses sizes whose workspace exceeds its 48 MiB array
    before any device call (this runs without a GPU), and names the limit."""
    f = lib.mc2_alltoall_quant_matmul_noalloc
    f.restype = ctypes.c_int
    I64 = ctypes.c_int64
    # rank_size 8, h 4096: 1536 tokens need 48 MiB of codes plus the scales
    st = f(A, 8, I64(8 * 1536), I64(4096), 2, B, I64(16), C, None, None, A, None, None, None, None, None)
    assert st == 5, st  # MC2_ERR_WORKSPACE
    assert "50331648" in _err(lib)
    # sizes the operator itself rejects keep their own status
    st = f(A, 3, I64(8 * 1536), I64(4096), 2, B, I64(16), C, None, None, A, None, None, None, None, None)
    assert st == 2, st  # MC2_ERR_SHAPE
