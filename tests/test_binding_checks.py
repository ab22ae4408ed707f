"""The Python binding rejects mismatched tensors before any device work.

The C ABI receives only pointers and sizes, so a tensor smaller than the sizes
the binding passes would be read or written out of bounds on the GPU.  These
tests run on the CPU: every check below fires before the binding touches a
device (CPU tensors of the right shapes are refused last, as host memory).
"""
import pytest
import torch

import comm_matmul_tensor_amd as mc2

bf, f16, i8, f32 = torch.bfloat16, torch.float16, torch.int8, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def shards(r=4, m=16, k=256, dtype=bf):
    return [z(m, k, dtype=dtype) for _ in range(r)]


@pytest.mark.parametrize("kwargs,exc,msg", [
    (dict(shards=[z(16, 256), z(15, 256)], x2=z(256, 64)), ValueError, r"shards\[1\] has shape"),
    (dict(shards=[z(16, 256), z(16, 256, dtype=f16)], x2=z(256, 64)), TypeError, r"shards\[1\] has dtype"),
    (dict(shards=shards(dtype=f32), x2=z(256, 64, dtype=f32)), TypeError, "float16 or bfloat16"),
    (dict(shards=shards(), x2=z(255, 64)), ValueError, "x2 has shape"),
    (dict(shards=shards(), x2=z(64, 255), x2_trans=True), ValueError, "x2 has shape"),
    (dict(shards=shards(), x2=z(256, 64, dtype=f16)), TypeError, "x2 has dtype"),
    (dict(shards=shards(), x2=z(256, 64), out=z(63, 64)), ValueError, "out has shape"),
    (dict(shards=shards(), x2=z(256, 64), out=z(64, 64, dtype=f16)), TypeError, "out has dtype"),
    (dict(shards=shards(), x2=z(256, 64), out=z(64, 65)[:, :64]), ValueError, "out must be contiguous"),
    (dict(shards=shards(), x2=z(256, 64), gather_out=z(64, 128)), ValueError, "gather_out has shape"),
    (dict(shards=shards(), x2=z(256, 64)), ValueError, "must be a device tensor"),
])
def test_allgather_matmul_checks(kwargs, exc, msg):
    s = kwargs.pop("shards")
    x2 = kwargs.pop("x2")
    with pytest.raises(exc, match=msg):
        mc2.mc2_allgather_matmul(s, x2, **kwargs)


def test_backward_checks():
    with pytest.raises(ValueError, match="w has shape"):
        mc2.mc2_matmul_grad_input(z(64, 32), z(31, 128))
    with pytest.raises(ValueError, match="out has shape"):
        mc2.mc2_matmul_grad_input(z(64, 32), z(32, 128), out=z(64, 127))
    with pytest.raises(TypeError, match="w has dtype"):
        mc2.mc2_matmul_grad_input(z(64, 32), z(32, 128, dtype=f16))
    with pytest.raises(ValueError, match="ag_x has shape"):
        mc2.mc2_matmul_grad_weight(z(64, 32), z(63, 128))
    with pytest.raises(ValueError, match="out has shape"):
        mc2.mc2_matmul_grad_weight(z(64, 32), z(64, 128), out=z(128, 32))
    with pytest.raises(ValueError, match="must be a device tensor"):
        mc2.mc2_matmul_grad_weight(z(64, 32), z(64, 128))


def test_reduce_scatter_checks():
    x, x2 = z(64, 256), z(256, 32)
    recv = [None, z(16, 32), z(16, 32), z(16, 32)]
    with pytest.raises(ValueError, match=r"recv\[2\] has shape"):
        mc2.mc2_matmul_reduce_scatter(x, x2, [None, z(16, 32), z(15, 32), z(16, 32)], 0)
    with pytest.raises(ValueError, match=r"recv\[1\] is required"):
        mc2.mc2_matmul_reduce_scatter(x, x2, [None, None, z(16, 32), z(16, 32)], 0)
    with pytest.raises(ValueError, match="rank_id"):
        mc2.mc2_matmul_reduce_scatter(x, x2, recv, 4)
    with pytest.raises(ValueError, match="x2 has shape"):
        mc2.mc2_matmul_reduce_scatter(x, z(255, 32), recv, 0)
    with pytest.raises(ValueError, match="partial_out has shape"):
        mc2.mc2_matmul_reduce_scatter(x, x2, recv, 0, partial_out=z(16, 32))
    with pytest.raises(ValueError, match="must be a device tensor"):
        mc2.mc2_matmul_reduce_scatter(x, x2, recv, 0)


R, BS, H, N = 4, 64, 256, 96


@pytest.mark.parametrize("kwargs,exc,msg", [
    (dict(x2=z(R * H, N)), TypeError, "x2 has dtype"),
    (dict(x2=z(R * H - 1, N, dtype=i8)), ValueError, "x2 has shape"),
    (dict(x2_scale=z(N - 1, dtype=f32)), ValueError, "x2_scale has shape"),
    (dict(x2_scale=z(N)), TypeError, "x2_scale has dtype"),
    (dict(x1_smooth=z(H)), ValueError, "x1_smooth has shape"),
    (dict(bias=z(N + 1)), ValueError, "bias has shape"),
    (dict(out=z(BS, N)), ValueError, "out has shape"),
    (dict(q_out=z(BS // R, R * H)), TypeError, "q_out has dtype"),
    (dict(x1_scale_out=z(BS, dtype=f32)), ValueError, "x1_scale_out has shape"),
    (dict(acc_out=z(BS // R, N, dtype=f32)), TypeError, "acc_out has dtype"),
    (dict(permuted_out=z(BS // R, H)), ValueError, "permuted_out has shape"),
    (dict(rank_size=3), ValueError, "multiple of rank_size"),
    (dict(), ValueError, "must be a device tensor"),
])
def test_alltoall_quant_matmul_checks(kwargs, exc, msg):
    args = dict(x1=z(BS, H), rank_size=R, x2=z(R * H, N, dtype=i8), x2_scale=z(N, dtype=f32))
    args.update(kwargs)
    with pytest.raises(exc, match=msg):
        mc2.mc2_alltoall_quant_matmul(args.pop("x1"), args.pop("rank_size"), args.pop("x2"), args.pop("x2_scale"),
                                      **args)


@pytest.mark.parametrize("kwargs,exc,msg", [
    (dict(x1=z(BS, H)), TypeError, "x1 must be int8"),
    (dict(x1_scale=z(BS, dtype=f32)), ValueError, "x1_scale has shape"),
    (dict(x2=z(R * H, N + 1, dtype=i8), x2_scale=z(N, dtype=f32)), ValueError, "x2_scale has shape"),
    (dict(out=z(BS // R, N, dtype=f32)), TypeError, "float16 or bfloat16"),
    (dict(bias=z(N, dtype=f16)), TypeError, "bias has dtype"),
    (dict(acc_out=z(BS // R, N - 1, dtype=torch.int32)), ValueError, "acc_out has shape"),
    (dict(), ValueError, "must be a device tensor"),
])
def test_alltoall_quant_matmul_static_checks(kwargs, exc, msg):
    args = dict(x1=z(BS, H, dtype=i8), rank_size=R, x1_scale=z(BS // R, dtype=f32), x2=z(R * H, N, dtype=i8),
                x2_scale=z(N, dtype=f32))
    args.update(kwargs)
    with pytest.raises(exc, match=msg):
        mc2.mc2_alltoall_quant_matmul_static(args.pop("x1"), args.pop("rank_size"), args.pop("x1_scale"),
                                             args.pop("x2"), args.pop("x2_scale"), **args)


def test_quant_all_reduce_checks():
    xs = [z(2, 256, dtype=i8) for _ in range(4)]
    sc = [z(2, 2, dtype=f32) for _ in range(4)]
    with pytest.raises(ValueError, match=r"x\[2\] has shape"):
        mc2.mc2_quant_all_reduce(xs[:2] + [z(2, 128, dtype=i8)] + xs[3:], sc)
    with pytest.raises(ValueError, match=r"scales\[1\] holds 2 scales"):
        mc2.mc2_quant_all_reduce(xs, [sc[0], z(2, 1, dtype=f32)] + sc[2:])
    with pytest.raises(ValueError, match="one tensor per rank"):
        mc2.mc2_quant_all_reduce(xs, sc[:3])
    with pytest.raises(ValueError, match="out has shape"):
        mc2.mc2_quant_all_reduce(xs, sc, out=z(2, 255, dtype=f32))
    with pytest.raises(ValueError, match="out has shape"):
        mc2.mc2_quant_reduce_scatter([z(4, 256, dtype=i8)] * 4, [z(4, 2, dtype=f32)] * 4, 1, out=z(4, 256, dtype=f32))
    with pytest.raises(ValueError, match="divisible by the number of ranks"):
        mc2.mc2_quant_reduce_scatter([z(3, 256, dtype=i8)] * 4, [z(3, 2, dtype=f32)] * 4, 0)
    with pytest.raises(ValueError, match="must be a device tensor"):
        mc2.mc2_quant_all_reduce(xs, sc)
