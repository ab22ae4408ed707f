"""Host-side pieces of the layer module (comm_matmul_tensor_amd.linear) on the CPU:
the sequence-dimension moves and their inverse, and argument checks that fire
before any device work."""
import pytest
import torch

from comm_matmul_tensor_amd.linear import MC2Linear, move_dim_to_front, move_front_to_dim, normalize_sequence_dim


@pytest.mark.parametrize("shape", [(3, 5, 7), (2, 3, 4, 5)])
def test_move_dims_are_inverse(shape):
    t = torch.arange(torch.tensor(shape).prod().item()).reshape(shape)
    for d in range(len(shape) - 1):
        f = move_dim_to_front(t, d)
        assert f.shape[0] == shape[d]
        assert torch.equal(move_front_to_dim(f, d), t)
        # element (i at dim d, rest) lands at (i, rest in order)
        idx = [1] * len(shape)
        idx[d] = shape[d] - 1
        rest = [idx[i] for i in range(len(shape)) if i != d]
        assert f[(idx[d], *rest)] == t[tuple(idx)]


def test_normalize_sequence_dim():
    assert normalize_sequence_dim(-1, 2) == 1 and normalize_sequence_dim(0, 2) == 0
    for bad in (2, -3):
        with pytest.raises(ValueError):
            normalize_sequence_dim(bad, 2)


def test_mc2linear_argument_checks():
    with pytest.raises(ValueError, match="mode"):
        MC2Linear(256, 256, 4, "ring", device="cpu")
    with pytest.raises(ValueError, match="out_features"):
        MC2Linear(256, 258, 4, "allgather", device="cpu")
    with pytest.raises(ValueError, match="in_features"):
        MC2Linear(258, 256, 4, "reduce_scatter", device="cpu")
    lin = MC2Linear(256, 1024, 4, "allgather", device="cpu")
    assert [tuple(w.shape) for w in lin.weights] == [(256, 256)] * 4 and len(lin.biases) == 4
    lin = MC2Linear(1024, 256, 4, "reduce_scatter", bias=False, device="cpu")
    assert [tuple(w.shape) for w in lin.weights] == [(256, 256)] * 4 and len(lin.biases) == 0
    with pytest.raises(ValueError, match="per-rank inputs"):
        lin([torch.zeros(4, 256)] * 3)
