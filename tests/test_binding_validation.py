"""Argument checks of the Python binding (CPU tensors, no library calls).

The C ABI receives raw pointers and takes K and N from the base descriptor, so
a wrong dtype, a non-contiguous view or a short tensor would reach the kernels
unnoticed; the binding rejects them before any pointer is passed on.
"""

import pytest
import torch

import lora_fine_tuning_amd as L

bf = torch.bfloat16


def _base(N=96, K=128, groups=1):
    codes = torch.zeros((groups, 16), dtype=torch.uint8)
    scales = torch.zeros((groups, 16), dtype=torch.float32)
    return L.PackedBase(L.LORA4_NF4, N, K, groups, codes, scales, None)


def _layer(M=40, N=96, K=128, r=8, groups=1):
    X = torch.zeros((M, K), dtype=bf)
    if groups == 1:
        A, B = torch.zeros((r, K), dtype=bf), torch.zeros((N, r), dtype=bf)
    else:
        A, B = torch.zeros((groups, r, K), dtype=bf), torch.zeros((groups, N, r), dtype=bf)
    return X, A, B


def test_valid_plain_and_grouped():
    b = _base()
    X, A, B = _layer()
    assert L.check_layer_args(b, X, A, B, dY=torch.zeros((40, 96), dtype=bf), Z=torch.zeros((40, 8), dtype=bf)) \
        == (40, 8, 1)
    g = _base(groups=3)
    X, A, B = _layer(groups=3)
    offs = torch.tensor([0, 10, 10, 40], dtype=torch.int64)
    assert L.check_layer_args(g, X, A, B, offsets=offs) == (40, 8, 3)
    # several adapters over one base
    X, A, B = _layer(groups=5)
    assert L.check_layer_args(b, X, A, B, offsets=torch.zeros(6, dtype=torch.int64), adapters=5) == (40, 8, 5)


@pytest.mark.parametrize("what", ["x_dtype", "x_k", "a_k", "b_n", "a_rank", "x_view", "dy_shape", "z_rank",
                                  "out_shape"])
def test_plain_layer_rejects(what):
    b = _base()
    X, A, B = _layer()
    dY = Z = None
    outputs = ()
    if what == "x_dtype":
        X = X.float()
    elif what == "x_k":
        X = torch.zeros((40, 64), dtype=bf)
    elif what == "a_k":
        A = torch.zeros((8, 64), dtype=bf)
    elif what == "b_n":
        B = torch.zeros((95, 8), dtype=bf)
    elif what == "a_rank":
        B = torch.zeros((96, 4), dtype=bf)
    elif what == "x_view":
        X = torch.zeros((128, 40), dtype=bf).t()
    elif what == "dy_shape":
        dY = torch.zeros((40, 95), dtype=bf)
    elif what == "z_rank":
        Z = torch.zeros((40, 4), dtype=bf)
    elif what == "out_shape":
        outputs = [("Y", torch.zeros((40, 95), dtype=bf), (40, 96))]
    with pytest.raises(ValueError):
        L.check_layer_args(b, X, A, B, dY=dY, Z=Z, outputs=outputs)


@pytest.mark.parametrize("what", ["no_offsets", "offsets_len", "offsets_dtype", "a_groups", "two_d_a",
                                  "offsets_plain"])
def test_grouped_rejects(what):
    g = _base(groups=3)
    X, A, B = _layer(groups=3)
    offs = torch.tensor([0, 10, 10, 40], dtype=torch.int64)
    if what == "no_offsets":
        offs = None
    elif what == "offsets_len":
        offs = torch.tensor([0, 10, 40], dtype=torch.int64)
    elif what == "offsets_dtype":
        offs = offs.int()
    elif what == "a_groups":
        A = torch.zeros((2, 8, 128), dtype=bf)
    elif what == "two_d_a":
        A = torch.zeros((8, 128), dtype=bf)
    if what == "offsets_plain":
        X, A, B = _layer()
        with pytest.raises(ValueError):
            L.check_layer_args(_base(), X, A, B, offsets=torch.tensor([0, 40], dtype=torch.int64))
        return
    with pytest.raises(ValueError):
        L.check_layer_args(g, X, A, B, offsets=offs)


def test_adapters_need_one_group_base():
    X, A, B = _layer(groups=2)
    with pytest.raises(ValueError):
        L.check_layer_args(_base(groups=2), X, A, B, offsets=torch.zeros(3, dtype=torch.int64), adapters=2)


def test_workspace_and_pack_inputs():
    ws = torch.zeros(100, dtype=torch.uint8)
    L._check_workspace(ws, 100, ws.device)
    with pytest.raises(ValueError):
        L._check_workspace(ws, 101, ws.device)
    with pytest.raises(ValueError):
        L._check_workspace(torch.zeros(100, dtype=torch.int16), 10, ws.device)
    L._check_pack_input(torch.zeros((4, 64), dtype=bf))
    for bad in (torch.zeros((4, 64)), torch.zeros((64, 4), dtype=bf).t(), torch.zeros(64, dtype=bf)):
        with pytest.raises(ValueError):
            L._check_pack_input(bad)
