"""The seeded input generator: determinism, shapes and distributions."""

import numpy as np
import torch

import synth


def test_to_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (synth.to_bf16(x) == ref).all()


def test_deterministic_and_shapes():
    lay = synth.layers(1)[0]
    a = synth.inputs(lay)
    b = synth.inputs(lay)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["X"].shape == (256, 1024) and a["W"].shape == (1024, 1024)
    assert a["A"].shape == (16, 1024) and a["B"].shape == (1024, 16) and a["dY"].shape == (256, 1024)


def test_distributions():
    lay = synth.layers(1)[0]
    t = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).double().numpy() for k, v in synth.inputs(lay).items()}
    assert abs(t["X"].std() - 1) < 0.01 and abs(t["dY"].std() - 1) < 0.01
    assert abs(t["W"].std() - 0.02) < 0.0005
    assert abs(t["B"].std() - 0.01) < 0.0005
    assert np.abs(t["A"]).max() <= 1 / 32 and abs(t["A"].std() - (1 / 32) / np.sqrt(3)) < 0.0005


def test_workload_shapes_and_flops():
    l2 = synth.layers(2)
    assert [(l.K, l.N) for l in l2] == [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096),
                                          (4096, 14336), (4096, 14336), (14336, 4096)]
    assert abs(sum(l.flops() for l in l2) / 1e9 - 3606) < 1
    assert abs(synth.layers(1)[0].flops() / 1e9 - 1.124) < 0.001
    assert abs(sum(l.flops() for l in synth.layers(3)) / 1e9 - 17876) < 1
    l4 = synth.layers(4)
    assert l4[0].M == 32768 and l4[0].experts == 64 and len(l4[0].offsets) == 65
    assert abs(sum(l.flops() for l in l4) / 1e9 - 5859) < 1
    assert abs(synth.layers(5)[0].flops() / 1e9 - 3694) < 1
    assert synth.layers(5)[0].fmt == synth.NF4_DQ and synth.layers(3)[0].block == 32
