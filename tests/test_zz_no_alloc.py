"""The allocation-free forward (lora4_forward_noalloc) against lora4_forward.

Two calls in a row on one GPU, the second with a smaller input (the scratch
keeps the first call's contents), through the C ABI; each output is compared
with lora4_forward's on the same inputs: bit for bit where both run the same
schedule, else within the relative Frobenius bar, and Y against the oracle.
A request past the scratch is refused with LORA4_ERR_SCRATCH.
"""

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from oracle import lora
from gpu_util import DEV, TOL, f64, oracle_dequant, oracle_pack, pack_gpu, print_case, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(M, K, N, r, fmt, index, E=1, offsets=None):
    lay = synth.small_layer(M, K, N, r, fmt=fmt, index=index, experts=E, offsets=offsets)
    t = synth.inputs(lay)
    base = pack_gpu(t["W"], fmt)
    X, A, B = (to_dev(t[k]) for k in ("X", "A", "B"))
    offs = None if E == 1 else torch.tensor(lay.offsets, dtype=torch.int64, device=DEV)
    return lay, t, base, X, A, B, offs


def _oracle_Y(lay, t):
    if lay.experts == 1:
        Wd = f64(oracle_dequant(oracle_pack(t["W"], lay.fmt), lay.fmt))
        return lora.forward(f64(t["X"]), Wd, f64(t["A"]), f64(t["B"]), lay.s)["Y"]
    Ws = [f64(oracle_dequant(oracle_pack(t["W"][e], lay.fmt), lay.fmt)) for e in range(lay.experts)]
    return lora.grouped_forward(f64(t["X"]), Ws, [f64(a) for a in t["A"]], [f64(b) for b in t["B"]], lay.s,
                                lay.offsets)["Y"]


@pytest.mark.parametrize("first,second", [
    ((1024, 1024, 1024, 16, synth.NF4, 1), (256, 1024, 1024, 16, synth.NF4, 2)),
    ((4096, 4096, 1024, 16, synth.NF4, 3), (700, 512, 320, 8, synth.MXFP4, 4)),
    ((600, 640, 384, 24, synth.NF4_DQ, 5), (130, 640, 384, 24, synth.NF4_DQ, 6)),
    ((520, 512, 384, 256, synth.NF4, 7), (130, 512, 384, 136, synth.MXFP4, 8)),   # ranks above 128
])
def test_noalloc_matches_forward_two_calls(first, second):
    for spec in (first, second):
        M, K, N, r, fmt, idx = spec
        print_case("noalloc", M, K, N, r, fmt)
        lay, t, base, X, A, B, offs = _case(M, K, N, r, fmt, 40 + idx)
        ref = L.forward(base, X, A, B, lay.s, group_offsets=offs)
        got = L.forward_noalloc(base, X, A, B, lay.s, group_offsets=offs)
        torch.cuda.synchronize()
        for k in ("Y", "Z"):
            g, e = to_host(got[k]), to_host(ref[k])
            if not np.array_equal(g, e):
                # a different schedule (unsplit tiles) sums in another order
                assert lora.rel_frobenius(f64(g), f64(e)) <= TOL, k
        assert lora.rel_frobenius(f64(to_host(got["Y"])), _oracle_Y(lay, t)) <= TOL


def test_noalloc_grouped_and_parts():
    lay, t, base, X, A, B, offs = _case(500, 256, 320, 16, synth.MXFP4, 50, E=3, offsets=[0, 200, 200, 500])
    ref = L.forward(base, X, A, B, lay.s, group_offsets=offs, want_parts=True)
    got = L.forward_noalloc(base, X, A, B, lay.s, group_offsets=offs, want_parts=True)
    torch.cuda.synchronize()
    for k in ("Y", "Z", "Y_base", "Y_lora"):
        assert np.array_equal(to_host(got[k]), to_host(ref[k])), k
    assert lora.rel_frobenius(f64(to_host(got["Y"])), _oracle_Y(lay, t)) <= TOL


def test_noalloc_refuses_past_scratch():
    # Z partials and s Z of 600k rows at rank 256 need more than the scratch
    M, K, N, r = 600_000, 64, 64, 256
    W = L.lora4_W(L.LORA4_NF4, 64, N, K, 1, 256, 256, None)
    st = L.lora4_forward_noalloc(W, 4096, M, 4096, 4096, r, 2.0, None, 4096, None, None, None, None)
    assert st == -8 and "scratch" in L.status_string(st)
