"""A base that ships already packed row-major (codes [N, K/2], scales
[N, K/block]) imported into the library's tiled storage
(lora4_import_rowmajor): the oracle's packing goes in, and the result must
equal, bit for bit, both the documented tile permutation of those bytes and
what the library's own packer writes for the same bf16 W; a forward on the
imported base matches the oracle."""

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from oracle import lora
from gpu_util import (DEV, TOL, f64, oracle_dequant, oracle_pack, pack_gpu, print_case, tile_codes, tile_scales,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


@pytest.mark.parametrize("fmt,N,K,E", [
    (synth.NF4, 200, 320, 1), (synth.NF4, 64, 4096, 2), (synth.NF4_DQ, 130, 384, 1), (synth.NF4_DQ, 96, 640, 3),
    (synth.MXFP4, 100, 352, 1), (synth.MXFP4, 256, 1024, 2), (synth.NVFP4, 70, 160, 1), (synth.NVFP4, 128, 512, 2),
])
def test_import_matches_packer_and_permutation(fmt, N, K, E):
    print_case("import", fmt, N, K, E)
    lay = synth.small_layer(64, K, N, 8, fmt=fmt, index=80 + N % 7, experts=E,
                            offsets=None if E == 1 else [0] + [64] * E)
    W = synth.inputs(lay, names=("W",))["W"]
    Ws = W if W.ndim == 3 else W[None]
    packs = [oracle_pack(Ws[e], fmt) for e in range(E)]
    codes_rm = np.stack([p[0] for p in packs])
    scales_rm = np.stack([p[1] for p in packs])
    s2 = np.stack([p[2] for p in packs]) if fmt == synth.NF4_DQ else None
    base = L.import_rowmajor(fmt, _dev_u8(codes_rm),
                             _dev_f32(scales_rm) if fmt == synth.NF4 else _dev_u8(scales_rm),
                             None if s2 is None else _dev_f32(s2))
    ref = pack_gpu(W, fmt)
    torch.cuda.synchronize()
    got_c, got_s = base.codes.cpu().numpy(), base.scales.cpu().numpy()
    assert np.array_equal(got_c, ref.codes.cpu().numpy())
    assert np.array_equal(got_s.view(np.uint8), ref.scales.cpu().numpy().view(np.uint8))
    for e in range(E):
        assert np.array_equal(got_c[e], tile_codes(codes_rm[e], N, K, fmt))
        assert np.array_equal(got_s[e].view(np.uint8), tile_scales(scales_rm[e], N, K).view(np.uint8))


def test_forward_on_imported_base():
    lay = synth.small_layer(300, 640, 200, 16, fmt=synth.MXFP4, index=90)
    t = synth.inputs(lay)
    codes, e8 = oracle_pack(t["W"], synth.MXFP4)
    base = L.import_rowmajor("mxfp4", _dev_u8(codes), _dev_u8(e8))
    X, A, B = (to_dev(t[k]) for k in ("X", "A", "B"))
    Y = L.forward(base, X, A, B, lay.s)["Y"]
    torch.cuda.synchronize()
    Wd = f64(oracle_dequant((codes, e8), synth.MXFP4))
    ref = lora.forward(f64(t["X"]), Wd, f64(t["A"]), f64(t["B"]), lay.s)["Y"]
    assert lora.rel_frobenius(f64(to_host(Y)), ref) <= TOL
