"""GPU parity at the full sizes of the benchmark workloads, on every element.

Every layer of the Llama-3-8B-shaped set (NF4), the Llama-70B-shaped MXFP4
layers, the 64-expert MoE layers (grouped, MXFP4; all 64 experts), the
long-context NF4 layer with double-quantized scales, the 16-adapter layers
over one base and NVFP4 bases of the 8B set run through the library's entry
points as bench.py calls them. The oracle then redoes each layer in full:

* packing: the whole packed base (codes, first- and second-level scales) equals
  the documented tile permutation of the oracle's row-major packing, bit for
  bit;
* Y, Z, dX, dA, dB: every element, with relative Frobenius error <= 5e-3 and
  |gpu - oracle| within the element bound of gpu_util.element_bound (bf16
  rounding of the output and of the one bf16 intermediate, Z or dZ, that
  feeds it);
* every output and both workspaces sit between guard bands that must come
  back untouched.

The oracle packs and dequantizes row ranges in host threads (packing is row
local; NF4-DQ's second-level step runs on the whole scale array) and runs the
products in float64 BLAS.
"""

import dataclasses

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from gpu_util import (DEV, compare_full, f64, guarded, oracle_dequant_full, oracle_pack_full, print_case,
                      tile_codes, tile_scales, to_dev, to_host, write_report)

pytestmark = pytest.mark.gpu


def _pack_gpu(W, fmt):
    Wd = to_dev(W)
    if fmt == synth.MXFP4:
        out = L.pack_mxfp4(Wd)
    elif fmt == synth.NVFP4:
        out = L.pack_nvfp4(Wd)
    else:
        out = L.pack_nf4(Wd, double_quant=(fmt == synth.NF4_DQ))
    del Wd
    return out


def run_layer_gpu(lay, t):
    """Forward + backward of one layer on the GPU into guarded buffers; returns
    host copies of the outputs and of the packed base."""
    E, M, N, K, r = lay.experts, lay.M, lay.N, lay.K, lay.r
    shared = lay.shared_base
    base = _pack_gpu(t["W"], lay.fmt)
    X, A, B, dY = (to_dev(t[k]) for k in ("X", "A", "B", "dY"))
    offs = None if E == 1 else torch.tensor(lay.offsets, dtype=torch.int64, device=DEV)
    W = base.abi()
    if shared:
        nf, nb = (L.lora4_workspace_bytes_multi(w, W, E, M, r) for w in (0, 1))
    else:
        nf, nb = (L.lora4_workspace_bytes(w, W, M, r) for w in (0, 1))
    ws_f, chk_wf = guarded((nf,), torch.uint8)
    ws_b, chk_wb = guarded((nb,), torch.uint8)
    Y, chk_y = guarded((M, N))
    Z, chk_z = guarded((M, r))
    dX, chk_dx = guarded((M, K))
    dA, chk_da = guarded(tuple(A.shape))
    dB, chk_db = guarded(tuple(B.shape))
    if shared:
        L.forward_multi(base, X, A, B, lay.s, adapter_offsets=offs, workspace=ws_f, out={"Y": Y, "Z": Z})
        L.backward_multi(base, X, dY, A, B, lay.s, Z=Z, adapter_offsets=offs, workspace=ws_b,
                         out={"dX": dX, "dA": dA, "dB": dB})
    else:
        L.forward(base, X, A, B, lay.s, group_offsets=offs, workspace=ws_f, out={"Y": Y, "Z": Z})
        L.backward(base, X, dY, A, B, lay.s, Z=Z, group_offsets=offs, workspace=ws_b,
                   out={"dX": dX, "dA": dA, "dB": dB})
    torch.cuda.synchronize()
    for chk, nm in ((chk_wf, "forward workspace"), (chk_wb, "backward workspace"), (chk_y, "Y"), (chk_z, "Z"),
                    (chk_dx, "dX"), (chk_da, "dA"), (chk_db, "dB")):
        chk(nm)
    out = {"Y": to_host(Y), "Z": to_host(Z), "dX": to_host(dX), "dA": to_host(dA), "dB": to_host(dB),
           "codes": base.codes.cpu().numpy(), "scales": base.scales.cpu().numpy(),
           "scales2": None if base.scales2 is None else base.scales2.cpu().numpy()}
    del X, A, B, dY, Y, Z, dX, dA, dB, ws_f, ws_b, base
    torch.cuda.empty_cache()
    return out


def check_packing(lay, got, packs):
    """The whole packed base against the oracle's packing, bit for bit."""
    for q, pk in enumerate(packs):
        assert np.array_equal(got["codes"][q], tile_codes(pk[0], lay.N, lay.K, lay.fmt)), f"codes of group {q}"
        assert np.array_equal(got["scales"][q].view(np.uint8), tile_scales(pk[1], lay.N, lay.K).view(np.uint8)), \
            f"scales of group {q}"
        if lay.fmt == synth.NF4_DQ:
            assert np.array_equal(got["scales2"][q].view(np.uint32), pk[2].view(np.uint32)), f"scales2 of group {q}"


def oracle_layer(lay, t, packs):
    """float64 reference outputs of the whole layer and, for each, the sum of
    absolute terms its bf16 intermediate (Z or dZ) enters."""
    E, M, N, K, r, s = lay.experts, lay.M, lay.N, lay.K, lay.r, lay.s
    shared = lay.shared_base
    ref = {"Y": np.empty((M, N)), "Z": np.empty((M, r)), "dX": np.empty((M, K))}
    inter = {"Y": np.empty((M, N)), "dX": np.empty((M, K))}
    shp_a, shp_b = (r, K) if E == 1 else (E, r, K), (N, r) if E == 1 else (E, N, r)
    ref["dA"], ref["dB"] = np.zeros(shp_a), np.zeros(shp_b)
    inter["dA"], inter["dB"] = np.zeros(shp_a), np.zeros(shp_b)
    offs = [0, M] if E == 1 else lay.offsets
    Wd = oracle_dequant_full(packs[0], lay.fmt) if shared or E == 1 else None
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        if b == a:
            continue
        We = Wd if Wd is not None else oracle_dequant_full(packs[e], lay.fmt)
        Ae = f64(t["A"] if E == 1 else t["A"][e])
        Be = f64(t["B"] if E == 1 else t["B"][e])
        Xe, dYe = f64(t["X"][a:b]), f64(t["dY"][a:b])
        Ze = Xe @ Ae.T
        ref["Z"][a:b] = Ze
        ref["Y"][a:b] = Xe @ We.T + s * (Ze @ Be.T)
        inter["Y"][a:b] = abs(s) * (np.abs(Ze) @ np.abs(Be).T)
        dZe = s * (dYe @ Be)
        ref["dX"][a:b] = dYe @ We + dZe @ Ae
        inter["dX"][a:b] = np.abs(dZe) @ np.abs(Ae)
        ia = slice(None) if E == 1 else e
        ref["dA"][ia] = dZe.T @ Xe
        inter["dA"][ia] = np.abs(dZe).T @ np.abs(Xe)
        ref["dB"][ia] = s * (dYe.T @ Ze)
        inter["dB"][ia] = abs(s) * (np.abs(dYe).T @ np.abs(Ze))
        del Xe, dYe
    return ref, inter


def check_layer_full(lay, case):
    print_case(case, lay.workload, lay.name, lay.M, lay.K, lay.N, lay.r, lay.fmt, lay.experts)
    t = synth.inputs(lay)
    got = run_layer_gpu(lay, t)
    E = lay.experts
    Ws = [t["W"]] if E == 1 or lay.shared_base else [t["W"][e] for e in range(E)]
    packs = [oracle_pack_full(W, lay.fmt) for W in Ws]
    check_packing(lay, got, packs)
    ref, inter = oracle_layer(lay, t, packs)
    report = {}
    for k in ("Y", "Z", "dX", "dA", "dB"):
        compare_full(k, got[k], ref[k], inter.get(k), report)
    print("[parity]", case, {k: "%.2e/%.3f" % (v["rel_frobenius"], v["max_err_over_bound"])
                             for k, v in report.items()}, flush=True)
    write_report(f"{case} {lay.name} M={lay.M} K={lay.K} N={lay.N} r={lay.r} {lay.fmt} E={E}", report)


def _layers(w):
    return [(w, i) for i in range(len(synth.layers(w)))]


@pytest.mark.parametrize("w,i", _layers(1) + _layers(2) + _layers(3) + _layers(4) + _layers(5))
def test_workload_layer(w, i):
    lay = synth.layers(w)[i]
    check_layer_full(lay, synth.WORKLOAD_NAMES[w])


@pytest.mark.parametrize("i", [0, 1, 4, 6])
def test_workload_layer_multilora(i):
    """Layers of the 8B set with 16 rank-16 adapters over the one NF4 base,
    4096 tokens cut into groups of 1 to ~700 rows, as bench.py --workload
    multilora runs them (several adapters inside most 256-row tiles)."""
    check_layer_full(synth.layers(6)[i], "multilora")


@pytest.mark.parametrize("i", [0, 4, 6])
def test_workload_layer_nvfp4(i):
    """Layers of the 8B set (4096 -> 4096, 4096 -> 14336, 14336 -> 4096) with an
    NVFP4 base, as bench.py --fmt nvfp4 runs them."""
    check_layer_full(dataclasses.replace(synth.layers(2)[i], fmt=synth.NVFP4), "llama8b-nvfp4")
