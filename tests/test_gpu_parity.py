"""GPU parity of lora4_forward / lora4_backward against the float64 oracle.

Bar: relative Frobenius error <= 5e-3 for Y, Z, dX, dA, dB (the outputs are
bf16; bf16 rounding alone contributes about 1.5e-3). Special cases that the
pages fix are checked exactly: B = 0 gives Y == Y^base and dA == 0; A = 0
gives dB == 0 ("Training LLMs on a Budget", section 2, "Initialization
matters").
"""

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from oracle import lora
from gpu_util import (DEV, TILE_PATHS, TOL, dequant_rows, f64, guarded, pack_gpu, print_case, rel, set_tiles,
                      to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=TILE_PATHS)
def tiles(request, monkeypatch):
    """Runs a test on each tile path of the library (gpu_util.set_tiles)."""
    return set_tiles(monkeypatch, request.param)


def _run(lay, t, s=None, Z_from_forward=True, offsets=None):
    """Forward and backward of one layer; every output and both workspaces sit
    inside guard bands that must come back untouched."""
    s = lay.s if s is None else s
    base = pack_gpu(t["W"], lay.fmt)
    X, A, B, dY = (to_dev(t[k]) for k in ("X", "A", "B", "dY"))
    offs = None if offsets is None else torch.tensor(offsets, dtype=torch.int64, device=DEV)
    M, r = X.shape[0], A.shape[-2]
    checks = []

    def g(name, shape, dtype=torch.bfloat16):
        v, c = guarded(shape, dtype)
        checks.append((name, c))
        return v

    ws0 = g("forward workspace", (L.lora4_workspace_bytes(0, base.abi(), M, r),), torch.uint8)
    ws1 = g("backward workspace", (L.lora4_workspace_bytes(1, base.abi(), M, r),), torch.uint8)
    fo = {"Y": g("Y", (M, base.N)), "Z": g("Z", (M, r)), "Y_base": g("Y_base", (M, base.N)),
          "Y_lora": g("Y_lora", (M, base.N))}
    bo = {"dX": g("dX", (M, base.K)), "dA": g("dA", tuple(A.shape)), "dB": g("dB", tuple(B.shape))}
    fw = L.forward(base, X, A, B, s, group_offsets=offs, want_parts=True, workspace=ws0, out=fo)
    bw = L.backward(base, X, dY, A, B, s, Z=fw["Z"] if Z_from_forward else None, group_offsets=offs,
                    workspace=ws1, out=bo)
    torch.cuda.synchronize()
    for name, c in checks:
        c(name)
    out = {k: to_host(v) for k, v in fw.items()}
    out.update({k: to_host(v) for k, v in bw.items()})
    return out


def _oracle(lay, t, s=None):
    s = lay.s if s is None else s
    Wd = dequant_rows(t["W"], np.arange(lay.N), lay.fmt)
    X, A, B, dY = (f64(t[k]) for k in ("X", "A", "B", "dY"))
    o = lora.forward(X, Wd, A, B, s)
    o.update(lora.backward(X, Wd, A, B, s, dY))
    return o


def _check_all(got, ref, keys=("Y", "Z", "Y_base", "Y_lora", "dX", "dA", "dB")):
    errs = {k: rel(got[k], ref[k]) for k in keys}
    print("[errs]", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= TOL, (k, v)
    return errs


def test_single_linear_workload_parity(tiles):
    lay = synth.layers(1)[0]
    print_case("workload single", lay)
    t = synth.inputs(lay)
    _check_all(_run(lay, t), _oracle(lay, t))


@pytest.mark.parametrize("fmt", [synth.NF4, synth.NF4_DQ, synth.MXFP4, synth.NVFP4])
@pytest.mark.parametrize("M,K,N,r", [(200, 192, 200, 8), (64, 320, 96, 24), (300, 256, 100, 4),
                                     (129, 1024, 264, 64), (17, 512, 136, 128), (1, 64, 8, 1),
                                     (33, 64, 3, 5), (5, 128, 1, 2)])
def test_ragged_shapes(fmt, M, K, N, r, tiles):
    if fmt in (synth.MXFP4, synth.NVFP4):
        K = K - 32 if K % 64 == 0 and K > 64 else K     # exercise K % 64 == 32
    lay = synth.small_layer(M, K, N, r, fmt=fmt, index=(M + K + N + r) % 97)
    print_case("ragged", fmt, M, K, N, r)
    t = synth.inputs(lay)
    _check_all(_run(lay, t, Z_from_forward=(M % 2 == 0)), _oracle(lay, t))


def test_b_zero_is_bitwise_base_and_kills_dA(tiles):
    lay = synth.small_layer(256, 512, 384, 16, index=11)
    t = synth.inputs(lay)
    t["B"] = np.zeros_like(t["B"])
    got = _run(lay, t)
    assert np.array_equal(got["Y"], got["Y_base"])
    assert (got["dA"] & 0x7FFF == 0).all()
    ref = _oracle(lay, t)
    _check_all(got, ref, keys=("Y", "dX", "dB"))


def test_a_zero_kills_dB():
    lay = synth.small_layer(256, 512, 384, 16, index=12)
    t = synth.inputs(lay)
    t["A"] = np.zeros_like(t["A"])
    got = _run(lay, t)
    assert (got["dB"] & 0x7FFF == 0).all()
    assert (got["Z"] & 0x7FFF == 0).all()
    assert np.array_equal(got["Y"], got["Y_base"])


def test_zero_base_isolates_the_lora_path(tiles):
    # deq(W) = 0: Y = Y^LoRA and dX = dZ A, checked at full relative precision
    lay = synth.small_layer(256, 512, 384, 32, index=13)
    t = synth.inputs(lay)
    t["W"] = np.zeros_like(t["W"])
    got = _run(lay, t)
    ref = _oracle(lay, t)
    assert (got["Y_base"] & 0x7FFF == 0).all()
    _check_all(got, ref, keys=("Y", "Y_lora", "dX", "dA", "dB"))


def test_grouped_small_with_empty_group(tiles):
    K, N, r, E = 256, 96, 16, 5
    offs = [0, 70, 70, 200, 201, 333]
    for fmt in (synth.MXFP4, synth.NF4, synth.NF4_DQ, synth.NVFP4):
        lay = synth.small_layer(offs[-1], K, N, r, fmt=fmt, index=21, experts=E, offsets=offs)
        print_case("grouped", fmt, offs)
        t = synth.inputs(lay)
        got = _run(lay, t, offsets=offs)
        Ws = [dequant_rows(t["W"][e], np.arange(N), fmt) for e in range(E)]
        X, dY = f64(t["X"]), f64(t["dY"])
        As = [f64(t["A"][e]) for e in range(E)]
        Bs = [f64(t["B"][e]) for e in range(E)]
        fo = lora.grouped_forward(X, Ws, As, Bs, lay.s, offs)
        bo = lora.grouped_backward(X, Ws, As, Bs, lay.s, dY, offs)
        assert rel(got["Y"], fo["Y"]) <= TOL
        assert rel(got["Z"], fo["Z"]) <= TOL
        assert rel(got["dX"], bo["dX"]) <= TOL
        for e in range(E):
            if offs[e + 1] == offs[e]:
                assert (got["dA"][e] & 0x7FFF == 0).all() and (got["dB"][e] & 0x7FFF == 0).all()
            else:
                assert rel(got["dA"][e], bo["dA"][e]) <= TOL, e
                assert rel(got["dB"][e], bo["dB"][e]) <= TOL, e


def test_zero_tokens():
    lay = synth.small_layer(4, 128, 64, 8, index=31)
    t = synth.inputs(lay)
    base = pack_gpu(t["W"], lay.fmt)
    X = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    A, B = to_dev(t["A"]), to_dev(t["B"])
    fw = L.forward(base, X, A, B, 2.0)
    assert fw["Y"].shape == (0, 64)
    bw = L.backward(base, X, dY, A, B, 2.0, Z=None)
    torch.cuda.synchronize()
    assert (to_host(bw["dA"]) == 0).all() and (to_host(bw["dB"]) == 0).all()


def test_deterministic(tiles):
    lay = synth.small_layer(512, 1024, 768, 16, index=41)
    t = synth.inputs(lay)
    a = _run(lay, t)
    b = _run(lay, t)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_validation_errors_launch_nothing():
    lay = synth.small_layer(64, 128, 64, 8, index=51)
    t = synth.inputs(lay)
    base = pack_gpu(t["W"], lay.fmt)
    X, A, B = to_dev(t["X"]), to_dev(t["A"]), to_dev(t["B"])
    Y = torch.full((64, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    # the library's own checks (raw ABI): a short workspace, a K off the block grid
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    assert L.lora4_forward(base.abi(), X.data_ptr(), 64, A.data_ptr(), B.data_ptr(), 8, 2.0, None, Y.data_ptr(),
                           None, None, None, small.data_ptr(), 16, st) == -5
    bad = L.PackedBase(base.fmt, base.N, 96, 1, base.codes, base.scales)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    assert L.lora4_forward(bad.abi(), X.data_ptr(), 64, A.data_ptr(), B.data_ptr(), 8, 2.0, None, Y.data_ptr(),
                           None, None, None, ws.data_ptr(), 1 << 20, st) == -2
    torch.cuda.synchronize()
    assert (Y.float() == 7.0).all()            # nothing was launched
    # the binding refuses both before calling the library
    with pytest.raises(ValueError):
        L.forward(base, X, A, B, 2.0, workspace=small)
    with pytest.raises(ValueError):
        L.forward(bad, X, A, B, 2.0, workspace=ws)


def test_large_tile_shape_selected_automatically(monkeypatch):
    # 1024 x 4096 output: 4 x 16 = 64 tiles of 256 -> small path; 4096 x 4096 -> large path.
    monkeypatch.delenv("LORA4_BIG", raising=False)
    lay = synth.small_layer(4096, 1024, 4096, 16, index=61)
    t = synth.inputs(lay)
    got = _run(lay, t)
    rows = np.random.default_rng(0).choice(lay.M, 96, replace=False)
    Wd = dequant_rows(t["W"], np.arange(lay.N), lay.fmt)
    X, A, B, dY = (f64(t[k]) for k in ("X", "A", "B", "dY"))
    ref = lora.forward(X[rows], Wd, A, B, lay.s)
    assert rel(got["Y"][rows], ref["Y"]) <= TOL
    bref = lora.backward(X, Wd, A, B, lay.s, dY)
    assert rel(got["dX"][rows], bref["dX"][rows]) <= TOL
    assert rel(got["dA"], bref["dA"]) <= TOL and rel(got["dB"], bref["dB"]) <= TOL


@pytest.mark.parametrize("fmt", [synth.NF4, synth.NF4_DQ, synth.MXFP4, synth.NVFP4])
@pytest.mark.parametrize("M,K,N,r", [(512, 4096, 256, 16),     # 2 tiles: 8-way split of 64 steps
                                     (700, 2048, 1000, 16),    # ragged rows, 12 tiles: 4-way split
                                     (300, 2048, 258, 8)])     # N % 4 != 0, ragged last columns
def test_forward_split_reduction(fmt, M, K, N, r, monkeypatch):
    """Forced onto the register-direct forward kernel, few-tile outputs split
    the reduction (fp32 partials + reduction); the rank-r tail is added once."""
    monkeypatch.setenv("LORA4_BIG", "1")
    if fmt in (synth.MXFP4, synth.NVFP4) and K % 64 == 0:
        K -= 32
    lay = synth.small_layer(M, K, N, r, fmt=fmt, index=(M + N) % 89)
    print_case("split", fmt, M, K, N, r)
    t = synth.inputs(lay)
    _check_all(_run(lay, t), _oracle(lay, t), keys=("Y", "Y_base", "Y_lora", "Z"))


def test_forward_split_grouped(monkeypatch):
    """Split reduction with grouped rows (one group empty)."""
    monkeypatch.setenv("LORA4_BIG", "1")
    K, N, r, E = 2048, 128, 16, 3
    offs = [0, 300, 300, 420]
    lay = synth.small_layer(offs[-1], K, N, r, fmt=synth.NF4, index=33, experts=E, offsets=offs)
    print_case("split grouped", offs)
    t = synth.inputs(lay)
    got = _run(lay, t, offsets=offs)
    Ws = [dequant_rows(t["W"][e], np.arange(N), synth.NF4) for e in range(E)]
    fo = lora.grouped_forward(f64(t["X"]), Ws, [f64(a) for a in t["A"]], [f64(b) for b in t["B"]], lay.s, offs)
    assert rel(got["Y"], fo["Y"]) <= TOL


@pytest.mark.parametrize("grouped", [False, True])
def test_small_grid_splits_the_reduction(grouped, monkeypatch):
    """A 128 x 128 grid that fills less than half the GPU (256 tokens x 1024:
    16 workgroups, 40 with three groups) splits the base GEMMs' reduction into
    ranges of fp32 partials that one launch sums in range order (reduce_y,
    reduce_dx), the rank-r term added in the last range. Checked against the
    oracle, with an empty group, and bitwise against a second identical call."""
    monkeypatch.setenv("LORA4_BIG", "0")
    M, K, N, r = 256, 1024, 1024, 16
    offs = [0, 100, 100, 256] if grouped else None
    lay = synth.small_layer(M, K, N, r, fmt=synth.NF4, index=61, experts=3 if grouped else 1, offsets=offs)
    print_case("small grid split", offs)
    t = synth.inputs(lay)
    L.timing_enable(True)
    try:
        L.timing_collect()
        got = _run(lay, t, offsets=offs)
        names = set(L.timing_collect())
    finally:
        L.timing_enable(False)
    assert "reduce_y" in names and "reduce_dx" in names, names
    again = _run(lay, t, offsets=offs)
    for k in ("Y", "Z", "dX", "dA", "dB"):
        assert np.array_equal(got[k], again[k]), k
    if not grouped:
        _check_all(got, _oracle(lay, t))
        return
    Ws = [dequant_rows(t["W"][e], np.arange(N), synth.NF4) for e in range(3)]
    As = [f64(a) for a in t["A"]]
    Bs = [f64(b) for b in t["B"]]
    fo = lora.grouped_forward(f64(t["X"]), Ws, As, Bs, lay.s, offs)
    bo = lora.grouped_backward(f64(t["X"]), Ws, As, Bs, lay.s, f64(t["dY"]), offs)
    for k in ("Y", "Z"):
        assert rel(got[k], fo[k]) <= TOL, k
    assert rel(got["dX"], bo["dX"]) <= TOL
    for e in (0, 2):
        assert rel(got["dA"][e], bo["dA"][e]) <= TOL and rel(got["dB"][e], bo["dB"][e]) <= TOL, e
    assert not (got["dA"][1] & 0x7FFF).any() and not (got["dB"][1] & 0x7FFF).any()   # (±0)


def test_forward_two_rounds_of_tiles(monkeypatch):
    """320 output tiles (more than one per CU): the XCD-aware block order over
    a partial second round. Checked on sampled columns of the first 96 column
    tiles and of the last 64 of the second row tile, all rows."""
    monkeypatch.setenv("LORA4_BIG", "1")
    M, K, N, r = 512, 1024, 160 * 256, 16
    lay = synth.small_layer(M, K, N, r, fmt=synth.NF4, index=7)
    print_case("two rounds", M, K, N, r)
    t = synth.inputs(lay)
    base = pack_gpu(t["W"], lay.fmt)
    X, A, B = (to_dev(t[k]) for k in ("X", "A", "B"))
    fw = L.forward(base, X, A, B, lay.s)
    torch.cuda.synchronize()
    Y = to_host(fw["Y"])
    rng = np.random.default_rng(5)
    cols = np.sort(np.concatenate([rng.choice(96 * 256, 48, replace=False),            # whole tiles only
                                   96 * 256 + rng.choice(64 * 256, 48, replace=False)]))
    Wn = dequant_rows(t["W"], cols, lay.fmt)
    Xf, Af, Bf = f64(t["X"]), f64(t["A"]), f64(t["B"])
    ref = Xf @ Wn.T + lay.s * ((Xf @ Af.T) @ Bf[cols].T)
    assert rel(Y[:, cols], ref) <= TOL


@pytest.mark.parametrize("r", [16, 12, 20])
@pytest.mark.parametrize("grouped", [False, True])
def test_tails_add_rank_r_partials(r, grouped, monkeypatch):
    """With the rank-r reductions split into ranges, the forward and dgrad
    GEMM tails add the fp32 range partials themselves (no separate reduction
    launch) and store Z / dZ for the passes that follow: r % 4 != 0 takes the
    element loads, r % 8 != 0 the element stores. (2100 rows: passes over
    fewer than 4 MiB of activations are not split.)"""
    monkeypatch.setenv("LORA4_BIG", "1")
    K, N = 1024, 1024
    offs = [0, 930, 930, 2100] if grouped else None
    M = 2100
    lay = synth.small_layer(M, K, N, r, fmt=synth.NF4, index=40 + r, experts=3 if grouped else 1, offsets=offs)
    print_case("tail partials", r, offs)
    t = synth.inputs(lay)
    L.timing_enable(True)
    try:
        L.timing_collect()
        got = _run(lay, t, offsets=offs)
        names = set(L.timing_collect())
    finally:
        L.timing_enable(False)
    assert "reduce_z" not in names and "reduce_dz" not in names, names
    assert "rows_skinny_z" in names and "rows_skinny_dz" in names, names
    if not grouped:
        _check_all(got, _oracle(lay, t))
    else:
        Ws = [dequant_rows(t["W"][e], np.arange(N), synth.NF4) for e in range(3)]
        As = [f64(a) for a in t["A"]]
        Bs = [f64(b) for b in t["B"]]
        fo = lora.grouped_forward(f64(t["X"]), Ws, As, Bs, lay.s, offs)
        bo = lora.grouped_backward(f64(t["X"]), Ws, As, Bs, lay.s, f64(t["dY"]), offs)
        for k in ("Y", "Z"):
            assert rel(got[k], fo[k]) <= TOL, k
        assert rel(got["dX"], bo["dX"]) <= TOL
        for e in (0, 2):
            assert rel(got["dA"][e], bo["dA"][e]) <= TOL and rel(got["dB"][e], bo["dB"][e]) <= TOL, e
    # no Z output requested: the tail still sums the partials for Y
    base = pack_gpu(t["W"], lay.fmt)
    o = None if offs is None else torch.tensor(offs, dtype=torch.int64, device=DEV)
    fw = L.forward(base, to_dev(t["X"]), to_dev(t["A"]), to_dev(t["B"]), lay.s, group_offsets=o, want_z=False)
    assert np.array_equal(to_host(fw["Y"]), got["Y"])


@pytest.mark.parametrize("fmt", [synth.NF4, synth.MXFP4])
@pytest.mark.parametrize("M,K,N,r", [(300, 512, 384, 256), (130, 256, 200, 200), (77, 192, 136, 136),
                                     (64, 128, 96, 130)])
def test_ranks_above_128(fmt, M, K, N, r, tiles):
    """Ranks above 128, up to the largest the library accepts (256): the
    rank-r passes then run more than one 128-wide block of rank columns (the
    grid's second dimension), the dA/dB pass more than one rank tile, and the
    GEMM heads and tails more than two 64-deep rank steps. r = 130 is not a
    multiple of 8 (the dZ pass takes the register kernel)."""
    lay = synth.small_layer(M, K, N, r, fmt=fmt, index=(M + r) % 89)
    print_case("rank above 128", fmt, M, K, N, r)
    t = synth.inputs(lay)
    _check_all(_run(lay, t, Z_from_forward=(M % 2 == 0)), _oracle(lay, t))


@pytest.mark.parametrize("fmt", [synth.NF4, synth.MXFP4, synth.NF4_DQ, synth.NVFP4])
def test_many_small_experts(fmt, tiles):
    """200 experts, each with its own base and adapter, of 0 to 9 rows (79 of
    them empty), 550 rows in all: every row tile is an expert's short last
    tile, and the grids hold more row slots for the experts than rows. Every
    expert's dA and dB against the oracle; the empty ones zero."""
    E, K, N, r = 200, 128, 96, 8
    rng = np.random.default_rng(2024)
    counts = rng.integers(0, 10, size=E)
    counts[rng.choice(E, E // 3, replace=False)] = 0
    offs = [0] + np.cumsum(counts).tolist()
    lay = synth.small_layer(offs[-1], K, N, r, fmt=fmt, index=29, experts=E, offsets=offs)
    print_case("many small experts", fmt, E, offs[-1])
    t = synth.inputs(lay)
    got = _run(lay, t, offsets=offs)
    Ws = [dequant_rows(t["W"][e], np.arange(N), fmt) for e in range(E)]
    As = [f64(a) for a in t["A"]]
    Bs = [f64(b) for b in t["B"]]
    fo = lora.grouped_forward(f64(t["X"]), Ws, As, Bs, lay.s, offs)
    bo = lora.grouped_backward(f64(t["X"]), Ws, As, Bs, lay.s, f64(t["dY"]), offs)
    for k in ("Y", "Z"):
        assert rel(got[k], fo[k]) <= TOL, k
    assert rel(got["dX"], bo["dX"]) <= TOL
    for e in range(E):
        if counts[e]:
            assert rel(got["dA"][e], bo["dA"][e]) <= TOL and rel(got["dB"][e], bo["dB"][e]) <= TOL, e
        else:
            assert not (got["dA"][e] & 0x7FFF).any() and not (got["dB"][e] & 0x7FFF).any(), e
