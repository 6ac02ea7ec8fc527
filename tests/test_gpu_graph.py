"""The forward and backward are capturable in a HIP graph: one layer's
forward + backward captured once and replayed three times, with eager work and
synchronizations between the replays, gives the eager results bit for bit
every time (the library clears memory with kernels, never hipMemsetAsync)."""

import numpy as np
import pytest
import torch

import lora_fine_tuning_amd as L
import synth
from gpu_util import DEV, pack_gpu, print_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [synth.NF4, synth.MXFP4])
def test_graph_replays_match_eager(fmt):
    M, K, N, r = 512, 2048, 1536, 16
    print_case("graph", fmt, M, K, N, r)
    lay = synth.small_layer(M, K, N, r, fmt=fmt, index=3)
    t = synth.inputs(lay)
    base = pack_gpu(t["W"], fmt)
    X, dY, A, B = (to_dev(t[k]) for k in ("X", "dY", "A", "B"))
    ws0 = L.workspace_for(0, base, M, r)
    ws1 = L.workspace_for(1, base, M, r)
    eager_f = L.forward(base, X, A, B, lay.s, workspace=ws0)
    eager_b = L.backward(base, X, dY, A, B, lay.s, Z=eager_f["Z"], workspace=ws1)
    torch.cuda.synchronize()

    out = {}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up on the capture stream's kind
        f = L.forward(base, X, A, B, lay.s, workspace=ws0)
        L.backward(base, X, dY, A, B, lay.s, Z=f["Z"], workspace=ws1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out.update(L.forward(base, X, A, B, lay.s, workspace=ws0))
        out.update(L.backward(base, X, dY, A, B, lay.s, Z=out["Z"], workspace=ws1))
    for rep in range(3):
        for v in (out["Y"], out["Z"], out["dX"], out["dA"], out["dB"]):
            v.fill_(0)                                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ref in (("Y", eager_f["Y"]), ("Z", eager_f["Z"]), ("dX", eager_b["dX"]), ("dA", eager_b["dA"]),
                       ("dB", eager_b["dB"])):
            assert torch.equal(out[k], ref), (rep, k)
