#!/usr/bin/env python3
"""Throughput of the unmerged-LoRA linear over a frozen 4-bit base on one MI355X.

A step is one forward and one backward pass of every layer of the workload
(forward through the layers in order, backward in reverse order, as in
training), with all inputs already resident in HBM and the base packed once
beforehand. The default workload is the Llama-3-8B-shaped layer set on 4096
tokens with an NF4 base (64-element blocks) and rank-16 adapters (alpha 32):
q and o 4096->4096, k and v 4096->1024, gate and up 4096->14336, down
14336->4096.

Prints one JSON line: fwd+bwd TFLOP/s (algorithmic flops 4MNK + 6Mr(N+K) per
layer), the fraction of the bf16 dense MFMA peak, the roofline of the dominant
kernel (timed live with HIP events on the launch stream) and the CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0         # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
WORKLOADS = {"single": 1, "llama8b": 2, "llama70b": 3, "moe": 4, "longctx": 5, "multilora": 6}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens per layer in the CPU oracle sample (capped at the layer's tokens)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="passes of the CPU oracle over its sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (counter calibration) and exit")
    ap.add_argument("--peak-probe", action="store_true",
                    help="only measure the roofline denominators (bf16 MFMA rate, HBM read and copy bandwidth) "
                         "and exit")
    ap.add_argument("--fmt", choices=["nf4", "nf4_dq", "mxfp4", "nvfp4"], default=None,
                    help="store every base of the workload in this format instead of its own")
    ap.add_argument("--mx", action="store_true",
                    help="forward through the MX-native path (MXFP8 activations x MXFP4 base on the scaled "
                         "MFMA); plain MXFP4 layer sets only")
    ap.add_argument("--loftq", action="store_true",
                    help="time the LoftQ initialisation (5 iterations, NF4) of the workload's bases instead of a step")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (the same kernels, fewer launch gaps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--blas-context", action="store_true",
                    help="also time torch's bf16 GEMMs (hipBLASLt) on already-dequantized W of the same shapes "
                         "(context only)")
    return ap.parse_args()


class Layer:
    """Device buffers of one layer (inputs, outputs, packed base)."""

    def __init__(self, spec, L, torch, synth, mx=False):
        self.spec = spec
        self.mx = mx
        t = synth.inputs(spec)
        dev = "cuda:0"

        def d(a):
            return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

        self.X, self.A, self.B, self.dY = d(t["X"]), d(t["A"]), d(t["B"]), d(t["dY"])
        W = d(t["W"])
        if spec.fmt == synth.MXFP4:
            self.base = L.pack_mxfp4(W)
        elif spec.fmt == synth.NVFP4:
            self.base = L.pack_nvfp4(W)
        else:
            self.base = L.pack_nf4(W, double_quant=(spec.fmt == synth.NF4_DQ))
        del W
        M, N, K, r, E = spec.M, spec.N, spec.K, spec.r, spec.experts
        self.offs = None
        if E > 1:
            self.offs = torch.tensor(spec.offsets, dtype=torch.int64, device=dev)
        self.Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.Z = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        self.dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        self.dA = torch.empty_like(self.A)
        self.dB = torch.empty_like(self.B)
        self.W = self.base.abi()
        if spec.shared_base:
            self.ws_bytes = max(L.lora4_workspace_bytes_multi(0, self.W, E, M, r),
                                L.lora4_workspace_bytes_multi(1, self.W, E, M, r))
        else:
            self.ws_bytes = max(L.lora4_workspace_bytes(0, self.W, M, r), L.lora4_workspace_bytes(1, self.W, M, r))
        if mx:
            self.ws_bytes = max(self.ws_bytes, L.lora4_workspace_bytes_mx(self.W, M, r))

    def fwd(self, L, ws, stream):
        s = self.spec
        if self.mx:
            st = L.lora4_forward_mx(self.W, self.X.data_ptr(), s.M, self.A.data_ptr(), self.B.data_ptr(), s.r, s.s,
                                    self.Y.data_ptr(), self.Z.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        elif s.shared_base:
            st = L.lora4_forward_multi(self.W, s.experts, self.X.data_ptr(), s.M, self.A.data_ptr(),
                                       self.B.data_ptr(), s.r, s.s, self.offs.data_ptr(), self.Y.data_ptr(),
                                       self.Z.data_ptr(), None, None, ws.data_ptr(), ws.numel(), stream)
        else:
            st = L.lora4_forward(self.W, self.X.data_ptr(), s.M, self.A.data_ptr(), self.B.data_ptr(), s.r, s.s,
                                 None if self.offs is None else self.offs.data_ptr(), self.Y.data_ptr(),
                                 self.Z.data_ptr(), None, None, ws.data_ptr(), ws.numel(), stream)
        if st:
            raise RuntimeError(f"lora4_forward failed: {L.status_string(st)}")

    def bwd(self, L, ws, stream):
        s = self.spec
        if s.shared_base:
            st = L.lora4_backward_multi(self.W, s.experts, self.X.data_ptr(), self.dY.data_ptr(), s.M,
                                        self.A.data_ptr(), self.B.data_ptr(), s.r, s.s, self.offs.data_ptr(),
                                        self.Z.data_ptr(), self.dX.data_ptr(), self.dA.data_ptr(),
                                        self.dB.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        else:
            st = L.lora4_backward(self.W, self.X.data_ptr(), self.dY.data_ptr(), s.M, self.A.data_ptr(),
                                  self.B.data_ptr(), s.r, s.s, None if self.offs is None else self.offs.data_ptr(),
                                  self.Z.data_ptr(), self.dX.data_ptr(), self.dA.data_ptr(), self.dB.data_ptr(),
                                  ws.data_ptr(), ws.numel(), stream)
        if st:
            raise RuntimeError(f"lora4_backward failed: {L.status_string(st)}")


def kernel_flops(name, spec):
    """Algorithmic flops of one launch of the named kernel for this layer."""
    M, N, K, r = spec.M, spec.N, spec.K, spec.r
    return {
        "gemm_nt_base": 2 * M * N * K + 2 * M * N * r,     # X deq(W)^T + (sZ) B^T
        "gemm_mx_base": 2 * M * N * K + 2 * M * N * r,     # mxfp8(X) W4^T + (sZ) B^T
        "gemm_nn_dgrad": 2 * M * N * K + 2 * M * K * r,    # dY deq(W) + dZ A
        "rows_skinny_z": 2 * M * K * r,                     # Z = X A^T
        "rows_skinny_dz": 2 * M * N * r,                    # dZ = s dY B
        "gemm_tn_dA_dB": 2 * M * r * K + 2 * M * r * N,   # dZ^T X and Z^T dY
    }.get(name, 0)


BITS_PER_WEIGHT = {"nf4": 4.5, "nf4_dq": 4.127, "mxfp4": 4.25, "nvfp4": 4.5}   # codes + scales


def kernel_bytes(name, spec):
    """Algorithmic HBM bytes of one launch of the named kernel for this layer:
    the rank-r passes' activation reads and small operands; the packed base
    (codes + scales) for the two dequant-GEMMs."""
    M, N, K, r, E = spec.M, spec.N, spec.K, spec.r, spec.experts
    wp = (1 if spec.shared_base else E) * N * K * BITS_PER_WEIGHT[spec.fmt] / 8
    return {
        "rows_skinny_z": 2 * M * K + 2 * E * r * K + 2 * M * r,       # X, A -> Z
        "rows_skinny_dz": 2 * M * N + 2 * E * N * r + 2 * M * r,      # dY, B -> dZ
        "gemm_tn_dA_dB": 2 * M * (K + N) + 4 * M * r,                 # X, dY, dZ, Z
        "gemm_nt_base": wp,
        "gemm_nn_dgrad": wp,
        "gemm_mx_base": wp,
        "quant_mxfp8": 2 * M * K + M * K + M * K // 32,                # X -> E4M3 codes + E8M0
    }.get(name, 0)


def hbm_summary(specs, kernels, steps):
    """Achieved HBM rates (GB/s, against the 8 TB/s peak): the packed base
    (codes + scales) over the time of each base GEMM, and the algorithmic bytes
    of the rank-r passes over theirs; for grouped layers also the packed bytes
    of one expert and its rows."""
    out = {"peak_gbps": PEAK_HBM_GBS}
    for name, v in kernels.items():
        if "algorithmic_gbps" in v:
            out[name + "_gbps"] = v["algorithmic_gbps"]
    s0 = specs[0]
    if s0.experts > 1 and not s0.shared_base:
        counts = [b - a for a, b in zip(s0.offsets[:-1], s0.offsets[1:])]
        per = [round(s.N * s.K * BITS_PER_WEIGHT[s.fmt] / 8) for s in specs]
        out["per_expert"] = {"experts": s0.experts, "rows_min": min(counts), "rows_avg": sum(counts) / len(counts),
                             "rows_max": max(counts), "packed_bytes_per_expert": per}
        for name in ("gemm_nt_base", "gemm_nn_dgrad"):
            if name in kernels:
                t_exp = kernels[name]["total_ms_per_step"] * 1e-3 / (len(specs) * s0.experts)
                out["per_expert"][name + "_us"] = round(t_exp * 1e6, 3)
                out["per_expert"][name + "_packed_gbps"] = round(sum(per) / len(per) / t_exp / 1e9, 1)
    return out


def csrc_digest():
    """sha256 over the HIP sources of the library (any kernel change alters it)."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lora_fine_tuning_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<workload>_<kernel>_traffic.md), or None when there is none or it
    was taken on other kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"{workload}_{kernel}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic:"):
                rec = dict(kv.split("=", 1) for kv in line.split()[1:])
    if rec.get("csrc_sha256") != csrc_digest():
        return None
    return {"bytes_per_launch": float(rec["bytes_per_launch"]), "fetch_bytes": float(rec["fetch_bytes"]),
            "write_bytes": float(rec["write_bytes"])}


def copy_probe(mib):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters: each launch reads and writes mib MiB."""
    import torch
    n = mib * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[copy] 3 launches of {mib} MiB read + {mib} MiB written")


def peak_probe():
    """Measured denominators: the rate of back-to-back v_mfma_f32_32x32x16_bf16
    on every SIMD (libpeakprobe), the HBM read bandwidth of a 4 GiB buffer read
    once with 16-byte loads, and a torch device copy of 2 GiB. Best of 5 runs
    each; one JSON line."""
    import ctypes
    import torch
    from lora_fine_tuning_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        B.build()
    P = ctypes.CDLL(B.PROBE_LIB)
    P.peak_probe_mfma_flops.restype = ctypes.c_double
    P.peak_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    P.peak_probe_mfma.restype = ctypes.c_float
    P.peak_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.peak_probe_read.restype = ctypes.c_float
    P.peak_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    blocks, iters = 2048, 2048
    out = torch.empty((blocks * 256,), dtype=torch.float32, device="cuda:0")
    P.peak_probe_mfma(blocks, 64, out.data_ptr(), st)          # warm-up
    ms = [P.peak_probe_mfma(blocks, iters, out.data_ptr(), st) for _ in range(5)]
    if min(ms) <= 0:
        raise RuntimeError("peak_probe_mfma failed")
    mfma = P.peak_probe_mfma_flops(blocks, iters) / (min(ms) * 1e-3) / 1e12
    log(f"[probe] bf16 MFMA {mfma:.1f} TFLOP/s (runs {', '.join(f'{m:.3f}' for m in ms)} ms)")
    nbytes = 4 << 30
    buf = torch.ones((nbytes // 4,), dtype=torch.float32, device="cuda:0")
    rblocks = 256 * 32
    rout = torch.empty((rblocks * 256,), dtype=torch.float32, device="cuda:0")
    P.peak_probe_read(buf.data_ptr(), nbytes, rblocks, rout.data_ptr(), st)
    rms = [P.peak_probe_read(buf.data_ptr(), nbytes, rblocks, rout.data_ptr(), st) for _ in range(5)]
    read = nbytes / (min(rms) * 1e-3) / 1e9
    log(f"[probe] HBM read {read:.0f} GB/s")
    half = buf[: nbytes // 8]
    dst = torch.empty_like(half)
    dst.copy_(half)
    torch.cuda.synchronize()
    cms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(half)
        e1.record()
        torch.cuda.synchronize()
        cms.append(e0.elapsed_time(e1))
    copy = 2 * half.numel() * 4 / (min(cms) * 1e-3) / 1e9
    log(f"[probe] device copy {copy:.0f} GB/s (read + write)")
    print(json.dumps({"metric": "measured roofline denominators", "bf16_mfma_tflops": round(mfma, 1),
                      "bf16_mfma_frac_of_spec": round(mfma / PEAK_BF16_TFLOPS, 4),
                      "hbm_read_gbps": round(read, 1), "hbm_copy_gbps": round(copy, 1),
                      "hbm_read_frac_of_spec": round(read / PEAK_HBM_GBS, 4),
                      "mfma_probe": {"blocks": blocks, "threads": 256, "iters": iters, "chains": 8,
                                     "ms": [round(m, 4) for m in ms]},
                      "read_probe": {"bytes": nbytes, "blocks": rblocks, "ms": [round(m, 4) for m in rms]}}),
          flush=True)


def blas_context(specs, torch, steps):
    """Context only: torch's bf16 GEMMs (hipBLASLt) for the two base products
    of every layer, X W^T and dY W, on a bf16 W of the same shape (as if it
    had been dequantized beforehand; the rank-r terms are left out)."""
    dev = "cuda:0"
    mats = []
    for s in specs:
        if s.experts > 1:
            continue
        g = torch.Generator(device=dev).manual_seed(1)
        X = torch.randn((s.M, s.K), device=dev, generator=g).bfloat16()
        dY = torch.randn((s.M, s.N), device=dev, generator=g).bfloat16()
        W = (torch.randn((s.N, s.K), device=dev, generator=g) * 0.02).bfloat16()
        mats.append((X, dY, W, W.t().contiguous()))

    def run():
        for X, dY, W, Wt in mats:
            torch.mm(X, Wt)
            torch.mm(dY, W)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = sum(4 * s.M * s.N * s.K for s in specs if s.experts == 1)
    return {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "what": "torch.mm bf16 (hipBLASLt), X W^T and dY W per layer, W already bf16"}


def cpu_baseline(specs, tokens, reps):
    """The oracle (never tuned) on a bounded sample: every layer of the workload,
    the first `tokens` rows. Oracle packing is done first, untimed; the timed
    part is what a step computes: dequant + forward + backward per layer."""
    import numpy as np
    import synth
    from oracle import lora, mxfp4, nf4, nvfp4

    prepared = []
    for spec in specs:
        t = synth.inputs(spec)
        E = spec.experts
        Ws = t["W"] if E > 1 and not spec.shared_base else t["W"][None]
        packs = []
        for e in range(len(Ws)):
            if spec.fmt == synth.MXFP4:
                packs.append(mxfp4.quantize(Ws[e]))
            elif spec.fmt == synth.NVFP4:
                packs.append(nvfp4.quantize(Ws[e]))
            else:
                c, sc = nf4.quantize(Ws[e])
                packs.append((c, *nf4.double_quantize(sc)) if spec.fmt == synth.NF4_DQ else (c, sc))
        m = min(tokens, spec.M)
        prepared.append((spec, packs, t["X"][:m], t["dY"][:m], t["A"], t["B"], m))
    flops = 0
    done = 0
    t0 = time.perf_counter()
    for _ in range(reps):
        if done and time.perf_counter() - t0 > 15.0:
            break                  # enough CPU time for a stable rate (large workloads)
        done += 1
        for spec, packs, X, dY, A, B, m in prepared:
            for e, pk in enumerate(packs):
                if spec.fmt == synth.MXFP4:
                    Wd = lora.as_f64(mxfp4.dequantize(*pk))
                elif spec.fmt == synth.NVFP4:
                    Wd = lora.as_f64(nvfp4.dequantize(*pk))
                elif spec.fmt == synth.NF4_DQ:
                    Wd = lora.as_f64(nf4.dequantize_dq(*pk))
                else:
                    Wd = lora.as_f64(nf4.dequantize(*pk))
                Ae = lora.as_f64(A if spec.experts == 1 else A[e])
                Be = lora.as_f64(B if spec.experts == 1 else B[e])
                Xf, dYf = lora.as_f64(X), lora.as_f64(dY)
                o = lora.forward(Xf, Wd, Ae, Be, spec.s)
                lora.backward(Xf, Wd, Ae, Be, spec.s, dYf, Z=o["Z"])
                flops += 4 * m * spec.N * spec.K + 6 * m * spec.r * (spec.N + spec.K)
                if spec.experts > 1:
                    break          # sample: the first expert of a grouped layer
    dt = time.perf_counter() - t0
    blas = blas_info()
    threads = blas.pop("threads", None) or len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": dt, "precision": "float64 (the oracle's own arithmetic)", "cpu": cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0)), "blas": blas,
            "sample": f"{done} passes over every layer of the workload at its first {tokens} tokens (capped at "
                      f"the layer's tokens; first expert of grouped layers): oracle dequant + forward + "
                      f"backward, float64 numpy"}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_info():
    """numpy's BLAS (name, version, threads in use) as threadpoolctl and numpy
    report it."""
    out = {}
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                out = {"library": d.get("internal_api"), "version": d.get("version"),
                       "threads": d.get("num_threads"), "arch": d.get("architecture")}
                break
    except Exception:
        pass
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        out.setdefault("library", b.get("name"))
        out["numpy_blas"] = f"{b.get('name')} {b.get('version')}"
    except Exception:
        pass
    return out


def loftq_bench(args, specs, L, torch, synth):
    """Wall time of lora4_loftq_init (5 iterations, NF4, the layer's rank and
    scale) over the workload's bases, with the library's per-kernel times."""
    Ws = []
    for s in specs:
        t = synth.inputs(s)
        W = t["W"] if s.experts == 1 else t["W"][0]
        Ws.append((s, torch.from_numpy(W.view("int16")).view(torch.bfloat16).to("cuda:0")))
    for s, W in Ws[:1]:
        L.loftq_init(W, s.r, iters=1, s=s.s)          # warm-up (first launches)
    torch.cuda.synchronize()
    L.timing_enable(True)
    L.timing_collect()
    t0 = time.perf_counter()
    for s, W in Ws:
        L.loftq_init(W, s.r, iters=5, s=s.s)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3
    kt = L.timing_collect()
    L.timing_enable(False)
    kernels = {k: {"launches": n, "total_ms": round(tot, 3)} for k, (n, tot) in kt.items()}
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"]):
        log(f"[loftq]   {k:18s} {v['launches']:6d} launches  {v['total_ms']:9.2f} ms")
    log(f"[loftq] {len(Ws)} bases, 5 iterations each: {ms:.1f} ms")
    print(json.dumps({"metric": "LoftQ initialisation time of the workload's bases (5 iterations, NF4)",
                      "value": round(ms, 2), "unit": "ms", "higher_is_better": False, "n_gpus": 1,
                      "config": {"workload": args.workload, "layers_KxN": [[s.K, s.N] for s in specs],
                                 "rank": specs[0].r},
                      "kernels": kernels}), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.peak_probe:
        peak_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import lora_fine_tuning_amd as L
    import synth
    if not os.path.exists(L.LIB_PATH):
        from lora_fine_tuning_amd import build as B
        B.build()
    L.lib()

    wl = WORKLOADS[args.workload]
    specs = synth.layers(wl)
    if args.fmt:
        import dataclasses
        specs = [dataclasses.replace(s, fmt=args.fmt) for s in specs]
    if args.mx and any(s.fmt != synth.MXFP4 or s.experts != 1 for s in specs):
        print("--mx needs a workload of plain MXFP4 layers (llama70b)", file=sys.stderr)
        sys.exit(2)
    if args.loftq:
        loftq_bench(args, specs, L, torch, synth)
        return
    log(f"[bench] workload {args.workload}: {len(specs)} layers, generating inputs")
    layers = [Layer(s, L, torch, synth, mx=args.mx) for s in specs]
    ws = torch.empty((max(l.ws_bytes for l in layers),), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    flops = sum(s.flops() for s in specs)

    def step_eager():
        st = torch.cuda.current_stream().cuda_stream   # the capturing stream inside a graph capture
        for l in layers:
            l.fwd(L, ws, st)
        for l in reversed(layers):
            l.bwd(L, ws, st)

    step = step_eager

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record()
        for _ in range(k):
            step()
        e1.record()
        torch.cuda.synchronize()
        w1 = time.perf_counter()
        return max(e0.elapsed_time(e1), (w1 - w0) * 1e3) / k

    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_eager()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_eager()
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        log("[bench] one step captured in a HIP graph; timing its replays")
    log(f"[bench] timing {args.steps} steps")
    ms = timed(args.steps)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {ms:.3f} ms/step, {value:.1f} TFLOP/s")

    # the two passes on their own (same loop, forward-only / backward-only steps)
    def timed_pass(fn, k):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(k):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    fwd_flops = sum(2 * s.M * s.N * s.K + 2 * s.M * s.r * (s.N + s.K) for s in specs)
    ms_f = timed_pass(lambda: [l.fwd(L, ws, stream) for l in layers], args.steps)
    ms_b = timed_pass(lambda: [l.bwd(L, ws, stream) for l in reversed(layers)], args.steps)
    passes = {"fwd_ms": round(ms_f, 4), "fwd_tflops": round(fwd_flops / (ms_f * 1e-3) / 1e12, 2),
              "bwd_ms": round(ms_b, 4), "bwd_tflops": round((flops - fwd_flops) / (ms_b * 1e-3) / 1e12, 2)}
    log(f"[bench] forward {ms_f:.3f} ms ({passes['fwd_tflops']} TFLOP/s), "
        f"backward {ms_b:.3f} ms ({passes['bwd_tflops']} TFLOP/s)")

    blas = None
    if args.blas_context:
        blas = blas_context(specs, torch, args.steps)
        log(f"[bench] hipBLASLt bf16 on dequantized W (context): {blas['ms']:.3f} ms/step, "
            f"{blas['tflops']:.1f} TFLOP/s")

    roofline = None
    kernels = {}
    hbm = None
    line_extra = {}
    if not args.no_kernel_timing:
        # the same timed loop with every launch bracketed by HIP events on its stream
        L.timing_enable(True)
        L.timing_collect()
        ms_ev = timed(args.steps)
        kt = L.timing_collect()
        L.timing_enable(False)
        # per-kernel algorithmic flops: every step launches each kernel once per layer
        kflops = {}
        for s in specs:
            for name in kt:
                kflops[name] = kflops.get(name, 0) + kernel_flops(name, s)
        kbytes = {}
        for s in specs:
            for name in kt:
                kbytes[name] = kbytes.get(name, 0) + kernel_bytes(name, s)
        for name, (n, tot) in kt.items():
            kernels[name] = {"launches": n, "avg_us": 1e3 * tot / n, "total_ms_per_step": tot / args.steps}
            if kbytes.get(name):
                # algorithmic bytes per step over the kernel's time per step (HBM peak 8 TB/s)
                kernels[name]["algorithmic_gbps"] = round(kbytes[name] / (tot / args.steps * 1e-3) / 1e9, 1)
        dom = max(kt, key=lambda k: kt[k][1])
        n, tot = kt[dom]
        per_launch = kflops[dom] / len(specs)
        achieved = (kflops[dom] * args.steps) / (tot * 1e-3) / 1e12
        tr = recorded_traffic(args.workload + ("_mx" if args.mx else ""), dom)
        # the MX GEMM multiplies E4M3 by E2M1: it is priced at the fp8 dense peak
        peak = PEAK_FP8_TFLOPS if dom == "gemm_mx_base" else PEAK_BF16_TFLOPS
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": None if tr is None else round(tr["bytes_per_launch"]),
                    "flops_per_launch_avg": per_launch, "avg_launch_us": round(1e3 * tot / n, 2),
                    "ms_per_step_with_events": round(ms_ev, 4)}
        for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms_per_step"]):
            log(f"[bench]   {k:22s} {v['launches']:5d} launches  avg {v['avg_us']:9.1f} us  "
                f"{v['total_ms_per_step']:.3f} ms/step")
        hbm = hbm_summary(specs, kernels, args.steps)

    if hbm is not None:
        line_extra["hbm"] = hbm
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) on {args.cpu_tokens} tokens per layer")
        cpu = cpu_baseline(specs, args.cpu_tokens, args.cpu_reps)
        log(f"[bench] cpu oracle {cpu['value']:.4f} TFLOP/s in {cpu['seconds']:.1f} s on {cpu['cores']} threads")

    s0 = specs[0]
    line = {
        "metric": "fwd+bwd TFLOP/s of 4-bit-base LoRA linear; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 x mxfp4 forward, bf16 backward" if args.mx else "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": {1: "single NF4 linear", 2: "Llama-3-8B-shaped layer set", 3: "Llama-70B-shaped MXFP4 layers",
                         4: "MoE grouped experts", 5: "long-context skinny rank",
                         6: "16 LoRA adapters over each Llama-3-8B-shaped base"}[wl]
                        + (" (MX-native forward)" if args.mx else ""),
            "tokens": s0.M,
            "format": s0.fmt,
            "rank": s0.r,
            "alpha": s0.alpha,
            "experts": 1 if s0.shared_base else s0.experts,
            "adapters": s0.experts if s0.shared_base else 1,
            "layers_KxN": [[s.K, s.N] for s in specs],
            "gflop_per_step": round(flops / 1e9, 2),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "passes": passes,
        "kernels": kernels,
    }
    if blas is not None:
        line["blas_context"] = blas
    line.update(line_extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
