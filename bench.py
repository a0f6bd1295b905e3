"""Benchmark of the W4 path on one MI355X.

Headline (``value``): W4A16 decode GEMV at M = 1 on the 8B-class MLP shapes
(up 14336 x 4096, down 4096 x 14336, asymmetric INT4, G = 128, fp16
scale/zero).  One step is a decode pass through ``--layers`` distinct up/down
weight pairs (default 16, about 1 GB of packed weights, four times the 256 MB
Infinity Cache, so every step streams its weights from HBM).  ``value`` is the
algorithmic bytes of the step (codes + scale/zero + activations + outputs)
divided by its time, in GB/s.

Also reported, in the same JSON line: the W4A16 and W4A8 GEMM at the 70B
prefill shape (M = 2048, N = 28672, K = 8192) in TFLOP/s, the W4A8 GEMV on the
12B-class shapes, the GEMV at M = 4 / 16, and the quantizer with the 11-way
MSE clip search on the 70B weight.  Times come from HIP events on the stream
the kernels are launched on.  Calls of a few tens of microseconds or less
(the M = 1 to 256 products on the 8B and 12B shapes, the gate + up pass at
M = 1 and 16, and the small workloads' products) are captured once in a HIP
graph and timed as replays of it, as a serving loop runs them: a call issued
from Python costs about as much host time as the GPU spends on it.  The headline step's rate issued call by
call from Python is reported beside it (``extra.decode_step_eager``).

``cpu_baseline``: the CPU oracle (plain C, OpenMP over the host's cores)
computing the same 8B up + down products at M = 1 in float64, repeated for a
bounded time; same unit as ``value``.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12   # plain (unpacked) fp32 VALU lane operations, 39.3 T/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mul_bytes(M, N, K, G, x_bytes=2):
    """Algorithmic HBM bytes of one product: codes, scale+zero, X, Y."""
    return N * K // 2 + N * (K // G) * 4 + M * K * x_bytes + M * N * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--only", default="all", help="all | decode | gemm | quant | extra")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the work, run a plain device copy of this many MiB three times "
                         "(the known-size kernel that scales the HBM byte counters)")
    return ap.parse_args()


# Source files that define the GEMV and GEMM kernels; a measured traffic figure
# is used only while these files are unchanged since it was taken.
KERNEL_SOURCES = ("w4_dequant_gemm_amd/csrc/skinny.hip", "w4_dequant_gemm_amd/csrc/gemm.hip",
                  "w4_dequant_gemm_amd/csrc/gemm_f8.hip", "w4_dequant_gemm_amd/csrc/rowquant.hip",
                  "w4_dequant_gemm_amd/csrc/device.hpp", "w4_dequant_gemm_amd/csrc/kernels.hpp")


def kernel_source_digest():
    """First 16 hex digits of sha256 over the code of KERNEL_SOURCES (in
    order), with comments and blank lines removed: an edit of a comment
    leaves the measured figures valid, any change of code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        code = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
        h.update("\n".join(line for line in code if line.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """Per-launch HBM bytes of a kernel from its committed counter summary.

    The summary (profiles/<name>.txt) holds ``key: value`` lines, among them
    ``traffic_bytes_per_launch`` and ``kernel_source_digest``; the figure is
    returned only when the digest matches the current kernel sources, else
    None (the counters no longer describe this code).
    """
    path = os.path.join(ROOT, "profiles", name + ".txt")
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "#", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_digest") != kernel_source_digest():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Timer:
    """HIP-event timing on the current (launch) stream."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, reps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps     # ms per call of fn


def captured(torch, fn, outputs):
    """Capture the launches of ``fn`` once in a HIP graph and return its
    replay.  Decode-sized calls take a few microseconds of GPU time, about what
    the Python binding needs to issue one, so they are timed the way a serving
    loop runs them: replayed from a graph.  A replay must reproduce the
    outputs of the eager launches bit for bit."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for o in outputs:
        o.zero_()
    g.replay()
    torch.cuda.synchronize()
    for o, r in zip(outputs, ref):
        if not torch.equal(o, r):
            raise RuntimeError("a graph replay differs from the eager launches")
    return g.replay


def quantize_to_gpu_layout(w4, torch, W, G, fracs):
    q = w4.w4_quantize_blockwise(torch.from_numpy(W).to("cuda:0"), G, "asym", fracs, want_clip=False)
    pk = w4.w4_prepack(q["packed"], q["scale"], q["zero"], G, "asym")
    del q
    return pk


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs the path on a single MI355X; "
              f"--gpus {args.gpus} is not supported (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import w4_dequant_gemm_amd as w4

    dev = torch.device("cuda:0")
    timer = Timer(torch)
    extra = {}
    result = {}

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    # ------------------------------------------------------- headline: decode
    wl8 = synth.WORKLOADS["llama8b_decode"]
    (Nu, Ku), (Nd, Kd) = wl8.shapes
    G = wl8.group
    if args.only in ("all", "decode", "extra"):
        log("[bench] 8B decode: drawing and quantizing the up/down weights on the GPU")
        up = quantize_to_gpu_layout(w4, torch, synth.weight(wl8, 0), G, (1.0,))
        down = quantize_to_gpu_layout(w4, torch, synth.weight(wl8, 1), G, (1.0,))
        L = args.layers
        ups = [up] + [{k: v.clone() for k, v in up.items()} for _ in range(L - 1)]
        downs = [down] + [{k: v.clone() for k, v in down.items()} for _ in range(L - 1)]
        x_up = bf16(synth.activations_bf16_bits(wl8, 1, Ku))
        x_dn = bf16(synth.activations_bf16_bits(wl8, 1, Kd))
        y_up = torch.empty((1, Nu), dtype=torch.bfloat16, device=dev)
        y_dn = torch.empty((1, Nd), dtype=torch.bfloat16, device=dev)

        def step():
            for i in range(L):
                w4.w4a16_gemm(x_up, ups[i]["wq"], ups[i]["sz"], G, Y=y_up)
                w4.w4a16_gemm(x_dn, downs[i]["wq"], downs[i]["sz"], G, Y=y_dn)

    if args.only in ("all", "decode"):
        log(f"[bench] decode step = {L} x (up + down) GEMV, M=1; warmup {args.warmup}, steps {args.steps}")
        # the step replayed from a HIP graph (the timed figure), and issued
        # call by call from Python (reported beside it: there the binding's
        # host time per call is close to the kernel's)
        replay = captured(torch, step, [y_up, y_dn])
        ms = timer.time(replay, args.steps, args.warmup)
        ms_eager = timer.time(step, max(args.steps // 4, 1), args.warmup)
        extra["decode_step_eager"] = {"ms_per_step": round(ms_eager, 5),
                                      "us_per_launch": round(ms_eager / (2 * L) * 1e3, 3)}
        b_up = mul_bytes(1, Nu, Ku, G)
        b_dn = mul_bytes(1, Nd, Kd, G)
        step_bytes = L * (b_up + b_dn)
        value = step_bytes / (ms * 1e-3) / 1e9
        per_launch_ms = ms / (2 * L)
        achieved = (b_up + b_dn) / 2 / (per_launch_ms * 1e-3) / 1e9
        result.update(ms_per_step=ms, value=value, step_bytes=step_bytes)
        result["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                              "traffic": measured_traffic("skinny_dot_w4a16_8b_m1"),
                              "kernel": "gemm_skinny_kernel<1, FJ, false, 3> (W4A16, M=1: v_dot2, "
                                        "activations staged in LDS; FJ = 2 up, 1 down)",
                              "bytes_per_launch": (b_up + b_dn) // 2,
                              "avg_launch_us": round(per_launch_ms * 1e3, 3)}
        log(f"[bench] decode: {ms:.4f} ms/step, {value:.1f} GB/s, per launch {per_launch_ms*1e3:.2f} us")

    if args.only in ("all", "extra"):
        # per-shape GEMV times at M = 1, 4, 16 and 64 (same rotation of weight copies;
        # 64 rows on the 64 x 128 tiles with their K split)
        for M in (1, 4, 16, 64):
            xu = bf16(synth.activations_bf16_bits(wl8, M, Ku))
            xd = bf16(synth.activations_bf16_bits(wl8, M, Kd))
            yu = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
            yd = torch.empty((M, Nd), dtype=torch.bfloat16, device=dev)
            for name, x, y, wts, N, K in (("up", xu, yu, ups, Nu, Ku), ("down", xd, yd, downs, Nd, Kd)):
                # the optional workspace of the K split (streaming kernel, or from 33 rows the tiles)
                wsp = torch.empty((max(w4.w4_gemm_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device=dev)

                def run(x=x, y=y, wts=wts, wsp=wsp):
                    for i in range(L):
                        w4.w4a16_gemm(x, wts[i]["wq"], wts[i]["sz"], G, Y=y, workspace=wsp)
                ms = timer.time(captured(torch, run, [y]), 20, 3) / L
                gbs = mul_bytes(M, N, K, G) / (ms * 1e-3) / 1e9
                extra[f"w4a16_gemv_8b_{name}_m{M}"] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
                log(f"[bench] W4A16 8B {name} M={M}: {ms*1e3:.2f} us, {gbs:.1f} GB/s")
        # gated MLP front half at decode: gate and up (two 14336 x 4096 weights,
        # consecutive copies) in one pass with the SiLU-and-multiply epilogue,
        # against the two products launched separately (from 33 rows with the
        # products' split workspace, as a caller would pass it)
        for M in (1, 16, 64, 256):
            x = bf16(synth.activations_bf16_bits(wl8, M, Ku))
            h = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
            y2 = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
            wsm = torch.empty((max(w4.w4_gemm_workspace_bytes(M, Ku, Nu), 16),), dtype=torch.uint8, device=dev)

            def fused(x=x, h=h):
                for i in range(0, L - 1, 2):
                    w4.w4a16_gate_up(x, ups[i], ups[i + 1], G, "silu", H=h)

            def apart(x=x, h=h, y2=y2, wsm=wsm):
                for i in range(0, L - 1, 2):
                    w4.w4a16_gemm(x, ups[i]["wq"], ups[i]["sz"], G, Y=h, workspace=wsm)
                    w4.w4a16_gemm(x, ups[i + 1]["wq"], ups[i + 1]["sz"], G, Y=y2, workspace=wsm)
            pairs = L // 2
            msf = timer.time(captured(torch, fused, [h]), 20, 3) / pairs
            msa = timer.time(captured(torch, apart, [h, y2]), 20, 3) / pairs
            by = 2 * mul_bytes(M, Nu, Ku, G) - M * Ku * 2 - M * Nu * 2    # x read once, one output
            extra[f"w4a16_gate_up_8b_m{M}"] = {"us": round(msf * 1e3, 3), "GB/s": round(by / (msf * 1e-3) / 1e9, 1),
                                               "TFLOP/s": round(4.0 * M * Nu * Ku / (msf * 1e-3) / 1e12, 2),
                                               "two_products_us": round(msa * 1e3, 3)}
            log(f"[bench] W4A16 8B gate+up M={M}: fused {msf*1e3:.2f} us ({by/(msf*1e-3)/1e9:.1f} GB/s), "
                f"two products {msa*1e3:.2f} us")
        # the same pair at prefill (M = 2048): the tiled pair GEMM against the
        # two GEMMs followed by torch's SiLU-and-multiply
        M = 2048
        x = bf16(synth.activations_bf16_bits(wl8, M, Ku))
        h = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
        ya = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
        yb = torch.empty((M, Nu), dtype=torch.bfloat16, device=dev)
        wsb = w4.w4_gemm_workspace_bytes(M, Ku, Nu)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev)

        wsg = torch.empty((max(w4.w4a16_gate_up_workspace_bytes(M, Ku, Nu), 16),), dtype=torch.uint8, device=dev)

        def fused_p():
            w4.w4a16_gate_up(x, ups[0], ups[1], G, "silu", H=h, workspace=wsg)

        def apart_p():
            w4.w4a16_gemm(x, ups[0]["wq"], ups[0]["sz"], G, Y=ya, workspace=ws)
            w4.w4a16_gemm(x, ups[1]["wq"], ups[1]["sz"], G, Y=yb, workspace=ws)
            torch.mul(torch.nn.functional.silu(ya), yb, out=h)
        # 30 untimed calls (about 15 ms of matrix work) first, as for the 70B
        # products below: the clocks ramp up under sustained matrix work
        msf = timer.time(fused_p, 20, 30)
        msa = timer.time(apart_p, 20, 10)
        fl = 2 * 2.0 * M * Nu * Ku
        extra["w4a16_gate_up_8b_m2048"] = {"ms": round(msf, 4), "TFLOP/s": round(fl / (msf * 1e-3) / 1e12, 1),
                                           "two_gemms_and_act_ms": round(msa, 4)}
        log(f"[bench] W4A16 8B gate+up M=2048: fused {msf:.3f} ms ({fl/(msf*1e-3)/1e12:.1f} TFLOP/s), "
            f"two GEMMs + SiLU*mul {msa:.3f} ms")
        # W4A8 form of the same pair (row quantization included), M = 256 and 2048
        for M8 in (256, 2048):
            x8 = x[:M8]
            h8 = h[:M8]
            xq8 = torch.empty((M8, Ku), dtype=torch.uint8, device=dev)
            xs8 = torch.empty((M8,), dtype=torch.float32, device=dev)
            hq8 = torch.empty((M8, Nu), dtype=torch.uint8, device=dev)
            hs8 = torch.empty((M8,), dtype=torch.float32, device=dev)
            wse = torch.empty((max(w4.w4a8_gate_up_workspace_bytes(M8, Ku, Nu), 16),), dtype=torch.uint8, device=dev)

            def fused8(x8=x8, h8=h8, xq8=xq8, xs8=xs8):
                w4.w4a8_gate_up(x8, ups[0], ups[1], G, "silu", H=h8, xq=xq8, xscale=xs8)

            def fused8e(x8=x8, h8=h8, xq8=xq8, xs8=xs8, hq8=hq8, hs8=hs8, wse=wse):
                w4.w4a8_gate_up(x8, ups[0], ups[1], G, "silu", H=h8, xq=xq8, xscale=xs8, hq=hq8, hscale=hs8,
                                workspace=wse)

            def fused8_rq(x8=x8, h8=h8, xq8=xq8, xs8=xs8, hq8=hq8, hs8=hs8):
                w4.w4a8_gate_up(x8, ups[0], ups[1], G, "silu", H=h8, xq=xq8, xscale=xs8)
                w4.w4_quantize_rows_e4m3(h8, xq=hq8, xscale=hs8)
            ms8 = timer.time(fused8, 20, 20)
            ms8e = timer.time(fused8e, 20, 5)
            ms8r = timer.time(fused8_rq, 20, 5)
            fl8 = 2 * 2.0 * M8 * Nu * Ku
            extra[f"w4a8_gate_up_8b_m{M8}"] = {"ms": round(ms8, 4), "TFLOP/s": round(fl8 / (ms8 * 1e-3) / 1e12, 1),
                                               "with_e4m3_H_ms": round(ms8e, 4),
                                               "then_row_quantizer_on_H_ms": round(ms8r, 4)}
            log(f"[bench] W4A8 8B gate+up M={M8}: fused {ms8:.3f} ms ({fl8/(ms8*1e-3)/1e12:.1f} TFLOP/s, incl. row "
                f"quant); emitting E4M3 H {ms8e:.3f} ms; row quantizer on H after it {ms8r:.3f} ms")
        del x, h, ya, yb, ws, x8, h8, xq8, xs8, hq8, hs8, wse

        # NF4 comparator at M = 1: the same up/down weights in NF4 (blocks of
        # 64, double-quantized scales), same rotation of copies
        for name, idx, x in (("up", 0, x_up), ("down", 1, x_dn)):
            Wd = torch.from_numpy(synth.weight(wl8, idx)).to(dev)
            base = w4.w4_nf4_quantize(Wd)
            del Wd
            copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(L - 1)]
            N, K = base["packed"].shape[0], 2 * base["packed"].shape[1]
            y = torch.empty((N,), dtype=torch.bfloat16, device=dev)

            def run_nf4(x=x, y=y, copies=copies):
                for c in copies:
                    w4.w4_nf4_gemv(x, c, y=y)
            ms = timer.time(captured(torch, run_nf4, [y]), 20, 3) / L
            nb = N * K // 64
            by = N * K // 2 + nb + 4 * ((nb + 255) // 256) + 2 * K + 2 * N
            gbs = by / (ms * 1e-3) / 1e9
            w4us = extra[f"w4a16_gemv_8b_{name}_m1"]["us"]
            extra[f"nf4_gemv_8b_{name}_m1"] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 1),
                                              "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "w4a16_us": w4us}
            log(f"[bench] NF4 8B {name} M=1: {ms*1e3:.2f} us, {gbs:.1f} GB/s (W4A16 G={G}: {w4us:.2f} us)")
            del copies, base
        del ups, downs
        torch.cuda.empty_cache()

        # Context for the decode figure: a plain streaming read of the same
        # 31.2 MB per launch (libw4probe.so, measurement only), launched back
        # to back over 17 rotating buffers as the products are; the best of a
        # few grid sizes is the achievable ceiling of one launch of this size.
        nbytes = mul_bytes(1, Nu, Ku, G)
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(17)]
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        probe = ctypes.CDLL(os.path.join(ROOT, "w4_dequant_gemm_amd", "libw4probe.so"))
        probe.w4probe_stream_read.restype = ctypes.c_int
        probe.w4probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        ptrs = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
        stream_h = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        best = None
        for blocks in (1024, 2048, 4096):
            def read_all(blocks=blocks):
                rc = probe.w4probe_stream_read(ptrs, len(bufs), nbytes, 2 * L, blocks, sink.data_ptr(), stream_h)
                if rc != 0:
                    raise RuntimeError(f"w4probe_stream_read returned {rc}")
            ms = timer.time(read_all, 20, 3) / (2 * L)
            log(f"[bench] plain streaming read, {blocks} workgroups: {ms*1e3:.2f} us per 31.2 MB, "
                f"{nbytes/(ms*1e-3)/1e9:.1f} GB/s")
            if best is None or ms < best[0]:
                best = (ms, blocks)
        ms, blocks = best
        extra["stream_read_31mb"] = {"us": round(ms * 1e3, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                     "workgroups": blocks, "launches_per_timing": 2 * L, "buffers": len(bufs)}
        del bufs, sink

        # W4A8 GEMV / small GEMM on the 12B shapes (weights with the 11-way clip search)
        wl12 = synth.WORKLOADS["gemma12b_w4a8"]
        for idx, (N, K) in enumerate(wl12.shapes):
            base = quantize_to_gpu_layout(w4, torch, synth.weight(wl12, idx), 128, synth.FRACS_11)
            copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(15)]
            for M in sorted(set(wl12.ms) | {128}):
                x = bf16(synth.activations_bf16_bits(wl12, M, K))
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
                xs = torch.empty((M,), dtype=torch.float32, device=dev)
                # split-K partial sums for shapes with few output tiles, and above
                # 128 rows the widened activations (the fastest W4A8 schedule)
                ws = torch.empty((max(w4.w4a8_gemm_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device=dev)

                def run(x=x, y=y, xq=xq, xs=xs, ws=ws, copies=copies):
                    for c in copies:
                        w4.w4a8_gemm(x, c["wq"], c["sz"], 128, Y=y, xq=xq, xscale=xs, workspace=ws)
                ms = timer.time(captured(torch, run, [y, xq, xs]), 10, 2) / len(copies)
                by = mul_bytes(M, N, K, 128)
                fl = 2.0 * M * N * K
                extra[f"w4a8_12b_{idx}_m{M}"] = {"us": round(ms * 1e3, 3),
                                                 "GB/s": round(by / (ms * 1e-3) / 1e9, 1),
                                                 "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2)}
                log(f"[bench] W4A8 12B[{idx}] M={M}: {ms*1e3:.2f} us, {by/(ms*1e-3)/1e9:.1f} GB/s, "
                    f"{fl/(ms*1e-3)/1e12:.2f} TFLOP/s (incl. row quant)")
            del copies, base
            torch.cuda.empty_cache()

    if args.only in ("all", "extra"):
        # the small workloads (tiny, SmolLM2 MLP) and the quantizer on every
        # workload: times only (launch-latency sized, no roofline claim; the
        # products replayed from a graph)
        for name, wl in synth.WORKLOADS.items():
            if name == "llama70b_prefill":
                continue
            fr = tuple(float(f) for f in synth.workload_fracs(wl))
            for idx, (N, K) in enumerate(wl.shapes):
                Wt = torch.from_numpy(synth.weight(wl, idx)).to(dev)
                for mode in wl.modes:
                    out = w4.w4_quantize_blockwise(Wt, wl.group, mode, fr)

                    def qrun(mode=mode, out=out):
                        w4.w4_quantize_blockwise(Wt, wl.group, mode, fr, packed=out["packed"], scale=out["scale"],
                                                 zero=out["zero"], clip_idx=out["clip_idx"])
                    msq = timer.time(qrun, 20, 3)
                    extra[f"quantize_{name}_{idx}_{mode}_n{len(fr)}"] = {
                        "us": round(msq * 1e3, 2), "weights_per_s": round(N * K / (msq * 1e-3), 0)}
                    if name in ("tiny", "smollm2_135m_mlp"):
                        pk = w4.w4_prepack(out["packed"], out["scale"], out["zero"], wl.group, mode)
                        for M in wl.ms:
                            x = bf16(synth.activations_bf16_bits(wl, M, K))
                            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                            # 20 calls per graph: one replay of a single small
                            # launch costs more than the launch itself
                            def small(x=x, y=y, pk=pk, G=wl.group):
                                for _ in range(20):
                                    w4.w4a16_gemm(x, pk["wq"], pk["sz"], G, Y=y)
                            msm = timer.time(captured(torch, small, [y]), 20, 3) / 20
                            extra[f"w4a16_{name}_{idx}_{mode}_m{M}"] = {
                                "us": round(msm * 1e3, 2),
                                "GB/s": round(mul_bytes(M, N, K, wl.group) / (msm * 1e-3) / 1e9, 1)}
                            log(f"[bench] {name}[{idx}] {mode} M={M}: {msm*1e3:.2f} us")
                    del out
                del Wt
        torch.cuda.empty_cache()

    # ------------------------------------------------ 70B prefill GEMM + quantizer
    if args.only in ("all", "gemm", "quant"):
        wl70 = synth.WORKLOADS["llama70b_prefill"]
        (N, K), = wl70.shapes
        M = wl70.ms[0]
        log("[bench] 70B prefill: drawing W and X")
        W = torch.from_numpy(synth.weight(wl70, 0)).to(dev)
        fr = tuple(float(f) for f in synth.FRACS_11)
        if args.only in ("all", "quant"):
            packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
            scale = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
            zero = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
            clip = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)

            def quant():
                w4.w4_quantize_blockwise(W, 128, "asym", fr, packed=packed, scale=scale, zero=zero, clip_idx=clip)
            ms = timer.time(quant, 5, 1)
            qbytes = N * K * 4 + N * K // 2 + N * (K // 128) * 5
            # ALU roofline: about 9 VALU operations per weight and candidate
            # (range, scale, zero, code, reconstruction, squared error, tree
            # add) against 256 CUs x 64 lanes x 2.4 GHz of plain fp32 VALU
            q_ops = 9.0 * N * K * len(fr)
            q_tops = q_ops / (ms * 1e-3) / 1e12
            extra["quantize_70b_clip11_alu"] = {"bound": "alu", "achieved": round(q_tops, 2), "peak": VALU_PEAK_TOPS,
                                                "unit": "Tops/s", "frac": round(q_tops / VALU_PEAK_TOPS, 4)}
            extra["quantize_70b_clip11"] = {"ms": round(ms, 3), "GB/s": round(qbytes / (ms * 1e-3) / 1e9, 1),
                                            "weights_per_s": round(N * K / (ms * 1e-3), 0)}
            log(f"[bench] quantize 70B (11 candidates): {ms:.3f} ms, {qbytes/(ms*1e-3)/1e9:.1f} GB/s")
            for nf in (1,):
                def quant1():
                    w4.w4_quantize_blockwise(W, 128, "asym", (1.0,), packed=packed, scale=scale, zero=zero,
                                             clip_idx=clip)
                ms1 = timer.time(quant1, 5, 1)
                extra["quantize_70b_plain"] = {"ms": round(ms1, 3), "GB/s": round(qbytes / (ms1 * 1e-3) / 1e9, 1)}
                log(f"[bench] quantize 70B (plain): {ms1:.3f} ms")
            pk = w4.w4_prepack(packed, scale, zero, 128, "asym")

            def prep():
                w4.w4_prepack(packed, scale, zero, 128, "asym", wq=pk["wq"], sz=pk["sz"])
            msp = timer.time(prep, 10, 2)
            pbytes = 2 * (N * K // 2 + N * (K // 128) * 4)
            extra["prepack_70b"] = {"us": round(msp * 1e3, 2), "GB/s": round(pbytes / (msp * 1e-3) / 1e9, 1)}
            del packed, scale, zero, clip
        else:
            pk = quantize_to_gpu_layout(w4, torch, W.cpu().numpy(), 128, fr)
        del W
        torch.cuda.empty_cache()
        if args.only in ("all", "gemm"):
            X = bf16(synth.activations_bf16_bits(wl70, M, K))
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
            xs = torch.empty((M,), dtype=torch.float32, device=dev)
            flops = 2.0 * M * N * K
            # fp32 partial tiles of the last round's tiles, whose K is split,
            # and (W4A8) the widened activations: the fastest schedule of both
            ws = torch.empty((max(w4.w4a8_gemm_workspace_bytes(M, K, N), 16),), dtype=torch.uint8, device=dev)
            # 50 untimed calls (about 50 ms) first: the clocks ramp up under
            # sustained matrix work, and a cold start would time the ramp
            ms16 = timer.time(lambda: w4.w4a16_gemm(X, pk["wq"], pk["sz"], 128, Y=Y, workspace=ws), 20, 50)
            ms8 = timer.time(lambda: w4.w4a8_gemm(X, pk["wq"], pk["sz"], 128, Y=Y, xq=xq, xscale=xs,
                                                  workspace=ws), 20, 50)
            t16 = flops / (ms16 * 1e-3) / 1e12
            t8 = flops / (ms8 * 1e-3) / 1e12
            extra["w4a16_gemm_70b_m2048"] = {"ms": round(ms16, 4), "TFLOP/s": round(t16, 1)}
            extra["w4a8_gemm_70b_m2048"] = {"ms": round(ms8, 4), "TFLOP/s": round(t8, 1)}
            result["roofline_gemm"] = {"bound": "mfma", "achieved": round(t16, 1), "peak": BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(t16 / BF16_PEAK_TFLOPS, 4),
                                       "traffic": measured_traffic("gemm256_breg_w4a16_70b_m2048"),
                                       "kernel": "gemm256_breg_kernel<false, 8> + splitk_reduce_kernel<256, 256> (the whole W4A16 "
                                                 "call, M=2048: 768 tiles whole, the last 128 in two K halves)",
                                       "flops_per_launch": flops, "avg_launch_us": round(ms16 * 1e3, 1)}
            result["roofline_w4a8"] = {"bound": "mfma", "achieved": round(t8, 1), "peak": FP8_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(t8 / FP8_PEAK_TFLOPS, 4),
                                       "traffic": measured_traffic("gemm_f8_w4a8_70b_m2048"),
                                       "kernel": "rowquant_kernel + gemm_f8_kernel<256, 256, 1, 8> + splitk_reduce_kernel<256, 256> "
                                                 "(the whole W4A8 call, M=2048: fp8 MFMA 16x16x128 on E4M3 "
                                                 "activations and exact u - z weight operands)",
                                       "flops_per_launch": flops, "avg_launch_us": round(ms8 * 1e3, 1)}
            log(f"[bench] 70B GEMM M=2048: W4A16 {ms16:.3f} ms = {t16:.1f} TFLOP/s; "
                f"W4A8 {ms8:.3f} ms = {t8:.1f} TFLOP/s ({t8 / FP8_PEAK_TFLOPS:.3f} of the fp8 peak)")

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.arange(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)       # elementwise: reads and writes n * 4 bytes
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written, 3 times")
        del src, dst

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu and args.only in ("all", "decode"):
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "W4A16 GEMV HBM GB/s (% peak) at M=1, 8B shapes; W4 GEMM TFLOP/s at M=2048",
        "value": round(result.get("value", 0.0), 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(result.get("ms_per_step", 0.0), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"llama8b_decode: W4A16 GEMV M=1 through {args.layers} distinct "
                               "up[14336x4096] + down[4096x14336] INT4 asym G=128 weight pairs",
                   "global_batch": 1, "group": 128, "layers": args.layers,
                   "step_bytes": result.get("step_bytes")},
        "roofline": result.get("roofline"),
        "roofline_gemm": result.get("roofline_gemm"),
        "roofline_w4a8": result.get("roofline_w4a8"),
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(seconds: float):
    """The oracle's float64 W4A16 product on the same 8B up + down layers, M = 1."""
    import numpy as np

    import oracle
    import synth
    wl = synth.WORKLOADS["llama8b_decode"]
    log("[bench] CPU oracle baseline: quantizing the 8B layers on the host")
    layers = []
    for idx, (N, K) in enumerate(wl.shapes):
        W = synth.weight(wl, idx)
        q = oracle.quantize(W, wl.group, "asym")
        del W
        x = oracle.bf16_bits_to_f64(synth.activations_bf16_bits(wl, 1, K))
        layers.append((q, x, N, K))
    total_bytes = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for q, x, N, K in layers:
            oracle.gemm_ref(x, q["packed"], q["scale"], q["zero"], wl.group, "asym")
            total_bytes += mul_bytes(1, N, K, wl.group)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 2000:
            break
    gbs = total_bytes / el / 1e9
    log(f"[bench] CPU oracle: {reps} x (up + down) in {el:.2f} s = {gbs:.3f} GB/s on {oracle.num_threads()} threads")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} decode passes (M=1) through one 8B up+down layer pair, float64 oracle product "
                      f"({el:.1f} s)",
            "per_config": cpu_per_config()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_per_config():
    """The oracle on every workload: its quantizer (with the workload's clip
    search) and its float64 product at every M, each on a bounded row sample,
    reported as seconds for the whole call (sample time scaled by the sampled
    fraction of rows) next to the sample that was timed."""
    import numpy as np

    import oracle
    import synth

    def timed(fn, min_s=0.05):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                return el / n
    out = {}
    for name, wl in synth.WORKLOADS.items():
        fr = synth.workload_fracs(wl)
        for idx, (N, K) in enumerate(wl.shapes):
            # quantizer: up to 2^21 weights of whole rows
            rows = max(1, min(N, (1 << 21) // K))
            W = synth.weight(wl, idx, rows=rows)
            for mode in wl.modes:
                t = timed(lambda: oracle.quantize(W, wl.group, mode, fracs=fr))
                out[f"{name}_{idx}_quantize_{mode}_n{len(fr)}"] = {
                    "cpu_s_full": round(t * N / rows, 6), "sample_rows": rows, "rows": N}
            q = oracle.quantize(W, wl.group, wl.modes[-1], fracs=fr)
            del W
            for M in wl.ms:
                # product: at most 2^26 multiply-adds of the sample (whole sampled weight rows)
                mr = max(1, min(M, (1 << 26) // (rows * K)))
                X = oracle.bf16_bits_to_f64(synth.activations_bf16_bits(wl, mr, K))
                t = timed(lambda: oracle.gemm_ref(X, q["packed"], q["scale"], q["zero"], wl.group, wl.modes[-1]))
                full = t * (M / mr) * (N / rows)
                out[f"{name}_{idx}_product_m{M}"] = {"cpu_s_full": round(full, 6), "sample_rows_x_cols": [mr, rows],
                                                     "shape": [M, N, K]}
    log(f"[bench] CPU oracle per workload: {len(out)} entries")
    return out


if __name__ == "__main__":
    main()
