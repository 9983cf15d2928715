#!/usr/bin/env python3
"""Decode throughput of the 64-layer 27B-shaped ternary projection stack on one GPU.

One step = one token through all 64 layers (tq_decode_stack).  Per layer, in
order, one launch each: quantise a fresh fp16 input and run the QKV
projection (5120 -> 10240); quantise a fresh fp16 input and run O
(8192 -> 5120); quantise O's output and run the fused gate/up/SwiGLU
(5120 -> 17408, two matrices); quantise h and run down (17408 -> 5120).  All
weights are distinct per layer (about 5.06 GB of B3-packed trits and fp16
scales), resident in HBM before timing starts.  Inputs are seeded synthetic
data with the shapes and distributions of the workload (trits P(0) = 1/2,
P(+-1) = 1/4; scales uniform in [0.005, 0.05]; activations N(0,1) in fp16).

Prints one JSON line.  --gpus N > 1 is refused: the library has no multi-GPU path.

  python bench.py --profile-summary TRACE_DIR FETCH_DIR WRITE_DIR
turns three rocprofv3 runs of this script (--kernel-trace --stats, then
--pmc FETCH_SIZE, then --pmc WRITE_SIZE) into the text summary kept under
profiles/ and the per-launch HBM traffic of the dominant kernel;
  python bench.py --counter-summary PMC_DIR...
prints per-kernel averages of the SQ counters of --pmc runs of this script.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ternary GEMV weight-stream GB/s (% HBM peak); 27B-stack decode tok/s"
HIDDEN, INTER, QKV_OUT, O_IN, LAYERS = 5120, 17408, 10240, 8192, 64
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_swiglu_stack_b3.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--fmt", choices=["b3", "2b"], default="b3")
    p.add_argument("--layers", type=int, default=LAYERS,
                   help="layers in the stack (the workload is 64; fewer is for quick checks)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline (0 = skip)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the prefill GEMM and small-batch measurements")
    p.add_argument("--profile-summary", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                   help="summarise rocprofv3 output directories of this script and exit")
    p.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR",
                   help="per-kernel averages of the counters in rocprofv3 --pmc directories "
                        "of this script (the stack's four projections, the prefill GEMM, the "
                        "small-batch GEMV), and exit")
    return p.parse_args()


# The sources the dominant kernel (the projection kernel) is built from.
DOMINANT_SOURCES = ("tq_proj.h", "tq_proj_kernel.h", "tq_proj.hip", "tq_proj_inst.hip", "tq_device.h",
                    "tq_layout.h")


def kernel_source_sha() -> str:
    """Hash of the dominant kernel's sources: traffic counted on other code is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_weight_base_amd", "csrc")
    for name in DOMINANT_SOURCES:
        with open(os.path.normpath(os.path.join(csrc, name)), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class Stack:
    """Packed weights of all layers, resident on the GPU."""

    SHAPES = {"qkv": (QKV_OUT, HIDDEN), "o": (HIDDEN, O_IN), "gate": (INTER, HIDDEN),
              "up": (INTER, HIDDEN), "down": (HIDDEN, INTER)}
    MATRIX_ID = {"qkv": 0, "o": 1, "gate": 2, "up": 3, "down": 4}

    def __init__(self, tq, synth, torch, fmt: int, layers: int):
        self.fmt, self.layers = fmt, layers
        self.bytes = {k: tq.tq_packed_bytes(fmt, n, k2) for k, (n, k2) in self.SHAPES.items()}
        self.W = {k: [] for k in self.SHAPES}
        for l in range(layers):
            for name, (N, K) in self.SHAPES.items():
                seed = synth.seed(3, 1000 + l, self.MATRIX_ID[name])
                t = synth.trits(synth.seed(seed, 1), N, K)
                s = synth.scales(synth.seed(seed, 2), N, K)
                blob = tq.tq_pack(fmt, t, s)
                self.W[name].append(torch.from_numpy(blob).cuda())
                del t, s, blob
        self.step_weight_bytes = layers * sum(self.bytes.values())


def main():
    args = parse()
    if args.profile_summary:
        profile_summary(*args.profile_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only; --gpus N with N > 1 is not "
              "supported (the library has no collectives).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import ternary_weight_base_amd as tq

    torch.cuda.set_device(0)
    dev = "cuda"
    fmt = tq.TQ_FMT_B3 if args.fmt == "b3" else tq.TQ_FMT_2B
    L = args.layers
    t0 = time.time()
    stack = Stack(tq, synth, torch, fmt, L)
    print(f"# stack packed and uploaded: {L} layers, {stack.step_weight_bytes / 1e9:.3f} GB "
          f"in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    x_in = torch.from_numpy(synth.normal_f16(synth.seed(3, 7, 1), L, HIDDEN)).to(dev)
    a_in = torch.from_numpy(synth.normal_f16(synth.seed(3, 7, 2), L, O_IN)).to(dev)
    y_qkv = torch.empty((L, QKV_OUT), dtype=torch.float32, device=dev)
    y_o = torch.empty((L, HIDDEN), dtype=torch.float32, device=dev)
    h = torch.empty((L, INTER), dtype=torch.float32, device=dev)
    y_dn = torch.empty((L, HIDDEN), dtype=torch.float32, device=dev)
    layers = tq.stack_layers([(stack.W["qkv"][l], stack.W["o"][l], stack.W["gate"][l],
                               stack.W["up"][l], stack.W["down"][l]) for l in range(L)])
    st_bytes = tq.tq_decode_stack_workspace_bytes(fmt, L, HIDDEN, INTER, QKV_OUT, O_IN)
    st_ws = torch.zeros((st_bytes + 15) // 16 * 4, dtype=torch.int32, device=dev)

    # the decode step: tq_decode_stack, 4 launches per layer
    def token():
        tq.tq_decode_stack(fmt, L, HIDDEN, INTER, QKV_OUT, O_IN, layers, x_in, a_in,
                           y_qkv, y_o, h, y_dn, st_ws)

    # the same token through the persistent kernel (one launch per 32 layers)
    def token_persistent():
        tq.tq_decode_stack(fmt, L, HIDDEN, INTER, QKV_OUT, O_IN, layers, x_in, a_in,
                           y_qkv, y_o, h, y_dn, st_ws, persistent=True)

    # the same token with the FFN input rotated online (block-64 Hadamard and
    # signs, folded into the O projection's epilogue)
    ffn_signs = torch.from_numpy(synth.signs(synth.seed(3, 7, 3), L * HIDDEN).reshape(L, HIDDEN)).to(dev)

    def token_rot():
        tq.tq_decode_stack(fmt, L, HIDDEN, INTER, QKV_OUT, O_IN, layers, x_in, a_in,
                           y_qkv, y_o, h, y_dn, st_ws, ffn_signs=ffn_signs)

    # the same token as 8 separate launches per layer (quantiser, then GEMV)
    q5, q8, q17 = (torch.empty((1, k), dtype=torch.int8, device=dev) for k in (HIDDEN, O_IN, INTER))
    sc = torch.empty(4, dtype=torch.float32, device=dev)
    y1, h1 = torch.empty((1, QKV_OUT), device=dev), torch.empty((1, INTER), device=dev)
    yo1, yd1 = torch.empty((1, HIDDEN), device=dev), torch.empty((1, HIDDEN), device=dev)
    ws_bytes = max(tq.tq_gemv_workspace_bytes(fmt, 1, n, k) for n, k in Stack.SHAPES.values())
    ws = torch.zeros(max(1, (ws_bytes + 15) // 16 * 4), dtype=torch.int32, device=dev)

    def token_separate():
        for l in range(L):
            tq.tq_quant_act(x_in[l:l + 1], q5, sc[0:1])
            tq.tq_gemv(fmt, 1, QKV_OUT, HIDDEN, stack.W["qkv"][l], q5, sc[0:1], y1, ws)
            tq.tq_quant_act(a_in[l:l + 1], q8, sc[1:2])
            tq.tq_gemv(fmt, 1, HIDDEN, O_IN, stack.W["o"][l], q8, sc[1:2], yo1, ws)
            tq.tq_quant_act(yo1, q5, sc[2:3])
            tq.tq_gemv_gate_up_swiglu(fmt, 1, INTER, HIDDEN, stack.W["gate"][l],
                                      stack.W["up"][l], q5, sc[2:3], h1, ws)
            tq.tq_quant_act(h1, q17, sc[3:4])
            tq.tq_gemv(fmt, 1, HIDDEN, INTER, stack.W["down"][l], q17, sc[3:4], yd1, ws)

    # The dominant kernel as the stack launches it: gate/up/SwiGLU on O's fp32
    # output and block maxima (made here once per layer by the same call).
    nb_o = HIDDEN // 64
    bmax_o = torch.empty((L, nb_o), dtype=torch.float32, device=dev)
    yo_l = torch.empty((L, HIDDEN), dtype=torch.float32, device=dev)
    hq = torch.empty((L, INTER), dtype=torch.float32, device=dev)
    q_bytes = max(tq.tq_gemv_quant_workspace_bytes(fmt, HIDDEN, O_IN),
                  tq.tq_gemv_quant_workspace_bytes(fmt, INTER, HIDDEN, True))
    q_ws = torch.zeros(max(4, (q_bytes + 15) // 16 * 4), dtype=torch.int32, device=dev)
    for l in range(L):
        tq.tq_gemv_quant(fmt, HIDDEN, O_IN, stack.W["o"][l], None, a_in[l], yo_l[l],
                         y_bmax=bmax_o[l], ws=q_ws)

    def gate_up_all():
        for l in range(L):
            tq.tq_gemv_quant(fmt, INTER, HIDDEN, stack.W["gate"][l], stack.W["up"][l], yo_l[l],
                             hq[l], x_bmax=bmax_o[l], ws=q_ws)

    # A plain device copy of known size (64 MiB read + 64 MiB written), untimed:
    # profiles of this command use it to calibrate the FETCH_SIZE / WRITE_SIZE
    # counters against bytes that are known exactly.
    calib_src = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    cap = torch.cuda.Stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def capture(fn):
        fn()  # eager run: loads kernels, checks arguments
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, steps, warmup):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # ---- timed region: K tokens through the stack ---------------------------
    graph = capture(token)
    ms_per_step = time_graph(graph, args.steps, args.warmup)
    assert torch.isfinite(y_dn).all().item() and torch.isfinite(h).all().item(), "non-finite"
    tok_s = 1000.0 / ms_per_step
    stream_gbps = stack.step_weight_bytes / (ms_per_step * 1e-3) / 1e9
    persistent_ms = time_graph(capture(token_persistent), max(3, args.steps // 4), 1)
    assert tq.stack_timeouts(st_ws) == 0, "a wait of the persistent stack kernel gave up"
    sep_ms = time_graph(capture(token_separate), max(3, args.steps // 4), 1)
    rot_ms = time_graph(capture(token_rot), max(3, args.steps // 4), 1)

    # ---- dominant kernel: the fused gate/up/SwiGLU projection, timed on its
    # own over the same 64 layers' weights (graph of L launches, HIP events)
    # weights + fp32 input and its block maxima + fp32 output
    gu_bytes = 2 * stack.bytes["gate"] + HIDDEN * 4 + (HIDDEN // 64) * 4 + INTER * 4
    gu_us = time_graph(capture(gate_up_all), 5, 1) * 1000.0 / L
    gu_gbps = gu_bytes / (gu_us * 1e-6) / 1e9
    traffic, trace = None, None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha") == kernel_source_sha() and tr.get("fmt") == args.fmt:
            traffic = tr.get("hbm_bytes_per_launch")
            if tr.get("trace_avg_launch_us"):
                t_us = tr["trace_avg_launch_us"]
                trace = {"avg_launch_us": t_us, "achieved": round(gu_bytes / (t_us * 1e-6) / 1e9, 1),
                         "frac": round(gu_bytes / (t_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                         "source": os.path.relpath(TRAFFIC_FILE, ROOT) + " (rocprofv3 kernel trace "
                                   "of this script, same kernel sources)"}
    # ---- measured HBM read ceiling: a plain streaming read of 2 GiB (beyond
    # the 256 MB MALL), beside which the byte rates above are also reported
    rd = torch.ones(1 << 29, dtype=torch.int32, device=dev)
    rd_sink = torch.empty(tq.TQ_STREAM_READ_WGS, dtype=torch.int32, device=dev)
    rd_ms = time_graph(capture(lambda: tq.tq_debug_stream_read(rd, rd_sink)), 10, 2)
    read_gbps = rd.numel() * 4 / (rd_ms * 1e-3) / 1e9
    read_ceiling = {"GBps": round(read_gbps, 1), "bytes": rd.numel() * 4,
                    "frac_of_8TBps": round(read_gbps / PEAK_HBM_GBPS, 4),
                    "kernel": "tq_debug_stream_read (8192 workgroups x 256 threads, 16-byte "
                              "nontemporal loads, 8 in flight per thread)"}
    del rd, rd_sink
    torch.cuda.empty_cache()
    roofline = {"bound": "hbm", "achieved": round(gu_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gu_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": "proj_kernel<fmt,2,fp32 input> (fused quantise + gate/up/SwiGLU, "
                          "2 x 17408x5120), as launched by the stack",
                "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 3),
                "trace": trace,
                "frac_of_measured_read_ceiling": round(gu_gbps / read_gbps, 4)}

    # ---- the other rows of the hot path, measured on the same weights -------
    extras = measure_extras(args, tq, synth, torch, fmt, stack, x_in, a_in, capture, time_graph)

    # ---- layout A/B: the same stack, inputs and seeds in each packed layout
    if extras is not None:
        # b3r: B3's bytes in row-major group order, without the re-tiling
        names = {tq.TQ_FMT_B3: "b3", tq.TQ_FMT_2B: "2b", tq.TQ_FMT_BP: "bp", tq.TQ_FMT_B3R: "b3r"}
        ab = {names[fmt]: {"tok_s": round(tok_s, 2), "weight_bytes_per_token": stack.step_weight_bytes}}
        for other in (tq.TQ_FMT_B3, tq.TQ_FMT_2B, tq.TQ_FMT_BP, tq.TQ_FMT_B3R):
            if other == fmt:
                continue
            st2 = Stack(tq, synth, torch, other, L)
            lay2 = tq.stack_layers([(st2.W["qkv"][l], st2.W["o"][l], st2.W["gate"][l], st2.W["up"][l],
                                     st2.W["down"][l]) for l in range(L)])
            nb2 = tq.tq_decode_stack_workspace_bytes(other, L, HIDDEN, INTER, QKV_OUT, O_IN)
            ws2 = torch.zeros((nb2 + 15) // 16 * 4, dtype=torch.int32, device=dev)

            def token2():
                tq.tq_decode_stack(other, L, HIDDEN, INTER, QKV_OUT, O_IN, lay2, x_in, a_in,
                                   y_qkv, y_o, h, y_dn, ws2)
            ms2 = time_graph(capture(token2), max(3, args.steps // 2), 2)
            ab[names[other]] = {"tok_s": round(1000.0 / ms2, 2),
                                "weight_bytes_per_token": st2.step_weight_bytes}
            del st2, lay2, ws2
            torch.cuda.empty_cache()
        extras["layout_ab"] = ab

    # ---- CPU baseline: the oracle on a bounded sample of the same workload,
    # and the oracle's check of the timed run's own outputs (layers 0 and L-1)
    cpu, parity = None, None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(synth, args.cpu_seconds, args.fmt)
        graph.replay()  # the timed token once more, then its outputs
        torch.cuda.synchronize()
        outs = [t.cpu().numpy() for t in (y_qkv, y_o, h, y_dn)]
        parity = stack_parity(synth, outs, x_in.cpu().numpy(), a_in.cpu().numpy(), sorted({0, L - 1}))

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8xtrit->int32, fp32 scale",
        "data": "synthetic (seeded trits/scales/N(0,1) fp16 inputs; no checkpoint)",
        "config": {"workload": f"27B-shaped {L}-layer ternary projection stack, decode batch 1",
                   "layers": L, "fmt": args.fmt, "hidden": HIDDEN, "intermediate": INTER,
                   "qkv_out": QKV_OUT, "o_in": O_IN, "group": 128,
                   "weight_bytes_per_token": stack.step_weight_bytes},
        "weight_stream_GBps": round(stream_gbps, 1),
        "weight_stream_frac_of_8TBps": round(stream_gbps / PEAK_HBM_GBPS, 4),
        "weight_stream_frac_of_measured_read_ceiling": round(stream_gbps / read_gbps, 4),
        "hbm_read_ceiling": read_ceiling,
        "stack_persistent_tok_s": round(1000.0 / persistent_ms, 2),
        "separate_launch_tok_s": round(1000.0 / sep_ms, 2),
        "ffn_hadamard_tok_s": round(1000.0 / rot_ms, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "other_rows": extras,
    }
    print(json.dumps(out))


def cpu_baseline(synth, budget_s: float, fmt_name: str):
    """The oracle (plain C, OpenMP over rows) on whole layers of the stack, from
    canonical packed blobs: unpack, quantise, project, SwiGLU, as the GPU does.
    Layers are run until the time budget is spent; tok/s = layers/s / 64."""
    import oracle

    avail = len(os.sched_getaffinity(0))
    cores = min(16, avail)
    oracle.set_threads(cores)
    fmt = oracle.FMT_B3 if fmt_name == "b3" else oracle.FMT_2B
    done, elapsed, l = 0, 0.0, 0
    while elapsed < budget_s and l < LAYERS:
        blobs = {}
        for name, (N, K) in Stack.SHAPES.items():
            seed = synth.seed(3, 1000 + l, Stack.MATRIX_ID[name])
            blobs[name] = oracle.pack(fmt, synth.trits(synth.seed(seed, 1), N, K),
                                      synth.scales(synth.seed(seed, 2), N, K))
        x = synth.normal_f16(synth.seed(3, 7, 1), LAYERS, HIDDEN)[l:l + 1]
        a = synth.normal_f16(synth.seed(3, 7, 2), LAYERS, O_IN)[l:l + 1]
        t0 = time.time()
        q, s = oracle.quant(x)
        oracle.project_packed(fmt, blobs["qkv"], QKV_OUT, HIDDEN, q, s)
        q, s = oracle.quant(a)
        yo = oracle.project_packed(fmt, blobs["o"], HIDDEN, O_IN, q, s)
        q, s = oracle.quant(yo)
        hh = oracle.swiglu(oracle.project_packed(fmt, blobs["gate"], INTER, HIDDEN, q, s),
                           oracle.project_packed(fmt, blobs["up"], INTER, HIDDEN, q, s))
        q, s = oracle.quant(hh)
        oracle.project_packed(fmt, blobs["down"], HIDDEN, INTER, q, s)
        elapsed += time.time() - t0
        done += 1
        l += 1
    layers_per_s = done / elapsed
    return {"value": round(layers_per_s / LAYERS, 4), "unit": "tok/s", "cores": cores,
            "host_cpus_available": avail, "kind": "oracle",
            "sample": f"{done} of {LAYERS} layers of the same stack (unpack+quant+project+SwiGLU "
                      f"from canonical packed blobs, {fmt_name}), {elapsed:.1f} s; tok/s = "
                      f"layers/s / {LAYERS}"}


def stack_parity(synth, outs, x_in, a_in, layers):
    """The timed stack's own outputs against the oracle, stage-isolated (each
    stage fed the GPU's input of that stage, so the int8 codes are bit-exact
    and the fp32 outputs compare within the tolerance), on the given layers.
    Runs with the CPU baseline (it is the oracle's part of this run)."""
    import oracle

    y_qkv, y_o, h, y_dn = outs
    worst_abs, worst_l2 = 0.0, 0.0

    def cmp(y, ref):
        nonlocal worst_abs, worst_l2
        y, ref = np.asarray(y, np.float64).ravel(), np.asarray(ref, np.float64).ravel()
        peak = np.abs(ref).max()
        worst_abs = max(worst_abs, float(np.abs(y - ref).max() / peak))
        worst_l2 = max(worst_l2, float(np.linalg.norm(y - ref) / np.linalg.norm(ref)))

    for l in layers:
        hw = {}
        for name, (N, K) in Stack.SHAPES.items():
            seed = synth.seed(3, 1000 + l, Stack.MATRIX_ID[name])
            hw[name] = (synth.trits(synth.seed(seed, 1), N, K), synth.scales(synth.seed(seed, 2), N, K))
        q, sc = oracle.quant(x_in[l:l + 1])
        cmp(y_qkv[l], oracle.gemv(*hw["qkv"], q, sc))
        q, sc = oracle.quant(a_in[l:l + 1])
        cmp(y_o[l], oracle.gemv(*hw["o"], q, sc))
        q, sc = oracle.quant(y_o[l:l + 1])
        cmp(h[l], oracle.swiglu(oracle.gemv(*hw["gate"], q, sc), oracle.gemv(*hw["up"], q, sc)))
        q, sc = oracle.quant(h[l:l + 1])
        cmp(y_dn[l], oracle.gemv(*hw["down"], q, sc))
        del hw
    return {"layers": list(layers), "max_abs_err_rel_to_peak": worst_abs, "max_rel_l2": worst_l2,
            "tolerance": {"max_abs_err_rel_to_peak": 1e-3, "rel_l2": 1e-5},
            "ok": worst_abs <= 1e-3 and worst_l2 <= 1e-5,
            "how": "stage-isolated against the oracle, every output of the four projections"}


def measure_extras(args, tq, synth, torch, fmt, stack, x_in, a_in, capture, time_graph):
    """The other configurations of the hot path, each on weights resident in HBM:
    - gemv_1k: one-token tq_gemv at N = K = 1024 (229,376 weight bytes, far
      below what fills the GPU: launch-latency-bound), per call over a graph
      of 2048 calls on 2048 distinct weight copies (470 MB, beyond the
      256 MB last-level cache);
    - quant_act_5120 / hadamard_quant_act_5120: the activation quantiser of
      one 5120-element token, alone and with the block-64 Hadamard rotation
      (per call over 64 calls; launch-latency-bound);
    - ffn_block: quant(x) -> gate/up/SwiGLU -> quant(h) -> down for one token,
      as two fused launches (tq_gemv_quant), per block over the stack's 64
      layers of FFN weights;
    - prefill GEMM (M = 512 on the gate and down matrices of the first 16
      layers, one launch per layer back to back in one graph, so that the
      graph's own launch cost is spread as in the decode measurements)
      against the int8 MFMA peak;
    - small-batch decode (M tokens per step through the whole stack:
      tq_quant_act + tq_gemv per projection, 8 launches a layer), and for
      M = 2..4 the batch stack (tq_decode_stack_batch: 4 launches a layer,
      quantisers fused, each weight group decoded once for all rows);
    - ternarize_host: the host ternariser on one fp32 gate matrix
      (17408 x 5120, 356 MB), the load-time step before tq_pack.
    (main() adds layout_ab: the decode stack in each packed layout.)"""
    if args.no_extras:
        return None
    dev = "cuda"
    out = {}
    # gemv_1k: 2048 copies of one packed 1024 x 1024 matrix
    n1 = 1024
    t1 = synth.trits(synth.seed(1, n1, n1), n1, n1)
    s1 = synth.scales(synth.seed(2, n1, n1), n1, n1)
    blob1 = torch.from_numpy(tq.tq_pack(fmt, t1, s1)).to(dev)
    copies = 2048
    W1 = blob1.repeat(copies).view(copies, -1)
    x1 = torch.from_numpy(synth.normal_f16(synth.seed(1, 7, 1), 1, n1)).to(dev)
    q1 = torch.empty((1, n1), dtype=torch.int8, device=dev)
    a1 = torch.empty(1, dtype=torch.float32, device=dev)
    tq.tq_quant_act(x1, q1, a1)
    y1 = torch.empty((1, n1), dtype=torch.float32, device=dev)
    ws1 = torch.zeros(max(4, (tq.tq_gemv_workspace_bytes(fmt, 1, n1, n1) + 15) // 16 * 4),
                      dtype=torch.int32, device=dev)

    def gemv_all():
        for c in range(copies):
            tq.tq_gemv(fmt, 1, n1, n1, W1[c], q1, a1, y1, ws1)
    us1 = time_graph(capture(gemv_all), 3, 1) * 1000.0 / copies
    out["gemv_1k"] = {"N": n1, "K": n1, "us_per_call": round(us1, 3),
                      "weight_GBps": round(blob1.numel() / (us1 * 1e-6) / 1e9, 1),
                      "bound": "launch latency"}
    del W1, blob1
    # the activation quantiser alone, and with the Hadamard rotation (M = 1, K = 5120)
    xq = torch.from_numpy(synth.normal_f16(synth.seed(1, 7, 2), 64, HIDDEN)).to(dev)
    qq = torch.empty((64, HIDDEN), dtype=torch.int8, device=dev)
    aq = torch.empty(64, dtype=torch.float32, device=dev)
    sq = torch.from_numpy(synth.signs(synth.seed(1, 7, 3), HIDDEN)).to(dev)
    us_q = time_graph(capture(lambda: [tq.tq_quant_act(xq[i:i + 1], qq[i:i + 1], aq[i:i + 1])
                                       for i in range(64)]), 5, 1) * 1000.0 / 64
    us_h = time_graph(capture(lambda: [tq.tq_hadamard_quant_act(xq[i:i + 1], sq, qq[i:i + 1], aq[i:i + 1])
                                       for i in range(64)]), 5, 1) * 1000.0 / 64
    out["quant_act_5120"] = {"us_per_call": round(us_q, 3), "bound": "launch latency"}
    wt = synth.normal_f32(synth.seed(6, 1), INTER, HIDDEN)
    t0 = time.time()
    tq.tq_ternarize(wt)
    sec = time.time() - t0
    out["ternarize_host"] = {"N": INTER, "K": HIDDEN, "s": round(sec, 3),
                             "input_GBps": round(wt.nbytes / sec / 1e9, 2),
                             "threads": int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))}
    del wt
    out["hadamard_quant_act_5120"] = {"us_per_call": round(us_h, 3), "bound": "launch latency"}
    # ffn_block over the stack's layers
    L = stack.layers
    xf = torch.from_numpy(synth.normal_f16(synth.seed(2, 7, 1), L, HIDDEN)).to(dev)
    hf = torch.empty((L, INTER), dtype=torch.float32, device=dev)
    bh = torch.empty((L, INTER // 64), dtype=torch.float32, device=dev)
    yf = torch.empty((L, HIDDEN), dtype=torch.float32, device=dev)
    nbf = max(tq.tq_gemv_quant_workspace_bytes(fmt, INTER, HIDDEN, True),
              tq.tq_gemv_quant_workspace_bytes(fmt, HIDDEN, INTER))
    wsf = torch.zeros(max(4, (nbf + 15) // 16 * 4), dtype=torch.int32, device=dev)

    def ffn_all():
        for l in range(L):
            tq.tq_gemv_quant(fmt, INTER, HIDDEN, stack.W["gate"][l], stack.W["up"][l], xf[l], hf[l],
                             y_bmax=bh[l], ws=wsf)
            tq.tq_gemv_quant(fmt, HIDDEN, INTER, stack.W["down"][l], None, hf[l], yf[l],
                             x_bmax=bh[l], ws=wsf)
    usf = time_graph(capture(ffn_all), 5, 1) * 1000.0 / L
    ffn_bytes = 2 * stack.bytes["gate"] + stack.bytes["down"]
    out["ffn_block"] = {"us": round(usf, 3), "weight_bytes": ffn_bytes,
                        "weight_GBps": round(ffn_bytes / (usf * 1e-6) / 1e9, 1),
                        "frac_of_8TBps": round(ffn_bytes / (usf * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    M = 512
    for name, (N, K) in (("gate", (INTER, HIDDEN)), ("down", (HIDDEN, INTER))):
        x = torch.from_numpy(synth.normal_f16(synth.seed(4, N, K), M, K)).to(dev)
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        a = torch.empty(M, dtype=torch.float32, device=dev)
        tq.tq_quant_act(x, q, a)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        Ws = [stack.W[name][l] for l in range(min(L, 16))]
        gws = tq.workspace(fmt, M, N, K)

        def gemm_layers():
            for W in Ws:
                tq.tq_gemm(fmt, M, N, K, W, q, a, y, gws)
        ms = time_graph(capture(gemm_layers), 5, 1) / len(Ws)
        tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[f"prefill_gemm_{name}"] = {"M": M, "N": N, "K": K, "us": round(ms * 1e3, 2), "launches": len(Ws),
                                       "TOP/s": round(tops, 1), "peak_int8_mfma_TOP/s": 5000.0,
                                       "frac": round(tops / 5000.0, 4)}
    for Mb in (2, 3, 4, 8, 16):
        xs = torch.from_numpy(synth.normal_f16(synth.seed(5, Mb, 1), L, Mb, HIDDEN)).to(dev)
        as_ = torch.from_numpy(synth.normal_f16(synth.seed(5, Mb, 2), L, Mb, O_IN)).to(dev)
        qh, qo, qi = (torch.empty((Mb, k), dtype=torch.int8, device=dev) for k in (HIDDEN, O_IN, INTER))
        sc = torch.empty((4, Mb), dtype=torch.float32, device=dev)
        yq = torch.empty((Mb, QKV_OUT), device=dev)
        yo = torch.empty((Mb, HIDDEN), device=dev)
        hh = torch.empty((Mb, INTER), device=dev)
        yd = torch.empty((Mb, HIDDEN), device=dev)
        nb = max(tq.tq_gemv_workspace_bytes(fmt, Mb, n, k) for n, k in Stack.SHAPES.values())
        ws = torch.zeros(max(4, (nb + 15) // 16 * 4), dtype=torch.int32, device=dev)
        W = stack.W

        def step():
            for l in range(L):
                tq.tq_quant_act(xs[l], qh, sc[0])
                tq.tq_gemv(fmt, Mb, QKV_OUT, HIDDEN, W["qkv"][l], qh, sc[0], yq, ws)
                tq.tq_quant_act(as_[l], qo, sc[1])
                tq.tq_gemv(fmt, Mb, HIDDEN, O_IN, W["o"][l], qo, sc[1], yo, ws)
                tq.tq_quant_act(yo, qh, sc[2])
                tq.tq_gemv_gate_up_swiglu(fmt, Mb, INTER, HIDDEN, W["gate"][l], W["up"][l], qh,
                                          sc[2], hh, ws)
                tq.tq_quant_act(hh, qi, sc[3])
                tq.tq_gemv(fmt, Mb, HIDDEN, INTER, W["down"][l], qi, sc[3], yd, ws)
        ms = time_graph(capture(step), 5, 1)
        out[f"small_batch_M{Mb}"] = {"tok/s": round(Mb * 1000.0 / ms, 1), "ms_per_step": round(ms, 3),
                                     "weight_stream_GBps": round(stack.step_weight_bytes / (ms * 1e-3) / 1e9, 1)}
    lay = tq.stack_layers([tuple(stack.W[k][l] for k in ("qkv", "o", "gate", "up", "down")) for l in range(L)])
    for Mb in range(2, tq.STACK_MAX_ROWS + 1):
        xs = torch.from_numpy(synth.normal_f16(synth.seed(5, Mb, 1), L, Mb, HIDDEN)).to(dev)
        as_ = torch.from_numpy(synth.normal_f16(synth.seed(5, Mb, 2), L, Mb, O_IN)).to(dev)
        outs = [torch.empty((L, Mb, n), device=dev) for n in (QKV_OUT, HIDDEN, INTER, HIDDEN)]
        nb = tq.tq_decode_stack_batch_workspace_bytes(fmt, Mb, L, HIDDEN, INTER, QKV_OUT, O_IN)
        ws = torch.zeros((nb + 15) // 16 * 4, dtype=torch.int32, device=dev)
        ms = time_graph(capture(lambda: tq.tq_decode_stack_batch(fmt, Mb, L, HIDDEN, INTER, QKV_OUT, O_IN, lay,
                                                                 xs, as_, *outs, ws)), 5, 1)
        out[f"small_batch_fused_M{Mb}"] = {
            "tok/s": round(Mb * 1000.0 / ms, 1), "ms_per_step": round(ms, 3),
            "weight_stream_GBps": round(stack.step_weight_bytes / (ms * 1e-3) / 1e9, 1)}
    return out


def _rocpd(d):
    """(per-kernel durations in ns, per-dispatch counter sums) from the rocprofv3
    SQLite outputs under directory d."""
    import glob
    import sqlite3
    durs, ctrs = {}, {}
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    for db in dbs:
        c = sqlite3.connect(db)
        tables = {r[0] for r in c.execute("select name from sqlite_master")}
        if "kernels" in tables:
            for name, dur in c.execute("select name, duration from kernels"):
                durs.setdefault(name, []).append(dur)
        if "counters_collection" in tables:
            for name, cn, disp, v in c.execute(
                    "select kernel_name, counter_name, dispatch_id, sum(value) from "
                    "counters_collection group by kernel_name, counter_name, dispatch_id"):
                ctrs.setdefault((name, cn), []).append(v)
    return durs, ctrs


# Kernels whose counters counter_summary reports (name parts, B3 instantiations;
# the last template argument of proj_kernel is the number of token rows).
COUNTER_KERNELS = (("QKV", "proj_kernel<0, 1, 1, 5, 2, false, true, false, 1>"),
                   ("O", "proj_kernel<0, 1, 1, 3, 2, false, true, false, 1>"),
                   ("gate/up", "proj_kernel<0, 2, 2, 6, 2, true, true, false, 1>"),
                   ("down", "proj_kernel<0, 1, 2, 6, 2, false, true, false, 1>"),
                   ("batch-stack gate/up, 4 token rows", "proj_kernel<0, 2, 2, 6, 2, true, true, false, 4>"),
                   ("prefill GEMM, 128-row tiles (gate shape)", "gemm_kernel<0, false, 2>"),
                   ("prefill GEMM, 256-row tiles (down shape)", "gemm_kernel<0, false, 4>"),
                   ("small-batch gate/up", "mgemv_kernel<0, 2, 5, false>"))


def counter_summary(dirs):
    """Per-dispatch averages (whole GPU) of every counter collected in the given
    rocprofv3 --pmc directories, for the kernels of COUNTER_KERNELS."""
    agg = {}
    for d in dirs:
        _, ctrs = _rocpd(d)
        for (kname, cname), vals in ctrs.items():
            for label, prefix in COUNTER_KERNELS:
                if prefix in kname:
                    agg.setdefault(label, {})[cname] = sum(vals) / len(vals)
    for label, _ in COUNTER_KERNELS:
        if label not in agg:
            continue
        print(label)
        for cname, v in sorted(agg[label].items()):
            print(f"  {cname:28s} {v:16.1f}")


def _short(name):
    """A kernel's name without return type, namespaces and parameter list, so
    that its template arguments fit a table column."""
    import re
    s = re.sub(r"^void ", "", name)
    s = re.sub(r"\(anonymous namespace\)::|tqproj::|tqstack::", "", s)
    depth = 0
    for i, ch in enumerate(s):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0 and i > 0:
            return s[:i]
    return s


def profile_summary(trace_dir, fetch_dir, write_dir):
    """Text summary of a profiled bench run (printed) and the dominant kernel's
    trace duration and HBM traffic per launch (written to TRAFFIC_FILE).
    FETCH_SIZE is scaled by what it reads for the 2 GiB streaming read of the
    same run (tq_debug_stream_read: every byte read exactly once, with the
    same nontemporal 16-byte loads as the weights), WRITE_SIZE by what it
    reads for the bench's 64 MiB device copy (64 MiB written)."""
    durs, _ = _rocpd(trace_dir)
    _, fetch = _rocpd(fetch_dir)
    _, write = _rocpd(write_dir)
    read_bytes, copy_bytes = 1 << 31, 64 << 20
    dom = [n for n in durs if "proj_kernel<0, 2, 2, 6, 2, true, true, false, 1>" in n]
    print("kernel                                                        calls   avg_us   total_ms")
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1]))[:32]:
        print(f"{_short(name)[:60]:60s} {len(v):7d} {sum(v) / len(v) / 1e3:8.3f} {sum(v) / 1e6:10.3f}")

    def per_dispatch(ctrs, cname, pick):
        return [x for (k, cn), v in ctrs.items() if cn == cname and pick(k) for x in v]

    fcal = per_dispatch(fetch, "FETCH_SIZE", lambda k: "stream_read_kernel" in k)
    # the copy: the runtime's buffer-copy dispatch whose count sits nearest to 64 MiB
    # (the other device copies are weight uploads of <= 20 MB); 1024 B per KiB
    wcal = per_dispatch(write, "WRITE_SIZE", lambda k: "copyBuffer" in k)
    if not dom or not fcal or not wcal:
        raise SystemExit("dominant kernel or calibration dispatches not found in the profiles")
    fscale = read_bytes / (sum(fcal) / len(fcal) * 1024)
    wbest = min(wcal, key=lambda v: abs(v - copy_bytes / 1024))
    wscale = copy_bytes / (wbest * 1024)
    f = per_dispatch(fetch, "FETCH_SIZE", lambda k: k in dom)
    w = per_dispatch(write, "WRITE_SIZE", lambda k: k in dom)
    fb = sum(f) / len(f) * 1024 * fscale
    wb = sum(w) / len(w) * 1024 * wscale
    dur = [x for n in dom for x in durs[n]]
    avg_us = sum(dur) / len(dur) / 1e3
    alg = 2 * 19496960 + 5120 * 4 + 80 * 4 + 17408 * 4  # weights, fp32 input, its maxima, output
    print(f"\ndominant kernel: {dom[0]}")
    print(f"  launches traced {len(dur)}, avg duration {avg_us:.3f} us -> {alg / (avg_us * 1e3):.1f} GB/s "
          f"algorithmic ({alg} B per launch), {alg / (avg_us * 1e3) / PEAK_HBM_GBPS:.4f} of 8 TB/s")
    print(f"  FETCH_SIZE per launch {sum(f) / len(f):.0f} KiB raw, x{fscale:.4f} (2 GiB streaming-read "
          f"calibration) = {fb / 1e6:.3f} MB")
    print(f"  WRITE_SIZE per launch {sum(w) / len(w):.0f} KiB raw, x{wscale:.4f} (64 MiB copy "
          f"calibration) = {wb / 1e6:.3f} MB")
    print(f"  calibration: streaming read of {read_bytes} B: FETCH_SIZE {sum(fcal) / len(fcal):.0f} KiB per "
          f"dispatch ({len(fcal)} dispatches); copy of {copy_bytes} B: WRITE_SIZE {wbest:.0f} KiB")
    out = {"kernel": dom[0], "fmt": "b3", "kernel_source_sha": kernel_source_sha(),
           "trace_avg_launch_us": round(avg_us, 3), "trace_launches": len(dur),
           "algorithmic_bytes_per_launch": alg,
           "hbm_bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
           "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
           "fetch_calibration": "stream_read_kernel, 2 GiB read once",
           "write_calibration": "64 MiB device copy"}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"\nwrote {os.path.relpath(TRAFFIC_FILE, ROOT)}")


if __name__ == "__main__":
    main()
