#!/usr/bin/env python3
"""Benchmark of the FP8-weight GEMM path on one MI355X.

Headline workload: the action-decoder GEMM pair at M = 50 rows with OCP
E4M3 per-channel-scaled weights, up-projection 1024 -> 4096 and
down-projection 4096 -> 1024 (bf16 activations ~N(0,1), weights ~N(0,0.02),
seeded; synthetic stand-ins for the camera observations and checkpoints the
pages measure on).  One step = one up call + one down call.  Inputs are
resident in HBM before timing starts.

Cache regime: "cold" (default) rotates every step through distinct copies of
the packed weights totalling >= 1 GiB, so weights stream from HBM rather than
the 256 MB Infinity Cache, and writes a 1 GiB buffer right before every timed
replay, so no copy the replay reads is cache-resident at any step count;
"warm" reuses one copy and skips the flush.

Timing: W untimed warmup steps, then K steps recorded once into a HIP graph
(the way the pages run inference), one untimed replay, the cache flush, and
one replay timed between HIP events on the launch stream, with
torch.cuda.synchronize() on both sides.  value = mean microseconds per GEMM
call of that replay (lower is better); six more flushed replays give the
p10/p50/p90 spread.  A one-workgroup marker kernel runs right before and
right after the timed replay (outside the events), so a kernel trace of this
command can pick out exactly the timed dispatches:

    rocprofv3 --kernel-trace --stats -d DIR -o run --output-format csv -- \
        python3 bench.py --gpus 1 --steps 20 --warmup 5
    python3 bench.py --trace-summary DIR --bench-json <the JSON line's file>

Prints one JSON line.  --gpus above 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA, published
FP8_PEAK_TFLOPS = 5000.0

M, H, I = 50, 1024, 4096
UP = (M, I, H)                 # (M, N, K): 50 x 1024 -> 4096
DOWN = (M, H, I)               # 50 x 4096 -> 1024


def alg_bytes_fp8w(m, n, k):
    """Algorithmic HBM bytes of one FP8-weight GEMM call: W + scales + A + Y."""
    return n * k + 4 * n + 2 * m * k + 2 * m * n


def alg_bytes_bf16w(m, n, k):
    return 2 * n * k + 2 * m * k + 2 * m * n


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cache", choices=["cold", "warm"], default="cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 8 times (scale reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--wide-only", action="store_true",
                    help="only run the M = 768 encoder GEMMs (W8A16 and FP8 x FP8, both shapes, 8 calls "
                         "each; the workload of the wide-kernel counter runs) and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="summarize a rocprofv3 kernel trace of this script (no GPU work): the dispatches "
                         "between the two marker kernels, i.e. the headline's timed replay, and exit")
    ap.add_argument("--bench-json", metavar="FILE", help="with --trace-summary: the bench's output, to compare")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="summarize rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of this script (no GPU work): "
                         "HBM bytes per dispatch of --kernel, scaled by a --calibrate-copy run of each, and exit")
    ap.add_argument("--kernel", default="skinny_gemm_kernel", help="with --pmc-summary: kernel name filter")
    ap.add_argument("--all-kernels-summary", metavar="DIR",
                    help="tabulate every launch configuration of a rocprofv3 kernel trace of this script (no GPU "
                         "work) and exit")
    ap.add_argument("--pmc-table", nargs="+", metavar="DIR",
                    help="mean per dispatch of every counter in rocprofv3 --pmc runs of this script, per launch "
                         "shape of --kernel (no GPU work), and exit")
    ap.add_argument("--mfma-trace-summary", metavar="DIR",
                    help="summarize a rocprofv3 kernel trace of --mfma-only (no GPU work) and exit")
    ap.add_argument("--algorithmic-bytes", type=int, help="with --pmc-summary: algorithmic bytes per launch")
    ap.add_argument("--mfma-only", action="store_true",
                    help="only run the matrix-core rate probe (zero and GEMM-like operands, four forms), print its "
                         "JSON and exit")
    ap.add_argument("--wide-shape", choices=["up", "down", "both"], default="both",
                    help="with --wide-only: the 2048 -> 16384 up-projection, the 16384 -> 2048 down-projection, "
                         "or both")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.bench_json)
        return
    if args.all_kernels_summary:
        all_kernels_summary(args.all_kernels_summary)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table, args.kernel)
        return
    if args.mfma_trace_summary:
        mfma_trace_summary(args.mfma_trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.kernel, args.algorithmic_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(it scales by replicas, one request per GPU with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.full((256 << 20,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "copies": 8}))
        return

    import bf16_gemm_vla_amd as vla
    import synthetic

    vla.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def up_bits(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a.copy()).to(dev)

    def quantize(W, wfmt=vla.VLA_WFMT_E4M3_OCP):
        N, K = W.shape
        q = torch.empty(vla.vla_packed_bytes(N, K, wfmt), dtype=torch.uint8, device=dev)
        s = torch.empty(N, dtype=torch.float32, device=dev) if wfmt != vla.VLA_WFMT_BF16 else None
        vla.vla_quantize_pack(up_bits(W), q, s, N, K, wfmt, vla.VLA_LAYOUT_MFMA)
        return q, s

    if args.mfma_only:
        print(json.dumps({"mfma_rate_TFLOPs": mfma_rates(vla, torch, dev)}))
        return

    if args.wide_only:
        Mw = 768
        shapes = {"up": [(16384, 2048)], "down": [(2048, 16384)], "both": [(16384, 2048), (2048, 16384)]}
        for n, k in shapes[args.wide_shape]:
            A = up_bits(synthetic.activations(Mw, k, 910 + n))
            q, s = quantize(synthetic.weights(n, k, 911 + n))
            qa = torch.empty(Mw * k, dtype=torch.uint8, device=dev)
            sa = torch.empty(1, dtype=torch.float32, device=dev)
            wq = torch.zeros(vla.vla_quantize_act_workspace_bytes(Mw, k), dtype=torch.uint8, device=dev)
            vla.vla_quantize_act(A, qa, sa, wq, wq.numel(), Mw, k)
            Y = torch.empty(Mw * n, dtype=torch.int16, device=dev)
            wsb = vla.vla_gemm_workspace_bytes(Mw, n, k, 1)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            for Ap, sap in ((A, None), (qa, sa)):
                for _ in range(8):
                    vla.vla_gemm_fp8w(Ap, sap, q, s, None, None, Y, ws, wsb, Mw, n, k)
                torch.cuda.synchronize()
        print(json.dumps({"wide_only": "done"}))
        return

    # ---------------------------------------------------------- headline
    log("building skinny workload")
    A_up = up_bits(synthetic.activations(M, H, synthetic.IDS["skinny.up.A"]))
    A_dn = up_bits(synthetic.activations(M, I, synthetic.IDS["skinny.down.A"]))
    W_up = synthetic.weights(I, H, synthetic.IDS["skinny.up.W"])
    W_dn = synthetic.weights(H, I, synthetic.IDS["skinny.down.W"])
    q_up, s_up = quantize(W_up)
    q_dn, s_dn = quantize(W_dn)
    copies = 1
    if args.cache == "cold":
        copies = max(1, (1 << 30) // (q_up.numel() + q_dn.numel()))
    qs_up = [q_up] + [q_up.clone() for _ in range(copies - 1)]
    qs_dn = [q_dn] + [q_dn.clone() for _ in range(copies - 1)]
    Y_up = torch.empty(M * I, dtype=torch.int16, device=dev)
    Y_dn = torch.empty(M * H, dtype=torch.int16, device=dev)
    ws_bytes = max(vla.vla_gemm_workspace_bytes(*UP, 1), vla.vla_gemm_workspace_bytes(*DOWN, 1))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)

    def step(i):
        c = i % copies
        vla.vla_gemm_fp8w(A_up, None, qs_up[c], s_up, None, None, Y_up, ws, ws_bytes, *UP)
        vla.vla_gemm_fp8w(A_dn, None, qs_dn[c], s_dn, None, None, Y_dn, ws, ws_bytes, *DOWN)

    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cache == "cold" else None
    flush_val = [0]
    marker_sink = torch.zeros(64, dtype=torch.int32, device=dev)

    def flush():
        """Write 1 GiB (4x the Infinity Cache) so nothing read next is cache-resident."""
        if flush_buf is not None:
            flush_val[0] = (flush_val[0] + 1) & 0xFF
            flush_buf.fill_(flush_val[0])

    def read_flush():
        """Read the same 1 GiB instead: evicts the caches and leaves no dirty
        lines to be written back during the timed replay (reported beside
        the protocol's write flush, never as the headline)."""
        if flush_buf is not None:
            vla.vla_probe_stream_read(flush_buf, flush_buf.numel(), marker_sink[32:], 2048)

    def marker():
        # one workgroup of the streaming-read probe over 16 bytes: the only
        # one-workgroup dispatch this script makes, so a kernel trace can
        # find the timed replay between two of them
        vla.vla_probe_stream_read(marker_sink, 16, marker_sink[16:], 1)

    def time_graph_all(fn, n, reps=1, cold=None, mark=False, flusher=None):
        """Record fn(0..n-1) into one graph, replay once untimed, then `reps`
        times, each after the cache flush (cold regime) and between HIP
        events; returns the ms of each timed replay."""
        flusher = flusher or flush
        cold = (args.cache == "cold") if cold is None else cold
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                fn(i)
        g.replay()                      # one untimed replay
        torch.cuda.synchronize()
        out = []
        for r in range(reps):
            if cold:
                flusher()
            if mark and r == 0:
                marker()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            if mark and r == 0:
                marker()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        del g
        return out

    def time_graph(fn, n, cold=None):
        return time_graph_all(fn, n, 1, cold)[0]

    def time_eager(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    log(f"warmup {args.warmup} steps ({copies} weight copies)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    reps = time_graph_all(step, args.steps, reps=7, mark=True)
    ms_graph = reps[0]                  # the headline: exactly K steps, one replay
    us_reps = np.array(reps) * 1000.0 / (2 * args.steps)
    us_read_flush = np.array(time_graph_all(step, args.steps, reps=5, flusher=read_flush)) * 1000.0 / (2 * args.steps)
    ms_eager = time_eager(step, args.steps)
    us_call = ms_graph * 1000.0 / (2 * args.steps)
    bytes_step = alg_bytes_fp8w(*UP) + alg_bytes_fp8w(*DOWN)
    achieved = bytes_step / (ms_graph * 1e-3 / args.steps) / 1e9
    floor_buf = torch.zeros(1, device=dev)
    floor_us = time_graph(lambda i: floor_buf.fill_(1.0), args.steps, cold=False) * 1000.0 / args.steps
    # streaming-read floor: one launch that only reads one call's 4 MiB of
    # packed weights (same cold rotation as the GEMM pair), best launch size
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    read_us = {}
    for blocks in (256, 512, 1024, 2048):
        def rd(i, blocks=blocks):
            q = (qs_up if i % 2 == 0 else qs_dn)[(i // 2) % copies]
            vla.vla_probe_stream_read(q, q.numel(), sink, blocks)
        read_us[blocks] = time_graph(rd, 2 * args.steps) * 1000.0 / (2 * args.steps)
    best_blocks = min(read_us, key=read_us.get)
    extra = {
        "us_per_call_p10_p50_p90": [round(float(np.percentile(us_reps, q)), 3) for q in (10, 50, 90)],
        "us_per_call_after_read_flush_p50": round(float(np.median(us_read_flush)), 3),
        "timed_replays_for_spread": len(reps),
        "us_per_call_eager": round(ms_eager * 1000.0 / (2 * args.steps), 3),
        "graph_launch_floor_us": round(floor_us, 3),
        "stream_read_4MiB_us": round(read_us[best_blocks], 3),
        "stream_read_4MiB_GBps": round(q_up.numel() / (read_us[best_blocks] * 1e-6) / 1e9, 1),
        "stream_read_blocks": best_blocks,
        "weight_copies": copies,
    }

    # per-shape split (same protocol)
    for name, shp, qs, A, s, Y in (("up", UP, qs_up, A_up, s_up, Y_up), ("down", DOWN, qs_dn, A_dn, s_dn, Y_dn)):
        def one(i, shp=shp, qs=qs, A=A, s=s, Y=Y):
            vla.vla_gemm_fp8w(A, None, qs[i % copies], s, None, None, Y, ws, ws_bytes, *shp)
        ms = time_graph(one, args.steps)
        extra[f"{name}_us"] = round(ms * 1000.0 / args.steps, 3)
        extra[f"{name}_GBps"] = round(alg_bytes_fp8w(*shp) / (ms * 1e-3 / args.steps) / 1e9, 1)
    # a call's time against the best time of a launch that only streams its
    # 4 MiB of weights (same cold rotation): the share of the single-call floor reached
    extra["read_floor_over_call"] = round(read_us[best_blocks] / (0.5 * (extra["up_us"] + extra["down_us"])), 3)
    if not args.no_extra:
        # one GPU's share of the up-projection split by output columns over
        # eight GPUs (no exchange): N/8 channels, a prefix of the packed
        # weights and scales, same cold rotation
        UPS = (M, I // 8, H)
        ws_s = torch.zeros(vla.vla_gemm_workspace_bytes(*UPS, 1), dtype=torch.uint8, device=dev)

        def up_shard(i):
            vla.vla_gemm_fp8w(A_up, None, qs_up[i % copies], s_up, None, None, Y_up, ws_s, ws_s.numel(), *UPS)
        ms = time_graph(up_shard, args.steps)
        extra["up_shard8_us"] = round(ms * 1000.0 / args.steps, 3)

    if not args.no_extra:
        # MXFP4 weights (E2M1 + an E8M0 scale per 32 values: 0.53 of the FP8
        # bytes), same shapes, activations and cold rotation over >= 1 GiB
        def quantize_mx(W):
            n_, k_ = W.shape
            q = torch.empty(vla.vla_packed_bytes(n_, k_, vla.VLA_WFMT_MXFP4), dtype=torch.uint8, device=dev)
            vla.vla_quantize_pack(up_bits(W), q, None, n_, k_, vla.VLA_WFMT_MXFP4, vla.VLA_LAYOUT_MFMA)
            return q
        mq_up, mq_dn = quantize_mx(W_up), quantize_mx(W_dn)
        mcopies = max(1, (1 << 30) // (mq_up.numel() + mq_dn.numel())) if args.cache == "cold" else 1
        mqs = {"up": [mq_up] + [mq_up.clone() for _ in range(mcopies - 1)],
               "down": [mq_dn] + [mq_dn.clone() for _ in range(mcopies - 1)]}
        wsm_bytes = max(vla.vla_gemm_workspace_bytes(*UP, vla.VLA_WFMT_MXFP4),
                        vla.vla_gemm_workspace_bytes(*DOWN, vla.VLA_WFMT_MXFP4))
        wsm = torch.zeros(wsm_bytes, dtype=torch.uint8, device=dev)
        for name, shp, A, Y in (("up", UP, A_up, Y_up), ("down", DOWN, A_dn, Y_dn)):
            def onem(i, name=name, shp=shp, A=A, Y=Y):
                vla.vla_gemm_mxfp4w(A, mqs[name][i % mcopies], None, None, Y, wsm, wsm_bytes, *shp)
            ms = time_graph(onem, args.steps)
            us = ms * 1000.0 / args.steps
            n_, k_ = shp[1], shp[2]
            mx_bytes = n_ * k_ // 2 + n_ * k_ // 32 + 2 * shp[0] * k_ + 2 * shp[0] * n_
            extra[f"mxfp4_{name}_us"] = round(us, 3)
            extra[f"mxfp4_{name}_GBps"] = round(mx_bytes / (us * 1e-6) / 1e9, 1)

        # the fused gate/up GEMM of the gated MLP (merged 2I x H weights,
        # GELU-tanh(gate) * up epilogue), same activations, cold rotation
        W_gu = np.concatenate([W_up, synthetic.weights(I, H, synthetic.IDS["skinny.up.W"] + 1000)])
        q_gu, s_gu = quantize(W_gu)
        gcopies = max(1, (1 << 30) // q_gu.numel()) if args.cache == "cold" else 1
        qs_gu = [q_gu] + [q_gu.clone() for _ in range(gcopies - 1)]
        act_gu = torch.empty(M * I, dtype=torch.int16, device=dev)
        wsg_bytes = vla.vla_gemm_workspace_bytes(M, 2 * I, H, 1)
        wsg = torch.zeros(wsg_bytes, dtype=torch.uint8, device=dev)

        def gateup(i):
            vla.vla_gemm_fp8w_gelu_mul(A_up, qs_gu[i % gcopies], s_gu, None, act_gu, None, wsg, wsg_bytes, M, I, H)
        ms = time_graph(gateup, args.steps)
        us = ms * 1000.0 / args.steps
        gu_bytes = 2 * I * H + 4 * 2 * I + 2 * M * H + 2 * M * I
        extra["gateup_us"] = round(us, 3)
        extra["gateup_GBps"] = round(gu_bytes / (us * 1e-6) / 1e9, 1)
        del qs_gu

        # the pages' own decoder row count (10 rows), same weights and rotation
        A10_up = up_bits(synthetic.activations(10, H, synthetic.IDS["skinny.up.A"]))
        A10_dn = up_bits(synthetic.activations(10, I, synthetic.IDS["skinny.down.A"]))
        ws10_bytes = max(vla.vla_gemm_workspace_bytes(10, I, H, 1), vla.vla_gemm_workspace_bytes(10, H, I, 1))
        ws10 = torch.zeros(ws10_bytes, dtype=torch.uint8, device=dev)
        for name, shp, qs, A, s in (("up", (10, I, H), qs_up, A10_up, s_up), ("down", (10, H, I), qs_dn, A10_dn, s_dn)):
            def one10(i, shp=shp, qs=qs, A=A, s=s):
                vla.vla_gemm_fp8w(A, None, qs[i % copies], s, None, None, Y_up, ws10, ws10_bytes, *shp)
            ms = time_graph(one10, args.steps)
            extra[f"m10_{name}_us"] = round(ms * 1000.0 / args.steps, 3)
            wsm10_bytes = vla.vla_gemm_workspace_bytes(*shp, vla.VLA_WFMT_MXFP4)
            wsm10 = torch.zeros(wsm10_bytes, dtype=torch.uint8, device=dev)

            def one10m(i, name=name, shp=shp, A=A, wsm10=wsm10, wsm10_bytes=wsm10_bytes):
                vla.vla_gemm_mxfp4w(A, mqs[name][i % mcopies], None, None, Y_up, wsm10, wsm10_bytes, *shp)
            ms = time_graph(one10m, args.steps)
            extra[f"m10_mxfp4_{name}_us"] = round(ms * 1000.0 / args.steps, 3)
        del mqs

    if not args.no_extra:
        extra.update(secondary(vla, torch, np, synthetic, dev, quantize, up_bits, time_graph, args))

    result = {
        "metric": "µs/call + achieved HBM GB/s (M≤64) / MFMA TFLOP/s (M≥512), FP8-weight GEMM",
        "value": round(us_call, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 activations, N(0,0.02) fp32 weights -> OCP E4M3 per-channel)",
        "config": {
            "workload": "action-decoder skinny FP8-weight GEMM pair, M=50: up 1024->4096 + down 4096->1024",
            "M": M, "hidden": H, "intermediate": I, "weights": "OCP E4M3, per-output-channel fp32 scale",
            "cache": args.cache + (" (1 GiB weight rotation + 1 GiB flush before the timed replay)"
                                   if args.cache == "cold" else ""),
            "timing": "HIP graph of K steps replayed once between HIP events",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "skinny_gemm_kernel (FP8 weights, bf16 activations), up and down launches",
            "bytes_per_launch": bytes_step // 2,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
        },
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, synthetic, W_up, W_dn)
    print(json.dumps(result), flush=True)


def secondary(vla, torch, np, synthetic, dev, quantize, up_bits, time_graph, args):
    """Encoder-size GEMMs, the 18-layer chain, the BF16-weight skinny GEMMs
    and the dialect conversion, each timed the same way (graph + events)."""
    out = {}
    log("secondary: bf16-weight skinny")
    for name, (m, n, k) in (("bf16_up", UP), ("bf16_down", DOWN)):
        A = up_bits(synthetic.activations(m, k, 900 + n))
        q, _ = quantize(synthetic.weights(n, k, 901 + n), vla.VLA_WFMT_BF16)
        copies = max(1, (1 << 30) // q.numel()) if args.cache == "cold" else 1
        qs = [q] + [q.clone() for _ in range(copies - 1)]
        Y = torch.empty(m * n, dtype=torch.int16, device=dev)
        wsb = vla.vla_gemm_workspace_bytes(m, n, k, 0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

        def one(i, A=A, qs=qs, Y=Y, ws=ws, wsb=wsb, m=m, n=n, k=k, copies=copies):
            vla.vla_gemm_bf16(A, qs[i % copies], None, None, Y, ws, wsb, m, n, k)
        ms = time_graph(one, 128)
        us = ms * 1000.0 / 128
        out[f"{name}_us"] = round(us, 3)
        out[f"{name}_GBps"] = round(alg_bytes_bf16w(m, n, k) / (us * 1e-6) / 1e9, 1)
        # the pages' 10 decoder rows, same weights and rotation (their FP8
        # vs BF16 comparison at that size)
        A10 = up_bits(synthetic.activations(10, k, 900 + n))
        ws10b = vla.vla_gemm_workspace_bytes(10, n, k, 0)
        ws10 = torch.zeros(ws10b, dtype=torch.uint8, device=dev)

        def one10(i, A10=A10, qs=qs, Y=Y, ws10=ws10, ws10b=ws10b, n=n, k=k, copies=copies):
            vla.vla_gemm_bf16(A10, qs[i % copies], None, None, Y, ws10, ws10b, 10, n, k)
        ms = time_graph(one10, 128)
        out[f"m10_{name}_us"] = round(ms * 1000.0 / 128, 3)
        del qs

    log("secondary: vendor library context")
    # torch.matmul in bf16 (hipBLASLt / rocBLAS underneath) on the same
    # shapes, bf16 weights transposed to K x N beforehand, weights in a
    # 1 GiB rotation for the decoder shapes as above: the comparison the
    # pages draw ("Beating the hipBLASLt baseline"); context, not the path
    for name, (m, n, k), rot in (("vendor_bf16_up", UP, True), ("vendor_bf16_down", DOWN, True),
                                 ("vendor_bf16_wide_up", (768, 16384, 2048), False),
                                 ("vendor_bf16_wide_down", (768, 2048, 16384), False)):
        A = torch.randn(m, k, device=dev).to(torch.bfloat16)
        Wt = (torch.randn(k, n, device=dev) * 0.02).to(torch.bfloat16).contiguous()
        copies = max(1, (1 << 30) // (Wt.numel() * 2)) if (rot and args.cache == "cold") else 1
        Wts = [Wt] + [Wt.clone() for _ in range(copies - 1)]
        Yv = torch.empty(m, n, dtype=torch.bfloat16, device=dev)

        def mm(i, A=A, Wts=Wts, Yv=Yv, copies=copies):
            torch.matmul(A, Wts[i % copies], out=Yv)
        mm(0)                       # the library's one-time set-up, outside the capture
        torch.cuda.synchronize()
        reps = 128 if rot else 20
        ms = time_graph(mm, reps)
        out[f"{name}_us"] = round(ms * 1000.0 / reps, 3)
        del Wts

    log("secondary: matrix-instruction rates")
    out["mfma_rate_TFLOPs"] = mfma_rates(vla, torch, dev)

    log("secondary: wide GEMMs")
    for Mw, prefix in ((768, "wide"), (571, "wide_m571")):
        for name, (n, k) in ((prefix + "_up", (16384, 2048)), (prefix + "_down", (2048, 16384))):
            A = up_bits(synthetic.activations(Mw, k, 910 + n))
            Wf = synthetic.weights(n, k, 911 + n)
            q, s = quantize(Wf)
            Y = torch.empty(Mw * n, dtype=torch.int16, device=dev)
            wsb = vla.vla_gemm_workspace_bytes(Mw, n, k, 1)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            qa = torch.empty(Mw * k, dtype=torch.uint8, device=dev)
            sa = torch.empty(1, dtype=torch.float32, device=dev)
            wq_b = vla.vla_quantize_act_workspace_bytes(Mw, k)
            wq = torch.zeros(wq_b, dtype=torch.uint8, device=dev)
            flops = 2.0 * Mw * n * k

            def w8a16(i):
                vla.vla_gemm_fp8w(A, None, q, s, None, None, Y, ws, wsb, Mw, n, k)

            def actq(i):
                vla.vla_quantize_act(A, qa, sa, wq, wq_b, Mw, k)

            def fp8fp8(i):
                vla.vla_gemm_fp8w(qa, sa, q, s, None, None, Y, ws, wsb, Mw, n, k)

            for tag, fn, peak in (("w8a16", w8a16, BF16_PEAK_TFLOPS), ("fp8xfp8", fp8fp8, FP8_PEAK_TFLOPS)):
                if tag == "fp8xfp8":
                    actq(0)
                ms = time_graph(fn, 20)
                us = ms * 1000.0 / 20
                tf = flops / (us * 1e-6) / 1e12
                out[f"{name}_{tag}_us"] = round(us, 2)
                out[f"{name}_{tag}_TFLOPs"] = round(tf, 1)
                out[f"{name}_{tag}_frac"] = round(tf / peak, 4)
                rate = out["mfma_rate_TFLOPs"]["bf16_32x32x16" if tag == "w8a16" else "fp8_32x32x64"]["normal"]
                out[f"{name}_{tag}_frac_of_mfma_rate"] = round(tf / rate, 4)
            ms = time_graph(actq, 20)
            out[f"{name}_act_quant_us"] = round(ms * 1000.0 / 20, 2)
            if Mw == 768 and name.endswith("_up"):
                # one GPU's share when the encoder up-projection is split by
                # output columns over eight GPUs: N/8 channels, W8A16
                n8 = n // 8
                wss = torch.zeros(vla.vla_gemm_workspace_bytes(Mw, n8, k, 1), dtype=torch.uint8, device=dev)

                def w8a16_shard(i):
                    vla.vla_gemm_fp8w(A, None, q, s, None, None, Y, wss, wss.numel(), Mw, n8, k)
                ms = time_graph(w8a16_shard, 20)
                us = ms * 1000.0 / 20
                out[f"{name}_w8a16_shard8_us"] = round(us, 2)
                out[f"{name}_w8a16_shard8_frac"] = round(2.0 * Mw * n8 * k / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)

            def actq_static(i):   # frozen scale (the one just calibrated): one pass, no absmax
                vla.vla_quantize_act_static(A, sa, qa, Mw, k)
            ms = time_graph(actq_static, 20)
            out[f"{name}_act_quant_static_us"] = round(ms * 1000.0 / 20, 2)

            if Mw == 768:   # MXFP4 weights, bf16 activations (converted to bf16 in registers, bf16 MFMA)
                qm = torch.empty(vla.vla_packed_bytes(n, k, vla.VLA_WFMT_MXFP4), dtype=torch.uint8, device=dev)
                vla.vla_quantize_pack(up_bits(Wf), qm, None, n, k, vla.VLA_WFMT_MXFP4, vla.VLA_LAYOUT_MFMA)
                wsmb = vla.vla_gemm_workspace_bytes(Mw, n, k, vla.VLA_WFMT_MXFP4)
                wsm_w = torch.zeros(wsmb, dtype=torch.uint8, device=dev)

                def w4a16(i):
                    vla.vla_gemm_mxfp4w(A, qm, None, None, Y, wsm_w, wsmb, Mw, n, k)
                ms = time_graph(w4a16, 20)
                us = ms * 1000.0 / 20
                tf = flops / (us * 1e-6) / 1e12
                out[f"{name}_mxfp4_us"] = round(us, 2)
                out[f"{name}_mxfp4_TFLOPs"] = round(tf, 1)
                out[f"{name}_mxfp4_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
                del qm, wsm_w
            del Wf

    log("secondary: fused decoder boundary")
    bx, by, bg, bs = (up_bits(t) for t in synthetic.boundary_inputs(M, H, M))
    b_out = [torch.empty(M * H, dtype=torch.int16, device=dev) for _ in range(3)]

    def boundary(i):
        vla.vla_gate_residual_ada_norm(bx, by, bg, bs, True, 1e-6, b_out[0], b_out[1], b_out[2], M, H)
    ms = time_graph(boundary, 256)
    b_us = ms * 1000.0 / 256
    b_bytes = (3 + 3) * M * H * 2 + 3 * M * H * 2          # reads x, out, gate, style; writes r, h, next gate
    out["boundary_us"] = round(b_us, 3)
    out["boundary_GBps"] = round(b_bytes / (b_us * 1e-6) / 1e9, 1)

    log("secondary: 18-layer chain")
    L = 18
    gate, up, down = synthetic.chain_weights(L, H, I)
    wgu, sgu, wd, sd = [], [], [], []
    for l in range(L):
        a, b = quantize(np.concatenate([gate[l], up[l]]))
        c, d = quantize(down[l])
        wgu.append(a); sgu.append(b); wd.append(c); sd.append(d)
    xin = up_bits(synthetic.activations(M, H, synthetic.IDS["chain.x"]))
    xout = torch.empty(M * H, dtype=torch.int16, device=dev)
    sb = vla.vla_mlp_chain_scratch_bytes(M, H, I)
    scratch = torch.zeros(sb + 256, dtype=torch.uint8, device=dev)
    cs = torch.cuda.Stream()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    rf_sink = torch.zeros(64, dtype=torch.int32, device=dev)
    chain_bytes = L * (2 * I * H + 8 * I + H * I + 4 * H) + 2 * 2 * M * H
    # the fused single launch (256-byte aligned scratch), then the graph of
    # 2L GEMM launches that a scratch without that alignment falls back to
    for prefix, sc in (("chain", scratch[:sb]), ("chain_graph_path", scratch[16:16 + sb])):
        torch.cuda.synchronize()
        h = vla.vla_mlp_chain_create(wgu, sgu, wd, sd, xin, xout, sc, sb, L, M, H, I, cs)
        try:
            for _ in range(5):
                vla.vla_mlp_chain_replay(h, cs)
            cs.synchronize()
            warm, cold, rcold = [], [], []
            for i in range(60):
                if i % 3 == 1:
                    flush.fill_(i & 0xFF)            # evict the 216 MiB of weights from cache
                    torch.cuda.synchronize()
                elif i % 3 == 2:                     # the same, reading: no dirty lines left behind
                    vla.vla_probe_stream_read(flush, flush.numel(), rf_sink, 2048, cs)
                    cs.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(cs)
                vla.vla_mlp_chain_replay(h, cs)
                e1.record(cs)
                cs.synchronize()
                (warm, cold, rcold)[i % 3].append(e0.elapsed_time(e1) * 1000.0)
            out[f"{prefix}_us_per_replay_warm"] = round(float(np.median(warm)), 2)
            out[f"{prefix}_us_per_replay_cold"] = round(float(np.median(cold)), 2)
            out[f"{prefix}_us_per_replay_after_read_flush"] = round(float(np.median(rcold)), 2)
            out[f"{prefix}_cold_GBps"] = round(chain_bytes / (np.median(cold) * 1e-6) / 1e9, 1)
        finally:
            vla.vla_mlp_chain_destroy(h)
    out["chain_fused_launch"] = bool(vla.vla_mlp_chain_fused_supported(M, H, I, L))

    log("secondary: 18-layer decoder-block chain (MLP + fused boundary per layer)")
    d_out = [torch.empty(M * H, dtype=torch.int16, device=dev) for _ in range(3)]
    dsb = vla.vla_decoder_chain_scratch_bytes(M, H, I)
    dscratch = torch.zeros(dsb + 256, dtype=torch.uint8, device=dev)
    styled = {}
    for per_row in (False, True):
        dx, dh, dg, dstyle = synthetic.decoder_chain_inputs(L, M, H, M if per_row else 1)
        styled[per_row] = ([up_bits(a) for a in (dx, dh, dg)], [up_bits(s_) for s_ in dstyle])
    # one style row for all rows (one sample's conditioning): the single
    # launch (256-byte aligned scratch) and the graph of three launches per
    # layer that an unaligned scratch falls back to; a style row per row
    # (the graph of launches at this M)
    for prefix, sc, per_row in (("decoder_chain", dscratch[:dsb], False),
                                ("decoder_chain_graph_path", dscratch[16:16 + dsb], False),
                                ("decoder_chain_style_per_row", dscratch[:dsb], True)):
        d_in, d_style = styled[per_row]
        out[f"{prefix}_fused_launch"] = bool(vla.vla_decoder_chain_fused_supported(M, H, I, L, per_row)) and \
            sc.data_ptr() % 256 == 0
        torch.cuda.synchronize()
        h = vla.vla_decoder_chain_create(wgu, sgu, wd, sd, d_style, per_row, 1e-6, *d_in, *d_out, sc, dsb,
                                         L, M, H, I, cs)
        try:
            for _ in range(5):
                vla.vla_mlp_chain_replay(h, cs)
            cs.synchronize()
            warm, cold, rcold = [], [], []
            for i in range(60):
                if i % 3 == 1:
                    flush.fill_(i & 0xFF)
                    torch.cuda.synchronize()
                elif i % 3 == 2:
                    vla.vla_probe_stream_read(flush, flush.numel(), rf_sink, 2048, cs)
                    cs.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(cs)
                vla.vla_mlp_chain_replay(h, cs)
                e1.record(cs)
                cs.synchronize()
                (warm, cold, rcold)[i % 3].append(e0.elapsed_time(e1) * 1000.0)
            out[f"{prefix}_us_per_replay_warm"] = round(float(np.median(warm)), 2)
            out[f"{prefix}_us_per_replay_cold"] = round(float(np.median(cold)), 2)
            out[f"{prefix}_us_per_replay_after_read_flush"] = round(float(np.median(rcold)), 2)
        finally:
            vla.vla_mlp_chain_destroy(h)
    del flush

    log("secondary: dialect conversion 16384 x 2048")
    N, K = 16384, 2048
    W = up_bits(synthetic.weights(N, K, synthetic.IDS["dialect.W"]))
    qf = torch.empty(N * K, dtype=torch.uint8, device=dev)
    sf = torch.empty(N, dtype=torch.float32, device=dev)
    qo = torch.empty(N * K, dtype=torch.uint8, device=dev)
    so = torch.empty(N, dtype=torch.float32, device=dev)
    qp = torch.empty(N * K, dtype=torch.uint8, device=dev)
    t_q = time_graph(lambda i: vla.vla_quantize_pack(W, qf, sf, N, K, vla.VLA_WFMT_E4M3_FNUZ,
                                                     vla.VLA_LAYOUT_ROWMAJOR), 10) * 100.0
    t_r = time_graph(lambda i: vla.vla_reencode_fnuz_to_ocp(qf, sf, qo, so, N, K, vla.VLA_LAYOUT_ROWMAJOR), 10) * 100.0
    t_p = time_graph(lambda i: vla.vla_pack_fp8(qo, qp, N, K), 10) * 100.0
    out["dialect_quantize_fnuz_us"] = round(t_q, 2)
    out["dialect_quantize_GBps"] = round((4 * N * K + N * K + 4 * N) / (t_q * 1e-6) / 1e9, 1)
    out["dialect_reencode_us"] = round(t_r, 2)
    out["dialect_reencode_GBps"] = round((2 * N * K + 8 * N) / (t_r * 1e-6) / 1e9, 1)
    out["dialect_pack_us"] = round(t_p, 2)
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "skinny_fp8_m50_pmc_traffic.txt")
# every source the skinny kernel is compiled from: a change to any of them
# invalidates the committed counter figures
KERNEL_SOURCES = [os.path.join(ROOT, "bf16_gemm_vla_amd", "csrc", f)
                  for f in ("gemm.hip", "gemm_common.h", "vla_device.h")]


def kernel_sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


MFMA_FORMS = (   # name, VLA_MFMA_* value, m*n*k, operand type, published dense peak (TFLOP/s)
    ("bf16_32x32x16", 0, 32 * 32 * 16, "bf16", BF16_PEAK_TFLOPS),
    ("bf16_16x16x32", 1, 16 * 16 * 32, "bf16", BF16_PEAK_TFLOPS),
    ("fp8_32x32x64", 2, 32 * 32 * 64, "fp8", FP8_PEAK_TFLOPS),
    ("fp8_16x16x128", 3, 16 * 16 * 128, "fp8", FP8_PEAK_TFLOPS),
)


def mfma_operands(torch, dev, kind, dtype, seed=1234):
    """The rate probe's 64 KiB operand buffer: zeros, or values distributed like
    the wide GEMMs' operands (bf16: N(0, 1) activations; FP8: E4M3 codes of
    absmax-scaled N(0, 1) data, i.e. N(0, ~100) clamped to the E4M3 range)."""
    if kind == "zero":
        return torch.zeros(256 * 64, dtype=torch.int32, device=dev)
    g = torch.Generator().manual_seed(seed)
    if dtype == "bf16":
        v = torch.randn(256 * 128, generator=g).to(torch.bfloat16).view(torch.int16)
    else:
        v = (torch.randn(256 * 256, generator=g) * 100.0).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return v.view(torch.int32).to(dev)


def mfma_iters(mnk, blocks=512):
    return max(1, int(2e12 / (blocks * 4 * 4 * 2.0 * mnk)))   # ~2 TFLOP per launch


def mfma_trace_summary(trace_dir, blocks=512, reps=5):
    """Matrix-core rates from a rocprofv3 kernel trace of --mfma-only: the
    probe's dispatches in launch order, one untimed and `reps` timed per
    (form, operands), in the order mfma_rates issues them."""
    import csv
    import glob
    import statistics

    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        sys.exit(f"no *kernel_trace.csv under {trace_dir}")
    rows = [r for r in csv.DictReader(open(files[0])) if "mfma_rate_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = reps + 1
    if len(rows) != per * 2 * len(MFMA_FORMS):
        sys.exit(f"expected {per * 2 * len(MFMA_FORMS)} probe dispatches, found {len(rows)}")
    print(f"# rocprofv3 kernel trace: {os.path.relpath(files[0], trace_dir)}; {blocks} workgroups x 256 threads")
    i = 0
    for name, form, mnk, dt, peak in MFMA_FORMS:
        iters = mfma_iters(mnk, blocks)
        flops = blocks * 4 * 4 * 2.0 * mnk * iters
        for kind in ("zero", "normal"):
            d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows[i + 1:i + per]]
            i += per
            med = statistics.median(d)
            tf = flops / (med * 1e-9) / 1e12
            print(f"{name} {kind:6s}: iters {iters}, median kernel {med / 1e3:.1f} us over {len(d)} launches "
                  f"-> {tf:.1f} TFLOP/s = {tf / peak:.4f} of the published {peak:.0f}")


def mfma_rates(vla, torch, dev, blocks=512, reps=5):
    """Issue rate of each matrix instruction the GEMMs use, on zero operands
    and on operands like the GEMMs' own (vla_probe_mfma_rate; two workgroups of
    four waves per CU, two waves per SIMD as in the wide kernel), with the
    shader clock each loop ran at.  The rate depends on the data through the
    clock (busy non-zero operands draw more power and the chip clocks down),
    so the wide GEMMs' fractions are read against the 'normal' figures as
    well as against the published peaks."""
    import numpy as np

    res = {}
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    for name, form, mnk, dt, peak in MFMA_FORMS:
        per_iter = blocks * 4 * 4 * 2.0 * mnk           # workgroups x waves x chains x flops
        iters = mfma_iters(mnk, blocks)
        r = {"iters": iters, "blocks": blocks}
        for kind in ("zero", "normal"):
            ops = mfma_operands(torch, dev, kind, dt)
            vla.vla_probe_mfma_rate(form, ops, iters, out, blocks)
            ts, ghz = [], []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                vla.vla_probe_mfma_rate(form, ops, iters, out, blocks, clocks=clocks)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
                c = clocks.cpu().numpy().astype(np.float64)
                ghz.append(float(np.median(c[0::2] / (c[1::2] * 10.0))))
            ms = sorted(ts)[len(ts) // 2]
            tf = per_iter * iters / (ms * 1e-3) / 1e12
            clk = sorted(ghz)[len(ghz) // 2]
            r[kind] = round(tf, 1)
            r[kind + "_frac_of_peak"] = round(tf / peak, 4)
            # the shader clock the loop ran at (the published peak assumes
            # 2.4 GHz) and the rate per clock against the peak's
            r[kind + "_clock_GHz"] = round(clk, 3)
            r[kind + "_frac_of_peak_per_clock"] = round(tf / (peak * clk / 2.4), 4)
        res[name] = r
    return res


def measured_traffic():
    """HBM bytes per launch of the skinny kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs, scaled by a plain copy's counters; None if
    the summary is missing or the kernel source changed since it was taken."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256") != kernel_sources_sha256():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def host_facts():
    """CPU model, the NUMA node of the GPU (from its PCI device) and of this
    process's CPUs, as far as the host exposes them."""
    facts = {"cpu_model": None, "nproc": os.cpu_count(), "gpu_numa_node": None, "process_numa_nodes": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                facts["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        import torch

        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
        facts["gpu_pci"] = bus
        facts["gpu_numa_node"] = int(open(f"/sys/bus/pci/devices/{bus}/numa_node").read())
    except Exception:       # properties or sysfs not available: leave it unknown
        pass
    try:
        cpus = os.sched_getaffinity(0)
        facts["process_cpus"] = len(cpus)
        nodes = set()
        base = "/sys/devices/system/node"
        for d in os.listdir(base):
            if d.startswith("node"):
                lst = open(os.path.join(base, d, "cpulist")).read().strip()
                ids = set()
                for part in lst.split(","):
                    if "-" in part:
                        a, b = part.split("-")
                        ids.update(range(int(a), int(b) + 1))
                    elif part:
                        ids.add(int(part))
                if ids & cpus:
                    nodes.add(int(d[4:]))
        facts["process_numa_nodes"] = sorted(nodes)
    except (OSError, ValueError):
        pass
    return facts


def cpu_baseline(np, synthetic, W_up, W_dn):
    """The oracle (unchanged) on the same workload: dequantize + fp64 GEMM per
    call, alternating up and down.  Three timed runs of about 4 s on all the
    threads OpenMP uses (median reported), then one pair of calls on a single
    thread."""
    import ctypes

    import oracle

    A_up = oracle.bf16_value(synthetic.activations(M, H, synthetic.IDS["skinny.up.A"]))
    A_dn = oracle.bf16_value(synthetic.activations(M, I, synthetic.IDS["skinny.down.A"]))
    q_up, s_up = oracle.quantize_rows(W_up, oracle.OCP)
    q_dn, s_dn = oracle.quantize_rows(W_dn, oracle.OCP)
    work = ((A_up, q_up, s_up), (A_dn, q_dn, s_dn))

    def run(seconds, max_pairs):
        calls = 0
        t0 = time.perf_counter()
        while True:
            for A, q, s in work:
                oracle.gemm(A, oracle.dequant_rows(q, s))
                calls += 1
            el = time.perf_counter() - t0
            if el >= seconds or calls >= 2 * max_pairs:
                return el * 1e6 / calls, calls, el

    gomp = None
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        threads = int(gomp.omp_get_max_threads())
    except OSError:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    runs = [run(4.0, 1000) for _ in range(3)]
    us = sorted(r[0] for r in runs)
    one = None
    if gomp is not None:
        gomp.omp_set_num_threads(1)
        one = run(0.0, 1)[0]               # one up + one down call
        gomp.omp_set_num_threads(threads)
    facts = host_facts()
    total_s = sum(r[2] for r in runs)
    return {"value": round(us[1], 1), "unit": "µs/call", "cores": threads, "kind": "oracle",
            "sample": (f"3 runs of {runs[0][1]}-{runs[-1][1]} calls (alternating up/down, M=50) of dequantize + "
                       f"fp64 GEMM, {total_s:.1f} s; value = median run, {threads} OpenMP threads"),
            "runs_us": [round(v, 1) for v in us],
            "one_thread_us": None if one is None else round(one, 1),
            "cpu_model": facts["cpu_model"], "nproc": facts["nproc"],
            "gpu_numa_node": facts["gpu_numa_node"], "process_numa_nodes": facts["process_numa_nodes"]}


def trace_summary(trace_dir, bench_json=None):
    """Summarize a rocprofv3 kernel trace of this script: the dispatches
    between the first two one-workgroup marker kernels (the headline's timed
    replay), per kernel name, against the bench's HIP-event figure."""
    import csv
    import glob
    import statistics

    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        sys.exit(f"no *kernel_trace.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))

    def col(row, *names):
        for n in names:
            if n in row:
                return row[n]
        raise KeyError(names)
    recs = []
    for r in rows:
        grid = int(col(r, "Grid_Size_X", "Grid_Size")) * int(r.get("Grid_Size_Y", 1)) * int(r.get("Grid_Size_Z", 1))
        wg = int(col(r, "Workgroup_Size_X", "Workgroup_Size")) * int(r.get("Workgroup_Size_Y", 1)) * \
            int(r.get("Workgroup_Size_Z", 1))
        recs.append((int(col(r, "Start_Timestamp")), int(col(r, "End_Timestamp")), col(r, "Kernel_Name"), grid, wg))
    recs.sort()
    marks = [i for i, r in enumerate(recs) if "stream_read" in r[2] and r[3] == r[4]]
    if len(marks) < 2:
        sys.exit("marker dispatches not found")
    timed = recs[marks[0] + 1:marks[1]]
    by = {}
    for st, en, name, grid, wg in timed:
        by.setdefault((name, grid // wg, wg), []).append(en - st)
    span_ns = timed[-1][1] - timed[0][0]
    gaps = [timed[i + 1][0] - timed[i][1] for i in range(len(timed) - 1)]
    print(f"# rocprofv3 kernel trace: {os.path.relpath(files[0], trace_dir)}")
    print(f"dispatches in the timed replay: {len(timed)}")
    total = 0.0
    for (name, groups, wg), d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        short = short_kernel_name(name)
        total += sum(d)
        print(f"kernel: {short}")
        print(f"  workgroups {groups} x {wg} threads; dispatches {len(d)}; mean {statistics.mean(d) / 1e3:.3f} us; "
              f"median {statistics.median(d) / 1e3:.3f} us; min {min(d) / 1e3:.3f} us; max {max(d) / 1e3:.3f} us")
    print(f"mean kernel duration over all timed dispatches: {total / len(timed) / 1e3:.3f} us")
    print(f"first start to last end: {span_ns / 1e3:.3f} us = {span_ns / 1e3 / len(timed):.3f} us per dispatch")
    print(f"gap between consecutive dispatches: mean {statistics.mean(gaps) / 1e3:.3f} us, "
          f"median {statistics.median(gaps) / 1e3:.3f} us")
    if bench_json:
        line = [l for l in open(bench_json) if l.startswith("{")][-1]
        b = json.loads(line)
        ev_us = b["ms_per_step"] * 1000.0 / 2
        print(f"bench (same run, HIP events around the same replay): {b['ms_per_step'] * 1000:.3f} us per step "
              f"= {ev_us:.3f} us per call")
        print(f"mean kernel duration x 2 = {2 * total / len(timed) / 1e3:.3f} us <= ms_per_step "
              f"{b['ms_per_step'] * 1000:.3f} us: {2 * total / len(timed) / 1e3 <= b['ms_per_step'] * 1000}")
        nbytes = b["roofline"].get("bytes_per_launch", (alg_bytes_fp8w(*UP) + alg_bytes_fp8w(*DOWN)) // 2)
        print(f"algorithmic bytes per launch {nbytes}: over the kernel's own duration "
              f"{nbytes / (total / len(timed)):.1f} GB/s ({nbytes / (total / len(timed)) / HBM_PEAK_GBS:.4f} of "
              f"8 TB/s); over the event time per call {nbytes / (ev_us * 1e3):.1f} GB/s "
              f"({nbytes / (ev_us * 1e3) / HBM_PEAK_GBS:.4f}, the bench's roofline.frac {b['roofline']['frac']})")


def short_kernel_name(name):
    """A kernel name without its trailing parameter list (names may contain
    parentheses of their own, as in '(anonymous namespace)')."""
    name = name.strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    return name[:160]


def all_kernels_summary(trace_dir):
    """One row per launch configuration of a rocprofv3 kernel trace (kernel,
    workgroup size, grid in workgroups, LDS bytes, VGPR+AGPR, scratch bytes):
    launches and their mean / median / min duration, by total time."""
    import csv
    import glob
    import statistics

    files = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        sys.exit(f"no *kernel_trace.csv under {trace_dir}")
    by = {}
    for r in csv.DictReader(open(files[0])):
        wg = [int(r.get(f"Workgroup_Size_{a}", 1) or 1) for a in "XYZ"]
        grid = tuple(int(r.get(f"Grid_Size_{a}", 1) or 1) // max(1, w) for a, w in zip("XYZ", wg))
        key = (short_kernel_name(r["Kernel_Name"]), wg[0] * wg[1] * wg[2], grid, int(r.get("LDS_Block_Size", 0) or 0),
               int(r.get("VGPR_Count", 0) or 0), int(r.get("Accum_VGPR_Count", 0) or 0),
               int(r.get("Scratch_Size", 0) or 0))
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# rocprofv3 kernel trace: {os.path.relpath(files[0], trace_dir)}")
    print(f"  {'kernel':34s} | {'wg':>5s} | {'grid':15s} | {'lds':>6s} | {'vgpr':7s} | {'scr':>3s} | {'calls':>5s} | "
          f"{'mean us':>9s} | {'median us':>9s} | {'min us':>8s}")
    for key, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        name, wg, grid, lds, vg, ag, scr = key
        print(f"  {name[:34]:34s} | {wg:5d} | {str(grid):15s} | {lds:6d} | {f'{vg}+{ag}':7s} | {scr:3d} | {len(d):5d} | "
              f"{statistics.mean(d):9.2f} | {statistics.median(d):9.2f} | {min(d):8.2f}")


def pmc_table(dirs, kernel):
    """Mean value per dispatch of every counter in rocprofv3 --pmc runs (one
    directory per run), per launch shape (grid, workgroup, LDS, VGPRs: this
    also separates template instances that share a truncated name) of the
    kernels whose name contains `kernel`; _sum counters also per compute
    unit (256)."""
    import csv
    import glob
    import statistics

    vals = {}
    for d in dirs:
        files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not files:
            sys.exit(f"no *counter_collection.csv under {d}")
        for r in csv.DictReader(open(files[0])):
            if kernel not in r["Kernel_Name"]:
                continue
            grid = int(float(r.get("Grid_Size", 0) or 0))
            wg = int(float(r.get("Workgroup_Size", 1) or 1))
            key = (short_kernel_name(r["Kernel_Name"]), grid // wg if grid >= wg > 0 else grid, wg,
                   int(float(r.get("LDS_Block_Size", 0) or 0)), int(float(r.get("VGPR_Count", 0) or 0)))
            vals.setdefault(key, {}).setdefault(r["Counter_Name"].strip(), []).append(float(r["Counter_Value"]))
    for (name, groups, wg, lds, vgpr), cs in sorted(vals.items()):
        print(f"{name}: {groups} workgroups x {wg} threads, LDS {lds} B, {vgpr} VGPRs")
        for c in sorted(cs):
            v = statistics.mean(cs[c])
            per_cu = f"  ({v / 256:.1f} per CU)" if c.endswith("_sum") else ""
            print(f"  {c:34s} {v:14.1f}{per_cu}   [{len(cs[c])} dispatches]")
        if "TCP_TCC_READ_REQ_sum" in cs:
            req = statistics.mean(cs["TCP_TCC_READ_REQ_sum"])
            print(f"  L1 -> L2 read requests x 128 B: {req * 128 / 2**20:.1f} MiB per dispatch")
            if "TCP_TCC_READ_REQ_LATENCY_sum" in cs and req > 0:
                print(f"  mean L1 -> L2 read latency: {statistics.mean(cs['TCP_TCC_READ_REQ_LATENCY_sum']) / req:.0f} cycles")


def pmc_summary(dirs, kernel, algorithmic=None):
    """Summarize rocprofv3 --pmc runs of FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch): dirs = [fetch, write, copy fetch, copy write]; the last two are
    runs of --calibrate-copy, whose 256 MiB copy scales each counter to bytes.
    Dispatches whose kernel name contains `kernel` are averaged per (name,
    launch shape) and over all of them."""
    import csv
    import glob
    import statistics

    def load_runs(d, counter):
        files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not files:
            sys.exit(f"no *counter_collection.csv under {d}")
        out = []
        for r in csv.DictReader(open(files[0])):
            if r.get("Counter_Name", "").strip() != counter:
                continue
            grid = int(float(r.get("Grid_Size", 0) or 0))
            wg = int(float(r.get("Workgroup_Size", 1) or 1))
            out.append((int(r.get("Dispatch_Id", len(out))), r["Kernel_Name"], grid, wg, float(r["Counter_Value"])))
        return out

    fetch, write, cfetch, cwrite = (load_runs(d, c) for d, c in zip(
        dirs, ("FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE")))
    copy_kib = (256 << 20) / 1024.0

    def copy_scale(rows):
        v = [x[4] for x in rows if "copy" in x[1].lower()]
        if not v:
            sys.exit("no copy dispatches in the calibration run")
        return copy_kib / statistics.mean(v), statistics.mean(v)

    fs, fraw = copy_scale(cfetch)
    ws, wraw = copy_scale(cwrite)
    print(f"# calibration: a plain 256 MiB device copy reads FETCH_SIZE {fraw:.1f} KiB and WRITE_SIZE "
          f"{wraw:.1f} KiB per dispatch against {copy_kib:.0f} KiB moved each way: fetch scale {fs:.4f}, "
          f"write scale {ws:.4f}")

    def group(rows):
        g = {}
        for _, name, grid, wg, v in rows:
            if kernel in name:
                groups = grid // wg if grid >= wg and wg > 0 else grid
                g.setdefault((short_kernel_name(name), groups, wg), []).append(v)
        return g
    gf, gw = group(fetch), group(write)
    allf = [v for vs in gf.values() for v in vs]
    allw = [v for vs in gw.values() for v in vs]
    if not allf or not allw:
        sys.exit(f"no dispatches of {kernel}")
    for key in sorted(gf):
        f, w = statistics.mean(gf[key]), statistics.mean(gw.get(key, [float("nan")]))
        print(f"kernel: {key[0]}")
        print(f"  workgroups {key[1]} x {key[2]} threads; dispatches {len(gf[key])} / {len(gw.get(key, []))}; "
              f"FETCH_SIZE {f:.1f} KiB, WRITE_SIZE {w:.1f} KiB per dispatch; HBM bytes per launch "
              f"{f * 1024 * fs + w * 1024 * ws:.0f} (read {f * 1024 * fs:.0f}, write {w * 1024 * ws:.0f})")
    f, w = statistics.mean(allf), statistics.mean(allw)
    hbm = f * 1024 * fs + w * 1024 * ws
    print(f"{kernel}_dispatches_fetch: {len(allf)}")
    print(f"{kernel}_dispatches_write: {len(allw)}")
    print(f"fetch_kib_per_launch_raw: {f:.1f}")
    print(f"write_kib_per_launch_raw: {w:.1f}")
    print(f"fetch_scale: {fs:.4f}")
    print(f"write_scale: {ws:.4f}")
    print(f"hbm_bytes_per_launch: {hbm:.0f}")
    if algorithmic:
        print(f"algorithmic_bytes_per_launch: {algorithmic}")
        print(f"traffic_over_algorithmic: {hbm / algorithmic:.3f}")
    if kernel == "skinny_gemm_kernel":
        print(f"kernel_source_sha256: {kernel_sources_sha256()}")


if __name__ == "__main__":
    main()
