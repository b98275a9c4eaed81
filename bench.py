#!/usr/bin/env python3
"""Throughput of the W8A8 INT8 projection path on one MI355X.

A step is one pass of the whole hot path over the workload's synthetic
input, all of it in the library's HIP kernels on one stream:
  per block: quantize X (shared by Q, K, V) -> Q, K and V (one GEMM over
  the concatenated weights where O reads X, else three); quantize X -> O GEMM;
  quantize X -> FC1 GEMM; SiLU+quantize of FC1's output -> FC2 GEMM;
  between blocks (the sweep): power-of-two renormalization of FC2's output
  feeds the next block, fused with that block's quantization for Q, K, V.
Inputs and weights are resident in HBM before timing starts.  Reported:
  value      = sum of 2*M*N*K over the step's GEMMs / step time (TOPS),
               quantization and glue time included, from K steps timed
               without per-call events;
  roofline   = the INT8 GEMM alone (one w8a8_gemm call: the main kernel
               launch and, where the last wave of tiles is short, its split-K
               tail launch and reduction): algorithmic ops / average call
               time (HIP events around every call, on the launch stream,
               over K more steps), against the dense INT8 MFMA peak of
               5.0 POP/s;
  cpu_baseline = the CPU oracle timed on a bounded row sample;
  bf16_baseline (context) = torch's BF16 linear (hipBLASLt) on the same
               shapes;
  int8_library_baseline (context) = hipBLASLt's INT8 GEMM (torch._int_mm)
               on the same codes and weights: INT32 accumulators only, no
               scales, bias or BF16 rounding;
  mfma_ceiling (context, MFMA-bound workloads) = the rate of the GEMM's
               MFMA sequence with register operands only (no memory
               traffic), on the workload's own codes and weights: the
               board's power limit makes the matrix cores' sustained rate
               depend on the data.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 0-6]
       [--qkv auto|fused|separate]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
GRAPH_GEMM_REPEATS = 20   # GEMM calls per timing graph (single projection)
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA, published
METRIC = ("W8A8 projection TOPS and % INT8 MFMA peak at DiT shapes "
          "(M~19k, K=5376)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=4, choices=range(7))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--no-int8-library-baseline", action="store_true")
    ap.add_argument("--no-mfma-ceiling", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--check-rows", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--qkv", choices=("auto", "fused", "separate"),
                    default="auto",
                    help="fused: Q, K and V as one GEMM over the "
                         "concatenated weights [3N, K] (the same outputs, "
                         "bit for bit); separate: three GEMMs; auto (the "
                         "default): fused wherever the attention output "
                         "projection reads the block input X")
    ap.add_argument("--fused-qkv", dest="qkv", action="store_const",
                    const="fused", help="the same as --qkv fused")
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="replay the step (and the GEMM-only timing) as a "
                         "HIP graph; auto = on for the single-projection "
                         "workload, whose kernels are shorter than the "
                         "Python launch path")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 4 times (a kernel "
                         "of known HBM traffic for scaling rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


def traffic_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "copies": 4}), flush=True)


def projections_of(wl, D):
    return list(wl.projs)


def main():
    args = parse()
    if args.traffic_calibration:
        traffic_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the projection would shard by tokens with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    from w8a8_int8_gemm_amd import binding as B
    from w8a8_int8_gemm_amd import block as BL
    from w8a8_int8_gemm_amd import datagen as D

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = D.WORKLOADS[args.config]
    M = wl.M
    single = len(wl.projs) == 1
    if args.qkv == "fused" and (single or wl.o_input != "x"):
        raise SystemExit("--qkv fused needs a block workload whose attention "
                         "output projection reads X")
    fused = (not single and wl.o_input == "x" and
             args.qkv in ("auto", "fused"))
    threads = min(16, os.cpu_count() or 8)

    # ---- oracle sample (row chain), computed while weights are on the host
    orc = None
    rows = None
    if not args.no_check or not args.no_cpu_baseline:
        import oracle
        orc = oracle.default()
    x0_host = D.activations(M, D.HIDDEN, wl.seed)
    if not args.no_check:
        rows = D.row_sample(M, max(args.check_rows - 2, 0), wl.seed)
        chk_x = x0_host[rows]
        chk_out = None

    # ---- weights: generated per block on the host, resident on the GPU
    t0 = time.time()
    blocks = []
    for b in range(wl.blocks):
        params = D.block_params(wl, b, threads=threads)
        dblk = {p.name: BL.upload_proj(p, params[p.name], dev)
                for p in wl.projs}
        if fused:
            dblk = BL.fuse_qkv(dblk)
        blocks.append(dblk)
        if rows is not None:
            if single:
                p = wl.projs[0]
                pp = params[p.name]
                chk_out = {p.name: orc.linear(chk_x, pp.w, pp.sw, pp.bias)}
            else:
                chk_out = oracle_block_rows(orc, wl, params, chk_x)
                if b + 1 < wl.blocks:
                    chk_x = orc.pow2_renorm(chk_out["fc2"])
        del params
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: M={M}, {wl.blocks} block(s), weights resident "
        f"({sum(p.w.numel() for blk in blocks for p in blk.values())/1e9:.2f}"
        f" GB INT8) in {time.time() - t0:.1f}s")

    x0 = BL.to_device_bf16(x0_host, dev)
    xbuf = [torch.empty_like(x0), torch.empty_like(x0)]
    runner = (BL.BlockRunner(M, dev, fused_qkv=fused,
                             projs=wl.projs, mlp=wl.mlp, o_input=wl.o_input)
              if not single else None)
    if single:
        p0 = wl.projs[0]
        qbuf = torch.empty((M, p0.K), dtype=torch.int8, device=dev)
        sbuf = torch.empty((M,), dtype=torch.float32, device=dev)
        ybuf = torch.empty((M, p0.N), dtype=torch.bfloat16, device=dev)
        wsb = torch.empty((max(B.gemm_workspace_bytes(M, p0.N, p0.K), 256),),
                          dtype=torch.uint8, device=dev)

    ops_per_step = 0
    for blk in blocks:
        for p in blk.values():
            ops_per_step += 2 * M * p.N * p.K

    gemm_events = []

    def on_gemm(name, phase):
        if gemm_events is None:
            return
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        gemm_events.append(ev)

    def step(record):
        nonlocal gemm_events
        gemm_events = [] if record else None
        if single:
            p = blocks[0][wl.projs[0].name]
            B.quantize_act(x0, out=(qbuf, sbuf))
            on_gemm(p.name, "begin")
            B.gemm(qbuf, sbuf, p.w, p.sw, p.bias, out=ybuf, workspace=wsb)
            on_gemm(p.name, "end")
            return {p.name: ybuf}
        x = x0
        out = None
        for b, blk in enumerate(blocks):
            out = runner.run(x, blk, on_gemm=on_gemm, x_quantized=b > 0)
            if b + 1 < len(blocks):
                # the next block's input and its quantization for Q, K, V
                nxt = xbuf[b % 2]
                B.pow2_renorm_quantize(out["fc2"], out=(nxt, runner.xq[0],
                                                        runner.xs[0]))
                x = nxt
        return out

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # Graph mode: the K timed steps captured once, back to back, and
    # replayed as one graph (a launch per replay, not per kernel); the
    # library records kernel launches only (no memsets, no host waits).
    use_graph = args.graph == "on" or (args.graph == "auto" and single)
    if use_graph:
        steps_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(steps_graph):
            for _ in range(args.steps):
                graph_out = step(False)
        steps_graph.replay()  # warm replay, outside the timed region
        torch.cuda.synchronize()

    # Timed region 1: the steps alone (value).  An event recorded between
    # two kernels costs a few microseconds of queue time, so the per-call
    # GEMM events are kept out of this region.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if use_graph:
        steps_graph.replay()
        out = graph_out
    else:
        for _ in range(args.steps):
            out = step(False)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / max(args.steps, 1)
    tops = ops_per_step / (ms_per_step * 1e-3) / 1e12

    # Timed region 2 (roofline: average duration of one GEMM call).  Eager:
    # the same steps with HIP events around every GEMM call on the launch
    # stream.  Graph mode: a graph of the step's GEMM calls alone (on the
    # buffers the step filled), replayed between two events.
    gemm_ms = 0.0
    launches = 0
    torch.cuda.synchronize()
    if use_graph:
        calls = []

        def gemm_call(name, phase):
            if phase == "begin":
                calls.append(name)
        gemm_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gemm_graph):
            if single:
                p = blocks[0][wl.projs[0].name]
                for _ in range(GRAPH_GEMM_REPEATS):
                    B.gemm(qbuf, sbuf, p.w, p.sw, p.bias, out=ybuf,
                           workspace=wsb)
                    calls.append(p.name)
            else:
                for blk in blocks:
                    runner.run_gemms(blk, on_gemm=gemm_call)
        gemm_graph.replay()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(args.steps):
            gemm_graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        gemm_ms = ev0.elapsed_time(ev1)
        launches = len(calls) * args.steps
        gemm_ops = args.steps * sum(
            2 * M * blocks[0][n].N * blocks[0][n].K for n in calls)
    else:
        all_gemm = []
        for _ in range(args.steps):
            out = step(True)
            all_gemm.append(gemm_events)
        torch.cuda.synchronize()
        for evs in all_gemm:
            for i in range(0, len(evs), 2):
                gemm_ms += evs[i].elapsed_time(evs[i + 1])
                launches += 1
        gemm_ops = ops_per_step * args.steps
    gemm_tops = gemm_ops / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    avg_launch_us = gemm_ms * 1e3 / max(launches, 1)
    log(f"[bench] step {ms_per_step:.3f} ms -> {tops:.1f} TOPS "
        f"({100 * tops / INT8_PEAK_TOPS:.1f}% of INT8 peak); GEMM kernel "
        f"{gemm_tops:.1f} TOPS, avg launch {avg_launch_us:.1f} us")

    # ---- sampled-row oracle check of the last step (outside timing)
    check = None
    if rows is not None:
        ri = torch.from_numpy(rows).to(dev)
        ok = True
        for n, ref in chk_out.items():
            got = BL.from_device_bf16(out[n][ri])
            ok &= bool(np.array_equal(got, ref))
        check = {"rows": rows.tolist(), "bit_exact": ok}
        log(f"[bench] oracle check of rows {rows.tolist()} through "
            f"{wl.blocks} block(s): {'bit-exact' if ok else 'MISMATCH'}")

    # ---- BF16 baseline (hipBLASLt through torch), same shapes, one block
    bf16 = None
    if not args.no_bf16_baseline:
        bf16 = bf16_baseline(torch, D, BL, wl, x0, blocks[0], dev,
                             args.warmup, max(args.steps, 3))
        log(f"[bench] BF16 baseline: {bf16['tflops']:.1f} TFLOPS")

    # ---- INT8 library baseline (hipBLASLt through torch), same codes
    int8lib = None
    if not args.no_int8_library_baseline:
        if single:
            codes = {wl.projs[0].name: qbuf}
        else:
            codes = runner.codes_by_projection(blocks[0])
        int8lib = int8_library_baseline(torch, blocks[0], codes, M,
                                        args.warmup, max(args.steps, 3),
                                        gemm_tops)
        log(f"[bench] INT8 library baseline: {int8lib['tops']:.1f} TOPS "
            f"(w8a8_gemm {int8lib['w8a8_gemm_speedup']:.3f}x)")

    # ---- register-only MFMA rate on the same codes and weights
    ceiling = None
    roofline = roofline_entry(blocks[0], M, gemm_tops, avg_launch_us,
                              launches, use_graph,
                              traffic_entry(wl, fused))
    if not args.no_mfma_ceiling and roofline["bound"] == "mfma":
        if single:
            xc, wc = qbuf, blocks[0][wl.projs[0].name].w
        else:
            xc, wc = runner.xq[0], blocks[0]["qkv" if fused else "q"].w
        ceiling = mfma_ceiling(torch, xc, wc, gemm_tops)
        log(f"[bench] MFMA ceiling on the workload's codes: "
            f"{ceiling['tops']:.1f} TOPS; the GEMM reaches "
            f"{ceiling['gemm_frac_of_ceiling']:.3f} of it")

    # ---- CPU baseline: the oracle on a bounded row sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(orc, D, wl, x0_host, args.cpu_seconds, threads)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} TOPS on {cpu['cores']} "
            f"threads ({cpu['sample']})")

    gemm_shapes = sorted({(M, p.N, p.K) for p in blocks[0].values()})
    result = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wl.name + ("+fused_qkv" if fused else ""),
            "tokens": M,
            "blocks": wl.blocks,
            "linears": wl.blocks * len(wl.projs),
            "gemm_shapes_MNK": [list(s) for s in gemm_shapes],
            "parallelism": "single_gpu",
        },
        "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "bf16_baseline": bf16,
        "int8_library_baseline": int8lib,
        "mfma_ceiling": ceiling,
        "oracle_check": check,
    }
    print(json.dumps(result), flush=True)


def gemm_call_bytes(M, N, K):
    """Algorithmic HBM bytes of one w8a8_gemm call: A and W read once, the
    BF16 output written once, the FP32 scales and the BF16 bias read."""
    return M * K + N * K + 2 * M * N + 4 * M + 4 * N + 2 * N


def roofline_entry(blk, M, gemm_tops, avg_launch_us, launches, graph,
                   traffic):
    """Roofline of the dominant kernel (one w8a8_gemm call).  A workload
    whose calls average fewer ops per byte than the chip's ridge point
    (5.0 POPS / 8 TB/s = 625) is bounded by HBM and reported in GB/s."""
    shapes = [(p.N, p.K) for p in blk.values()]
    ops = sum(2 * M * N * K for N, K in shapes) / len(shapes)
    nbytes = sum(gemm_call_bytes(M, N, K) for N, K in shapes) / len(shapes)
    hbm = ops / nbytes < INT8_PEAK_TOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm:
        achieved = nbytes / (avg_launch_us * 1e-6) / 1e9 if avg_launch_us \
            else None
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = gemm_tops, INT8_PEAK_TOPS, "TOP/s"
    return {
        "kernel": ("w8a8_gemm call: gemm_kernel (INT8 MFMA + fused "
                   "epilogue), plus its split-K tail launch and tail "
                   "reduction where the last wave of tiles is short, or "
                   "its split-K reduction for skinny M"),
        "bound": "hbm" if hbm else "mfma",
        "achieved": round(achieved, 2) if achieved else None,
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4) if achieved else None,
        "algorithmic_bytes_per_call": int(nbytes),
        "algorithmic_ops_per_call": int(ops),
        "avg_launch_us": round(avg_launch_us, 2),
        "launches_timed": launches,
        "timing": ("graph of back-to-back calls between two HIP events"
                   if graph else "HIP events around every call"),
        "traffic": traffic,
    }


def gemm_mix(wl, fused_qkv):
    """(tokens, sorted (N, K) of a block's GEMM calls) for a workload, with
    Q, K and V as one [3N, K] call when fused."""
    shapes = [(p.N, p.K) for p in wl.projs
              if not (fused_qkv and p.name in ("q", "k", "v"))]
    if fused_qkv:
        q = next(p for p in wl.projs if p.name == "q")
        shapes.append((3 * q.N, q.K))
    return wl.M, sorted(shapes)


def traffic_entry(wl, fused_qkv):
    """Measured HBM bytes per GEMM launch from committed rocprofv3 counter
    summaries: each record is valid only for the call mix it was taken on
    (a block's GEMM calls at its token count and shapes) and only while the
    kernel source is unchanged."""
    f = ROOT / "profiles" / "gemm_traffic.json"
    if not f.exists():
        return None
    tokens, shapes = gemm_mix(wl, fused_qkv)
    for rec in json.loads(f.read_text()).get("records", []):
        if rec.get("kernel_sha256") != kernel_source_sha256():
            continue
        mix = rec.get("workload", {})
        if (mix.get("tokens") == tokens and
                sorted(map(tuple, mix.get("shapes_NK", []))) == shapes):
            return rec.get("traffic")
    return None


def kernel_source_sha256():
    """Hash of the GEMM kernel's sources (the kernel file and the shared
    device header); traffic figures are only valid for this exact code."""
    import hashlib
    csrc = ROOT / "w8a8_int8_gemm_amd" / "csrc"
    h = hashlib.sha256()
    for name in ("gemm.hip", "internal.h"):
        h.update((csrc / name).read_bytes())
    return h.hexdigest()


def bf16_baseline(torch, D, BL, wl, x0, blk, dev, warmup, reps):
    """torch.nn.functional.linear in BF16 (hipBLASLt) on the same shapes:
    weights are the dequantized INT8 weights rounded to BF16."""
    F = torch.nn.functional
    ws = {n: (p.w.to(torch.float32) * p.sw[:, None]).to(torch.bfloat16)
          for n, p in blk.items()}
    bs = {n: p.bias for n, p in blk.items()}
    ops = sum(2 * x0.shape[0] * p.N * p.K for p in blk.values())

    def run():
        if len(blk) == 1:
            n = next(iter(blk))
            return F.linear(x0, ws[n], bs[n])
        out = {}
        for n in blk:
            if n not in ("o", "fc1", "fc2"):
                out[n] = F.linear(x0, ws[n], bs[n])
        F.linear(out["v"] if wl.o_input == "v" else x0, ws["o"], bs["o"])
        h = F.linear(x0, ws["fc1"], bs["fc1"])
        if wl.mlp == "swiglu":
            g, u = h.chunk(2, dim=-1)
            h = F.silu(g) * u
        else:
            h = F.silu(h)
        return F.linear(h, ws["fc2"], bs["fc2"])

    for _ in range(warmup + 1):
        run()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    tflops = ops / (ms * 1e-3) / 1e12
    del ws
    return {"tflops": round(tflops, 2), "ms_per_block": round(ms, 4),
            "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
            "what": "torch.nn.functional.linear, BF16 weights, one block "
                    "(SiLU or SwiGLU included)"}


def int8_library_baseline(torch, blk, codes, M, warmup, reps, gemm_tops):
    """hipBLASLt's INT8 GEMM through torch._int_mm on one block's shapes,
    fed the codes the step's own quantizations produced and the resident
    INT8 weights (consumed transposed, as stored).  It returns INT32
    accumulators only: no per-token / per-channel scales, no bias and no
    BF16 rounding, and it writes 4 bytes per output against w8a8_gemm's 2."""
    calls = [(codes[n], p.w) for n, p in blk.items()]
    ops = sum(2 * M * p.N * p.K for p in blk.values())

    def run():
        for q, w in calls:
            torch._int_mm(q, w.t())

    for _ in range(warmup + 1):
        run()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    tops = ops / (ms * 1e-3) / 1e12
    return {"tops": round(tops, 2), "ms_per_block": round(ms, 4),
            "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
            "w8a8_gemm_speedup": round(gemm_tops / tops, 3)
            if gemm_tops else None,
            "what": "torch._int_mm (hipBLASLt), INT32 output only, same "
                    "codes and weights, one block's GEMMs"}


def mfma_ceiling(torch, x_codes, w_codes, gemm_tops, blocks=1024,
                 iters=2048, reps=20):
    """Sustained rate of the GEMM's v_mfma_i32_32x32x32_i8 sequence with
    register operands only, fed fragments of the given token codes and
    weights (libw8a8_ceiling.so, a measurement kernel outside the library):
    8 waves per CU, 1024 work groups per launch, `reps` launches back to
    back after a warm one, so the board reaches its power-limited clock."""
    import ctypes
    from w8a8_int8_gemm_amd import build as LB
    if not LB.CEILING_LIB.exists():
        raise RuntimeError(f"{LB.CEILING_LIB} is not built "
                           "(run __graft_entry__.build())")
    lib = ctypes.CDLL(str(LB.CEILING_LIB))
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w8a8_ceiling_run.restype = ci
    lib.w8a8_ceiling_run.argtypes = [vp, i64, vp, i64, i64, ci, ci, vp, vp]
    lib.w8a8_ceiling_ops.restype = ctypes.c_double
    lib.w8a8_ceiling_ops.argtypes = [ci, ci]
    lib.w8a8_ceiling_out_len.restype = i64
    lib.w8a8_ceiling_out_len.argtypes = [ci]
    if x_codes.shape[1] != w_codes.shape[1]:
        raise ValueError("codes and weights disagree on K")
    out = torch.empty((lib.w8a8_ceiling_out_len(blocks),), dtype=torch.int32,
                      device=x_codes.device)
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        rc = lib.w8a8_ceiling_run(
            x_codes.data_ptr(), x_codes.shape[0], w_codes.data_ptr(),
            w_codes.shape[0], x_codes.shape[1], blocks, iters,
            out.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"w8a8_ceiling_run failed ({rc})")

    run()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        run()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    tops = lib.w8a8_ceiling_ops(blocks, iters) / (ms * 1e-3) / 1e12
    return {"tops": round(tops, 2),
            "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
            "gemm_frac_of_ceiling": round(gemm_tops / tops, 4)
            if gemm_tops else None,
            "what": "v_mfma_i32_32x32x32_i8, the GEMM's MFMA order, register "
                    "operands only (4 k-steps of 2 token and 4 weight "
                    "fragments per wave, 8 waves per CU), on the workload's "
                    "token codes and weights"}


def oracle_block_rows(orc, wl, params, x_rows):
    """One block's BF16 outputs for some token rows through the oracle
    (rows are independent through every step of the block)."""
    out = {}
    for n in ("q", "k", "v", "fc1"):
        pp = params[n]
        out[n] = orc.linear(x_rows, pp.w, pp.sw, pp.bias)
    pp = params["o"]
    out["o"] = orc.linear(out["v"] if wl.o_input == "v" else x_rows, pp.w,
                          pp.sw, pp.bias)
    h = (orc.swiglu_bf16(out["fc1"]) if wl.mlp == "swiglu"
         else orc.silu_bf16(out["fc1"]))
    pp = params["fc2"]
    out["fc2"] = orc.linear(h, pp.w, pp.sw, pp.bias)
    return out


def cpu_baseline(orc, D, wl, x0_host, seconds, threads):
    """The oracle as it stands, timed on the first rows of block 0's
    projections; rows are doubled until the run lasts `seconds`/4, then one
    final timed run with about `seconds` of work."""
    params = D.block_params(wl, 0, threads=threads)

    def run(R):
        x = x0_host[:R]
        t = time.perf_counter()
        if len(wl.projs) == 1:
            p = wl.projs[0]
            pp = params[p.name]
            orc.linear(x, pp.w, pp.sw, pp.bias)
        else:
            oracle_block_rows(orc, wl, params, x)
        macs = sum(R * p.N * p.K for p in wl.projs)
        return time.perf_counter() - t, macs

    R = 4
    dt, _ = run(R)
    while dt < seconds / 4 and R < wl.M:
        R = min(R * 2, wl.M)
        dt, _ = run(R)
    R = int(min(wl.M, max(1, R * seconds / max(dt, 1e-3))))
    dt, macs = run(R)
    return {"value": round(2 * macs / dt / 1e12, 6), "unit": "TOPS",
            "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"first {R} of {wl.M} token rows through block 0's "
                      f"{len(wl.projs)} projection(s), {dt:.1f} s"}


if __name__ == "__main__":
    main()
