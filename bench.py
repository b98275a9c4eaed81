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
               between two events (per-step events give the median and the
               sample standard deviation);
  roofline   = the INT8 GEMM alone (one w8a8_gemm call: the main kernel
               launch and, where the last wave of tiles is short, its split-K
               tail launch and reduction): algorithmic ops / average call
               time (HIP events around every call, on the launch stream,
               over K more steps), against the dense INT8 MFMA peak of
               5.0 POP/s (GB/s against 8 TB/s below the ridge point);
  phases     = the same per-call timing for every kind of call: each
               projection's GEMM, the quantizers (GB/s of their algorithmic
               bytes) and the renormalization between blocks;
  oracle_check = sampled token rows of every projection of every block,
               the block inputs and their INT8 codes and scales, compared
               bit for bit with the CPU oracle run through the whole chain;
  per_config = the other single-GPU workloads (one projection at 64 tokens,
               one block at 4096, 19077 and 37503 tokens) measured the same
               way in the same run, with their own oracle checks;
  cpu_baseline = the CPU oracle timed on a bounded row sample, with the
               host's CPU model, affinity and thread count;
  power_clock (context) = board power and the 8 XCD clocks sampled with
               amd-smi while the timed steps ran;
  measured_peaks (context) = a device copy's HBM rate and torch's BF16 GEMM
               rate on this machine, beside the published peaks;
  bf16_baseline (context) = torch's BF16 linear (hipBLASLt) on the same
               shapes, and how many times faster the W8A8 step runs a
               block (w8a8_speedup);
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
import math
import os
import shutil
import signal
import statistics
import subprocess
import sys
import tempfile
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
GRAPH_GEMM_REPEATS = 20   # GEMM calls per timing graph (single projection)
GRAPH_STAT_REPLAYS = 7    # replays of the step graph for the median / std
# Untimed work queued ahead of each eager timed region: the host then
# enqueues the region's launches and events before the GPU reaches them, so
# no event pair spans a pause of the host (short calls of the one-block
# workloads otherwise let the GPU drain between launches).  By default that
# work is steps of the workload itself, about LEAD_MS of them: after the
# host synchronization before a region the board's clock takes a few
# hundred milliseconds of load to settle, so the region starts at the clock
# the workload runs at when it runs continuously.  With --lead spin it is a
# spin kernel of QUEUE_AHEAD_CYCLES GPU clock cycles instead.  Timed graph
# replays are led the same way by about LEAD_MS of replays of the graph.
QUEUE_AHEAD_CYCLES = 100_000_000
LEAD_MS = 500.0
LEAD_MAX_STEPS = 1000
LEAD_MAX_REPLAYS = 1024
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA, published
PER_CONFIGS = (0, 1, 2, 3)  # single-GPU workloads reported beside the main
METRIC = ("W8A8 projection TOPS and % INT8 MFMA peak at DiT shapes "
          "(M~19k, K=5376)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
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
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the other single-GPU workloads")
    ap.add_argument("--per-config-steps", type=int, default=7,
                    help="timed steps of each per-config workload (after 2 "
                         "warm-up steps)")
    ap.add_argument("--no-power-clock", action="store_true",
                    help="do not sample board power and clocks")
    ap.add_argument("--no-measured-peaks", action="store_true")
    ap.add_argument("--check-rows", type=int, default=16)
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
    ap.add_argument("--lead-ms", type=float, default=LEAD_MS,
                    help="milliseconds of untimed steps (or graph replays) "
                         "queued ahead of each timed region")
    ap.add_argument("--lead", choices=("steps", "spin"), default="steps",
                    help="untimed work queued right before each eager timed "
                         "region while the host enqueues it: steps of the "
                         "workload (default) or a bounded spin kernel")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="only copy a 1 GiB device buffer 4 times (a kernel "
                         "of known HBM traffic for scaling rocprofv3's "
                         "FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args(argv)


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


# ---------------------------------------------------------------------------
# board power and clocks (context)
# ---------------------------------------------------------------------------

class PowerClockSampler:
    """Board power and the XCD clocks read with `amd-smi metric` (read-only
    queries, about four per second) by a child shell started before this
    process initializes the GPU; readings are stamped with the host clock
    so the timed regions can pick theirs.  Absent amd-smi: no readings."""

    def __init__(self):
        self.proc = None
        self.path = None
        exe = shutil.which("amd-smi")
        if exe is None:
            return
        fd, self.path = tempfile.mkstemp(prefix="w8a8_smi_", suffix=".txt")
        script = (f'while true; do echo "T $(date +%s.%N)"; '
                  f'"{exe}" metric -p -c --json 2>/dev/null; sleep 0.2; done')
        self.proc = subprocess.Popen(["bash", "-c", script], stdout=fd,
                                     stderr=subprocess.DEVNULL,
                                     start_new_session=True)
        os.close(fd)

    def stop(self):
        if self.proc is not None and self.proc.poll() is None:
            try:
                os.killpg(self.proc.pid, signal.SIGTERM)
            except ProcessLookupError:
                pass
            self.proc.wait(timeout=10)

    def samples(self):
        """[(host time, socket power W or None, [gfx clocks MHz])]."""
        if self.path is None or not os.path.exists(self.path):
            return []
        out = []
        blocks, cur = [], None
        for line in Path(self.path).read_text(errors="replace").splitlines():
            head = line.split()
            if len(head) == 2 and head[0] == "T":
                try:
                    cur = [float(head[1]), []]
                    blocks.append(cur)
                    continue
                except ValueError:
                    pass
            if cur is not None:
                cur[1].append(line)
        for t, lines in blocks:
            body = "\n".join(lines)
            try:
                j = json.loads(body[body.index("{"):])
            except (ValueError, json.JSONDecodeError):
                continue
            gpus = j.get("gpu_data", j if isinstance(j, list) else [])
            if not gpus:
                continue
            g = gpus[0]
            p = g.get("power", {}).get("socket_power", {})
            power = p.get("value") if isinstance(p, dict) else None
            clocks = [v["clk"]["value"] for k, v in g.get("clock", {}).items()
                      if k.startswith("gfx_") and isinstance(v, dict) and
                      isinstance(v.get("clk"), dict) and
                      isinstance(v["clk"].get("value"), (int, float))]
            out.append((t, power if isinstance(power, (int, float)) else None,
                        clocks))
        return out

    def window(self, t0, t1):
        """Readings taken between host times t0 and t1, summarized."""
        s = [x for x in self.samples() if t0 <= x[0] <= t1]
        if not s:
            return None
        pw = [x[1] for x in s if x[1] is not None]
        ck = [c for x in s for c in x[2]]
        return {"samples": len(s),
                "socket_power_w": [min(pw), max(pw)] if pw else None,
                "gfx_clock_mhz_min_mean_max":
                    [min(ck), round(sum(ck) / len(ck)), max(ck)]
                    if ck else None,
                "xcds": max(len(x[2]) for x in s),
                "source": "amd-smi metric -p -c, about 4 readings per "
                          "second"}

    def close(self):
        self.stop()
        if self.path and os.path.exists(self.path):
            os.unlink(self.path)


# ---------------------------------------------------------------------------
# host facts for the CPU baseline
# ---------------------------------------------------------------------------

def cpu_model() -> str | None:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# one workload: weights, oracle references, steps, timings, checks
# ---------------------------------------------------------------------------

def quant_bytes(kind, M, K):
    """Algorithmic HBM bytes of one quantization call over M rows whose
    codes are K wide: BF16 read (twice as wide for the gated form), INT8
    codes and FP32 scales written; the renormalization also writes the
    renormalized BF16 row."""
    read = 2 * M * K * (2 if kind == "swiglu_quant" else 1)
    write = M * K + 4 * M + (2 * M * K if kind == "renorm_quant" else 0)
    return read + write


class Workload:
    """One workload of datagen.WORKLOADS, resident on the device."""

    def __init__(self, wl, dev, qkv, check_rows, orc, threads, graph,
                 lead="steps", lead_ms=LEAD_MS):
        import torch
        from w8a8_int8_gemm_amd import binding as B
        from w8a8_int8_gemm_amd import block as BL
        from w8a8_int8_gemm_amd import datagen as D
        self.torch, self.B, self.BL, self.D = torch, B, BL, D
        self.wl, self.dev, self.orc = wl, dev, orc
        M = self.M = wl.M
        self.single = len(wl.projs) == 1
        if qkv == "fused" and (self.single or wl.o_input != "x"):
            raise SystemExit("--qkv fused needs a block workload whose "
                             "attention output projection reads X")
        self.fused = (not self.single and wl.o_input == "x" and
                      qkv in ("auto", "fused"))
        self.graph = graph == "on" or (graph == "auto" and self.single)
        x0_host = D.activations(M, D.HIDDEN, wl.seed)
        self.x0_host = x0_host
        self.rows = (D.row_sample(M, max(check_rows - 2, 0), wl.seed)
                     if check_rows > 0 else None)
        self.refs = []
        chk_x = x0_host[self.rows] if self.rows is not None else None
        t0 = time.time()
        self.blocks = []
        for b in range(wl.blocks):
            params = D.block_params(wl, b, threads=threads)
            dblk = {p.name: BL.upload_proj(p, params[p.name], dev)
                    for p in wl.projs}
            if self.fused:
                dblk = BL.fuse_qkv(dblk)
            self.blocks.append(dblk)
            if chk_x is not None:
                ref = oracle_rows(orc, wl, params, chk_x)
                self.refs.append(ref)
                if b + 1 < wl.blocks:
                    chk_x = orc.pow2_renorm(ref["fc2"])
            del params
        torch.cuda.synchronize()
        self.weight_bytes = sum(p.w.numel() for blk in self.blocks
                                for p in blk.values())
        log(f"[bench] {wl.name}: M={M}, {wl.blocks} block(s), weights "
            f"resident ({self.weight_bytes / 1e9:.2f} GB INT8) in "
            f"{time.time() - t0:.1f}s")
        self.x0 = BL.to_device_bf16(x0_host, dev)
        self.xbuf = [torch.empty_like(self.x0), torch.empty_like(self.x0)]
        if self.single:
            p0 = wl.projs[0]
            e = lambda *s, dt: torch.empty(s, dtype=dt, device=dev)
            self.qbuf = e(M, p0.K, dt=torch.int8)
            self.sbuf = e(M, dt=torch.float32)
            self.ybuf = e(M, p0.N, dt=torch.bfloat16)
            self.wsb = e(max(B.gemm_workspace_bytes(M, p0.N, p0.K), 256),
                         dt=torch.uint8)
            self.runner = None
        else:
            self.runner = BL.BlockRunner(M, dev, fused_qkv=self.fused,
                                         projs=wl.projs, mlp=wl.mlp,
                                         o_input=wl.o_input)
        self.ops_per_step = sum(2 * M * p.N * p.K for blk in self.blocks
                                for p in blk.values())
        self.lead, self.lead_steps, self.lead_ms = lead, 1, lead_ms

    # -- one step ------------------------------------------------------------
    def step(self, on_gemm=None, on_quant=None, on_block=None):
        B = self.B
        if self.single:
            p = self.blocks[0][self.wl.projs[0].name]
            if on_quant:
                on_quant("quant", "begin")
            B.quantize_act(self.x0, out=(self.qbuf, self.sbuf))
            if on_quant:
                on_quant("quant", "end")
            if on_gemm:
                on_gemm(p.name, "begin")
            B.gemm(self.qbuf, self.sbuf, p.w, p.sw, p.bias, out=self.ybuf,
                   workspace=self.wsb)
            if on_gemm:
                on_gemm(p.name, "end")
            out = {p.name: self.ybuf}
            if on_block:
                on_block(0, self.x0, out)
            return out
        x = self.x0
        out = None
        r = self.runner
        for b, blk in enumerate(self.blocks):
            out = r.run(x, blk, on_gemm=on_gemm, on_quant=on_quant,
                        x_quantized=b > 0)
            if on_block:
                on_block(b, x, out)
            if b + 1 < len(self.blocks):
                # the next block's input and its quantization for Q, K, V
                nxt = self.xbuf[b % 2]
                if on_quant:
                    on_quant("renorm_quant", "begin")
                B.pow2_renorm_quantize(out["fc2"], out=(nxt, r.xq[0],
                                                        r.xs[0]))
                if on_quant:
                    on_quant("renorm_quant", "end")
                x = nxt
        return out

    def warmup(self, n):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        # steps run ahead of each eager timed region (untimed), enough to
        # keep the GPU busy for LEAD_MS while the host enqueues the region
        est = e0.elapsed_time(e1) / max(n, 1)
        self.lead_steps = max(1, min(LEAD_MAX_STEPS,
                                     math.ceil(self.lead_ms / max(est, 1e-3))))

    def graph_lead_in(self, g):
        """Replays of graph ``g`` queued right before its timed replays
        (about LEAD_MS of them, at least one), from a timed warm replay."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        n = max(1, min(LEAD_MAX_REPLAYS, math.ceil(
            self.lead_ms / max(e0.elapsed_time(e1), 1e-3))))
        for _ in range(n):
            g.replay()

    def lead_in(self):
        """Untimed work queued right before an eager timed region, so that
        the host enqueues the region's launches and events while the GPU is
        busy: real steps (the GPU stays at its working clock), or with
        ``--lead spin`` a bounded spin kernel."""
        if self.lead == "spin":
            self.torch.cuda._sleep(QUEUE_AHEAD_CYCLES)
            return
        for _ in range(self.lead_steps):
            self.step()

    # -- timed region 1: whole steps -------------------------------------------
    def time_steps(self, K):
        """(ms per step over exactly K steps between two events, per-step
        ms list for the median and standard deviation)."""
        torch = self.torch
        Ev = lambda: torch.cuda.Event(enable_timing=True)
        if self.graph:
            # the K steps captured once and replayed as one graph (a launch
            # per replay, not per kernel); the library enqueues kernel
            # launches only, so replays reproduce the eager results
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(K):
                    self.step()
            g.replay()
            torch.cuda.synchronize()
            evs = [Ev() for _ in range(GRAPH_STAT_REPLAYS + 1)]
            self.graph_lead_in(g)
            evs[0].record()
            for i in range(GRAPH_STAT_REPLAYS):
                g.replay()
                evs[i + 1].record()
            torch.cuda.synchronize()
            per = [evs[i].elapsed_time(evs[i + 1]) / K
                   for i in range(GRAPH_STAT_REPLAYS)]
            self._graph_keep = g
            return per[0], per, "graph of the K steps, replayed " \
                f"{GRAPH_STAT_REPLAYS} times (value from the first)"
        evs = [Ev() for _ in range(K + 1)]
        torch.cuda.synchronize()
        self.lead_in()
        evs[0].record()
        for i in range(K):
            self.step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
        return evs[0].elapsed_time(evs[K]) / K, per, \
            "K eager steps between two events (an event after each step)"

    # -- timed region 2: every call ----------------------------------------------
    def time_calls(self, K):
        """Average duration of every kind of call: {kind: (calls, total
        ms, [(M, N, K) or (M, K) per call])}."""
        torch = self.torch
        B = self.B
        stats = {}

        def add(kind, ms, shape):
            c = stats.setdefault(kind, [0, 0.0, []])
            c[0] += 1
            c[1] += ms
            c[2].append(shape)

        if self.graph:
            # graphs of back-to-back calls of one kind, between two events
            p = self.blocks[0][self.wl.projs[0].name]
            for kind, call, shape in (
                    ("gemm:" + p.name,
                     lambda: B.gemm(self.qbuf, self.sbuf, p.w, p.sw, p.bias,
                                    out=self.ybuf, workspace=self.wsb),
                     (self.M, p.N, p.K)),
                    ("quant", lambda: B.quantize_act(
                        self.x0, out=(self.qbuf, self.sbuf)),
                     (self.M, p.K))):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(GRAPH_GEMM_REPEATS):
                        call()
                g.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                self.graph_lead_in(g)
                e0.record()
                for _ in range(K):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / (K * GRAPH_GEMM_REPEATS)
                for _ in range(K * GRAPH_GEMM_REPEATS):
                    add(kind, ms, shape)
            return stats, "graphs of back-to-back calls between two events"
        pending = []
        open_ev = {}
        calls = [0]

        def count(name, phase):
            calls[0] += phase == "begin"
        self.step(on_gemm=count, on_quant=count)
        pool = [torch.cuda.Event(enable_timing=True)
                for _ in range(2 * K * calls[0])]

        def hook(kind):
            def f(name, phase):
                ev = pool.pop()
                ev.record()
                key = f"{kind}:{name}" if kind == "gemm" else name
                if phase == "begin":
                    open_ev[key] = ev
                else:
                    pending.append((key, open_ev.pop(key), ev))
            return f

        torch.cuda.synchronize()
        self.lead_in()
        for _ in range(K):
            self.step(on_gemm=hook("gemm"), on_quant=hook("quant"))
        torch.cuda.synchronize()
        shapes = self.call_shapes()
        for key, a, b in pending:
            add(key, a.elapsed_time(b), shapes[key])
        return stats, "HIP events around every call, on the launch stream"

    def call_shapes(self):
        blk = self.blocks[0]
        out = {f"gemm:{n}": (self.M, p.N, p.K) for n, p in blk.items()}
        H = self.D.HIDDEN
        out["quant"] = (self.M, H)
        out["quant_o"] = (self.M, blk["o"].K) if "o" in blk else None
        out["renorm_quant"] = (self.M, H)
        out["silu_quant"] = (self.M, blk["fc2"].K) if "fc2" in blk else None
        out["swiglu_quant"] = out["silu_quant"]
        return out

    # -- sampled-row oracle check ------------------------------------------------
    def check(self):
        """Rows of every block's input, of its INT8 codes and scales and of
        every projection's output (and FC2's input codes) from one more
        step, against the oracle run through the whole chain."""
        if self.rows is None:
            return None
        torch = self.torch
        ri = torch.from_numpy(self.rows).to(self.dev)
        got = []
        r = self.runner

        def on_block(b, x, out):
            g = {"x": self.BL.from_device_bf16(x[ri])}
            for n, t in out.items():
                if n != "qkv":
                    g[n] = self.BL.from_device_bf16(t[ri])
            if self.single:
                g["xq"] = self.qbuf[ri].cpu().numpy()
                g["xs"] = self.sbuf[ri].cpu().numpy()
            else:
                g["xq"] = r.xq[0][ri].cpu().numpy()
                g["xs"] = r.xs[0][ri].cpu().numpy()
                g["hq"] = r.hq[ri].cpu().numpy()
                g["hs"] = r.hs[ri].cpu().numpy()
                if r.oq is not None:
                    g["oq"] = r.oq[ri].cpu().numpy()
                    g["os"] = r.xs[1][ri].cpu().numpy()
            got.append(g)

        self.step(on_block=on_block)
        torch.cuda.synchronize()
        values = mismatched = 0
        keys = set()
        first_bad = None
        for b, (g, ref) in enumerate(zip(got, self.refs)):
            for k, want in ref.items():
                have = g[k]
                if want.dtype == np.float32:
                    have, want = have.view(np.uint32), want.view(np.uint32)
                bad = int(np.count_nonzero(have != want))
                values += want.size
                mismatched += bad
                keys.add(k)
                if bad and first_bad is None:
                    first_bad = f"block {b} {k}"
        return {"rows": self.rows.tolist(), "blocks": len(got),
                "compared": sorted(keys), "values_compared": values,
                "mismatches": mismatched, "first_mismatch": first_bad,
                "bit_exact": mismatched == 0 and values > 0}

    def gemm_ops_per_call(self):
        blk = self.blocks[0]
        return sum(2 * self.M * p.N * p.K for p in blk.values()) / len(blk)


def oracle_rows(orc, wl, params, x_rows):
    """The oracle on some token rows of a workload's block input: the
    input itself, its codes and scales, every projection's BF16 output and
    FC2's input codes and scales (rows are independent through every step
    of a block)."""
    out = {"x": x_rows}
    out["xq"], out["xs"] = orc.quantize_act(x_rows)
    if len(wl.projs) == 1:
        p = wl.projs[0]
        pp = params[p.name]
        out[p.name] = orc.linear(x_rows, pp.w, pp.sw, pp.bias)
        return out
    for n in ("q", "k", "v", "fc1"):
        pp = params[n]
        out[n] = orc.linear(x_rows, pp.w, pp.sw, pp.bias)
    o_in = out["v"] if wl.o_input == "v" else x_rows
    if wl.o_input == "v":
        out["oq"], out["os"] = orc.quantize_act(o_in)
    pp = params["o"]
    out["o"] = orc.linear(o_in, pp.w, pp.sw, pp.bias)
    h = (orc.swiglu_bf16(out["fc1"]) if wl.mlp == "swiglu"
         else orc.silu_bf16(out["fc1"]))
    out["hq"], out["hs"] = orc.quantize_act(h)
    pp = params["fc2"]
    out["fc2"] = orc.linear(h, pp.w, pp.sw, pp.bias)
    return out


def step_stats(per):
    return {"median": round(statistics.median(per), 4),
            "std": round(statistics.stdev(per), 4) if len(per) > 1 else 0.0,
            "min": round(min(per), 4), "max": round(max(per), 4),
            "n": len(per)}


def phases_entry(stats, M):
    """Per kind of call: calls timed, average us, and the rate of its
    algorithmic work (TOP/s for GEMMs, GB/s for the quantizers)."""
    out = {}
    for kind, (n, ms, shapes) in sorted(stats.items()):
        us = ms * 1e3 / n
        e = {"calls": n, "avg_us": round(us, 2)}
        if kind.startswith("gemm:"):
            Mm, N, K = shapes[0]
            e["tops"] = round(2 * Mm * N * K / (us * 1e-6) / 1e12, 2)
            e["gbs"] = round(gemm_call_bytes(Mm, N, K) / (us * 1e-6) / 1e9, 1)
        elif shapes[0] is not None:
            Mm, K = shapes[0]
            nb = quant_bytes(kind, Mm, K)
            e["bytes_per_call"] = nb
            e["gbs"] = round(nb / (us * 1e-6) / 1e9, 1)
            e["frac_hbm_peak"] = round(e["gbs"] / HBM_PEAK_GBS, 4)
        out[kind] = e
    return out


def gemm_totals(stats):
    n = sum(v[0] for k, v in stats.items() if k.startswith("gemm:"))
    ms = sum(v[1] for k, v in stats.items() if k.startswith("gemm:"))
    ops = sum(2 * s[0] * s[1] * s[2] for k, v in stats.items()
              if k.startswith("gemm:") for s in v[2])
    return n, ms, ops


def measure(w, steps, warmup, sampler=None):
    """Timed regions of one workload; returns the pieces of its entry."""
    w.warmup(warmup)
    t0 = time.time()
    ms_step, per, how = w.time_steps(steps)
    t1 = time.time()
    stats, call_how = w.time_calls(steps)
    t2 = time.time()
    tops = w.ops_per_step / (ms_step * 1e-3) / 1e12
    n, gms, gops = gemm_totals(stats)
    gemm_tops = gops / (gms * 1e-3) / 1e12
    return {"tops": tops, "ms_step": ms_step, "per": per, "how": how,
            "stats": stats, "call_how": call_how, "gemm_calls": n,
            "gemm_ms": gms, "gemm_tops": gemm_tops,
            "avg_launch_us": gms * 1e3 / max(n, 1),
            "window_steps": (t0, t1), "window_calls": (t1, t2)}


def run(args, sampler):
    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    from w8a8_int8_gemm_amd import datagen as D

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    threads = min(16, len(os.sched_getaffinity(0)))
    orc = None
    if not args.no_check or not args.no_cpu_baseline or not args.no_per_config:
        import oracle
        orc = oracle.default()
    wl = D.WORKLOADS[args.config]
    w = Workload(wl, dev, args.qkv, 0 if args.no_check else args.check_rows,
                 orc, threads, args.graph, args.lead, args.lead_ms)
    m = measure(w, args.steps, args.warmup, sampler)
    log(f"[bench] step {m['ms_step']:.3f} ms -> {m['tops']:.1f} TOPS "
        f"({100 * m['tops'] / INT8_PEAK_TOPS:.1f}% of INT8 peak); GEMM calls "
        f"{m['gemm_tops']:.1f} TOP/s, avg call {m['avg_launch_us']:.1f} us")
    power = None
    if sampler is not None:
        time.sleep(0.5)  # the last reading of the window
        power = {"timed_steps": sampler.window(*m["window_steps"]),
                 "timed_calls": sampler.window(*m["window_calls"])}
        sampler.stop()
    check = None if args.no_check else w.check()
    if check is not None:
        log(f"[bench] oracle check: {check['values_compared']} values of "
            f"{len(check['rows'])} rows x {check['blocks']} block(s) "
            f"({', '.join(check['compared'])}): "
            f"{'bit-exact' if check['bit_exact'] else 'MISMATCH'}")

    # ---- baselines on the same shapes (context)
    bf16 = None
    if not args.no_bf16_baseline:
        bf16 = bf16_baseline(torch, wl, w.x0, w.blocks[0],
                             args.warmup, max(args.steps, 3))
        bf16["w8a8_speedup"] = speedup_vs_bf16(bf16, m["ms_step"], wl.blocks)
        log(f"[bench] BF16 baseline: {bf16['tflops']:.1f} TFLOPS (the W8A8 "
            f"step {bf16['w8a8_speedup']:.3f}x faster per block)")
    int8lib = None
    if not args.no_int8_library_baseline:
        codes = ({wl.projs[0].name: w.qbuf} if w.single
                 else w.runner.codes_by_projection(w.blocks[0]))
        int8lib = int8_library_baseline(torch, w.blocks[0], codes, w.M,
                                        args.warmup, max(args.steps, 3),
                                        m["gemm_tops"])
        log(f"[bench] INT8 library baseline: {int8lib['tops']:.1f} TOPS "
            f"(w8a8_gemm {int8lib['w8a8_gemm_speedup']:.3f}x)")
    roofline = roofline_entry(w.blocks[0], w.M, m["gemm_tops"],
                              m["avg_launch_us"], m["gemm_calls"], w.graph,
                              traffic_entry(wl, w.fused))
    ceiling = None
    if not args.no_mfma_ceiling and roofline["bound"] == "mfma":
        if w.single:
            xc, wc = w.qbuf, w.blocks[0][wl.projs[0].name].w
        else:
            xc, wc = w.runner.xq[0], w.blocks[0]["qkv" if w.fused else "q"].w
        ceiling = mfma_ceiling(torch, xc, wc, m["gemm_tops"])
        log(f"[bench] MFMA ceiling on the workload's codes: "
            f"{ceiling['tops']:.1f} TOPS; the GEMM reaches "
            f"{ceiling['gemm_frac_of_ceiling']:.3f} of it")
    fused = w.fused
    gemm_shapes = sorted({(w.M, p.N, p.K) for p in w.blocks[0].values()})
    phases = phases_entry(m["stats"], w.M)
    del w
    torch.cuda.empty_cache()

    # ---- the other single-GPU workloads, measured the same way
    per_config = None
    if not args.no_per_config:
        per_config = {}
        for c in PER_CONFIGS:
            if c == args.config:
                continue
            per_config[str(c)] = per_config_entry(
                D.WORKLOADS[c], dev, orc, threads, args)
            torch.cuda.empty_cache()

    peaks = None if args.no_measured_peaks else measured_peaks(torch)
    if peaks:
        log(f"[bench] measured on this box: device copy "
            f"{peaks['hbm_copy_gbs']:.0f} GB/s, BF16 GEMM "
            f"{peaks['bf16_gemm_tflops']:.0f} TFLOPS")

    # ---- CPU baseline: the oracle on a bounded row sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(orc, D, wl, args.cpu_seconds, threads)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} TOPS on {cpu['cores']} "
            f"threads ({cpu['sample']})")

    return {
        "metric": METRIC,
        "value": round(m["tops"], 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wl.name + ("+fused_qkv" if fused else ""),
            "tokens": wl.M,
            "blocks": wl.blocks,
            "linears": wl.blocks * len(wl.projs),
            "gemm_shapes_MNK": [list(s) for s in gemm_shapes],
            "parallelism": "single_gpu",
        },
        "pct_int8_peak": round(100 * m["tops"] / INT8_PEAK_TOPS, 2),
        "step_ms": {**step_stats(m["per"]), "timing": m["how"]},
        "roofline": roofline,
        "phases": phases,
        "oracle_check": check,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "power_clock": power,
        "measured_peaks": peaks,
        "bf16_baseline": bf16,
        "int8_library_baseline": int8lib,
        "mfma_ceiling": ceiling,
    }


def per_config_entry(wl, dev, orc, threads, args):
    """A compact entry for another workload: value, step statistics, the
    GEMM call's roofline, per-phase rates and its own oracle check."""
    w = Workload(wl, dev, "auto", 8, orc, threads, "auto", args.lead,
                 args.lead_ms)
    m = measure(w, args.per_config_steps, 2)
    check = w.check()
    r = roofline_entry(w.blocks[0], w.M, m["gemm_tops"], m["avg_launch_us"],
                       m["gemm_calls"], w.graph, None)
    entry = {
        "workload": wl.name + ("+fused_qkv" if w.fused else ""),
        "value": round(m["tops"], 2), "unit": "TOPS",
        "ms_per_step": step_stats(m["per"]),
        "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit",
                                       "frac", "avg_launch_us")},
        "phases": phases_entry(m["stats"], w.M),
        "oracle_check": {k: check[k] for k in ("blocks", "values_compared",
                                               "mismatches", "bit_exact")}
        | {"rows": len(check["rows"])},
    }
    log(f"[bench] config {wl.name}: {entry['value']:.1f} TOPS, GEMM "
        f"{r['achieved']} {r['unit']} (frac {r['frac']}), oracle "
        f"{'bit-exact' if check['bit_exact'] else 'MISMATCH'}")
    del w
    return entry


def measured_peaks(torch):
    """This box's device-copy rate (bytes read + written) and torch's BF16
    GEMM rate (hipBLASLt, 8192 x 8192 x 8192), beside the published
    8 TB/s and 2.5 PFLOP/s."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    S = 8192
    a = torch.randn((S, S), device="cuda").to(torch.bfloat16)
    b = torch.randn((S, S), device="cuda").to(torch.bfloat16)
    for _ in range(3):
        a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        a @ b
    e1.record()
    torch.cuda.synchronize()
    tflops = 2 * S ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"hbm_copy_gbs": round(copy_gbs, 1),
            "hbm_published_gbs": HBM_PEAK_GBS,
            "bf16_gemm_tflops": round(tflops, 1),
            "bf16_published_tflops": BF16_PEAK_TFLOPS,
            "what": "1 GiB device copy (read + write bytes); torch BF16 "
                    "matmul 8192^3 (hipBLASLt), 10 reps each"}


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
    # started before this process touches the GPU
    sampler = None if args.no_power_clock else PowerClockSampler()
    try:
        result = run(args, sampler)
    finally:
        if sampler is not None:
            sampler.close()
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


def speedup_vs_bf16(bf16, ms_step, blocks):
    """How many times faster the W8A8 step runs one block (quantizations,
    GEMMs and glue) than the BF16 baseline runs the same block."""
    return round(bf16["ms_per_block"] / (ms_step / blocks), 3)


def bf16_baseline(torch, wl, x0, blk, warmup, reps):
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


def cpu_baseline(orc, D, wl, seconds, threads):
    """The oracle as it stands, timed on the first rows of block 0's
    projections; rows are doubled until the run lasts `seconds`/4, then one
    final timed run with about `seconds` of work.  Reported with the host's
    CPU model, the CPUs this process may run on and OMP_NUM_THREADS."""
    params = D.block_params(wl, 0, threads=threads)
    x0_host = D.activations(wl.M, D.HIDDEN, wl.seed)

    def run(R):
        x = x0_host[:R]
        t = time.perf_counter()
        oracle_rows(orc, wl, params, x)
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
                      f"{len(wl.projs)} projection(s), {dt:.1f} s",
            "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "extrapolated_full_step_s": round(
                2 * sum(wl.M * p.N * p.K for p in wl.projs) * wl.blocks /
                (2 * macs / dt), 1)}


if __name__ == "__main__":
    main()
