"""bench.py's host-side contract and roofline arithmetic (no GPU needed)."""
from __future__ import annotations

import json
import subprocess
import sys
from pathlib import Path
from types import SimpleNamespace

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
from w8a8_int8_gemm_amd import datagen as D  # noqa: E402


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_gemm_call_bytes():
    # Q at M=19077: A 102.6 MB + W 28.9 MB + BF16 out 205.1 MB + scales/bias
    M, N, K = 19077, 5376, 5376
    assert bench.gemm_call_bytes(M, N, K) == \
        M * K + N * K + 2 * M * N + 4 * M + 4 * N + 2 * N


def _blk(shapes):
    return {f"p{i}": SimpleNamespace(N=n, K=k) for i, (n, k) in
            enumerate(shapes)}


def test_roofline_mfma_bound_block():
    blk = _blk([(p.N, p.K) for p in D.BLOCK_PROJS])
    r = bench.roofline_entry(blk, 19077, 2400.0, 919.0, 1500, False, None)
    assert r["bound"] == "mfma" and r["unit"] == "TOP/s"
    assert r["peak"] == bench.INT8_PEAK_TOPS
    assert r["frac"] == round(2400.0 / bench.INT8_PEAK_TOPS, 4)
    ops = sum(2 * 19077 * p.N * p.K for p in D.BLOCK_PROJS) / 6
    assert r["algorithmic_ops_per_call"] == int(ops)


def test_roofline_hbm_bound_single_projection():
    # M = 64: about 123 ops per byte, below the 625 ops/byte ridge
    blk = _blk([(5376, 5376)])
    us = 12.5
    r = bench.roofline_entry(blk, 64, None, us, 100, True, None)
    nbytes = bench.gemm_call_bytes(64, 5376, 5376)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == round(nbytes / (us * 1e-6) / 1e9, 2)
    assert r["peak"] == bench.HBM_PEAK_GBS
    assert r["timing"].startswith("graph")


def test_traffic_only_for_its_projection_mix():
    recs = json.loads(
        (ROOT / "profiles" / "gemm_traffic.json").read_text())["records"]
    sha = bench.kernel_source_sha256()
    wl2 = D.WORKLOADS[2]
    for fused in (False, True):
        tokens, shapes = bench.gemm_mix(wl2, fused)
        match = [r for r in recs if r["kernel_sha256"] == sha and
                 r["workload"]["tokens"] == tokens and
                 sorted(map(tuple, r["workload"]["shapes_NK"])) == shapes]
        t = bench.traffic_entry(wl2, fused)
        # a record taken on an older kernel, or none for this mix: no traffic
        assert t == (match[0]["traffic"] if match else None)
    assert bench.traffic_entry(D.WORKLOADS[0], False) is None  # M = 64
    assert bench.traffic_entry(D.WORKLOADS[5], False) is None  # page shapes


def test_gemm_mix_fuses_qkv_into_one_call():
    tokens, sep = bench.gemm_mix(D.WORKLOADS[2], False)
    _, fused = bench.gemm_mix(D.WORKLOADS[2], True)
    assert tokens == 19077 and len(sep) == 6 and len(fused) == 4
    assert (3 * 5376, 5376) in fused and sep.count((5376, 5376)) == 4
    assert sum(n for n, _ in sep) == sum(n for n, _ in fused)


def test_defaults_check_sixteen_rows_and_other_configs():
    a = bench.parse([])
    assert a.check_rows >= 16 and a.config == 4 and not a.no_per_config
    assert set(bench.PER_CONFIGS) == {0, 1, 2, 3}


def test_quant_bytes():
    M, K = 19077, 5376
    assert bench.quant_bytes("quant", M, K) == 2 * M * K + M * K + 4 * M
    assert bench.quant_bytes("silu_quant", M, 21504) == 3 * M * 21504 + 4 * M
    # gated: reads gate and up (2K wide), writes K codes
    assert bench.quant_bytes("swiglu_quant", M, K) == 4 * M * K + M * K + 4 * M
    # renormalization writes the BF16 row as well as the codes
    assert bench.quant_bytes("renorm_quant", M, K) == 5 * M * K + 4 * M


def test_step_stats_and_phases():
    st = bench.step_stats([2.0, 4.0, 3.0])
    assert st["median"] == 3.0 and st["n"] == 3 and st["std"] == 1.0
    M = 100
    stats = {"gemm:q": [2, 0.02, [(M, 256, 512)] * 2],
             "quant": [4, 0.008, [(M, 512)] * 4]}
    ph = bench.phases_entry(stats, M)
    assert ph["gemm:q"]["avg_us"] == 10.0
    assert ph["gemm:q"]["tops"] == round(2 * M * 256 * 512 / 1e-5 / 1e12, 2)
    assert ph["quant"]["avg_us"] == 2.0
    assert ph["quant"]["gbs"] == round(bench.quant_bytes("quant", M, 512)
                                       / 2e-6 / 1e9, 1)
    n, ms, ops = bench.gemm_totals(stats)
    assert n == 2 and ms == 0.02 and ops == 2 * 2 * M * 256 * 512


def test_power_clock_sampler_parses_amd_smi_json(tmp_path):
    s = bench.PowerClockSampler.__new__(bench.PowerClockSampler)
    s.proc = None
    s.path = str(tmp_path / "smi.txt")
    reading = {"gpu_data": [{"gpu": 0,
                             "power": {"socket_power": {"value": 1400,
                                                        "unit": "W"}},
                             "clock": {f"gfx_{i}": {"clk": {"value": 1700 + i,
                                                            "unit": "MHz"}}
                                       for i in range(8)}}]}
    with open(s.path, "w") as f:
        for t in (10.0, 11.0, 12.0):
            f.write(f"T {t}\n{json.dumps(reading)}\n")
        f.write("T 13.0\nnot json\n")
    assert len(s.samples()) == 3
    w = s.window(10.5, 12.5)
    assert w["samples"] == 2 and w["socket_power_w"] == [1400, 1400]
    assert w["gfx_clock_mhz_min_mean_max"] == [1700, 1704, 1707]
    assert w["xcds"] == 8
    assert s.window(20, 30) is None


def test_speedup_vs_bf16_is_per_block():
    # 50 blocks in 300 ms against a BF16 block of 10.2 ms: 1.7x per block
    assert bench.speedup_vs_bf16({"ms_per_block": 10.2}, 300.0, 50) == 1.7
