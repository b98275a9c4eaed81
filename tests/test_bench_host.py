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
