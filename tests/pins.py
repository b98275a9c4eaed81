"""Pins of the CPU oracle to facts other than the oracle itself.

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError (or
``oracle.OracleError``) when the oracle disagrees with:
  * hand-worked cases stored under tests/golden/ (cited there);
  * closed forms and brute force (integer products);
  * invariants of per-token symmetric quantization;
  * exact rational arithmetic with explicit IEEE rounding (tests/exact.py);
  * library routines for the special cases they cover (torch's BF16 cast,
    torch's float64 SiLU).
The same checks run against deliberately broken builds of the oracle in
test_oracle_mutants.py, where at least one of them must fail.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

from tests import exact as ex

GOLDEN = Path(__file__).resolve().parent / "golden"


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def bf16_bits_exact(values) -> np.ndarray:
    """Exact values (Fractions) -> BF16 bits; each must be representable."""
    out = []
    for v in values:
        r = ex.rn_bf16(v)
        assert r == v, f"{v} is not a BF16 value"
        bits = ex.value_to_bf16_bits(r)
        if r == 0 and str(v).startswith("-"):
            bits = 0x8000
        out.append(bits)
    return np.array(out, np.uint16)


def _parse_table(name: str):
    rows = []
    for line in (GOLDEN / name).read_text().splitlines():
        if not line.strip() or line.lstrip().startswith("#"):
            continue
        rows.append([c.strip() for c in line.split("|")])
    return rows


def ordered(bits: np.ndarray) -> np.ndarray:
    """BF16 bits -> integers ordered like the values (+0 and -0 equal)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def torch_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_rows(seed: int, M: int, K: int) -> np.ndarray:
    """BF16 rows of assorted magnitudes, signs and outliers."""
    g = np.random.default_rng([seed, 77])
    x = g.standard_normal((M, K)).astype(np.float32)
    x[g.random((M, K)) < 0.01] *= 20.0
    scale = np.float32(2.0) ** g.integers(-20, 20, size=(M, 1)).astype(
        np.float32)
    x = x * scale
    if M > 2:
        x[1] = -np.abs(x[1])  # argmax negative
        x[2, : K // 2] = 0.0  # half zeros
    return torch_bf16_bits(x)


# --------------------------------------------------------------------------
# quantization
# --------------------------------------------------------------------------

def check_quant_hand_worked(orc):
    rows = _parse_table("quant_hand_worked.txt")
    assert len(rows) >= 9
    for name, xs, scale, codes in rows:
        vals = [ex.from_hex_or_rational(t) for t in xs.split()]
        bits = bf16_bits_exact(vals)
        for i, t in enumerate(xs.split()):
            if t.startswith("-") and vals[i] == 0:
                bits[i] = 0x8000
        q, sa = orc.quantize_act(bits.reshape(1, -1))
        want_s = ex.rn_f32(ex.from_hex_or_rational(scale))
        got_s = Fraction(float(sa[0]))
        assert got_s == want_s, f"{name}: scale {got_s} != {want_s}"
        want_q = [int(c) for c in codes.split()]
        assert q[0].tolist() == want_q, f"{name}: codes {q[0]} != {want_q}"
        # The stored codes were derived by hand; confirm them from the
        # rounded scale with exact arithmetic as well.
        if want_s != 0:
            for v, c in zip(vals, want_q):
                t = ex.rn_f32(v / want_s)
                assert max(-127, min(127, ex.round_half_even_int(t))) == c


def check_quant_invariants(orc):
    for seed, (M, K) in enumerate([(6, 1), (5, 7), (9, 128), (4, 300),
                                   (3, 5376)]):
        x = random_rows(seed, M, K)
        q, sa = orc.quantize_act(x)
        xf = x.view(np.uint16).astype(np.uint32) << 16
        xf = xf.view(np.float32).reshape(M, K).astype(np.float64)
        for m in range(M):
            row, qr, s = xf[m], q[m].astype(np.int64), float(sa[m])
            amax = np.abs(row).max()
            if amax == 0:
                assert s == 0 and not qr.any()
                continue
            # scale is amax/127 rounded once to binary32
            assert Fraction(s) == ex.rn_f32(Fraction(amax) / 127)
            # codes in range, the largest magnitudes map to +-127
            assert qr.min() >= -127 and qr.max() <= 127
            big = np.abs(row) == amax
            assert np.all(qr[big] == np.sign(row[big]) * 127)
            # signs agree (or zero) and the map is monotone
            assert np.all((np.sign(qr) == np.sign(row)) | (qr == 0))
            order = np.argsort(row, kind="stable")
            assert np.all(np.diff(qr[order]) >= 0)
            # reconstruction error within half a step (+ division rounding)
            err = np.abs(row - qr * s)
            assert np.all(err <= s * (0.5 + 2.0 ** -17)), m
        # negation: codes negate, scales unchanged
        qn, san = orc.quantize_act(x ^ np.uint16(0x8000))
        assert np.array_equal(qn, -q) and np.array_equal(san, sa)
        # power-of-two scaling: codes unchanged, scale scaled exactly
        for j in (-3, 4):
            y = xf * 2.0 ** j
            yb = torch_bf16_bits(y.astype(np.float32))
            assert np.array_equal(
                (yb.astype(np.uint32) << 16).view(np.float32).astype(
                    np.float64), y), "test data must scale exactly"
            q2, sa2 = orc.quantize_act(yb)
            assert np.array_equal(q2, q)
            assert np.array_equal(sa2.astype(np.float64),
                                  sa.astype(np.float64) * 2.0 ** j)


def check_quant_rejects_nonfinite(orc):
    import oracle as orc_mod
    x = np.array([[0x3F80, 0x7F80]], np.uint16)  # 1.0, +Inf
    try:
        orc.quantize_act(x)
    except orc_mod.OracleError as e:
        assert e.code == 3
    else:
        raise AssertionError("non-finite activation accepted")


# --------------------------------------------------------------------------
# integer matrix product
# --------------------------------------------------------------------------

def check_gemm_bruteforce(orc):
    g = np.random.default_rng(5)
    for M, N, K in [(1, 1, 1), (2, 3, 5), (17, 9, 130), (3, 128, 256),
                    (5, 2, 1000)]:
        a = g.integers(-128, 128, (M, K), dtype=np.int8)
        w = g.integers(-128, 128, (N, K), dtype=np.int8)
        want = a.astype(np.int64) @ w.astype(np.int64).T
        got = orc.gemm_i32(a, w)
        assert np.array_equal(got.astype(np.int64), want), (M, N, K)


def check_gemm_closed_forms(orc):
    # all 127: 127*127*K; at K = 21504 that is 346 838 016 < 2^31
    K = 21504
    a = np.full((2, K), 127, np.int8)
    w = np.full((3, K), 127, np.int8)
    assert np.all(orc.gemm_i32(a, w) == 16129 * K)
    w[1] = -127
    assert np.all(orc.gemm_i32(a, w)[:, 1] == -16129 * K)
    # all ones: K
    assert np.all(orc.gemm_i32(np.ones((1, 384), np.int8),
                               np.ones((2, 384), np.int8)) == 384)
    # one-hot weight rows pick activation columns
    g = np.random.default_rng(6)
    a = g.integers(-127, 128, (4, 256), dtype=np.int8)
    perm = g.permutation(256)[:64]
    w = np.zeros((64, 256), np.int8)
    w[np.arange(64), perm] = 1
    assert np.array_equal(orc.gemm_i32(a, w), a[:, perm].astype(np.int32))
    # largest magnitude that still fits: (-128)^2 * 131071 < 2^31
    K = 131071
    a = np.full((1, K), -128, np.int8)
    assert orc.gemm_i32(a, a)[0, 0] == 16384 * K
    # one more term leaves INT32 and must be reported
    import oracle as orc_mod
    a = np.full((1, K + 1), -128, np.int8)
    try:
        orc.gemm_i32(a, a)
    except orc_mod.OracleError as e:
        assert e.code == 5
    else:
        raise AssertionError("INT32 overflow not reported")


# --------------------------------------------------------------------------
# epilogue
# --------------------------------------------------------------------------

def check_epilogue_hand_worked(orc):
    rows = _parse_table("epilogue_hand_worked.txt")
    assert len(rows) >= 12
    for acc, sa, sw, bias, want_f, want_b in rows:
        acc_a = np.array([[int(acc)]], np.int32)
        sa_a = np.array([float(ex.from_hex_or_rational(sa))], np.float32)
        sw_a = np.array([float(ex.from_hex_or_rational(sw))], np.float32)
        b = None
        if bias != "-":
            b = bf16_bits_exact([ex.from_hex_or_rational(bias)])
        yf, yb = orc.epilogue(acc_a, sa_a, sw_a, b)
        if want_f == "inf":
            assert math.isinf(yf[0, 0]) and yf[0, 0] > 0
        else:
            assert Fraction(float(yf[0, 0])) == ex.from_hex_or_rational(
                want_f), (acc, sa, sw, bias, yf[0, 0])
        assert int(yb[0, 0]) == int(want_b, 16), (acc, hex(yb[0, 0]))


def _exact_epilogue(acc: int, sa: float, sw: float, b):
    t = ex.rn_f32(Fraction(acc))
    t = ex.rn_f32(t * Fraction(float(sa)))
    t = ex.rn_f32(t * Fraction(float(sw)))
    if b is not None:
        t = ex.rn_f32(t + b)
    return t


def check_epilogue_exact(orc):
    g = np.random.default_rng(7)
    M, N = 7, 29
    acc = g.integers(-2**31, 2**31, (M, N), dtype=np.int64).astype(np.int32)
    acc[0, :5] = [0, 1, -1, 2**24 + 1, -(2**24 + 3)]
    sa = np.exp(g.normal(-4, 2, M)).astype(np.float32)
    sw = np.exp(g.normal(-6, 0.3, N)).astype(np.float32)
    bias = torch_bf16_bits(g.normal(0, 0.02, N).astype(np.float32))
    yf, yb = orc.epilogue(acc, sa, sw, bias)
    yf0, yb0 = orc.epilogue(acc, sa, sw, None)
    order_sensitive = 0
    for m in range(M):
        for n in range(N):
            b = ex.bf16_bits_to_fraction(bias[n])
            t = _exact_epilogue(int(acc[m, n]), sa[m], sw[n], b)
            assert Fraction(float(yf[m, n])) == t, (m, n)
            assert int(yb[m, n]) == ex.value_to_bf16_bits(ex.rn_bf16(t))
            t0 = _exact_epilogue(int(acc[m, n]), sa[m], sw[n], None)
            assert Fraction(float(yf0[m, n])) == t0
            # does the other association give another binary32 value?
            alt = ex.rn_f32(ex.rn_f32(Fraction(int(acc[m, n]))) *
                            ex.rn_f32(Fraction(float(sa[m])) *
                                      Fraction(float(sw[n]))))
            order_sensitive += alt != t0
    assert order_sensitive > 0, "data must distinguish the two orders"


def check_epilogue_rejects_bad_scales(orc):
    import oracle as orc_mod
    acc = np.zeros((1, 2), np.int32)
    sa = np.ones(1, np.float32)
    for bad in (0.0, -1.0, np.inf, np.nan):
        try:
            orc.epilogue(acc, sa, np.array([1.0, bad], np.float32))
        except orc_mod.OracleError as e:
            assert e.code == 4
        else:
            raise AssertionError(f"weight scale {bad} accepted")


# --------------------------------------------------------------------------
# BF16 rounding
# --------------------------------------------------------------------------

def check_bf16_rounding(orc):
    g = np.random.default_rng(8)
    bits = g.integers(0, 2**32, 6000, dtype=np.uint64).astype(np.uint32)
    # ties with even and odd kept parts, subnormals, near-overflow
    hi = g.integers(0, 2**16, 2000, dtype=np.uint64).astype(np.uint32)
    ties = (hi << 16) | 0x8000
    specials = np.array([0x00000001, 0x00008000, 0x00018000, 0x7F7F8000,
                         0x7F7FFFFF, 0x7F7F7FFF, 0xFF7F8000, 0x80000000,
                         0x3F808000, 0x3F818000, 0x7F800000, 0xFF800000],
                        np.uint32)
    allb = np.concatenate([bits, ties, specials])
    f = allb.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    got = orc.f32_to_bf16(f)
    want = torch_bf16_bits(f)
    assert np.array_equal(got, want)
    # binary64 -> BF16 with a single rounding, against exact arithmetic
    d = np.concatenate([
        g.standard_normal(1500) * 10.0 ** g.integers(-40, 39, 1500),
        np.ldexp(g.random(300) + 1.0, g.integers(-150, -120, 300)),
        [0.0, -0.0, 3.4e38, 3.39e38, -3.5e38, 2.0 ** -134, 2.0 ** -135,
         1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 3 * 2.0 ** -8]])
    got = orc.f64_to_bf16(d)
    for v, b in zip(d, got):
        r = ex.rn_bf16(Fraction(float(v)))
        want = ex.value_to_bf16_bits(r)
        if r == 0 and math.copysign(1.0, v) < 0:
            want = 0x8000
        assert int(b) == want, (v, hex(b), hex(want))


# --------------------------------------------------------------------------
# whole linear
# --------------------------------------------------------------------------

def check_linear_hand_worked(orc):
    """Rows whose largest magnitude is 127 have scale exactly 1, so their
    integer entries are their own codes; power-of-two weight scales and a
    BF16 bias then make every FP32 step exact and leave one rounding."""
    M, K, N = 2, 128, 128
    xq = np.zeros((M, K), np.int64)
    xq[0, :] = 127
    xq[1, 0] = -127
    xq[1, 1:] = (np.arange(1, K) % 7) - 3
    kk, nn = np.meshgrid(np.arange(K), np.arange(N))
    w = ((kk * 3 + nn * 5) % 11 - 5).astype(np.int8)
    sw_exp = 8 + (np.arange(N) % 3)
    sw = (2.0 ** -sw_exp).astype(np.float32)
    bias_vals = [Fraction(((n % 5) - 2), 8) for n in range(N)]
    x = bf16_bits_exact([Fraction(int(v)) for v in xq.ravel()]).reshape(M, K)
    bias = bf16_bits_exact(bias_vals)
    y = orc.linear(x, w, sw, bias)
    for m in range(M):
        for n in range(N):
            acc = sum(int(xq[m, k]) * int(w[n, k]) for k in range(K))
            v = Fraction(acc) / 2 ** int(sw_exp[n]) + bias_vals[n]
            want = ex.value_to_bf16_bits(ex.rn_bf16(v))
            if ex.rn_bf16(v) == 0 and v < 0:
                want = 0x8000
            assert int(y[m, n]) == want, (m, n, hex(y[m, n]), hex(want))
    # the composite equals the three stages run one after another
    g = np.random.default_rng(9)
    x = random_rows(10, 5, 256)
    w = g.integers(-127, 128, (40, 256), dtype=np.int8)
    sw = np.exp(g.normal(-6, 0.3, 40)).astype(np.float32)
    b = torch_bf16_bits(g.normal(0, 0.02, 40).astype(np.float32))
    q, sa = orc.quantize_act(x)
    _, yb = orc.epilogue(orc.gemm_i32(q, w), sa, sw, b)
    assert np.array_equal(orc.linear(x, w, sw, b), yb)


# --------------------------------------------------------------------------
# weight quantization (converter side) and the scale contract
# --------------------------------------------------------------------------

def _bits_of(tokens):
    vals = [ex.from_hex_or_rational(t) for t in tokens]
    bits = bf16_bits_exact(vals)
    for i, t in enumerate(tokens):
        if t.startswith("-") and vals[i] == 0:
            bits[i] = 0x8000
    return vals, bits


def check_weight_quant_hand_worked(orc):
    rows = _parse_table("weight_quant_hand_worked.txt")
    assert len(rows) >= 5
    width = max(len(r[1].split()) for r in rows)
    for name, ws, scale, codes in rows:
        vals, bits = _bits_of(ws.split())
        # pad every row to one width with zeros (do not change amax)
        w = np.zeros((2, width), np.uint16)
        w[0, : len(bits)] = bits
        q, sw = orc.quantize_weight(w)
        want_s = ex.rn_f32(ex.from_hex_or_rational(scale))
        assert Fraction(float(sw[0])) == want_s, f"{name}: scale {sw[0]}"
        assert q[0, : len(bits)].tolist() == [int(c) for c in codes.split()]
        assert not q[0, len(bits):].any()
        # the all-zero second row: codes 0, scale exactly 1
        assert float(sw[1]) == 1.0 and not q[1].any()


def check_weight_quant_rows(orc):
    # random rows: every code from exact rational arithmetic, every scale
    # finite and positive
    w = random_rows(21, 7, 96)
    w[3] = 0
    q, sw = orc.quantize_weight(w)
    assert np.all(np.isfinite(sw)) and np.all(sw > 0)
    for n in range(w.shape[0]):
        vals = [Fraction(float(v)) for v in
                (w[n].astype(np.uint32) << 16).view(np.float32)]
        amax = max(abs(v) for v in vals)
        if amax == 0:
            assert float(sw[n]) == 1.0 and not q[n].any()
            continue
        s = ex.rn_f32(amax / 127)
        assert Fraction(float(sw[n])) == s
        want = [max(-127, min(127, ex.round_half_even_int(ex.rn_f32(v / s))))
                for v in vals]
        assert q[n].tolist() == want


def check_scale_contract(orc):
    sw = np.array([1.0, 0.0, -0.0, -1.0, np.inf, -np.inf, np.nan, 1e-45,
                   3.4e38, 2.5e-3], np.float32)
    # bad: 0, -0, -1, +inf, -inf, nan  (a positive subnormal is fine)
    assert orc.check_scales(sw) == 6
    assert orc.check_scales(np.ones(5, np.float32)) == 0
    assert orc.check_scales(np.zeros(0, np.float32)) == 0


# --------------------------------------------------------------------------
# harness glue
# --------------------------------------------------------------------------

def all_finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (b >> 7) & 0xFF
    return b[e != 0xFF]


def check_silu(orc):
    x = all_finite_bf16()
    y = orc.silu_bf16(x)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = torch.nn.functional.silu(torch.from_numpy(xv)).numpy()
    # torch's float64 SiLU rounded once to BF16 with exact arithmetic
    want = np.array([ex.value_to_bf16_bits(ex.rn_bf16(Fraction(float(v))))
                     if v != 0 else (0x8000 if math.copysign(1, v) < 0
                                     else 0)
                     for v in ref], np.uint16)
    d = np.abs(ordered(y) - ordered(want))
    assert d.max() <= 1
    assert np.count_nonzero(d) <= 8, np.count_nonzero(d)
    # silu(0) = 0; silu(x) = x for large x
    assert int(orc.silu_bf16(np.array([0], np.uint16))[0]) == 0
    big = torch_bf16_bits(np.array([64.0, 1000.0, 3e38], np.float32))
    assert np.array_equal(orc.silu_bf16(big), big)


def check_pow2_renorm(orc):
    x = random_rows(11, 6, 300)
    x[3] = 0
    x[4, :] = np.array([1, 0x8002, 5], np.uint16).repeat(100)  # subnormals
    y = orc.pow2_renorm(x)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(y[3], x[3])
    for m in range(6):
        amax = np.abs(xv[m]).max()
        if amax == 0:
            continue
        e = math.floor(math.log2(amax))
        assert 1.0 <= np.abs(yv[m]).max() < 2.0
        for a, b in zip(xv[m], yv[m]):
            want = ex.rn_bf16(Fraction(float(a)) / Fraction(2) ** e)
            assert Fraction(float(b)) == want


def check_swiglu_hand_worked(orc):
    rows = _parse_table("swiglu_hand_worked.txt")
    assert len(rows) >= 5
    for name, gs, us, ys in rows:
        _, g = _bits_of(gs.split())
        _, u = _bits_of(us.split())
        yv, want = _bits_of(ys.split())
        h = np.concatenate([g, u]).reshape(1, -1)
        y = orc.swiglu_bf16(h)
        assert y[0].tolist() == want.tolist(), f"{name}: {y[0]} != {want}"


def check_swiglu_composition(orc):
    # y = BF16(BF16(silu(g)) * u) with the gate first: the SiLU values come
    # from the oracle's SiLU (pinned by check_silu), the product and its
    # rounding from exact rational arithmetic
    g = np.random.default_rng([31, 5])
    M, F = 3, 200
    gate = torch_bf16_bits((g.standard_normal((M, F)) * 4).astype(np.float32))
    up = torch_bf16_bits((g.standard_normal((M, F)) * 3).astype(np.float32))
    h = np.concatenate([gate, up], axis=1)
    y = orc.swiglu_bf16(h)
    s = orc.silu_bf16(gate)
    sv = (s.astype(np.uint32) << 16).view(np.float32)
    uv = (up.astype(np.uint32) << 16).view(np.float32)
    yv = (y.astype(np.uint32) << 16).view(np.float32)
    for a, b, c in zip(sv.ravel(), uv.ravel(), yv.ravel()):
        want = ex.rn_bf16(Fraction(float(a)) * Fraction(float(b)))
        assert Fraction(float(c)) == want


ALL_CHECKS = [
    check_quant_hand_worked,
    check_quant_invariants,
    check_quant_rejects_nonfinite,
    check_gemm_bruteforce,
    check_gemm_closed_forms,
    check_epilogue_hand_worked,
    check_epilogue_exact,
    check_epilogue_rejects_bad_scales,
    check_bf16_rounding,
    check_linear_hand_worked,
    check_silu,
    check_pow2_renorm,
    check_weight_quant_hand_worked,
    check_weight_quant_rows,
    check_scale_contract,
    check_swiglu_hand_worked,
    check_swiglu_composition,
]
