"""Pins for the MXFP8 part of the oracle (OCP MX v1.0 reading of the MXFP8 paragraph of
section 02 of the MoK article, kucoin.com/es).

The oracle's E4M3 rounding works from log2 and rint; the pins below use a second,
independent quantiser (a table of the 256 E4M3 codes built by enumerating sign,
exponent and mantissa, nearest entry by bisection, ties to the even code, saturation)
over every bf16 value at several scales, hand-worked blocks, closed forms of the shared
exponent found by repeated doubling, and a pure-Python brute force of one quantised
expert.  A plausible slip (ties away from zero, NaN instead of saturation, an off-by-one
scale exponent, subnormals flushed, h left unquantised) fails one of them.
"""
import bisect
import json
import math
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import mx_oracle as MX

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- table quantiser
def _e4m3_table():
    """(value, code) for every finite non-negative E4M3 code, from the bit-field definition."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                  # S.1111.111 is NaN
            v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
            out.append((v, (e << 3) | m))
    out.sort()
    return out


TABLE = _e4m3_table()
TVALS = [v for v, _ in TABLE]
TCODES = [c for _, c in TABLE]


def table_code(y: float) -> int:
    """Nearest E4M3 code of y (ties to even mantissa, saturate at 448) by table lookup."""
    s = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a >= TVALS[-1]:
        return s | TCODES[-1]
    i = bisect.bisect_left(TVALS, a)
    if TVALS[i] == a:
        return s | TCODES[i]
    lo, hi = i - 1, i
    dl, dh = a - TVALS[lo], TVALS[hi] - a
    if dl < dh:
        j = lo
    elif dh < dl:
        j = hi
    else:
        j = lo if (TCODES[lo] & 1) == 0 else hi
    return s | TCODES[j]


def table_value(code: int) -> float:
    v = dict((c, val) for val, c in TABLE)[code & 0x7F]
    return -v if code & 0x80 else v


def brute_block(vals):
    """Quantise one block of 32 with the table quantiser; exponent found by doubling."""
    amax = max(abs(float(v)) for v in vals)
    if amax == 0.0:
        return 0, [0] * len(vals), [0.0] * len(vals)
    p = 0
    while 2.0 ** (p + 1) <= amax:
        p += 1
    while 2.0 ** p > amax:
        p -= 1
    e = max(-127, min(127, p - 8))
    codes = [table_code(float(v) / 2.0 ** e) for v in vals]
    return e + 127, codes, [table_value(c) * 2.0 ** e for c in codes]


def _all_bf16_finite():
    p = np.arange(65536, dtype=np.uint32)
    keep = ((p >> 7) & 0xFF) != 0xFF
    return (p[keep] << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- pins
def test_table_has_the_e4m3_landmarks():
    assert len(TABLE) == 127 and TVALS[0] == 0.0
    assert TVALS[1] == 2.0 ** -9 and TVALS[-1] == 448.0
    assert TVALS[8] == 2.0 ** -6            # first normal value


@pytest.mark.parametrize("scale_exp", [0, -3, 5, 9, -20, 100, -126])
def test_e4m3_round_matches_table_on_every_bf16(scale_exp):
    v = _all_bf16_finite()
    y = v / 2.0 ** scale_exp
    q = MX.e4m3_round(y)
    codes = MX.e4m3_encode(q)
    # the table side, vectorised by bisection on the sorted values
    a = np.abs(y)
    tv = np.asarray(TVALS)
    tc = np.asarray(TCODES)
    i = np.clip(np.searchsorted(tv, a), 1, len(tv) - 1)
    lo, hi = tv[i - 1], tv[i]
    pick_hi = (hi - a < a - lo) | ((hi - a == a - lo) & ((tc[i - 1] & 1) == 1))
    j = np.where(pick_hi, i, i - 1)
    j = np.where(a >= 448.0, len(tv) - 1, j)
    ref = tc[j].astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)
    assert np.array_equal(codes, ref)
    assert np.array_equal(MX.e4m3_decode(codes), np.copysign(tv[j], y))
    # spot-check the vectorised side against the scalar table lookup
    for t in range(0, len(y), 997):
        assert table_code(float(y[t])) == int(ref[t])


def test_decode_encode_round_trip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = MX.e4m3_decode(codes)
    assert np.array_equal(MX.e4m3_encode(vals), codes)
    for c in codes:
        assert vals[list(codes).index(c)] == table_value(int(c)) or (vals[list(codes).index(c)] == 0 and table_value(int(c)) == 0)
    assert np.isnan(MX.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_golden_blocks():
    g = json.load(open(os.path.join(GOLD, "mx_block_examples.json")))
    for b in g["blocks"]:
        x = np.asarray(b["x"], dtype=np.float64)[None, :]
        codes, sc, deq = MX.quantize(x)
        assert int(sc[0, 0]) == b["scale_code"], b["name"]
        assert deq[0].tolist() == [float(v) for v in b["deq"]], b["name"]
        for i, c in b["codes_at"].items():
            assert int(codes[0, int(i)]) == c, (b["name"], i)
        assert np.array_equal(MX.dequantize(codes, sc), deq)


@pytest.mark.parametrize("amax,code", [(1.0, 119), (448.0, 127), (511.0, 127), (512.0, 128), (0.999, 118),
                                       (2.0 ** -140, 0), (2.0 ** -119, 0), (2.0 ** -118, 1),
                                       (3.0e38, 246), (0.0, 0)])
def test_scale_code_closed_forms(amax, code):
    assert int(MX.block_scale_code(np.array([amax]))[0]) == code


def test_quantize_matches_brute_force_blocks():
    rng = np.random.default_rng(11)
    blocks = []
    for t in range(120):
        mag = 2.0 ** rng.integers(-30, 30)
        b = rng.standard_normal(32) * mag
        if t % 7 == 0:
            b[rng.integers(0, 32)] *= 1000.0       # one outlier: small values go subnormal
        if t % 11 == 0:
            b[:] = 0.0
        if t % 13 == 0:
            b = np.round(b / mag * 4) / 4 * mag     # many exact grid points and ties
        blocks.append(b)
    x = np.stack(blocks).reshape(4, 30 * 32)
    codes, sc, deq = MX.quantize(x)
    flat_c = codes.reshape(-1, 32)
    flat_s = sc.reshape(-1)
    flat_d = deq.reshape(-1, 32)
    for i, b in enumerate(blocks):
        s, c, d = brute_block(b.tolist())
        assert int(flat_s[i]) == s, i
        assert flat_c[i].tolist() == c, i
        assert flat_d[i].tolist() == d, i


def test_quantize_error_bound_and_idempotence():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-5, 5, size=(64, 1)))
    codes, sc, deq = MX.quantize(x)
    xb, db = x.reshape(64, 8, 32), deq.reshape(64, 8, 32)
    scale = np.exp2(sc.astype(np.float64) - 127)[..., None]
    # error <= half a grid step at the element's binade (or the subnormal step), unless the
    # element saturated (|x| / scale in (448, 512))
    y = np.abs(xb) / scale
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -20))), -6) - 3)
    sat = y > 448.0
    err = np.abs(db - xb) / scale
    assert np.all((err <= step / 2 + 1e-300) | sat)
    assert np.all(np.abs(db[sat]) == 448.0 * np.broadcast_to(scale, db.shape)[sat])
    c2, s2, d2 = MX.quantize(deq)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sc) and np.array_equal(d2, deq)


def test_swiglu_ffn_q_matches_loops_with_table_quantiser():
    rng = np.random.default_rng(2)
    d, F, M = 64, 96, 3
    x = rng.standard_normal((M, d))
    w1 = rng.standard_normal((F, d)) / 8
    w3 = rng.standard_normal((F, d)) / 8
    w2 = rng.standard_normal((d, F)) / 10
    y = MX.swiglu_ffn_q(x, w1, w3, w2)
    for m in range(M):
        h = []
        for f in range(F):
            a = sum(float(w1[f][i]) * float(x[m][i]) for i in range(d))
            b = sum(float(w3[f][i]) * float(x[m][i]) for i in range(d))
            h.append(a / (1.0 + math.exp(-a)) * b)
        hq = []
        for blk in range(F // 32):
            hq += brute_block(h[32 * blk:32 * blk + 32])[2]
        for i in range(d):
            ref = sum(float(w2[i][f]) * hq[f] for f in range(F))
            assert abs(y[m][i] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_forward_q_assembly_matches_per_token_and_fp64_forward():
    rng = np.random.default_rng(9)
    R, T, d, F, E, El, k = 2, 24, 64, 64, 6, 4, 2
    logits = rng.standard_normal((R, T, E)).astype(np.float32)
    x = rng.standard_normal((R, T, d))
    w1 = rng.standard_normal((El, F, d)) / 8
    w3 = rng.standard_normal((El, F, d)) / 8
    w2 = rng.standard_normal((El, d, F)) / 8
    e2l = np.array([2, -1, 0, 3, -1, 1], dtype=np.int32)
    wq = [MX.quantize(w)[2] for w in (w1, w3, w2)]
    out = MX.forward_q(logits, x, *wq, e2l, El, k, minibatch=8)
    for r in range(R):
        for t in range(T):
            ref = MX.token_output_q(x[r, t], out["idx"][r, t], out["gates"][r, t], e2l, *wq)
            np.testing.assert_allclose(out["y"][r, t], ref, rtol=0, atol=1e-12)
    # E4M3 keeps 3 mantissa bits: each quantised operand carries ~3.6 % rms relative
    # error, so the quantised forward sits ~8 % (relative Frobenius) from the exact one.
    # The band catches a codec that is not applied at all or is badly off.
    exact = O.forward(logits, x, w1, w3, w2, e2l, El, k, minibatch=8)["y"]
    live = np.abs(exact).max(axis=-1) > 0
    fro = np.linalg.norm(out["y"][live] - exact[live]) / np.linalg.norm(exact[live])
    assert 0.03 < fro < 0.12, fro
    assert np.array_equal(out["y"][~live], np.zeros_like(out["y"][~live]))
