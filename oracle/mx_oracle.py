"""CPU oracle for the MXFP8 forward: E4M3 elements with one E8M0 scale per 32 along K.

TEST INFRASTRUCTURE ONLY (imported by tests/ and bench.py's cpu_baseline only; shares
no code with the HIP path).

Source: the MoK article (kucoin.com/es "Cursor's MoK logra un aumento del 2.37x ...",
section 02, MXFP8 paragraph) says activation quantisation is fused into the dispatch,
grouped GEMM and SwiGLU data paths.  The pages give nothing MX-specific, so the
reading is the OCP Microscaling (MX) v1.0 format:

  * block: 32 consecutive values along the contraction (K) axis;
  * scale: E8M0, value 2^(code - 127); code = floor(log2 amax) - 8 + 127, clamped to
    [0, 254] (8 = exponent of E4M3's largest power of two); an all-zero block gets code 0
    and zero elements;
  * element: E4M3 (OCP "E4M3FN": bias 7, 3 mantissa bits, subnormals down to 2^-9, no
    infinities, largest finite 448), value / 2^e rounded to nearest, ties to even, and
    saturated to +-448.

Quantised operands: token rows x (during the gather), expert weights (offline, the same
rule), and h (in the GEMM1 epilogue).  "Oracle-Q" is the fp64 forward on the dequantised
operands; h is quantised from its fp64 value.

Parity status: the codec is pinned by tests/test_mx_oracle.py (an independent table
quantiser over every bf16 value at several scales, closed forms); the Oracle-Q forward
reuses the pinned fp64 oracle around the pinned codec.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as O

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8            # exponent of the largest power of two in E4M3
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value of y (ties to even), saturated to +-448; float64 in and out.

    The grid step at |y| is 2^(max(floor(log2 |y|), -6) - 3): 3 mantissa bits in a normal
    binade, the subnormal step 2^-9 below 2^-6.  np.rint rounds half to even."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)                        # a = m * 2^ex with m in [0.5, 1): floor(log2 a) = ex - 1
    step = np.ldexp(1.0, np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP) - E4M3_MANT_BITS)
    q = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    return np.copysign(q, y)


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """Bit pattern (uint8) of E4M3 values q (already on the E4M3 grid): S.EEEE.MMM with
    bias 7; exponent field 0 holds the subnormals m * 2^-9."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    _, ex = np.frexp(a)
    e = ex - 1
    normal = a >= 2.0 ** E4M3_MIN_NORMAL_EXP
    code_norm = ((e + 7) << 3) + np.rint((np.ldexp(a, -e) - 1.0) * 8).astype(np.int64)
    code_sub = np.rint(a / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, code_sub).astype(np.uint8)
    return code | (np.signbit(q).astype(np.uint8) << 7)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of E4M3 bit patterns (S.1111.111 = NaN is never produced by the quantiser)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def block_scale_code(amax: np.ndarray) -> np.ndarray:
    """E8M0 code of the shared scale of blocks with max magnitude amax (0 -> code 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    code = np.clip(ex - 1 - E4M3_EMAX + 127, 0, 254)
    return np.where(amax > 0, code, 0).astype(np.uint8)


def quantize(x: np.ndarray):
    """MX-quantise the last axis of x (length a multiple of 32).

    Returns (codes uint8 [..., K], scale codes uint8 [..., K/32], dequantised float64)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    lead = x.shape[:-1]
    rows = x.reshape(-1, K)
    codes = np.empty(rows.shape, dtype=np.uint8)
    sc = np.empty((rows.shape[0], K // BLOCK), dtype=np.uint8)
    deq = np.empty(rows.shape, dtype=np.float64)
    # every block is independent; rows go through in groups only to keep temporaries small
    step = max(1, (1 << 20) // K)
    for r0 in range(0, rows.shape[0], step):
        xb = rows[r0:r0 + step].reshape(-1, K // BLOCK, BLOCK)
        amax = np.abs(xb).max(axis=-1)
        s = block_scale_code(amax)
        scale = np.ldexp(1.0, s.astype(np.int64) - 127)[..., None]
        q = np.where((amax == 0)[..., None], 0.0, e4m3_round(xb / scale))
        n = xb.shape[0]
        codes[r0:r0 + n] = e4m3_encode(q).reshape(n, K)
        sc[r0:r0 + n] = s
        deq[r0:r0 + n] = (q * scale).reshape(n, K)
    return codes.reshape(x.shape), sc.reshape(*lead, K // BLOCK), deq.reshape(x.shape)


def dequantize(codes: np.ndarray, scale_codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes)
    K = codes.shape[-1]
    v = e4m3_decode(codes).reshape(*codes.shape[:-1], K // BLOCK, BLOCK)
    s = np.exp2(np.asarray(scale_codes, dtype=np.float64) - 127.0)[..., None]
    return (v * s).reshape(codes.shape)


def swiglu_ffn_q(rows_q: np.ndarray, w1q, w3q, w2q) -> np.ndarray:
    """One expert on dequantised rows and weights; h quantised along F before W2."""
    x = np.asarray(rows_q, dtype=np.float64)
    a = x @ np.asarray(w1q, dtype=np.float64).T
    b = x @ np.asarray(w3q, dtype=np.float64).T
    h = O.silu(a) * b
    _, _, hq = quantize(h)
    return hq @ np.asarray(w2q, dtype=np.float64).T


def forward_q(logits, x, w1q, w3q, w2q, expert_to_local, E_local, k, minibatch=128) -> dict:
    """Oracle-Q: route and lay out exactly as the fp64 oracle; x quantised per row along d;
    weights given already dequantised (offline quantisation); h quantised along F."""
    idx, gates = O.route(logits, k)
    lay = O.layout(idx, expert_to_local, E_local, minibatch)
    xe = O.dispatch(x, lay["pull_src"])
    _, _, xeq = quantize(xe)
    ye = np.empty((xe.shape[0], np.asarray(w2q[0]).shape[0]), dtype=np.float64)
    off = lay["offsets"]
    for l in range(len(off) - 1):
        a, b = int(off[l]), int(off[l + 1])
        if b > a:
            ye[a:b] = swiglu_ffn_q(xeq[a:b], w1q[l], w3q[l], w2q[l])
    recv = O.combine_push(ye, lay["pull_src"], lay["slot_of"])
    y = O.weighted_merge(recv, gates, np.asarray(x).shape[2])
    out = dict(lay)
    out.update(idx=idx, gates=gates, xeq=xeq, ye=ye, y=y)
    return out


def token_output_q(x_row, idx_row, gates_row, expert_to_local, w1q, w3q, w2q) -> np.ndarray:
    """Oracle-Q output row of one token computed on its own."""
    _, _, xq = quantize(np.asarray(x_row, dtype=np.float64)[None, :])
    y = np.zeros(xq.shape[1], dtype=np.float64)
    for j in range(len(idx_row)):
        l = int(expert_to_local[int(idx_row[j])])
        if l >= 0:
            y += gates_row[j] * swiglu_ffn_q(xq, w1q[l], w3q[l], w2q[l])[0]
    return y
