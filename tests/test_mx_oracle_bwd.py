"""Pins for the MXFP8 backward oracle (oracle/mx_oracle_bwd.py).

* With the identity in place of the MX quantiser it is the pinned bf16 backward oracle.
* Its forward steps equal Oracle-Q's forward_q (the pinned quantised forward).
* Each data-gradient GEMM (dh = dO W2, dX = da W1 + db W3) and GEMM1's a = x W1^T equal a
  product computed here block by block with the independent table quantiser of
  test_mx_oracle, each operand quantised along that GEMM's K -- a transposed quantisation
  axis, a missing quantisation or a quantised weight gradient fails it.
* Against the exact (unquantised) backward its relative Frobenius error lies in the band of
  the MX forward's (a few percent, not zero and not whole).
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle_bwd as B
from oracle import mx_oracle as MX
from oracle import mx_oracle_bwd as QB
from tests.test_mx_oracle import brute_block


def _case(El, seed, R=1, T=48, d=64, E=8, k=2, F=64):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((R, T, E)).astype(np.float32)
    x = rng.standard_normal((R, T, d))
    w1 = rng.standard_normal((El, F, d)) / math.sqrt(d)
    w3 = rng.standard_normal((El, F, d)) / math.sqrt(d)
    w2 = rng.standard_normal((El, d, F)) / math.sqrt(F)
    e2l = np.full(E, -1, dtype=np.int32)
    e2l[rng.permutation(E)[:El]] = np.arange(El)
    dy = rng.standard_normal((R, T, d))
    return dict(logits=logits, x=x, w1=w1, w3=w3, w2=w2, e2l=e2l, El=El, k=k, dy=dy)


def _run(c, **kw):
    return QB.backward_q(c["logits"], c["x"], c["w1"], c["w3"], c["w2"], c["e2l"], c["El"], c["k"], c["dy"],
                         minibatch=16, **kw)


def _brute_rows(a):
    """Dequantised rows of a, each block of 32 through the table quantiser."""
    a = np.asarray(a, dtype=np.float64)
    out = np.empty_like(a)
    for i in range(a.shape[0]):
        for b0 in range(0, a.shape[1], 32):
            out[i, b0:b0 + 32] = brute_block(a[i, b0:b0 + 32])[2]
    return out


def _brute_mx_matmul(A, Bm):
    """sum_k A[i][k] Bm[k][j] with A's rows and Bm's columns quantised along k."""
    return _brute_rows(A) @ _brute_rows(np.asarray(Bm).T).T


@pytest.mark.parametrize("El,seed", [(4, 0), (8, 1)])
def test_identity_quantiser_is_the_bf16_backward(El, seed):
    c = _case(El, seed)
    g = _run(c, q=lambda a: np.asarray(a, dtype=np.float64))
    ref = B.backward(c["logits"], c["x"], c["w1"], c["w3"], c["w2"], c["e2l"], c["El"], c["k"], c["dy"],
                     minibatch=16)
    for key in ("dx", "dw1", "dw3", "dw2", "dlogits", "dh", "da", "db", "dX", "ye"):
        np.testing.assert_allclose(g[key], ref[key], rtol=0, atol=1e-11, err_msg=key)


def test_forward_steps_equal_forward_q():
    c = _case(4, 3)
    g = _run(c)
    W = g["weights"]
    f = MX.forward_q(c["logits"], c["x"], W["w1q"], W["w3q"], W["w2q"], c["e2l"], c["El"], c["k"], minibatch=16)
    np.testing.assert_array_equal(g["xeq"], f["xeq"])
    np.testing.assert_allclose(g["ye"], f["ye"], rtol=0, atol=1e-12)


def test_data_gradient_gemms_match_blockwise_products():
    c = _case(4, 5)
    g = _run(c)
    off = g["offsets"]
    checked = 0
    for l in range(c["El"]):
        lo, hi = int(off[l]), int(off[l + 1])
        if hi == lo:
            continue
        sl = slice(lo, min(hi, lo + 6))              # a few rows per expert keep the loops short
        W1, W3, W2 = c["w1"][l], c["w3"][l], c["w2"][l]
        # GEMM1's a: x along d, W1 along d (its rows)
        np.testing.assert_allclose(g["a"][sl], _brute_mx_matmul(g["xe"][sl], W1.T), rtol=0, atol=1e-12)
        # dh = dO W2: dO along d, W2 along d (its columns)
        np.testing.assert_allclose(g["dh"][sl], _brute_mx_matmul(g["dO"][sl], W2), rtol=0, atol=1e-12)
        # dX = da W1 + db W3: da, db along F, W1 and W3 along F (their columns)
        want = _brute_mx_matmul(g["da"][sl], W1) + _brute_mx_matmul(g["db"][sl], W3)
        np.testing.assert_allclose(g["dX"][sl], want, rtol=0, atol=1e-12)
        # weight gradients stay unquantised
        np.testing.assert_allclose(g["dw1"][l], g["da"][lo:hi].T @ g["xe"][lo:hi], rtol=0, atol=1e-12)
        checked += 1
    assert checked >= 3


def test_error_band_against_exact_backward():
    c = _case(8, 2, T=128, d=128, F=128)
    g = _run(c)
    ref = B.backward(c["logits"], c["x"], c["w1"], c["w3"], c["w2"], c["e2l"], c["El"], c["k"], c["dy"],
                     minibatch=16)
    for key, lo, hi in (("dx", 0.02, 0.15), ("dw1", 0.02, 0.15), ("dw2", 0.01, 0.15)):
        rel = np.linalg.norm(g[key] - ref[key]) / np.linalg.norm(ref[key])
        assert lo < rel < hi, (key, rel)
