"""Pins for the backward oracle: central finite differences of the (pinned) forward oracle.

The loss is L = sum <dY, y>.  Each gradient the backward returns is checked against
(L(theta + eps v) - L(theta - eps v)) / (2 eps) for random whole-tensor directions v and for
single entries, on the tiny slice R1 T64 d64 E8 k2 F128 with half and with all experts
local.  Logit perturbations are an exact fp32 step (2^-10) and stay inside every token's
top-k margin, so the routing does not change.  A plausible slip (silu' on the wrong
branch, a missing gate factor in the pull, dW transposed, the softmax Jacobian sign, remote
pairs counted) fails one of these.
"""
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle import moe_oracle_bwd as B


def _case(El, seed, R=1, T=64, d=64, E=8, k=2, F=128):
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


def _L(c, **over):
    p = dict(c)
    p.update(over)
    return B.loss(p["logits"], p["x"], p["w1"], p["w3"], p["w2"], p["e2l"], p["El"], p["k"], p["dy"], minibatch=16)


def _grads(c):
    return B.backward(c["logits"], c["x"], c["w1"], c["w3"], c["w2"], c["e2l"], c["El"], c["k"], c["dy"],
                      minibatch=16)


def _margin(logits, k):
    s = -np.sort(-logits.astype(np.float64), axis=-1)
    return float((s[..., k - 1] - s[..., k]).min())


@pytest.mark.parametrize("El,seed", [(4, 0), (8, 1)])
def test_directional_finite_differences(El, seed):
    c = _case(El, seed)
    g = _grads(c)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-5
    for name, key in (("x", "dx"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2")):
        for _ in range(2):
            v = rng.standard_normal(np.shape(c[name]))
            fd = (_L(c, **{name: c[name] + eps * v}) - _L(c, **{name: c[name] - eps * v})) / (2 * eps)
            an = float(np.sum(g[key] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    # logits: an exact fp32 step inside the top-k margin
    e = 2.0 ** -10
    assert _margin(c["logits"], c["k"]) > 2 * e, "seed gives a top-k margin too small for the step"
    for _ in range(2):
        v = np.sign(rng.standard_normal(c["logits"].shape)).astype(np.float32)
        lp = (c["logits"] + np.float32(e) * v).astype(np.float32)
        lm = (c["logits"] - np.float32(e) * v).astype(np.float32)
        fd = (_L(c, logits=lp) - _L(c, logits=lm)) / (2 * e)
        an = float(np.sum(g["dlogits"] * v))
        assert abs(fd - an) <= 1e-5 * max(1.0, abs(an)), (fd, an)


def test_single_entry_finite_differences():
    c = _case(4, 7)
    g = _grads(c)
    rng = np.random.default_rng(3)
    eps = 1e-5
    for name, key in (("x", "dx"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2")):
        shp = np.shape(c[name])
        for _ in range(6):
            i = tuple(int(rng.integers(0, n)) for n in shp)
            p = np.array(c[name], dtype=np.float64)
            m = np.array(c[name], dtype=np.float64)
            p[i] += eps
            m[i] -= eps
            fd = (_L(c, **{name: p}) - _L(c, **{name: m})) / (2 * eps)
            assert abs(fd - g[key][i]) <= 1e-7 * max(1.0, abs(fd)), (name, i, fd, g[key][i])
    # a kept logit of a few tokens, and a logit that is not kept (gradient 0)
    e = 2.0 ** -10
    for t in (0, 5, 33):
        for j in range(c["k"]):
            ex = int(g["idx"][0, t, j])
            p = c["logits"].copy()
            m = c["logits"].copy()
            p[0, t, ex] += np.float32(e)
            m[0, t, ex] -= np.float32(e)
            fd = (_L(c, logits=p) - _L(c, logits=m)) / (2 * e)
            assert abs(fd - g["dlogits"][0, t, ex]) <= 1e-6 * max(1.0, abs(fd)), (t, ex)
        kept = set(int(v) for v in g["idx"][0, t])
        other = [e_ for e_ in range(8) if e_ not in kept][0]
        assert g["dlogits"][0, t, other] == 0.0


def test_remote_pairs_contribute_nothing():
    """With no local expert at all every gradient is zero; a token whose kept experts are all
    remote gets dx = 0 and zero logit gradients on this GPU's share."""
    c = _case(4, 11)
    g = _grads(c)
    so = g["slot_of"]
    none_local = ~(so >= 0).any(-1)
    assert none_local.any()
    assert np.all(g["dx"][none_local] == 0.0)
    assert np.all(g["dlogits"][none_local] == 0.0)


def test_zero_gradient_and_linearity():
    c = _case(4, 5)
    g1 = _grads(c)
    c0 = dict(c, dy=np.zeros_like(c["dy"]))
    g0 = _grads(c0)
    for key in ("dx", "dw1", "dw3", "dw2", "dlogits"):
        assert np.all(g0[key] == 0.0), key
    rng = np.random.default_rng(9)
    dy2 = rng.standard_normal(c["dy"].shape)
    g2 = _grads(dict(c, dy=dy2))
    g12 = _grads(dict(c, dy=c["dy"] + 2.0 * dy2))
    for key in ("dx", "dw1", "dw3", "dw2", "dlogits"):
        np.testing.assert_allclose(g12[key], g1[key] + 2.0 * g2[key], rtol=0, atol=1e-11)


def test_logit_gradient_rows_sum_to_zero():
    g = _grads(_case(8, 2))
    np.testing.assert_allclose(g["dlogits"].sum(-1), 0.0, atol=1e-13)


def test_silu_grad_closed_form():
    a = np.array([-3.0, -0.5, 0.0, 0.7, 4.0])
    fd = (O.silu(a + 1e-6) - O.silu(a - 1e-6)) / 2e-6
    np.testing.assert_allclose(B.silu_grad(a), fd, rtol=0, atol=1e-9)
    assert B.silu_grad(np.array([0.0]))[0] == 0.5
