"""CPU oracle for the backward of one GPU's share of the MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` (and ``bench.py``'s ``cpu_baseline`` leg) may
import or call this module.  It shares no code with the HIP path.  Plain float64 NumPy;
the forward pieces come from ``moe_oracle`` (already pinned).

Sources:
  [kucoin] "Cursor's MoK logra un aumento del 2.37x ..." (kucoin.com/es), section 01:
           training adds a backward pass with two more communication rounds in the
           opposite direction; section 02 (push/pull paragraph): the backward uses a pull
           reverse-combine and a push reverse-dispatch; section 03: backward speed-ups.

The pages do not write the backward out; it is the derivative of the forward the oracle
already fixes (readings listed with the design notes):
  * loss L = sum over (r, t) of <dY[r, t], y[r, t]>, so dY is the incoming gradient of y;
  * pull reverse-combine: expert row s of pair (r, t, j) pulls dO_s = g_j * dY[r, t]
    by the forward's pull schedule; the gate gradient of that pair is dg_j = <dY[r, t], o_s>;
  * SwiGLU backward: dh = dO W2, da = dh * b * silu'(a), db = dh * silu(a),
    silu'(a) = sigma(a) * (1 + a * (1 - sigma(a)));
  * dX_s = da W1 + db W3 (row s), pushed back to its (r, t, j) and summed over ascending
    local j into dx[r, t] (push reverse-dispatch, then an ordered sum);
  * dW1 = sum_s da_s^T x_s, dW3 = sum_s db_s^T x_s, dW2 = sum_s dO_s^T h_s per local expert;
  * gates are a softmax over the k kept logits, so for kept expert i of a token
    dl_i = g_i (dg_i - sum_j g_j dg_j); logits not kept get 0.  On one GPU's share dg_j
    of a remote expert is 0 (its contribution comes from the GPU that holds it; the
    expression is linear in dg, so the shares add up to the full gradient).

Parity status: pinned by tests/test_oracle_bwd.py against central finite differences of
the forward oracle (whole-tensor directional derivatives and single entries), plus
invariants (zero incoming gradient, linearity in dY, per-token logit gradients summing to 0).
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as O


def sigmoid(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d silu(a) / da = sigma(a) (1 + a (1 - sigma(a)))."""
    s = sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def pair_j(slot_of: np.ndarray, s: int, r: int, t: int) -> int:
    """The j of the pair whose row is s."""
    hit = np.nonzero(slot_of[r, t] == s)[0]
    assert len(hit) == 1
    return int(hit[0])


def backward(logits, x, w1, w3, w2, expert_to_local, E_local, k, dy, minibatch=128) -> dict:
    """Gradients of L = sum <dy, y> with respect to x, the local experts' weights and the logits.

    Returns the forward dict plus dO, dg (per row), dh, da, db, h, dX (per row), dx [R][T][d],
    dw1, dw3 [E_local][F][d], dw2 [E_local][d][F], dlogits [R][T][E]."""
    fwd = O.forward(logits, x, w1, w3, w2, expert_to_local, E_local, k, minibatch)
    dy = np.asarray(dy, dtype=np.float64)
    R, T, d = dy.shape
    E = np.asarray(logits).shape[2]
    gates, pull_src, slot_of, off = fwd["gates"], fwd["pull_src"], fwd["slot_of"], fwd["offsets"]
    N = fwd["N"]
    xe, ye = fwd["xe"], fwd["ye"]
    F = np.asarray(w1[0]).shape[0] if E_local > 0 else 0

    # pull reverse-combine: each expert row pulls its token's incoming gradient, times its gate
    dO = np.zeros((N, d))
    dg = np.zeros(N)
    for s in range(N):
        r, t = int(pull_src[s, 0]), int(pull_src[s, 1])
        j = pair_j(slot_of, s, r, t)
        dO[s] = gates[r, t, j] * dy[r, t]
        dg[s] = dy[r, t] @ ye[s]

    # SwiGLU backward per local expert, and the weight gradients
    h = np.zeros((N, F))
    dh = np.zeros((N, F))
    da = np.zeros((N, F))
    db = np.zeros((N, F))
    dX = np.zeros((N, d))
    dw1 = np.zeros((E_local, F, d))
    dw3 = np.zeros((E_local, F, d))
    dw2 = np.zeros((E_local, d, F))
    for l in range(E_local):
        lo, hi = int(off[l]), int(off[l + 1])
        if hi == lo:
            continue
        X = xe[lo:hi]
        W1 = np.asarray(w1[l], dtype=np.float64)
        W3 = np.asarray(w3[l], dtype=np.float64)
        W2 = np.asarray(w2[l], dtype=np.float64)
        a = X @ W1.T
        b = X @ W3.T
        sa = O.silu(a)
        h[lo:hi] = sa * b
        dh[lo:hi] = dO[lo:hi] @ W2
        db[lo:hi] = dh[lo:hi] * sa
        da[lo:hi] = dh[lo:hi] * b * silu_grad(a)
        dX[lo:hi] = da[lo:hi] @ W1 + db[lo:hi] @ W3
        dw1[l] = da[lo:hi].T @ X
        dw3[l] = db[lo:hi].T @ X
        dw2[l] = dO[lo:hi].T @ h[lo:hi]

    # push reverse-dispatch, then the ordered sum over local j
    dx = np.zeros((R, T, d))
    dlogits = np.zeros((R, T, E))
    idx = fwd["idx"]
    for r in range(R):
        for t in range(T):
            dgt = np.zeros(k)
            for j in range(k):
                s = int(slot_of[r, t, j])
                if s >= 0:
                    dx[r, t] += dX[s]
                    dgt[j] = dg[s]
            g = gates[r, t]
            dl = g * (dgt - np.dot(g, dgt))
            for j in range(k):
                dlogits[r, t, int(idx[r, t, j])] = dl[j]
    out = dict(fwd)
    out.update(dO=dO, dg=dg, h=h, dh=dh, da=da, db=db, dX=dX, dx=dx, dw1=dw1, dw3=dw3, dw2=dw2,
               dlogits=dlogits)
    return out


def loss(logits, x, w1, w3, w2, expert_to_local, E_local, k, dy, minibatch=128) -> float:
    """L = sum <dy, y> through the forward oracle (what the finite differences perturb)."""
    y = O.forward(logits, x, w1, w3, w2, expert_to_local, E_local, k, minibatch)["y"]
    return float(np.sum(np.asarray(dy, dtype=np.float64) * y))
