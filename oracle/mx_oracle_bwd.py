"""CPU oracle for the backward of one GPU's share with MXFP8 expert GEMMs ("Oracle-Q backward").

TEST INFRASTRUCTURE ONLY.  Only ``tests/`` (and ``bench.py``'s ``cpu_baseline`` leg) may
import or call this module.  It shares no code with the HIP path.  Plain float64 NumPy.

Sources:
  [kucoin] "Cursor's MoK logra un aumento del 2.37x ..." (kucoin.com/es), section 01
           (training adds a backward pass), section 02 (MXFP8 quantisation fused into the
           expert data path; the backward's pull reverse-combine and push reverse-dispatch).

The pages name MXFP8 and the backward but give neither the backward's quantisation points
nor its rule.  Reading (listed with the design notes): the backward is the bf16 backward of
``moe_oracle_bwd`` with every operand of its two data-gradient GEMMs quantised by the OCP MX
rule of ``mx_oracle`` in blocks of 32 along that GEMM's K:
  * dh = dO W2:         dO along d (rows), W2 along d (its columns: W2^T quantised by rows);
  * dX = da W1 + db W3: da, db along F (rows), W1 and W3 along F (their columns);
  * a = x W1^T, b = x W3^T are the forward's MXFP8 products (x along d, W1 and W3 along d);
  * the weight gradients dW1 = da^T x, dW3 = db^T x, dW2 = dO^T h contract over an expert's
    rows, where 32-row blocks would straddle experts, and stay unquantised (bf16 on the GPU);
  * h in dW2 is the unquantised silu(a) * b (the quantised h only feeds the forward output).
The forward steps (routing, gates, and ye for dg = <dY, o>) are Oracle-Q's, written out
here because the backward needs its a and b (checked equal to ``forward_q``).

Parity status: pinned by tests/test_mx_oracle_bwd.py -- with the identity in place of the
quantiser it equals the pinned bf16 backward oracle; each data-gradient GEMM equals a
brute-force block-by-block MX product written independently in the test (which also fixes
the quantisation axis of every operand); and its error against the exact backward lies in
the band the MX forward's does.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as O
from . import moe_oracle_bwd as B
from . import mx_oracle as MX


def mx_rows(a: np.ndarray) -> np.ndarray:
    """Dequantised MX quantisation of a along its last axis (blocks of 32)."""
    return MX.quantize(np.asarray(a, dtype=np.float64))[2]


def weights_q(w1, w3, w2, E_local, q=mx_rows):
    """Every quantised weight the MX forward and backward use, per local expert:
    forward orientation (W1, W3 along d; W2 along F) and backward orientation (W2 along
    d; W1, W3 along F), all dequantised, float64."""
    qc = (lambda w: q(np.asarray(w, dtype=np.float64).T).T)
    out = {"w1q": [], "w3q": [], "w2q": [], "w2q_d": [], "w1q_f": [], "w3q_f": []}
    for l in range(E_local):
        W1 = np.asarray(w1[l], dtype=np.float64)
        W3 = np.asarray(w3[l], dtype=np.float64)
        W2 = np.asarray(w2[l], dtype=np.float64)
        out["w1q"].append(q(W1))
        out["w3q"].append(q(W3))
        out["w2q"].append(q(W2))
        out["w2q_d"].append(qc(W2))
        out["w1q_f"].append(qc(W1))
        out["w3q_f"].append(qc(W3))
    return out


def backward_q(logits, x, w1, w3, w2, expert_to_local, E_local, k, dy, minibatch=128, q=mx_rows, W=None) -> dict:
    """Gradients of L = sum <dy, y> through the MXFP8 share (see the module notes).

    w1, w3 [E_local][F][d] and w2 [E_local][d][F] are the unquantised (bf16) weights; q is
    the row quantiser (MX by default; the identity reduces this to the bf16 backward).  W,
    if given, is weights_q(w1, w3, w2, E_local, q) computed beforehand."""
    if W is None:
        W = weights_q(w1, w3, w2, E_local, q)
    # forward: routing, layout, MX x, SwiGLU with MX h, merge
    idx, gates = O.route(logits, k)
    lay = O.layout(idx, expert_to_local, E_local, minibatch)
    xe = O.dispatch(x, lay["pull_src"])
    xeq = q(xe)
    N = xe.shape[0]
    dy = np.asarray(dy, dtype=np.float64)
    R, T, d = dy.shape
    E = np.asarray(logits).shape[2]
    F = W["w1q"][0].shape[0] if E_local > 0 else 0
    off, pull_src, slot_of = lay["offsets"], lay["pull_src"], lay["slot_of"]
    a = np.zeros((N, F))
    b = np.zeros((N, F))
    ye = np.zeros((N, d))
    for l in range(E_local):
        lo, hi = int(off[l]), int(off[l + 1])
        if hi == lo:
            continue
        a[lo:hi] = xeq[lo:hi] @ W["w1q"][l].T
        b[lo:hi] = xeq[lo:hi] @ W["w3q"][l].T
        ye[lo:hi] = q(O.silu(a[lo:hi]) * b[lo:hi]) @ W["w2q"][l].T

    # pull reverse-combine
    dO = np.zeros((N, d))
    dg = np.zeros(N)
    for s in range(N):
        r, t = int(pull_src[s, 0]), int(pull_src[s, 1])
        j = B.pair_j(slot_of, s, r, t)
        dO[s] = gates[r, t, j] * dy[r, t]
        dg[s] = dy[r, t] @ ye[s]
    dOq = q(dO)

    # expert backward: MX data-gradient GEMMs, unquantised weight gradients
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
        al, bl = a[lo:hi], b[lo:hi]
        sa = O.silu(al)
        h[lo:hi] = sa * bl
        dh[lo:hi] = dOq[lo:hi] @ W["w2q_d"][l]
        db[lo:hi] = dh[lo:hi] * sa
        da[lo:hi] = dh[lo:hi] * bl * B.silu_grad(al)
        dX[lo:hi] = q(da[lo:hi]) @ W["w1q_f"][l] + q(db[lo:hi]) @ W["w3q_f"][l]
        dw1[l] = da[lo:hi].T @ xe[lo:hi]
        dw3[l] = db[lo:hi].T @ xe[lo:hi]
        dw2[l] = dO[lo:hi].T @ h[lo:hi]

    # push reverse-dispatch, ordered sum, gate gradients
    dx = np.zeros((R, T, d))
    dlogits = np.zeros((R, T, E))
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
    out = dict(lay)
    out.update(idx=idx, gates=gates, xe=xe, xeq=xeq, ye=ye, a=a, b=b, dO=dO, dOq=dOq, dg=dg, h=h, dh=dh, da=da,
               db=db, dX=dX, dx=dx, dw1=dw1, dw3=dw3, dw2=dw2, dlogits=dlogits, weights=W)
    return out
