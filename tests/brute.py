"""Brute-force MoE forward for tiny shapes, in pure Python floats.

It shares nothing with the oracle: the gate is the literal reading (softmax over
all E experts, keep the k largest probabilities by repeated scanning, renormalise),
every local expert is evaluated on every token with explicit loops, and the
outputs are masked to the chosen experts.  Used only to pin the oracle.
"""
import math


def literal_gates(logit_row, k):
    E = len(logit_row)
    m = max(logit_row)
    p = [math.exp(float(v) - m) for v in logit_row]
    z = sum(p)
    p = [v / z for v in p]
    chosen = []
    for _ in range(k):
        best = -1
        for e in range(E):
            if e in chosen:
                continue
            # strict '>' keeps the lower id on ties; compare on the logits, which
            # order the same way as the probabilities but cannot tie spuriously
            if best < 0 or float(logit_row[e]) > float(logit_row[best]):
                best = e
        chosen.append(best)
    s = sum(p[e] for e in chosen)
    return chosen, [p[e] / s for e in chosen]


def ffn_loops(xrow, w1, w3, w2):
    F = len(w1)
    d = len(xrow)
    h = []
    for f in range(F):
        a = 0.0
        b = 0.0
        for i in range(d):
            a += float(w1[f][i]) * float(xrow[i])
            b += float(w3[f][i]) * float(xrow[i])
        h.append(a / (1.0 + math.exp(-a)) * b)
    out = []
    for i in range(d):
        acc = 0.0
        for f in range(F):
            acc += float(w2[i][f]) * h[f]
        out.append(acc)
    return out


def brute_forward(logits, x, w1, w3, w2, expert_to_local, k):
    """y[r][t] as nested lists; every local expert runs on every token, then masks."""
    R, T = len(logits), len(logits[0])
    E = len(expert_to_local)
    d = len(x[0][0])
    y = []
    for r in range(R):
        yr = []
        for t in range(T):
            chosen, g = literal_gates([float(v) for v in logits[r][t]], k)
            acc = [0.0] * d
            for e in range(E):
                l = int(expert_to_local[e])
                if l < 0:
                    continue
                o = ffn_loops(x[r][t], w1[l], w3[l], w2[l])
                mask = 1.0 if e in chosen else 0.0
                ge = g[chosen.index(e)] if e in chosen else 0.0
                acc = [a + mask * ge * v for a, v in zip(acc, o)]
            yr.append(acc)
        y.append(yr)
    return y
