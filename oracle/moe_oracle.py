"""CPU oracle for one GPU's share of a Mixture-of-Experts layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP path (``mixture_experts_layer_histogram_amd``) and imports
nothing from it.  It is plain, slow and written to be checked by eye: float64
arithmetic throughout, NumPy sort and matmul as the only library primitives.

Sources (the pages this follows):
  [kucoin]   "Cursor's MoK logra un aumento del 2.37x en el rendimiento en NVIDIA
             GB300 NVL72" (kucoin.com/es news flash; also published in Vietnamese,
             Hindi and Chinese with the same sections 01/02/03).
  [qubstore] "Смесь котят: как Cursor создал открытое ядро, ускоряющее обучение
             ИИ до 2,4 раз" (qubstore.ru), paragraphs on the MoE primer, pull
             dispatch, the ring buffer and the megakernel.

Readings taken where the pages are silent (every one is listed with the
design notes):
  * gate = softmax over the k selected logits (softmax over all experts, keep the
    top k, renormalise to sum 1 -- the same numbers);
  * ties in the top-k go to the lower expert id, selection is on the raw logits;
    the k chosen ids are listed in descending logit order;
  * inside one expert's segment, rows are in ascending (rank, token, j) order of
    the (token, expert) pairs -- a stable counting order, no sort;
  * a token that picks two local experts occupies two rows (no de-duplication);
  * SwiGLU expert: h = silu(x W1^T) * (x W3^T), out = h W2^T, silu(a) = a / (1 + e^-a),
    no biases;
  * the gate weight is applied in the final weighted merge, summed over j in
    ascending order; a token with no local expert gets an all-zero output row.

Parity status: every function here is pinned by ``tests/test_oracle.py``
(brute force, closed forms, invariants and hand-worked fixtures under
``tests/golden/``).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# a1. top-k routing  [kucoin §01: the router picks several experts per token and
#     re-decides every step; qubstore, MoE primer paragraph]
# ----------------------------------------------------------------------------
def route(logits: np.ndarray, k: int):
    """Top-k expert choice and gate weights for every token.

    logits: [..., E] float32.  Returns (idx [..., k] int32, gates [..., k] float64).
    Experts are ordered by (-logit, expert id); the first k are kept.  The gate of
    the j-th kept expert is exp(l_j - l_0) / sum_i exp(l_i - l_0) over the kept ones.
    """
    l = np.asarray(logits, dtype=np.float32)
    E = l.shape[-1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # stable sort on the negated logit: equal logits keep ascending expert id
    order = np.argsort(-l.astype(np.float64), axis=-1, kind="stable")
    idx = order[..., :k].astype(np.int32)
    sel = np.take_along_axis(l, order[..., :k], axis=-1).astype(np.float64)
    z = np.exp(sel - sel[..., :1])
    gates = z / z.sum(axis=-1, keepdims=True)
    return idx, gates


# ----------------------------------------------------------------------------
# a2-a4. layout: per-expert histogram, exclusive prefix over local experts,
#     stable slot per pair, pull schedule of (source rank, source row)
#     [kucoin §01: count tokens per expert, decide where they land, keep one
#     expert's tokens together for the grouped GEMM; kucoin §02: the puller only
#     needs the source GPU and the position in the source, and chooses the local
#     placement itself; qubstore, pull paragraph: a two-column schedule built
#     without sorting]
# ----------------------------------------------------------------------------
def layout(idx: np.ndarray, expert_to_local: np.ndarray, E_local: int, minibatch: int = 128):
    """Destination rows for the (token, expert) pairs that land on this GPU.

    idx: [R][T][k] expert ids.  expert_to_local: [E] local id or -1.
    Returns a dict with
      counts   [E]          pairs routed to each global expert (all ranks)
      offsets  [E_local+1]  exclusive prefix of the local experts' counts
      pull_src [N][2]       (source rank, source token) of every local row
      slot_of  [R][T][k]    row of each pair, -1 if its expert is not local
      chunks   list of (local expert, first row, rows), <= minibatch rows each
    """
    idx = np.asarray(idx)
    R, T, k = idx.shape
    e2l = np.asarray(expert_to_local)
    E = e2l.shape[0]

    counts = np.zeros(E, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[int(e)] += 1

    local_to_global = np.full(E_local, -1, dtype=np.int64)
    for e in range(E):
        if e2l[e] >= 0:
            local_to_global[e2l[e]] = e
    offsets = np.zeros(E_local + 1, dtype=np.int64)
    for l in range(E_local):
        offsets[l + 1] = offsets[l] + counts[local_to_global[l]]
    N = int(offsets[E_local])

    pull_src = np.zeros((N, 2), dtype=np.int64)
    slot_of = np.full((R, T, k), -1, dtype=np.int64)
    seen = np.zeros(E_local, dtype=np.int64)
    for r in range(R):
        for t in range(T):
            for j in range(k):
                l = int(e2l[int(idx[r, t, j])])
                if l < 0:
                    continue
                s = int(offsets[l] + seen[l])
                seen[l] += 1
                pull_src[s] = (r, t)
                slot_of[r, t, j] = s

    chunks = []
    for l in range(E_local):
        row = int(offsets[l])
        while row < offsets[l + 1]:
            n = min(minibatch, int(offsets[l + 1]) - row)
            chunks.append((l, row, n))
            row += n
    return {"counts": counts, "offsets": offsets, "pull_src": pull_src,
            "slot_of": slot_of, "chunks": chunks, "N": N}


# ----------------------------------------------------------------------------
# a5. pull dispatch [kucoin §02: the expert side reads the rows it needs]
# ----------------------------------------------------------------------------
def dispatch(x: np.ndarray, pull_src: np.ndarray) -> np.ndarray:
    """Expert-ordered rows: row s is x[src rank][src token].  x: [R][T][d]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty((pull_src.shape[0], x.shape[2]), dtype=np.float64)
    for s, (r, t) in enumerate(pull_src):
        out[s] = x[r, t]
    return out


# ----------------------------------------------------------------------------
# a6. expert SwiGLU FFN [kucoin §01: grouped GEMM over expert-grouped input;
#     kucoin §02: SwiGLU in the expert path]
# ----------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_ffn(rows: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One expert on a block of rows.  rows [n][d]; w1, w3 [F][d]; w2 [d][F]."""
    x = np.asarray(rows, dtype=np.float64)
    a = x @ np.asarray(w1, dtype=np.float64).T
    b = x @ np.asarray(w3, dtype=np.float64).T
    h = silu(a) * b
    return h @ np.asarray(w2, dtype=np.float64).T


def expert_ffn(xe: np.ndarray, offsets: np.ndarray, w1, w3, w2) -> np.ndarray:
    """Grouped FFN: rows [offsets[l], offsets[l+1]) go through local expert l."""
    out = np.empty((xe.shape[0], w2.shape[1]), dtype=np.float64)
    for l in range(len(offsets) - 1):
        a, b = int(offsets[l]), int(offsets[l + 1])
        if b > a:
            out[a:b] = swiglu_ffn(xe[a:b], w1[l], w3[l], w2[l])
    return out


# ----------------------------------------------------------------------------
# a7-a8. push combine and final weighted merge [kucoin §01: combine returns each
#     result to the token's original position; kucoin §02: combine is a push
#     because the destination is known; kucoin §03: the final weighted merge is
#     a step of its own]
# ----------------------------------------------------------------------------
def combine_push(ye: np.ndarray, pull_src: np.ndarray, slot_of: np.ndarray) -> dict:
    """Map (r, t, j) -> expert output row for every local pair (the recv contents)."""
    recv = {}
    R, T, k = slot_of.shape
    for r in range(R):
        for t in range(T):
            for j in range(k):
                s = int(slot_of[r, t, j])
                if s >= 0:
                    assert tuple(pull_src[s]) == (r, t)
                    recv[(r, t, j)] = ye[s]
    return recv


def weighted_merge(recv: dict, gates: np.ndarray, shape) -> np.ndarray:
    """y[r, t] = sum over ascending j of g[r,t,j] * recv[r,t,j] (local pairs only)."""
    R, T, k = gates.shape
    d = shape
    y = np.zeros((R, T, d), dtype=np.float64)
    for r in range(R):
        for t in range(T):
            for j in range(k):
                if (r, t, j) in recv:
                    y[r, t] += gates[r, t, j] * recv[(r, t, j)]
    return y


def forward(logits, x, w1, w3, w2, expert_to_local, E_local, k, minibatch=128) -> dict:
    """The whole share: route, lay out, pull, FFN, push, merge.  Returns every stage."""
    idx, gates = route(logits, k)
    lay = layout(idx, expert_to_local, E_local, minibatch)
    xe = dispatch(x, lay["pull_src"])
    ye = expert_ffn(xe, lay["offsets"], w1, w3, w2)
    recv = combine_push(ye, lay["pull_src"], lay["slot_of"])
    y = weighted_merge(recv, gates, np.asarray(x).shape[2])
    out = dict(lay)
    out.update(idx=idx, gates=gates, xe=xe, ye=ye, y=y)
    return out


def token_output(x_row, idx_row, gates_row, expert_to_local, w1, w3, w2) -> np.ndarray:
    """Output row of one token computed on its own (used to sample large shapes)."""
    d = np.asarray(x_row).shape[0]
    y = np.zeros(d, dtype=np.float64)
    for j in range(len(idx_row)):
        l = int(expert_to_local[int(idx_row[j])])
        if l >= 0:
            y += gates_row[j] * swiglu_ffn(np.asarray(x_row)[None, :], w1[l], w3[l], w2[l])[0]
    return y
