"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic (no routing, no layout, no FFN), so
the CPU oracle and the HIP path can both be fed from it without sharing any
computation.

Recipe (one generator per tensor, NumPy PCG64 seeded with ``[seed, tag, i]``):

* ``x_r``      ~ N(0, 1), one ``[T][d]`` buffer per source rank r.
* ``W_r``      ~ N(0, 1/d) router weights ``[d][E]``.
* router logits = fp32( fp64(x) @ fp64(W_r) ), computed here, on the host,
  because logits are an *input* of the layer's boundary (the caller owns the
  router projection).
* ``W1, W3``   ~ N(0, 1/d), ``[E_local][F][d]``;  ``W2`` ~ N(0, 1/F), ``[E_local][d][F]``.
* ``dY_r``     ~ N(0, 1), one ``[T][d]`` buffer per rank: the incoming gradient of the
  layer output for the backward (``make_dy``).
* skewed load: ``logit[t, e] = tau * ln p[pi(e)] + Gumbel(0, 1)`` with ``p`` the
  Zipf(s) distribution over popularity ranks 1..E and ``pi`` a seeded
  permutation, swapped so that the most popular expert is local.

bf16 tensors are produced by round-to-nearest-even of the fp32 draw and are
returned as raw ``uint16`` bit patterns together with their exact float32
widening, so both sides read identical bits.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor tags for the seed sequence (fixed per tensor kind)
TAG_X, TAG_WR, TAG_W1, TAG_W3, TAG_W2, TAG_GUMBEL, TAG_PERM, TAG_DY = range(8)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction (no NaN handling needed)."""
    b = np.ascontiguousarray(a, dtype=np.float32).copy().view(np.uint32)
    lsb = (b >> 16) & 1
    b += 0x7FFF
    b += lsb
    b >>= 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (u.astype(np.uint32) << 16).view(np.float32)


@dataclass
class MoEInputs:
    """Host copies of one layer invocation's inputs.

    ``*_bits`` hold the storage-format payload (uint16 bf16 patterns or float32);
    ``*_f32`` hold the exact float32 value of every stored element.
    """
    cfg: object
    logits: np.ndarray                 # [R][T][E] float32
    x_f32: np.ndarray                  # [R][T][d] float32 (exact values of x)
    w1_f32: object                     # [E_l][F][d]; indexable per expert (see Widened)
    w3_f32: object                     # [E_l][F][d]
    w2_f32: object                     # [E_l][d][F]
    expert_to_local: np.ndarray        # [E] int32, -1 = not on this GPU
    x_store: np.ndarray = field(repr=False, default=None)   # storage payload of x
    w1_store: np.ndarray = field(repr=False, default=None)
    w3_store: np.ndarray = field(repr=False, default=None)
    w2_store: np.ndarray = field(repr=False, default=None)


def _rng(seed: int, tag: int, i: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), int(i)])


def _normal_into(out: np.ndarray, seed, tag, i, std, dtype):
    """Fill ``out`` (storage type) with one N(0, std^2) tensor."""
    a = _rng(seed, tag, i).standard_normal(out.size, dtype=np.float32)
    a *= np.float32(std)
    if dtype == "f32":
        out.reshape(-1)[:] = a
    else:
        out.reshape(-1)[:] = f32_to_bf16_bits(a)


def _normal_stack(seed, tag, n, shape, std, dtype, threads):
    """n independent tensors of ``shape`` (stream i = tensor i), filled in parallel."""
    out = np.empty((n, *shape), dtype=np.float32 if dtype == "f32" else np.uint16)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(lambda i: _normal_into(out[i], seed, tag, i, std, dtype), range(n)))
    return out


class Widened:
    """Per-index exact float32 view of a bf16-bit tensor (widened on access)."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits
        self.shape = bits.shape
        self.dtype = np.float32

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, i):
        return bf16_bits_to_f32(self.bits[i])

    def __array__(self, dtype=None, copy=None):
        a = bf16_bits_to_f32(self.bits)
        return a if dtype is None else a.astype(dtype)


def _values(store: np.ndarray, dtype: str):
    return store if dtype == "f32" else Widened(store)


def make_inputs(cfg, seed: int = 0, want_f32_weights: bool = True,
                threads: int | None = None) -> MoEInputs:
    """Draw every input tensor of config ``cfg`` (see ``configs.py``)."""
    threads = threads or min(16, os.cpu_count() or 1)
    R, T, d, E, El, F = cfg.R, cfg.T, cfg.d, cfg.E, cfg.E_local, cfg.F
    st = "f32" if cfg.dtype == "f32" else "bf16"

    e2l = np.full(E, -1, dtype=np.int32)
    local_ids = np.asarray(cfg.local_experts(), dtype=np.int64)
    e2l[local_ids] = np.arange(El, dtype=np.int32)

    # token rows, one buffer per source rank
    x_store = _normal_stack(seed, TAG_X, R, (T, d), 1.0, st, threads)
    x_f32 = x_store if st == "f32" else bf16_bits_to_f32(x_store)

    if cfg.load == "skew":
        logits = skewed_logits(cfg, seed, e2l)
    else:
        wr = _rng(seed, TAG_WR).standard_normal((d, E)) / np.sqrt(d)
        logits = np.empty((R, T, E), dtype=np.float32)
        for r in range(R):
            logits[r] = (x_f32[r].astype(np.float64) @ wr).astype(np.float32)

    w1_store = _normal_stack(seed, TAG_W1, El, (F, d), 1.0 / np.sqrt(d), st, threads)
    w3_store = _normal_stack(seed, TAG_W3, El, (F, d), 1.0 / np.sqrt(d), st, threads)
    w2_store = _normal_stack(seed, TAG_W2, El, (d, F), 1.0 / np.sqrt(F), st, threads)
    if want_f32_weights:
        w1_f32, w3_f32, w2_f32 = (_values(w, st) for w in (w1_store, w3_store, w2_store))
    else:
        w1_f32 = w3_f32 = w2_f32 = None

    return MoEInputs(cfg=cfg, logits=logits, x_f32=x_f32, w1_f32=w1_f32, w3_f32=w3_f32,
                     w2_f32=w2_f32, expert_to_local=e2l, x_store=x_store,
                     w1_store=w1_store, w3_store=w3_store, w2_store=w2_store)


def make_dy(cfg, seed: int = 0, threads: int | None = None):
    """Incoming gradient of y: ([R][T][d] bf16 bits, their exact float32 values)."""
    threads = threads or min(16, os.cpu_count() or 1)
    bits = _normal_stack(seed, TAG_DY, cfg.R, (cfg.T, cfg.d), 1.0, "bf16", threads)
    return bits, bf16_bits_to_f32(bits)


def zipf_probs(E: int, s: float) -> np.ndarray:
    """Zipf(s) probabilities over popularity ranks 1..E."""
    w = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    return w / w.sum()


def skewed_logits(cfg, seed: int, e2l: np.ndarray) -> np.ndarray:
    """Gumbel-perturbed Zipf log-popularities (a seeded, skewed expert load)."""
    R, T, E = cfg.R, cfg.T, cfg.E
    p = zipf_probs(E, cfg.zipf_s)
    perm = _rng(seed, TAG_PERM).permutation(E)      # expert e has popularity rank perm[e]
    hot = int(np.argmin(perm))                      # expert holding rank 1
    if e2l[hot] < 0:                                # make the hottest expert local
        first_local = int(np.flatnonzero(e2l >= 0)[0])
        perm[hot], perm[first_local] = perm[first_local], perm[hot]
    base = cfg.tau * np.log(p[perm])                # [E]
    g = _rng(seed, TAG_GUMBEL).gumbel(size=(R, T, E))
    return (base[None, None, :] + g).astype(np.float32)


def random_logits(shape, seed: int = 0, tag: int = 99) -> np.ndarray:
    """Plain N(0,1) fp32 logits (used by layout-only cases)."""
    return _rng(seed, tag).standard_normal(shape).astype(np.float32)
