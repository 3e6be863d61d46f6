"""Workload shapes for one GPU's share of a MoE layer forward.

R = emulated source ranks (each with its own token buffer), T = tokens per
rank, d = hidden size, E = global experts, E_local = experts resident here
(global ids 0..E_local-1), k = experts per token, F = expert SwiGLU width.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    R: int
    T: int
    d: int
    E: int
    E_local: int
    k: int
    F: int
    dtype: str = "bf16"          # "f32" | "bf16" | "mxfp8"
    load: str = "router"         # "router": logits = x @ W_r ; "skew": Zipf/Gumbel logits
    zipf_s: float = 1.2
    tau: float = 0.5
    ring_mib: int = 256          # ring buffer of the persistent path
    minibatch: int = 128         # rows per expert released to compute at once

    def local_experts(self):
        return list(range(self.E_local))

    @property
    def G(self) -> int:
        """GPUs the experts would be spread over in the multi-GPU layer."""
        return self.E // self.E_local

    @property
    def pairs_max(self) -> int:
        """Worst-case local (token, expert) pairs: every token picks min(k, E_local) local experts."""
        return self.R * self.T * min(self.k, self.E_local)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


# Tiny fp32 case: T=256, d=128, 8 experts (all local), top-2, F=256.
TINY = MoEConfig("tiny-fp32 T256 d128 E8 k2 F256", R=1, T=256, d=128, E=8, E_local=8, k=2,
                 F=256, dtype="f32")
# Mid bf16 case: T=4096, d=2048, 64 experts (all local), top-6, F=1408.
MID = MoEConfig("mid-bf16 T4096 d2048 E64 k6 F1408", R=1, T=4096, d=2048, E=64, E_local=64,
                k=6, F=1408, dtype="bf16")
# DeepSeek-V3-shaped one-GPU share: 8 source ranks x 4096 tokens, d=7168, 256 experts of
# which 32 are resident, top-8, F=2048, bf16, 128-row minibatches.  The persistent path's
# ring is 512 MiB: 227 slots of 128 rows (x and h rows, 2.25 MiB a slot), 28 per XCD
# pipeline, so each pipeline's ~36 chunks cycle through its slots, in groups of up to 4 row
# tiles of one expert (measured 3.52 ms/step, against 3.71 with a 256 MiB ring and groups of
# 2, whose weight panels are read about twice as often).
DSV3 = MoEConfig("dsv3-share-bf16 R8 T4096 d7168 E256/32 k8 F2048", R=8, T=4096, d=7168, E=256,
                 E_local=32, k=8, F=2048, dtype="bf16", ring_mib=512)
# Same shape with Zipf(1.2) expert popularity.
DSV3_SKEW = replace(DSV3, name="dsv3-share-bf16-zipf1.2 R8 T4096 d7168 E256/32 k8 F2048",
                    load="skew")
# Same shape with MXFP8 expert GEMMs.
DSV3_MX = replace(DSV3, name="dsv3-share-mxfp8 R8 T4096 d7168 E256/32 k8 F2048", dtype="mxfp8")

CONFIGS = {"tiny": TINY, "mid": MID, "dsv3": DSV3, "dsv3_skew": DSV3_SKEW, "dsv3_mx": DSV3_MX}
