"""Device buffers for one layer invocation (torch allocation and upload only).

``DeviceProblem`` owns every input and output tensor the C ABI needs for one
config, uploads the seeded host inputs once, and calls the binding.  No
arithmetic of the layer happens here.
"""
from __future__ import annotations

import numpy as np

from . import moe


def _to_device_store(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


class DeviceProblem:
    def __init__(self, cfg, inp, device="cuda:0", minibatch=None, alloc_outputs=True):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        dt = cfg.dtype
        self.shape = moe.Shape(cfg.R, cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, moe.DTYPE_CODE[dt])
        self.e2l = torch.from_numpy(np.ascontiguousarray(inp.expert_to_local, dtype=np.int32)).to(self.device)
        self.placement = moe.Placement(self.e2l.data_ptr(), cfg.E_local)
        self.ex = moe.Exec(minibatch or cfg.minibatch, 0, 0, 0, 0)
        self.logits = [torch.from_numpy(np.ascontiguousarray(inp.logits[r])).to(self.device)
                       for r in range(cfg.R)]
        self.x = [_to_device_store(inp.x_store[r], dt, self.device) for r in range(cfg.R)]
        self.w1 = _to_device_store(inp.w1_store, dt, self.device)
        self.w3 = _to_device_store(inp.w3_store, dt, self.device)
        self.w2 = _to_device_store(inp.w2_store, dt, self.device)
        self.w_scales = None
        if dt == "mxfp8":
            self.quantize_weights()
        self.nmax = moe.moe_max_pairs(self.shape, self.placement)
        self.ws_bytes = moe.moe_workspace_bytes(self.shape, self.placement, self.ex)
        if self.ws_bytes == 0:
            raise ValueError("shape rejected by moe_workspace_bytes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        if alloc_outputs:
            self.alloc_outputs()

    def quantize_weights(self, stream=None):
        """MXFP8 codes and block scales of the bf16 expert weights (the offline step, on the device)."""
        torch = self.torch
        self.wq, self.ws_codes = [], []
        for w in (self.w1, self.w3, self.w2):
            K = w.shape[-1]
            rows = w.numel() // K
            q = torch.empty(w.shape, dtype=torch.uint8, device=self.device)
            sc = torch.empty((K // 128, rows, 4), dtype=torch.uint8, device=self.device)   # K-tile-major
            moe.moe_mx_quantize(w, moe.MOE_BF16, rows, K, q, sc, stream=stream)
            self.wq.append(q)
            self.ws_codes.append(sc)
        self.w_scales = moe.MXScales(*(t.data_ptr() for t in self.ws_codes))

    def weights(self):
        """The weight tensors the FFN reads: bf16/fp32 rows, or MXFP8 codes."""
        return self.wq if self.cfg.dtype == "mxfp8" else (self.w1, self.w3, self.w2)

    def alloc_outputs(self):
        torch, cfg, dev = self.torch, self.cfg, self.device
        ed = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
        R, T, k, d = cfg.R, cfg.T, cfg.k, cfg.d
        self.topk_idx = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((R, T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(cfg.E_local + 1, dtype=torch.int32, device=dev)
        self.pull_src = torch.empty((self.nmax, 2), dtype=torch.int32, device=dev)
        self.slot_of = torch.empty((R, T, k), dtype=torch.int32, device=dev)
        if cfg.dtype == "mxfp8":
            self.xe = torch.empty((self.nmax, d), dtype=torch.uint8, device=dev)
            self.xe_scales = torch.empty((d // 128, self.nmax, 4), dtype=torch.uint8, device=dev)
        else:
            self.xe = torch.empty((self.nmax, d), dtype=ed, device=dev)
            self.xe_scales = None
        self.ye = torch.empty((self.nmax, d), dtype=ed, device=dev)
        self.recv = [torch.zeros((T, k, d), dtype=ed, device=dev) for _ in range(R)]
        self.y = [torch.empty((T, d), dtype=ed, device=dev) for _ in range(R)]

    # ---- the C entry points on this problem's buffers ----
    def layout(self, stream=None):
        moe.moe_layout(self.shape, self.placement, self.ex, self.logits, self.topk_idx, self.topk_w,
                       self.counts, self.offsets, self.pull_src, self.slot_of, self.ws, stream=stream)

    def dispatch(self, stream=None):
        moe.moe_dispatch_pull(self.shape, self.placement, self.x, self.pull_src, self.offsets, self.xe,
                              self.ws, stream=stream, xe_scales=self.xe_scales)

    def ffn(self, stream=None):
        w1, w3, w2 = self.weights()
        moe.moe_expert_ffn(self.shape, self.placement, self.ex, self.xe, self.offsets, w1, w3, w2, self.ye,
                           self.ws, stream=stream, xe_scales=self.xe_scales, w_scales=self.w_scales)

    def combine(self, stream=None):
        moe.moe_combine_push(self.shape, self.placement, self.ye, self.pull_src, self.slot_of, self.topk_w,
                             self.offsets, self.recv, self.y, self.ws, stream=stream)

    def ffn_push(self, stream=None, pull=False):
        """The FFN with the push fused into the down GEMM (writes recv, not ye); with pull=True
        (fp32, bf16) the gate/up GEMM also reads its rows straight from x (no xe)."""
        w1, w3, w2 = self.weights()
        moe.moe_expert_ffn_push(self.shape, self.placement, self.ex, self.xe, self.offsets, w1, w3, w2,
                                self.pull_src, self.slot_of, self.recv, self.ws, stream=stream,
                                xe_scales=self.xe_scales, w_scales=self.w_scales, x=self.x if pull else None)

    def merge(self, stream=None):
        moe.moe_weighted_merge(self.shape, self.placement, self.slot_of, self.topk_w, self.recv, self.y,
                               stream=stream)

    def forward_fused(self, stream=None):
        w1, w3, w2 = self.weights()
        moe.moe_forward_fused(self.shape, self.placement, self.ex, self.logits, self.x, w1, w3, w2, self.xe,
                              self.recv, self.y, self.topk_idx, self.topk_w, self.counts, self.offsets,
                              self.pull_src, self.slot_of, self.ws, stream=stream, w_scales=self.w_scales,
                              xe_scales=self.xe_scales)

    def forward(self, stream=None):
        w1, w3, w2 = self.weights()
        moe.moe_forward(self.shape, self.placement, self.ex, self.logits, self.x, w1, w3, w2, self.xe, self.ye,
                        self.recv, self.y, self.topk_idx, self.topk_w, self.counts, self.offsets, self.pull_src,
                        self.slot_of, self.ws, stream=stream, w_scales=self.w_scales, xe_scales=self.xe_scales)

    # ---- backward (bf16) ----
    def alloc_backward(self, dy_bits=None):
        """Backward buffers: gradients, the backward workspace, and dy."""
        torch, cfg, dev = self.torch, self.cfg, self.device
        R, T, d, E, El, F, k = cfg.R, cfg.T, cfg.d, cfg.E, cfg.E_local, cfg.F, cfg.k
        bf = torch.bfloat16
        self.dx = [torch.empty((T, d), dtype=bf, device=dev) for _ in range(R)]
        self.dlogits = [torch.empty((T, E), dtype=torch.float32, device=dev) for _ in range(R)]
        self.dw1 = torch.empty((El, F, d), dtype=bf, device=dev)
        self.dw3 = torch.empty((El, F, d), dtype=bf, device=dev)
        self.dw2 = torch.empty((El, d, F), dtype=bf, device=dev)
        self.bws_bytes = moe.moe_backward_workspace_bytes(self.shape, self.placement)
        if self.bws_bytes == 0:
            raise ValueError("shape rejected by moe_backward_workspace_bytes")
        self.bws = torch.empty(self.bws_bytes, dtype=torch.uint8, device=dev)
        if cfg.dtype == "mxfp8":
            u8 = torch.uint8
            self.w2t = torch.empty((El, F, d), dtype=u8, device=dev)
            self.w2t_scales = torch.empty((d // 128, El * F, 4), dtype=u8, device=dev)
            self.w13t = torch.empty((El, d, 2 * F), dtype=u8, device=dev)
            self.w13t_scales = torch.empty((2 * F // 128, El * d, 4), dtype=u8, device=dev)
        if dy_bits is not None:
            self.dy = [_to_device_store(dy_bits[r], "bf16", dev) for r in range(R)]

    def combine_reverse(self, stream=None):
        moe.moe_combine_pull_reverse(self.shape, self.placement, self.dy, self.ye, self.pull_src, self.slot_of,
                                     self.topk_w, self.ws, self.bws, stream=stream)

    def ffn_backward(self, stream=None):
        moe.moe_expert_ffn_backward(self.shape, self.placement, self.xe, self.offsets, self.w1, self.w3, self.w2,
                                    self.ws, self.dw1, self.dw3, self.dw2, self.bws, stream=stream)

    def dispatch_reverse(self, stream=None):
        moe.moe_dispatch_push_reverse(self.shape, self.placement, self.pull_src, self.slot_of, self.topk_idx,
                                      self.topk_w, self.ws, self.recv, self.dx, self.dlogits, self.bws, stream=stream)

    def prepare_backward_mx(self, stream=None):
        """The weights in the backward's orientation, MX-quantised (once per weight update)."""
        moe.moe_backward_prepare_mx(self.shape, self.placement, self.w1, self.w3, self.w2, self.w2t, self.w2t_scales,
                                    self.w13t, self.w13t_scales, stream=stream)

    def backward_mx(self, stream=None, check=True):
        w1q, w3q, _ = self.weights()
        return moe.moe_backward_mx(self.shape, self.placement, self.dy, self.x, self.xe, self.xe_scales, self.ye, w1q,
                                   w3q, self.w_scales, self.w2t, self.w2t_scales, self.w13t, self.w13t_scales,
                                   self.topk_idx, self.topk_w, self.offsets, self.pull_src, self.slot_of, self.ws,
                                   self.recv, self.dx, self.dlogits, self.dw1, self.dw3, self.dw2, self.bws,
                                   stream=stream, check=check)

    def backward_ring(self, use_ring=True, ex=None, stream=None, check=True):
        """moe_backward_ring after forward_persistent (same ex): token rows still in the ring are
        read there (use_ring=False pulls every row again); expert outputs come from recv; xe is
        staging for the rows not in the ring."""
        return moe.moe_backward_ring(self.shape, self.placement, ex if ex is not None else self.pex, self.dy, self.x,
                                     self.ring if use_ring else None, self.ws, self.w1, self.w3, self.w2,
                                     self.topk_idx, self.topk_w, self.offsets, self.pull_src, self.slot_of,
                                     self.recv, self.dx, self.dlogits, self.dw1, self.dw3, self.dw2, self.xe,
                                     self.bws, stream=stream, check=check)

    def backward(self, stream=None, check=True):
        return moe.moe_backward(self.shape, self.placement, self.dy, self.xe, self.ye, self.w1, self.w3, self.w2,
                                self.topk_idx, self.topk_w, self.offsets, self.pull_src, self.slot_of,
                                self.ws, self.recv, self.dx, self.dlogits, self.dw1, self.dw3, self.dw2, self.bws,
                                stream=stream, check=check)

    def alloc_ring(self, ring_mib=None, ex=None):
        """Ring buffer for the persistent path (ring_mib MiB, default the config's)."""
        torch = self.torch
        mib = self.cfg.ring_mib if ring_mib is None else ring_mib
        self.ring = torch.empty(int(mib * (1 << 20)), dtype=torch.uint8, device=self.device)
        self.pex = ex if ex is not None else self.ex
        return self.ring

    def forward_persistent(self, ex=None, stream=None, check=True):
        if not hasattr(self, "ring"):
            self.alloc_ring()
        w1, w3, w2 = self.weights()
        return moe.moe_forward_persistent(self.shape, self.placement, ex if ex is not None else self.pex,
                                          self.logits, self.x, w1, w3, w2, self.ring, self.recv,
                                          self.y, self.topk_idx, self.topk_w, self.counts, self.offsets,
                                          self.pull_src, self.slot_of, self.ws, stream=stream, check=check,
                                          w_scales=self.w_scales)

    def persistent_dfc(self, ex=None, stream=None, check=True):
        """The persistent kernel alone (dispatch, FFN, push) after layout() with the same ex."""
        if not hasattr(self, "ring"):
            self.alloc_ring()
        w1, w3, w2 = self.weights()
        return moe.moe_persistent_dispatch_ffn_combine(self.shape, self.placement, ex if ex is not None else self.pex,
                                                       self.x, w1, w3, w2, self.ring, self.pull_src,
                                                       self.slot_of, self.offsets, self.recv, self.ws, stream=stream,
                                                       check=check, w_scales=self.w_scales)

    def status(self, stream=None) -> int:
        return moe.moe_read_status(self.ws, stream)

    # ---- host copies ----
    @staticmethod
    def scales_rowmajor(t, rows=None) -> np.ndarray:
        """[rows][K/32] scale codes from a [K/128][rows][4] device array (first `rows` rows)."""
        a = t.cpu().numpy()
        kt, n, _ = a.shape
        rows = n if rows is None else rows
        return np.ascontiguousarray(a[:, :rows, :].transpose(1, 0, 2).reshape(rows, kt * 4))

    def N(self) -> int:
        return int(self.offsets[-1].item())

    @staticmethod
    def rows_f64(t) -> np.ndarray:
        """Exact float64 values of a device tensor (fp32 or bf16)."""
        return t.float().cpu().numpy().astype(np.float64)
