"""Thin ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmoe.so.  Tensors are torch device tensors (PyTorch is used for device memory
and streams); each function takes the same arguments as its C namesake and
raises MoEError on a non-zero return code.  There is no fallback: importing the
binding without the built library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}
MOE_MAX_RANKS = 64
ERRORS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EALIGN", -3: "MOE_ENOSPC", -4: "MOE_EHIP",
          -5: "MOE_ETIMEOUT", -6: "MOE_EUNSUP", -7: "MOE_EINCOMPLETE"}

# every symbol include/moe.h declares
EXPORTS = ["moe_max_pairs", "moe_workspace_bytes", "moe_mx_quantize", "moe_layout", "moe_dispatch_pull",
           "moe_expert_ffn", "moe_expert_ffn_push", "moe_weighted_merge", "moe_combine_push", "moe_forward",
           "moe_forward_fused", "moe_forward_persistent", "moe_persistent_dispatch_ffn_combine",
           "moe_forward_persistent_noalloc", "moe_ring_slot_bytes", "moe_persistent_workspace_bytes", "moe_persistent_trace_info",
           "moe_persistent_resident_info",
           "moe_backward_workspace_bytes",
           "moe_combine_pull_reverse", "moe_expert_ffn_backward",
           "moe_dispatch_push_reverse", "moe_backward", "moe_backward_ring", "moe_backward_prepare_mx",
           "moe_backward_mx",
           "moe_signal_probe_bytes", "moe_signal_probe", "moe_ceiling_probe_bytes", "moe_ceiling_probe",
           "moe_read_status", "moe_strerror", "moe_version"]


class MoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({strerror(code)})")


class Shape(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("T", ctypes.c_int32), ("d", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("F", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Placement(ctypes.Structure):
    _fields_ = [("expert_to_local", ctypes.c_void_p), ("E_local", ctypes.c_int32)]


class MXScales(ctypes.Structure):
    """moe_mx_scales_t: device pointers of the E8M0 block scales of w1, w3, w2."""
    _fields_ = [("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class Exec(ctypes.Structure):
    _fields_ = [("minibatch_rows", ctypes.c_int32), ("comm_cus", ctypes.c_int32),
                ("ring_slots", ctypes.c_int32), ("trace", ctypes.c_int32),
                ("watchdog_us", ctypes.c_uint64), ("reverse_ring", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe.so not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, I32, SZ = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        S, PL, EX, MS = P(Shape), P(Placement), P(Exec), P(MXScales)
        L.moe_max_pairs.argtypes = [S, PL]
        L.moe_max_pairs.restype = ctypes.c_int64
        L.moe_workspace_bytes.argtypes = [S, PL, EX]
        L.moe_workspace_bytes.restype = SZ
        L.moe_mx_quantize.argtypes = [VP, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, VP, VP, VP]
        L.moe_layout.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_dispatch_pull.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_expert_ffn.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, MS, VP, VP, SZ, VP]
        L.moe_expert_ffn_push.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, VP, MS, VP, VP, VP, VP, SZ, VP]
        L.moe_weighted_merge.argtypes = [S, PL, VP, VP, VP, VP, VP]
        L.moe_combine_push.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_forward_fused.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, MS, VP, VP, VP, VP,
                                        VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_forward.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, MS, VP, VP, VP, VP, VP,
                                  VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_forward_persistent.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, VP, SZ, VP, VP,
                                             VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_persistent_dispatch_ffn_combine.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, SZ, VP, VP, VP, VP,
                                                          VP, SZ, VP]
        L.moe_forward_persistent_noalloc.argtypes = [S, PL, EX, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP,
                                                     VP, VP, VP]
        L.moe_ring_slot_bytes.argtypes = [S, EX]
        L.moe_ring_slot_bytes.restype = SZ
        L.moe_persistent_workspace_bytes.argtypes = [S, PL, EX]
        L.moe_persistent_workspace_bytes.restype = SZ
        L.moe_persistent_trace_info.argtypes = [S, PL, EX, P(SZ), P(ctypes.c_int32), P(ctypes.c_int32)]
        L.moe_persistent_trace_info.restype = I32
        L.moe_persistent_resident_info.argtypes = [S, PL, P(SZ), P(ctypes.c_int32)]
        L.moe_persistent_resident_info.restype = I32
        L.moe_backward_workspace_bytes.argtypes = [S, PL]
        L.moe_backward_workspace_bytes.restype = SZ
        L.moe_combine_pull_reverse.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, SZ, VP, SZ, VP]
        L.moe_expert_ffn_backward.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, SZ, VP, VP, VP, VP, SZ, VP]
        L.moe_dispatch_push_reverse.argtypes = [S, PL, VP, VP, VP, VP, VP, SZ, VP, VP, VP, VP, SZ, VP]
        L.moe_backward.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ,
                                   VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_backward_ring.argtypes = [S, PL, EX, VP, VP, VP, SZ, VP, SZ, VP, VP, VP, VP, VP, VP, VP, VP,
                                        VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_backward_prepare_mx.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, VP, VP]
        L.moe_backward_mx.argtypes = [S, PL, VP, VP, VP, VP, VP, VP, VP, MS, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP,
                                      SZ, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_signal_probe_bytes.argtypes = [I32]
        L.moe_signal_probe_bytes.restype = SZ
        L.moe_signal_probe.argtypes = [I32, I32, I32, I32, VP, SZ, VP, VP, VP, VP, VP]
        L.moe_ceiling_probe_bytes.argtypes = []
        L.moe_ceiling_probe_bytes.restype = SZ
        L.moe_ceiling_probe.argtypes = [I32, I32, VP, SZ, VP, SZ, VP, VP, VP]
        L.moe_read_status.argtypes = [VP, VP]
        L.moe_strerror.argtypes = [I32]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_version.restype = ctypes.c_char_p
        for f in ("moe_mx_quantize", "moe_layout", "moe_dispatch_pull", "moe_expert_ffn", "moe_combine_push",
                  "moe_expert_ffn_push", "moe_weighted_merge", "moe_forward_fused",
                  "moe_forward", "moe_forward_persistent", "moe_persistent_dispatch_ffn_combine",
                  "moe_forward_persistent_noalloc",
                  "moe_combine_pull_reverse", "moe_expert_ffn_backward", "moe_dispatch_push_reverse", "moe_backward", "moe_backward_prepare_mx",
                  "moe_backward_ring", "moe_backward_mx", "moe_signal_probe", "moe_ceiling_probe", "moe_read_status"):
            getattr(L, f).restype = I32
        _lib = L
    return _lib


# --------------------------------------------------------------------------- marshalling
def _p(t):
    """Device pointer of a tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _table(ts):
    """Host array of R device pointers."""
    if ts is None:
        return None
    ptrs = [_p(t) for t in ts]
    return ctypes.cast((ctypes.c_void_p * len(ptrs))(*ptrs), ctypes.c_void_p)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> int:
    if rc != 0:
        raise MoEError(rc, where)
    return rc


def strerror(code: int) -> str:
    return lib().moe_strerror(int(code)).decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_max_pairs(shape: Shape, placement: Placement) -> int:
    return int(lib().moe_max_pairs(ctypes.byref(shape), ctypes.byref(placement)))


def moe_workspace_bytes(shape: Shape, placement: Placement, ex: Exec | None = None) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape), ctypes.byref(placement),
                                         ctypes.byref(ex) if ex is not None else None))


def _ref(st):
    return ctypes.byref(st) if st is not None else None


def moe_mx_quantize(src, src_dtype, rows, K, codes, scales, stream=None, check=True):
    rc = lib().moe_mx_quantize(_p(src), int(src_dtype), int(rows), int(K), _p(codes), _p(scales), _stream(stream))
    return _check(rc, "moe_mx_quantize") if check else rc


def moe_layout(shape, placement, ex, logits, topk_idx, topk_w, counts, offsets, pull_src, slot_of,
               ws, ws_bytes=None, stream=None, check=True):
    rc = lib().moe_layout(ctypes.byref(shape), ctypes.byref(placement),
                          ctypes.byref(ex) if ex is not None else None, _table(logits), _p(topk_idx),
                          _p(topk_w), _p(counts), _p(offsets), _p(pull_src), _p(slot_of), _p(ws),
                          ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_layout") if check else rc


def moe_dispatch_pull(shape, placement, x, pull_src, offsets, xe, ws, ws_bytes=None, stream=None,
                      check=True, xe_scales=None):
    rc = lib().moe_dispatch_pull(ctypes.byref(shape), ctypes.byref(placement), _table(x), _p(pull_src),
                                 _p(offsets), _p(xe), _p(xe_scales), _p(ws),
                                 ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_dispatch_pull") if check else rc


def moe_expert_ffn(shape, placement, ex, xe, offsets, w1, w3, w2, ye, ws, ws_bytes=None, stream=None,
                   check=True, xe_scales=None, w_scales=None):
    rc = lib().moe_expert_ffn(ctypes.byref(shape), ctypes.byref(placement), _ref(ex), _p(xe), _p(xe_scales),
                              _p(offsets), _p(w1), _p(w3), _p(w2), _ref(w_scales), _p(ye), _p(ws),
                              ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_expert_ffn") if check else rc


def moe_expert_ffn_push(shape, placement, ex, xe, offsets, w1, w3, w2, pull_src, slot_of, recv, ws, ws_bytes=None,
                        stream=None, check=True, xe_scales=None, w_scales=None, x=None):
    rc = lib().moe_expert_ffn_push(ctypes.byref(shape), ctypes.byref(placement), _ref(ex), _table(x), _p(xe),
                                   _p(xe_scales),
                                   _p(offsets), _p(w1), _p(w3), _p(w2), _ref(w_scales), _p(pull_src), _p(slot_of),
                                   _table(recv), _p(ws), ws.numel() if ws_bytes is None else ws_bytes,
                                   _stream(stream))
    return _check(rc, "moe_expert_ffn_push") if check else rc


def moe_weighted_merge(shape, placement, slot_of, topk_w, recv, y, stream=None, check=True):
    rc = lib().moe_weighted_merge(ctypes.byref(shape), ctypes.byref(placement), _p(slot_of), _p(topk_w),
                                  _table(recv), _table(y), _stream(stream))
    return _check(rc, "moe_weighted_merge") if check else rc


def moe_combine_push(shape, placement, ye, pull_src, slot_of, topk_w, offsets, recv, y, ws, ws_bytes=None,
                     stream=None, check=True):
    rc = lib().moe_combine_push(ctypes.byref(shape), ctypes.byref(placement), _p(ye), _p(pull_src),
                                _p(slot_of), _p(topk_w), _p(offsets), _table(recv), _table(y), _p(ws),
                                ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_combine_push") if check else rc


def moe_forward(shape, placement, ex, logits, x, w1, w3, w2, xe, ye, recv, y, topk_idx, topk_w, counts,
                offsets, pull_src, slot_of, ws, ws_bytes=None, stream=None, check=True, w_scales=None,
                xe_scales=None):
    rc = lib().moe_forward(ctypes.byref(shape), ctypes.byref(placement), _ref(ex), _table(logits), _table(x),
                           _p(w1), _p(w3), _p(w2), _ref(w_scales), _p(xe), _p(xe_scales), _p(ye), _table(recv),
                           _table(y), _p(topk_idx),
                           _p(topk_w), _p(counts), _p(offsets), _p(pull_src), _p(slot_of), _p(ws),
                           ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_forward") if check else rc


def moe_forward_fused(shape, placement, ex, logits, x, w1, w3, w2, xe, recv, y, topk_idx, topk_w, counts,
                      offsets, pull_src, slot_of, ws, ws_bytes=None, stream=None, check=True, w_scales=None,
                      xe_scales=None):
    rc = lib().moe_forward_fused(ctypes.byref(shape), ctypes.byref(placement), _ref(ex), _table(logits), _table(x),
                                 _p(w1), _p(w3), _p(w2), _ref(w_scales), _p(xe), _p(xe_scales), _table(recv),
                                 _table(y), _p(topk_idx), _p(topk_w), _p(counts), _p(offsets), _p(pull_src),
                                 _p(slot_of), _p(ws), ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_forward_fused") if check else rc


def moe_forward_persistent(shape, placement, ex, logits, x, w1, w3, w2, ring, recv, y, topk_idx, topk_w,
                           counts, offsets, pull_src, slot_of, ws, ring_bytes=None, ws_bytes=None, stream=None,
                           check=True, w_scales=None):
    rc = lib().moe_forward_persistent(ctypes.byref(shape), ctypes.byref(placement),
                                      ctypes.byref(ex) if ex is not None else None, _table(logits), _table(x),
                                      _p(w1), _p(w3), _p(w2), _ref(w_scales), _p(ring),
                                      ring.numel() if ring_bytes is None else ring_bytes, _table(recv),
                                      _table(y), _p(topk_idx), _p(topk_w), _p(counts), _p(offsets),
                                      _p(pull_src), _p(slot_of), _p(ws),
                                      ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_forward_persistent") if check else rc


def moe_persistent_dispatch_ffn_combine(shape, placement, ex, x, w1, w3, w2, ring, pull_src, slot_of, offsets, recv,
                                        ws, ring_bytes=None, ws_bytes=None, stream=None, check=True, w_scales=None):
    rc = lib().moe_persistent_dispatch_ffn_combine(ctypes.byref(shape), ctypes.byref(placement),
                                                   ctypes.byref(ex) if ex is not None else None, _table(x), _p(w1),
                                                   _p(w3), _p(w2), _ref(w_scales), _p(ring),
                                                   ring.numel() if ring_bytes is None else ring_bytes,
                                                   _p(pull_src), _p(slot_of), _p(offsets), _table(recv), _p(ws),
                                                   ws.numel() if ws_bytes is None else ws_bytes, _stream(stream))
    return _check(rc, "moe_persistent_dispatch_ffn_combine") if check else rc


NOALLOC_SCRATCH_BYTES = 128 << 20
NOALLOC_WORKSPACE_BYTES = 8 << 20


def moe_forward_persistent_noalloc(shape, placement, ex, logits, x, w1, w3, w2, recv, y, topk_idx, topk_w, counts,
                                   offsets, pull_src, slot_of, status=None, stream=None, check=True):
    rc = lib().moe_forward_persistent_noalloc(ctypes.byref(shape), ctypes.byref(placement),
                                              ctypes.byref(ex) if ex is not None else None, _table(logits), _table(x),
                                              _p(w1), _p(w3), _p(w2), _table(recv), _table(y), _p(topk_idx),
                                              _p(topk_w), _p(counts), _p(offsets), _p(pull_src), _p(slot_of),
                                              _p(status), _stream(stream))
    return _check(rc, "moe_forward_persistent_noalloc") if check else rc


def moe_ring_slot_bytes(shape: Shape, ex: Exec | None = None) -> int:
    return int(lib().moe_ring_slot_bytes(ctypes.byref(shape), ctypes.byref(ex) if ex is not None else None))


def moe_persistent_workspace_bytes(shape: Shape, placement: Placement, ex: Exec | None = None) -> int:
    return int(lib().moe_persistent_workspace_bytes(ctypes.byref(shape), ctypes.byref(placement),
                                                    ctypes.byref(ex) if ex is not None else None))


# one moe_trace_event_t (include/moe.h), as a numpy structured dtype
TRACE_EVENT_FIELDS = [("t_begin", "<i8"), ("t_end", "<i8"), ("t_wait", "<i4"), ("index", "<i4"),
                      ("workgroup", "<i4"), ("kind", "<i2"), ("pipeline", "<i2")]
TRACE_KINDS = {0: "start", 1: "gather", 2: "push", 3: "gate_up", 4: "down", 5: "end"}


def moe_persistent_trace_info(shape: Shape, placement: Placement, ex: Exec):
    """(byte offset of the trace in the workspace, event capacity, ticks per us)."""
    off, cap, tpu = ctypes.c_size_t(), ctypes.c_int32(), ctypes.c_int32()
    rc = lib().moe_persistent_trace_info(ctypes.byref(shape), ctypes.byref(placement), ctypes.byref(ex),
                                         ctypes.byref(off), ctypes.byref(cap), ctypes.byref(tpu))
    _check(rc, "moe_persistent_trace_info")
    return int(off.value), int(cap.value), int(tpu.value)


def read_trace(ws, shape: Shape, placement: Placement, ex: Exec):
    """Copy the persistent kernel's trace out of the workspace tensor: (events, ticks per us).
    Host-side parsing only (numpy structured array of the recorded events)."""
    import numpy as np
    off, cap, tpu = moe_persistent_trace_info(shape, placement, ex)
    n = int(ws[off:off + 4].cpu().numpy().view(np.int32)[0])
    n = min(n, cap)
    dt = np.dtype(TRACE_EVENT_FIELDS)
    raw = ws[off + 256: off + 256 + n * dt.itemsize].cpu().numpy()
    return raw.view(dt).copy(), tpu


def moe_backward_workspace_bytes(shape: Shape, placement: Placement) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(shape), ctypes.byref(placement)))


def moe_combine_pull_reverse(shape, placement, dy, ye, pull_src, slot_of, topk_w, ws, bws, ws_bytes=None,
                             bws_bytes=None, stream=None, check=True):
    rc = lib().moe_combine_pull_reverse(ctypes.byref(shape), ctypes.byref(placement), _table(dy), _p(ye),
                                        _p(pull_src), _p(slot_of), _p(topk_w), _p(ws),
                                        ws.numel() if ws_bytes is None else ws_bytes, _p(bws),
                                        bws.numel() if bws_bytes is None else bws_bytes, _stream(stream))
    return _check(rc, "moe_combine_pull_reverse") if check else rc


def moe_expert_ffn_backward(shape, placement, xe, offsets, w1, w3, w2, ws, dw1, dw3, dw2, bws,
                            ws_bytes=None, bws_bytes=None, stream=None, check=True):
    rc = lib().moe_expert_ffn_backward(ctypes.byref(shape), ctypes.byref(placement), _p(xe), _p(offsets), _p(w1),
                                       _p(w3), _p(w2), _p(ws),
                                       ws.numel() if ws_bytes is None else ws_bytes, _p(dw1), _p(dw3), _p(dw2),
                                       _p(bws), bws.numel() if bws_bytes is None else bws_bytes, _stream(stream))
    return _check(rc, "moe_expert_ffn_backward") if check else rc


def moe_dispatch_push_reverse(shape, placement, pull_src, slot_of, topk_idx, topk_w, ws, recv, dx, dlogits, bws,
                              ws_bytes=None, bws_bytes=None, stream=None, check=True):
    rc = lib().moe_dispatch_push_reverse(ctypes.byref(shape), ctypes.byref(placement), _p(pull_src), _p(slot_of),
                                         _p(topk_idx), _p(topk_w), _p(ws),
                                         ws.numel() if ws_bytes is None else ws_bytes, _table(recv), _table(dx),
                                         _table(dlogits), _p(bws), bws.numel() if bws_bytes is None else bws_bytes,
                                         _stream(stream))
    return _check(rc, "moe_dispatch_push_reverse") if check else rc


def moe_backward(shape, placement, dy, xe, ye, w1, w3, w2, topk_idx, topk_w, offsets, pull_src, slot_of,
                 ws, recv, dx, dlogits, dw1, dw3, dw2, bws, ws_bytes=None, bws_bytes=None, stream=None, check=True):
    rc = lib().moe_backward(ctypes.byref(shape), ctypes.byref(placement), _table(dy), _p(xe), _p(ye), _p(w1),
                            _p(w3), _p(w2), _p(topk_idx), _p(topk_w), _p(offsets), _p(pull_src),
                            _p(slot_of), _p(ws), ws.numel() if ws_bytes is None else ws_bytes, _table(recv),
                            _table(dx), _table(dlogits), _p(dw1), _p(dw3), _p(dw2), _p(bws),
                            bws.numel() if bws_bytes is None else bws_bytes, _stream(stream))
    return _check(rc, "moe_backward") if check else rc


def read_resident(ws, shape, placement):
    """The persistent forward's record of which ring slot holds each chunk (host int32 array,
    entry 4 m + h = 1 + slot, or 0)."""
    off, n = ctypes.c_size_t(), ctypes.c_int32()
    _check(lib().moe_persistent_resident_info(ctypes.byref(shape), ctypes.byref(placement), ctypes.byref(off),
                                              ctypes.byref(n)), "moe_persistent_resident_info")
    import numpy as np
    raw = ws[off.value:off.value + 4 * n.value].cpu().numpy()
    return raw.view(np.int32).copy()


def moe_backward_ring(shape, placement, ex, dy, x, ring, pws, w1, w3, w2, topk_idx, topk_w, offsets, pull_src,
                      slot_of, recv, dx, dlogits, dw1, dw3, dw2, xe, bws, ring_bytes=None, pws_bytes=None,
                      bws_bytes=None, stream=None, check=True):
    """ring = None: every token row is pulled again (nothing is read from the ring)."""
    rb = 0 if ring is None else (ring.numel() if ring_bytes is None else ring_bytes)
    rc = lib().moe_backward_ring(ctypes.byref(shape), ctypes.byref(placement), ctypes.byref(ex), _table(dy), _table(x),
                                 None if ring is None else _p(ring), rb, _p(pws),
                                 pws.numel() if pws_bytes is None else pws_bytes, _p(w1), _p(w3), _p(w2),
                                 _p(topk_idx), _p(topk_w), _p(offsets), _p(pull_src), _p(slot_of), _table(recv),
                                 _table(dx), _table(dlogits), _p(dw1), _p(dw3), _p(dw2), _p(xe), _p(bws),
                                 bws.numel() if bws_bytes is None else bws_bytes, _stream(stream))
    return _check(rc, "moe_backward_ring") if check else rc


def moe_backward_prepare_mx(shape, placement, w1, w3, w2, w2t, w2t_scales, w13t, w13t_scales, stream=None,
                            check=True):
    rc = lib().moe_backward_prepare_mx(ctypes.byref(shape), ctypes.byref(placement), _p(w1), _p(w3), _p(w2), _p(w2t),
                                       _p(w2t_scales), _p(w13t), _p(w13t_scales), _stream(stream))
    return _check(rc, "moe_backward_prepare_mx") if check else rc


def moe_backward_mx(shape, placement, dy, x, xe, xe_scales, ye, w1q, w3q, w_scales, w2t, w2t_scales, w13t,
                    w13t_scales, topk_idx, topk_w, offsets, pull_src, slot_of, ws, recv, dx, dlogits, dw1, dw3, dw2,
                    bws, ws_bytes=None, bws_bytes=None, stream=None, check=True):
    rc = lib().moe_backward_mx(ctypes.byref(shape), ctypes.byref(placement), _table(dy), _table(x), _p(xe),
                               _p(xe_scales), _p(ye), _p(w1q), _p(w3q), _ref(w_scales), _p(w2t), _p(w2t_scales),
                               _p(w13t), _p(w13t_scales), _p(topk_idx), _p(topk_w), _p(offsets), _p(pull_src),
                               _p(slot_of), _p(ws), ws.numel() if ws_bytes is None else ws_bytes, _table(recv),
                               _table(dx), _table(dlogits), _p(dw1), _p(dw3), _p(dw2), _p(bws),
                               bws.numel() if bws_bytes is None else bws_bytes, _stream(stream))
    return _check(rc, "moe_backward_mx") if check else rc


def moe_read_status(ws, stream=None) -> int:
    return int(lib().moe_read_status(_p(ws), _stream(stream)))


def moe_signal_probe_bytes(payload_words: int) -> int:
    return int(lib().moe_signal_probe_bytes(int(payload_words)))


def moe_signal_probe(cross_xcd: int, scope: int, payload_words: int, rounds: int, scratch, scratch_bytes=None,
                     stream=None, check=True):
    """Returns (rc, us_per_round, stale_words, timeouts, pairs_same_xcd)."""
    us = ctypes.c_float(0.0)
    stale, tmo, same = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    rc = lib().moe_signal_probe(int(cross_xcd), int(scope), int(payload_words), int(rounds), _p(scratch),
                                scratch.numel() if scratch_bytes is None else scratch_bytes, ctypes.byref(us),
                                ctypes.byref(stale), ctypes.byref(tmo), ctypes.byref(same), _stream(stream))
    if check:
        _check(rc, "moe_signal_probe")
    return rc, float(us.value), int(stale.value), int(tmo.value), int(same.value)


def moe_ceiling_probe_bytes() -> int:
    return int(lib().moe_ceiling_probe_bytes())


def moe_ceiling_probe(kind: int, reps: int, src, src_bytes: int, scratch, scratch_bytes=None, stream=None, check=True):
    """Returns (rc, work, ms): FLOP (kinds 0, 1) or bytes (kinds 2, 3) of the timed launch and its time."""
    work = ctypes.c_double(0.0)
    ms = ctypes.c_float(0.0)
    rc = lib().moe_ceiling_probe(int(kind), int(reps), _p(src), int(src_bytes), _p(scratch),
                                 scratch.numel() * scratch.element_size() if scratch_bytes is None else scratch_bytes,
                                 ctypes.byref(work), ctypes.byref(ms), _stream(stream))
    if check:
        _check(rc, "moe_ceiling_probe")
    return rc, float(work.value), float(ms.value)
