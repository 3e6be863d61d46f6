"""C-ABI host-side tests (no GPU): the library loads, exports what include/moe.h
declares, sizes its workspace, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_histogram_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# aligned fake device addresses: every call below must fail its checks before using them
FAKE = 0x7F0000000000


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    declared = _declared_symbols()
    assert declared, "no declarations parsed"
    assert set(declared) == set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_strerror():
    assert "gfx950" in moe.moe_version()
    for code in moe.ERRORS:
        assert moe.strerror(code)
    assert moe.strerror(-99) == "unknown error"


def _shape(**kw):
    d = dict(R=8, T=4096, d=7168, E=256, k=8, F=2048, dtype=moe.MOE_BF16)
    d.update(kw)
    return moe.Shape(d["R"], d["T"], d["d"], d["E"], d["k"], d["F"], d["dtype"])


def _pl(El=32):
    return moe.Placement(FAKE, El)


def test_max_pairs_and_workspace():
    s, p = _shape(), _pl()
    assert moe.moe_max_pairs(s, p) == 8 * 4096 * 8
    assert moe.moe_max_pairs(_shape(k=8), _pl(4)) == 8 * 4096 * 4
    ws = moe.moe_workspace_bytes(s, p)
    # the GEMM1 output staging (max pairs x F bf16) dominates
    assert ws >= 8 * 4096 * 8 * 2048 * 2
    assert ws % 256 == 0
    assert moe.moe_workspace_bytes(_shape(T=8192), p) > ws
    assert moe.moe_workspace_bytes(_shape(k=0), p) == 0


@pytest.mark.parametrize("kw,El,code", [
    (dict(k=0), 32, -1),
    (dict(k=17, E=256), 32, -1),
    (dict(k=9, E=8), 8, -1),
    (dict(E=2048), 32, -1),
    (dict(R=65), 32, -1),
    (dict(T=0), 32, -1),
    (dict(), 0, -1),
    (dict(), 300, -1),
    (dict(dtype=7), 32, -1),
    (dict(dtype=moe.MOE_MXFP8, d=7168 + 64), 32, -2),   # MXFP8 GEMM stage needs d % 128 == 0
    (dict(dtype=moe.MOE_MXFP8, F=2048 + 64), 32, -2),
    (dict(d=7160), 32, -2),                         # bf16 K step needs d % 64 == 0
    (dict(F=2000), 32, -2),
    (dict(d=130, dtype=moe.MOE_F32), 32, -2),       # fp32 row of 520 B is not 16-byte aligned
])
def test_bad_shapes_rejected_before_launch(kw, El, code):
    s, p = _shape(**kw), _pl(El)
    tab = (ctypes.c_void_p * 64)(*([FAKE] * 64))
    rc = moe.lib().moe_layout(ctypes.byref(s), ctypes.byref(p), None, ctypes.cast(tab, ctypes.c_void_p),
                              FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == code


def test_null_and_misaligned_pointers_rejected():
    s, p = _shape(), _pl()
    L = moe.lib()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    # null output
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), None, tabp, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                        FAKE, big, None) == -1
    # null placement map
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(moe.Placement(None, 32)), None, tabp, FAKE, FAKE,
                        FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    # null rank pointer
    tab2 = (ctypes.c_void_p * 8)(*([FAKE] * 7 + [None]))
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), None, ctypes.cast(tab2, ctypes.c_void_p), FAKE,
                        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    # misaligned rank pointer / workspace / row buffer
    tab3 = (ctypes.c_void_p * 8)(*([FAKE] * 7 + [FAKE + 4]))
    assert L.moe_dispatch_pull(ctypes.byref(s), ctypes.byref(p), ctypes.cast(tab3, ctypes.c_void_p), FAKE,
                               FAKE, FAKE, None, FAKE, big, None) == -2
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), None, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE + 64, big, None) == -2
    assert L.moe_dispatch_pull(ctypes.byref(s), ctypes.byref(p), tabp, FAKE, FAKE, FAKE + 8, None, FAKE, big,
                               None) == -2
    # workspace too small
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), None, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, 1024, None) == -3
    assert L.moe_expert_ffn(ctypes.byref(s), ctypes.byref(p), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, None,
                            FAKE, FAKE, 1024, None) == -3
    assert L.moe_combine_push(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, tabp, None,
                              FAKE, big, None) == -1
    # negative minibatch
    ex = moe.Exec(-1, 0, 0, 0, 0)
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), tabp, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, FAKE, big, None) == -1
    assert L.moe_read_status(None, None) == -1


def test_forward_checks_every_stage_before_launching():
    s, p = _shape(), _pl()
    L = moe.lib()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    # y table missing: must fail up front, not after launching the layout
    rc = L.moe_forward(ctypes.byref(s), ctypes.byref(p), None, tabp, tabp, FAKE, FAKE, FAKE, None, FAKE, None,
                       FAKE, tabp, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == -1


def test_mx_quantize_rejects_bad_arguments_before_launch():
    L = moe.lib()
    q = L.moe_mx_quantize
    assert q(FAKE, moe.MOE_MXFP8, 4, 128, FAKE, FAKE, None) == -1       # source must be bf16 or fp32
    assert q(FAKE, moe.MOE_BF16, -1, 128, FAKE, FAKE, None) == -1
    assert q(FAKE, moe.MOE_BF16, 4, 0, FAKE, FAKE, None) == -1
    assert q(FAKE, moe.MOE_BF16, 4, 48, FAKE, FAKE, None) == -2         # K % 128: whole scale words
    assert q(FAKE, moe.MOE_BF16, 4, 64, FAKE, FAKE, None) == -2
    assert q(None, moe.MOE_BF16, 4, 128, FAKE, FAKE, None) == -1
    assert q(FAKE, moe.MOE_BF16, 4, 128, FAKE, None, None) == -1
    assert q(FAKE + 8, moe.MOE_BF16, 4, 128, FAKE, FAKE, None) == -2
    assert q(FAKE, moe.MOE_F32, 4, 128, FAKE + 4, FAKE, None) == -2
    assert q(FAKE, moe.MOE_BF16, 0, 128, FAKE, FAKE, None) == 0         # nothing to do, nothing launched


def test_mx_entry_points_need_their_scales():
    L = moe.lib()
    s, p = _shape(dtype=moe.MOE_MXFP8), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    ws = moe.moe_workspace_bytes(s, p)
    assert 0 < ws < moe.moe_workspace_bytes(_shape(), p)                # h is one byte per value
    ok = moe.MXScales(FAKE, FAKE, FAKE)
    assert L.moe_dispatch_pull(ctypes.byref(s), ctypes.byref(p), tabp, FAKE, FAKE, FAKE, None, FAKE, big,
                               None) == -1
    assert L.moe_dispatch_pull(ctypes.byref(s), ctypes.byref(p), tabp, FAKE, FAKE, FAKE, FAKE + 2, FAKE, big,
                               None) == -2

    def ffn(xs, wsc):
        return L.moe_expert_ffn(ctypes.byref(s), ctypes.byref(p), None, FAKE, xs, FAKE, FAKE, FAKE, FAKE,
                                ctypes.byref(wsc) if wsc is not None else None, FAKE, FAKE, 1024, None)
    assert ffn(FAKE, None) == -1
    assert ffn(None, ok) == -1
    assert ffn(FAKE, moe.MXScales(FAKE, None, FAKE)) == -1
    assert ffn(FAKE, moe.MXScales(FAKE, FAKE, FAKE + 1)) == -2
    assert ffn(FAKE, ok) == -3                                          # then the workspace check
    rc = L.moe_forward(ctypes.byref(s), ctypes.byref(p), None, tabp, tabp, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                       FAKE, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None)
    assert rc == -1
    # the persistent path takes MXFP8 weights with their scales; the ring slot holds codes and
    # scale words of the token rows and of h, each part 256-byte aligned
    def pers(wsc, ws_bytes=big):
        return L.moe_forward_persistent(ctypes.byref(s), ctypes.byref(p), None, tabp, tabp, FAKE, FAKE, FAKE,
                                        ctypes.byref(wsc) if wsc is not None else None, FAKE, big, tabp, tabp, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert pers(None) == -1
    assert pers(moe.MXScales(FAKE, FAKE, FAKE + 1)) == -2
    assert pers(ok, ws_bytes=1024) == -3
    ex = moe.Exec(128, 0, 0, 0, 0)
    slot = moe.moe_ring_slot_bytes(s, ex)
    a = lambda n: (n + 255) // 256 * 256
    assert slot == a(128 * 7168) + a(128 * 7168 // 32) + a(128 * 2048) + a(128 * 2048 // 32)
    assert moe.moe_ring_slot_bytes(_shape(dtype=moe.MOE_MXFP8, d=7168 + 64), ex) == 0    # d % 128
    # the pair address table is part of the MXFP8 workspace, reverse ring or not
    assert moe.moe_persistent_workspace_bytes(s, p, ex) == moe.moe_persistent_workspace_bytes(
        s, p, moe.Exec(128, 0, 0, 0, 0, 1))
    assert moe.moe_persistent_workspace_bytes(s, p, ex) == moe.moe_persistent_workspace_bytes(
        _shape(), p, moe.Exec(128, 0, 0, 0, 0, 1))


def test_persistent_entry_rejects_bad_arguments_before_launch():
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    slot = moe.moe_ring_slot_bytes(s, moe.Exec(128, 0, 0, 0, 0))
    assert slot == 128 * (7168 + 2048) * 2
    assert moe.moe_ring_slot_bytes(s, moe.Exec(96, 0, 0, 0, 0)) == 0
    assert 0 < moe.moe_persistent_workspace_bytes(s, p) < moe.moe_workspace_bytes(s, p)

    def call(shape=s, ex=None, ring_bytes=big, ring=FAKE, ws_bytes=big):
        return L.moe_forward_persistent(ctypes.byref(shape), ctypes.byref(p), ctypes.byref(ex) if ex else None,
                                        tabp, tabp, FAKE, FAKE, FAKE, None, ring, ring_bytes, tabp, tabp, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert call(shape=_shape(dtype=moe.MOE_F32)) == -6                 # bf16 only
    assert call(ex=moe.Exec(96, 0, 0, 0, 0)) == -6                      # chunk must divide 256
    assert call(ring_bytes=slot) == -3                                  # below one 256-row tile
    assert call(ring=FAKE + 16) == -2                                   # ring alignment
    assert call(ws_bytes=1024) == -3
    assert call(ring=None) == -1


def test_persistent_trace_layout_and_workspace():
    """The trace region sits after the persistent workspace proper; its record is 32 bytes."""
    import numpy as np
    s, p = _shape(), _pl()
    ex0, ex1 = moe.Exec(128, 16, 0, 0, 0), moe.Exec(128, 16, 0, 1, 0)
    base = moe.moe_persistent_workspace_bytes(s, p, ex0)
    with_trace = moe.moe_persistent_workspace_bytes(s, p, ex1)
    off, cap, tpu = moe.moe_persistent_trace_info(s, p, ex1)
    assert off == base and off % 256 == 0
    assert np.dtype(moe.TRACE_EVENT_FIELDS).itemsize == 32
    assert with_trace >= base + 256 + cap * 32
    # every task of the worst case fits: gathers (2 per row tile), pushes, 16 + 28 GEMM tiles
    max_mtiles = (8 * 4096 * 8 + 255) // 256 + 32
    assert cap >= max_mtiles * (2 + 1 + 16 + 28)
    assert tpu > 0
    with pytest.raises(moe.MoEError):
        moe.moe_persistent_trace_info(s, p, ex0)                       # trace must be on


def test_trace_is_rejected_outside_the_persistent_path():
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    ex = moe.Exec(128, 0, 0, 1, 0)
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), tabp, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, big, None) == -1
    assert L.moe_expert_ffn(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), FAKE, None, FAKE, FAKE, FAKE, FAKE,
                            None, FAKE, FAKE, big, None) == -1
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), tabp, tabp, FAKE, FAKE, FAKE, None,
                         FAKE, None, FAKE, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert L.moe_forward_fused(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), tabp, tabp, FAKE, FAKE, FAKE,
                               None, None, None, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                               None) == -1
    # the persistent path takes 0 or 1 only
    bad = moe.Exec(128, 0, 0, 2, 0)
    assert L.moe_forward_persistent(ctypes.byref(s), ctypes.byref(p), ctypes.byref(bad), tabp, tabp, FAKE, FAKE,
                                    FAKE, None, FAKE, big, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                    None) == -1


def test_persistent_entry_rejects_a_partition_without_compute():
    """comm_cus leaving no CU for the expert GEMMs is rejected before any launch."""
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    ex = moe.Exec(128, 4096, 0, 0, 0)
    assert L.moe_forward_persistent(ctypes.byref(s), ctypes.byref(p), ctypes.byref(ex), tabp, tabp, FAKE, FAKE,
                                    FAKE, None, FAKE, 1 << 40, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1 << 40, None) == -1


def test_backward_entry_points_reject_bad_arguments_before_launch():
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    bws = moe.moe_backward_workspace_bytes(s, p)
    assert bws > 0 and bws % 256 == 0
    # the per-row gradients (dO, dX [d]; dh, h [F]; [da|db] [2F]) dominate
    assert bws >= 8 * 4096 * 8 * (7168 * 2 + 2048 * 4) * 2
    # MXFP8 adds its codes, scales and the bf16 token rows; fp32 has no backward
    assert moe.moe_backward_workspace_bytes(_shape(dtype=moe.MOE_MXFP8), p) > bws
    assert moe.moe_backward_workspace_bytes(_shape(dtype=moe.MOE_F32), p) == 0

    def bwd(shape=s, xe=FAKE, dy=tabp, dlog=tabp, ws_bytes=big, bws_ptr=FAKE, bws_bytes=big, dw2=FAKE):
        return L.moe_backward(ctypes.byref(shape), ctypes.byref(p), dy, xe, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, FAKE, ws_bytes, tabp, tabp, dlog, FAKE, FAKE, dw2, bws_ptr,
                              bws_bytes, None)
    assert bwd(shape=_shape(dtype=moe.MOE_MXFP8)) == -6
    assert bwd(shape=_shape(k=0)) == -1
    assert bwd(xe=None) == -1
    assert bwd(xe=FAKE + 8) == -2
    assert bwd(dw2=None) == -1
    assert bwd(dy=None) == -1
    assert bwd(dlog=None) == -1
    assert bwd(ws_bytes=1024) == -3                                     # the forward's workspace
    assert bwd(bws_ptr=None) == -1
    assert bwd(bws_ptr=FAKE + 16) == -2
    assert bwd(bws_bytes=bws - 1) == -3


def test_backward_stage_entries_reject_bad_arguments_before_launch():
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    bws = moe.moe_backward_workspace_bytes(s, p)
    mx = _shape(dtype=moe.MOE_MXFP8)

    def pull(shape=s, dy=tabp, ye=FAKE, bb=big):
        return L.moe_combine_pull_reverse(ctypes.byref(shape), ctypes.byref(p), dy, ye, FAKE, FAKE, FAKE, FAKE, big,
                                          FAKE, bb, None)
    assert pull(shape=mx) == -6
    assert pull(dy=None) == -1
    assert pull(ye=FAKE + 2) == -2
    assert pull(bb=bws - 256) == -3

    def ffn(shape=s, xe=FAKE, dw1=FAKE, ws_bytes=big):
        return L.moe_expert_ffn_backward(ctypes.byref(shape), ctypes.byref(p), xe, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         ws_bytes, dw1, FAKE, FAKE, FAKE, big, None)
    assert ffn(shape=mx) == -6
    assert ffn(xe=None) == -1
    assert ffn(dw1=FAKE + 4) == -2
    assert ffn(ws_bytes=0) == -3

    def push(shape=s, recv=tabp, dlog=tabp, bptr=FAKE):
        return L.moe_dispatch_push_reverse(ctypes.byref(shape), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                           recv, tabp, dlog, bptr, big, None)
    assert push(shape=mx) == -6
    assert push(recv=None) == -1
    assert push(dlog=None) == -1
    assert push(bptr=FAKE + 128) == -2


def test_mx_backward_entries_reject_bad_arguments_before_launch():
    L = moe.lib()
    s, p = _shape(dtype=moe.MOE_MXFP8), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    bws = moe.moe_backward_workspace_bytes(s, p)
    ok = moe.MXScales(FAKE, FAKE, FAKE)

    def prep(shape=s, w=FAKE, sc=FAKE):
        return L.moe_backward_prepare_mx(ctypes.byref(shape), ctypes.byref(p), w, FAKE, FAKE, FAKE, sc, FAKE, FAKE,
                                         None)
    assert prep(shape=_shape()) == -6                                    # MXFP8 only
    assert prep(w=None) == -1
    assert prep(w=FAKE + 8) == -2
    assert prep(sc=FAKE + 1) == -2
    assert prep(shape=_shape(dtype=moe.MOE_MXFP8, d=7168 + 64)) == -2   # d % 128

    def bwd(shape=s, x=tabp, xs=FAKE, wsc=ok, bb=big, dw1=FAKE):
        return L.moe_backward_mx(ctypes.byref(shape), ctypes.byref(p), tabp, x, FAKE, xs, FAKE, FAKE, FAKE,
                                 ctypes.byref(wsc) if wsc is not None else None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, FAKE, big, tabp, tabp, tabp, dw1, FAKE, FAKE, FAKE, bb, None)
    assert bwd(shape=_shape()) == -6                                     # bf16 uses moe_backward
    assert bwd(x=None) == -1
    assert bwd(xs=None) == -1
    assert bwd(wsc=None) == -1
    assert bwd(wsc=moe.MXScales(FAKE, FAKE + 2, FAKE)) == -2
    assert bwd(dw1=FAKE + 4) == -2
    assert bwd(bb=bws - 256) == -3


def test_signal_probe_sizes_and_rejects_bad_arguments_before_launch():
    L = moe.lib()
    assert moe.moe_signal_probe_bytes(0) > 0
    assert moe.moe_signal_probe_bytes(16384) >= 128 * 16384 * 4
    assert moe.moe_signal_probe_bytes(-1) == 0 and moe.moe_signal_probe_bytes(1 << 21) == 0
    need = moe.moe_signal_probe_bytes(1024)
    us, n1, n2, n3 = ctypes.c_float(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    outs = [ctypes.byref(us), ctypes.byref(n1), ctypes.byref(n2), ctypes.byref(n3)]

    def call(cross=0, scope=1, words=1024, rounds=10, scratch=FAKE, nbytes=need, out=outs):
        return L.moe_signal_probe(cross, scope, words, rounds, scratch, nbytes, *out, None)
    assert call(cross=2) == -1
    assert call(scope=-1) == -1
    assert call(scope=4) == -1
    assert call(words=-5) == -1
    assert call(rounds=0) == -1
    assert call(rounds=100001) == -1
    assert call(scratch=None) == -1
    assert call(out=[None] + outs[1:]) == -1
    assert call(scratch=FAKE + 64) == -2
    assert call(nbytes=need - 1) == -3


def test_ceiling_probe_rejects_bad_arguments_before_launch():
    L = moe.lib()
    work, ms = ctypes.c_double(), ctypes.c_float()

    def call(kind=0, reps=10, src=FAKE, nbytes=1 << 30, scratch=FAKE, sbytes=1 << 20, w=ctypes.byref(work),
             t=ctypes.byref(ms)):
        return L.moe_ceiling_probe(kind, reps, src, nbytes, scratch, sbytes, w, t, None)
    assert call(kind=-1) == -1
    assert call(kind=4) == -1
    assert call(reps=0) == -1
    assert call(reps=1000001) == -1
    assert call(scratch=None) == -1
    assert call(w=None) == -1
    assert call(t=None) == -1
    assert call(scratch=FAKE + 64) == -2


def test_fused_push_entries_reject_bad_arguments_before_launch():
    s, p = _shape(), _pl()
    L = moe.lib()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    # moe_expert_ffn_push: missing pull_src, slot_of or recv table; misaligned recv row; small workspace
    args = lambda pull, so, rv, ws_bytes, x=None: (ctypes.byref(s), ctypes.byref(p), None, x, FAKE, None, FAKE,  # noqa: E731
                                                   FAKE, FAKE, FAKE, None, pull, so, rv, FAKE, ws_bytes, None)
    assert L.moe_expert_ffn_push(*args(None, FAKE, tabp, big)) == -1
    assert L.moe_expert_ffn_push(*args(FAKE, None, tabp, big)) == -1
    assert L.moe_expert_ffn_push(*args(FAKE, FAKE, None, big)) == -1
    tab3 = (ctypes.c_void_p * 8)(*([FAKE] * 7 + [FAKE + 4]))
    assert L.moe_expert_ffn_push(*args(FAKE, FAKE, ctypes.cast(tab3, ctypes.c_void_p), big)) == -2
    assert L.moe_expert_ffn_push(*args(FAKE, FAKE, tabp, 1024)) == -3
    # the fused pull: a null or misaligned x entry
    tab2 = (ctypes.c_void_p * 8)(*([FAKE] * 7 + [None]))
    assert L.moe_expert_ffn_push(*args(FAKE, FAKE, tabp, big, ctypes.cast(tab2, ctypes.c_void_p))) == -1
    assert L.moe_expert_ffn_push(*args(FAKE, FAKE, tabp, big, ctypes.cast(tab3, ctypes.c_void_p))) == -2
    # moe_weighted_merge: missing topk_w, missing y table
    assert L.moe_weighted_merge(ctypes.byref(s), ctypes.byref(p), FAKE, None, tabp, tabp, None) == -1
    assert L.moe_weighted_merge(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, tabp, None, None) == -1
    # moe_forward_fused: every stage checked up front (y table missing)
    rc = L.moe_forward_fused(ctypes.byref(s), ctypes.byref(p), None, tabp, tabp, FAKE, FAKE, FAKE, None, FAKE, None,
                             tabp, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None)
    assert rc == -1
    # MXFP8 without scales
    smx = moe.Shape(8, 4096, 7168, 256, 8, 2048, moe.MOE_MXFP8)
    assert L.moe_expert_ffn_push(ctypes.byref(smx), ctypes.byref(p), None, None, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, FAKE, tabp, FAKE, big, None) == -1
    # MXFP8 cannot fuse the pull (its rows are quantised by the gather)
    sc = moe.MXScales(FAKE, FAKE, FAKE)
    assert L.moe_expert_ffn_push(ctypes.byref(smx), ctypes.byref(p), None, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 ctypes.byref(sc), FAKE, FAKE, tabp, FAKE, big, None) == -6


def test_reverse_ring_layout_and_rejection():
    """reverse_ring adds the per-pair recv address table to the persistent workspace (before
    the trace region); the resident-chunk record lies inside the workspace proper; every
    entry point other than the persistent ones rejects reverse_ring, and those take 0 or 1."""
    L = moe.lib()
    s, p = _shape(), _pl()
    assert ctypes.sizeof(moe.Exec) == 32
    ex0 = moe.Exec(128, 16, 0, 0, 0)
    exr = moe.Exec(128, 16, 0, 0, 0, 1)
    exrt = moe.Exec(128, 16, 0, 1, 0, 1)
    base = moe.moe_persistent_workspace_bytes(s, p, ex0)
    npairs = moe.moe_max_pairs(s, p)
    with_table = moe.moe_persistent_workspace_bytes(s, p, exr)
    assert with_table == base + (npairs * 8 + 255) // 256 * 256
    off, cap, _ = moe.moe_persistent_trace_info(s, p, exrt)
    assert off == with_table
    roff, n = ctypes.c_size_t(), ctypes.c_int32()
    assert L.moe_persistent_resident_info(ctypes.byref(s), ctypes.byref(p), ctypes.byref(roff), ctypes.byref(n)) == 0
    max_mtiles = (npairs + 255) // 256 + 32
    assert n.value == 4 * max_mtiles
    assert roff.value % 4 == 0 and roff.value + 4 * n.value <= base
    assert L.moe_persistent_resident_info(ctypes.byref(s), ctypes.byref(p), None, ctypes.byref(n)) == -1
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    assert L.moe_layout(ctypes.byref(s), ctypes.byref(p), ctypes.byref(exr), tabp, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, big, None) == -1
    assert L.moe_forward(ctypes.byref(s), ctypes.byref(p), ctypes.byref(exr), tabp, tabp, FAKE, FAKE, FAKE, None,
                         FAKE, None, FAKE, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    bad = moe.Exec(128, 0, 0, 0, 0, 2)
    assert L.moe_forward_persistent(ctypes.byref(s), ctypes.byref(p), ctypes.byref(bad), tabp, tabp, FAKE, FAKE,
                                    FAKE, None, FAKE, big, tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                                    None) == -1


def test_backward_ring_rejects_bad_arguments_before_launch():
    L = moe.lib()
    s, p = _shape(), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    big = 1 << 40
    ex = moe.Exec(128, 16, 0, 0, 0, 1)

    def call(shape=s, exx=ex, ring=FAKE, pws=FAKE, pws_bytes=big, xe=FAKE, bws=FAKE, bws_bytes=big, dlog=tabp):
        return L.moe_backward_ring(ctypes.byref(shape), ctypes.byref(p), ctypes.byref(exx), tabp, tabp, ring, big,
                                   pws, pws_bytes, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, tabp, tabp, dlog,
                                   FAKE, FAKE, FAKE, xe, bws, bws_bytes, None)
    assert call(shape=_shape(dtype=moe.MOE_MXFP8)) == -6
    assert call(shape=_shape(k=0)) == -1
    assert call(pws=None) == -1
    assert call(pws=FAKE + 16) == -2
    assert call(pws_bytes=1024) == -3
    assert call(bws_bytes=1024) == -3
    assert call(bws=FAKE + 16) == -2
    assert call(ring=FAKE + 16) == -2
    assert call(xe=None) == -1
    assert call(dlog=None) == -1
    assert call(exx=moe.Exec(96, 16, 0, 0, 0, 1)) == -6            # chunk must divide 256
    assert call(exx=moe.Exec(128, 16, 0, 0, 0, 2)) == -1


def test_noalloc_entry_refuses_mxfp8_before_touching_the_device():
    """The no-allocation entry point takes no weight scales: an MXFP8 shape is refused before
    the device array is looked up."""
    L = moe.lib()
    s, p = _shape(dtype=moe.MOE_MXFP8), _pl()
    tab = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    tabp = ctypes.cast(tab, ctypes.c_void_p)
    rc = L.moe_forward_persistent_noalloc(ctypes.byref(s), ctypes.byref(p), None, tabp, tabp, FAKE, FAKE, FAKE,
                                          tabp, tabp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert rc == -6
