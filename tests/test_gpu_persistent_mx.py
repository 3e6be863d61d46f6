"""GPU tests of moe_forward_persistent with MXFP8 expert weights: the gather quantises each
token row into the ring slot (E4M3 codes and K-tile-major scale words), the gate/up GEMM
reads them from the slot and writes h's codes and scale words back into it, and the down
GEMM stores its bf16 rows straight to recv.  recv (local-pair entries) and y must be
bit-identical to the unfused MXFP8 path (moe_forward with w_scales, which test_gpu_mx pins
to the oracle's MX codec and quantised forward): the same quantiser, the same tile code and
the same K order on both sides.  Across ring sizes, minibatch sizes, data-movement
partitions, skewed load, both ring walks, and moe_persistent_dispatch_ffn_combine alone."""
import sys

import pytest

from mixture_experts_layer_histogram_amd import configs, inputs, moe

pytestmark = pytest.mark.gpu

WATCHDOG_US = 500_000


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = configs.MID.scaled(name="small-ragged-mx R2 T300 d256 E16/8 k4 F256", R=2, T=300, d=256, F=256, E=16,
                           E_local=8, k=4, dtype="mxfp8")
MID_SMALL = configs.MID.scaled(name="mid-ragged-mx R2 T777 d2048 E64/64 k6 F1408", R=2, T=777, dtype="mxfp8")
SLICE = configs.DSV3_MX.scaled(name="dsv3-slice-mx R4 T1024 d7168 E64/8 k8 F2048", R=4, T=1024, E=64, E_local=8)
SLICE_SKEW = SLICE.scaled(name="dsv3-slice-mx-zipf", load="skew")

CFG = {"small": SMALL, "mid-ragged": MID_SMALL, "dsv3-slice": SLICE, "dsv3-slice-zipf": SLICE_SKEW}

_cache = {}


def _reference(cfg, seed=0):
    """Inputs on the device plus the unfused MXFP8 path's outputs."""
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    key = (cfg.name, seed)
    if key not in _cache:
        _cache.clear()
        inp = inputs.make_inputs(cfg, seed=seed)
        P = DeviceProblem(cfg, inp)
        P.forward()
        assert P.status() == 0
        torch.cuda.synchronize()
        _cache[key] = (P, {"y": [t.clone() for t in P.y], "recv": [t.clone() for t in P.recv],
                           "slot_of": P.slot_of.clone()})
    return _cache[key]


def _clear(P):
    for t in P.y:
        t.fill_(7.0)
    for t in P.recv:
        t.fill_(-3.0)


def _assert_same(P, ref):
    import torch
    for a, b in zip(P.y, ref["y"]):
        assert torch.equal(a, b)
    so = ref["slot_of"]
    for r in range(len(P.recv)):
        m = so[r] >= 0
        assert torch.equal(P.recv[r][m], ref["recv"][r][m])


CASES = [
    # (config, minibatch, comm_cus, ring_slots, ring MiB, reverse ring): smallest first
    ("small", 128, 0, 0, 16, 0),       # eight pipelines
    ("small", 128, 8, 2, 16, 0),       # one row tile of ring: one pipeline, no look-ahead
    ("small", 64, 16, 32, 16, 1),
    ("small", 256, 8, 0, 16, 1),
    ("mid-ragged", 128, 16, 0, 64, 0),
    ("mid-ragged", 64, 8, 24, 64, 1),  # four pipelines (agent-scope hand-offs)
    ("dsv3-slice", 128, 8, 0, 256, 0),
    ("dsv3-slice", 128, 8, 0, 256, 1),
    ("dsv3-slice", 128, 8, 16, 256, 1),  # eight pipelines, 2 slots each
    ("dsv3-slice", 64, 16, 0, 256, 0),
    ("dsv3-slice", 256, 16, 0, 256, 1),
    ("dsv3-slice-zipf", 128, 8, 0, 256, 1),
]


@pytest.mark.parametrize("name,mb,comm,slots,mib,rev", CASES)
def test_persistent_mx_equals_unfused(name, mb, comm, slots, mib, rev):
    import torch
    cfg = CFG[name]
    _say(f"[persistent-mx] {name} minibatch={mb} comm_cus={comm} ring_slots={slots} ring={mib}MiB reverse={rev}")
    P, ref = _reference(cfg)
    ex = moe.Exec(mb, comm, slots, 0, WATCHDOG_US, rev)
    _clear(P)
    P.alloc_ring(mib, ex)
    P.forward_persistent()
    st = P.status()
    torch.cuda.synchronize()
    assert st == 0, moe.ERRORS.get(st, st)
    _assert_same(P, ref)


def test_persistent_mx_dfc_alone():
    """The persistent kernel alone after moe_layout: recv's local-pair rows as the unfused path."""
    import torch
    P, ref = _reference(SLICE)
    _say("[persistent-mx] dispatch-ffn-combine alone")
    ex = moe.Exec(128, 8, 0, 0, WATCHDOG_US, 1)
    _clear(P)
    P.alloc_ring(256, ex)
    P.layout()
    P.persistent_dfc(ex)
    st = P.status()
    torch.cuda.synchronize()
    assert st == 0
    so = ref["slot_of"]
    for r in range(len(P.recv)):
        m = so[r] >= 0
        assert torch.equal(P.recv[r][m], ref["recv"][r][m])


def test_persistent_mx_repeatable():
    import torch
    P, ref = _reference(SLICE_SKEW)
    _say("[persistent-mx] repeat x3")
    ex = moe.Exec(128, 8, 0, 0, WATCHDOG_US, 1)
    P.alloc_ring(256, ex)
    for _ in range(3):
        _clear(P)
        P.forward_persistent()
        assert P.status() == 0
        torch.cuda.synchronize()
        _assert_same(P, ref)
