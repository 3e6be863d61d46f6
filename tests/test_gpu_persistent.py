"""GPU tests of moe_forward_persistent: bit-identical to the unfused path (which the
oracle pins), across ring sizes (per-XCD pipelines with L2-local hand-offs, and
cross-XCD pipelines with agent-scope hand-offs when the ring is small), minibatch
sizes and data-movement partition sizes; deterministic; and a watchdog expiry forced
from the host that ends the kernel cleanly with MOE_ETIMEOUT."""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from mixture_experts_layer_histogram_amd import configs, inputs, moe

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="moe_forward_persistent is switched off (returns MOE_EUNSUP): its one GPU run "
                            "did not complete and the cause is not yet shown; see the design notes"),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SLICE = configs.DSV3.scaled(name="dsv3-slice R4 T1024 d7168 E64/8 k8 F2048", R=4, T=1024, E=64, E_local=8)
SLICE_SKEW = SLICE.scaled(name="dsv3-slice-zipf", load="skew")
MID_SMALL = configs.MID.scaled(name="mid-ragged R2 T777 d2048 E64/64 k6 F1408", R=2, T=777)

_cache = {}


def _reference(cfg, seed=0):
    """Inputs on the device plus the unfused path's outputs (pinned to the oracle by
    test_gpu_parity)."""
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    key = (cfg.name, seed)
    if key not in _cache:
        inp = inputs.make_inputs(cfg, seed=seed)
        P = DeviceProblem(cfg, inp)
        P.forward()
        assert P.status() == 0
        torch.cuda.synchronize()
        ref = {"y": [t.clone() for t in P.y], "recv": [t.clone() for t in P.recv],
               "slot_of": P.slot_of.clone(), "offsets": P.offsets.clone()}
        _cache.clear()
        _cache[key] = (inp, P, ref)
    return _cache[key]


def _run_persistent(P, ex, ring_mib):
    import torch
    for t in P.y:
        t.fill_(7.0)
    for t in P.recv:
        t.fill_(-3.0)
    P.alloc_ring(ring_mib, ex)
    P.forward_persistent()
    st = P.status()
    torch.cuda.synchronize()
    return st


def _assert_same(P, ref):
    import torch
    for a, b in zip(P.y, ref["y"]):
        assert torch.equal(a, b)
    so = ref["slot_of"]
    for r in range(len(P.recv)):
        m = so[r] >= 0
        assert torch.equal(P.recv[r][m], ref["recv"][r][m])


CASES = [
    # (config, minibatch, comm_cus, ring_slots, ring MiB)
    ("dsv3-slice", 128, 0, 0, 256),
    ("dsv3-slice", 128, 0, 2, 256),       # one row tile of ring: single cross-XCD pipeline
    ("dsv3-slice", 128, 0, 7, 256),       # 3 pipelines' worth -> two pipelines
    ("dsv3-slice", 128, 8, 16, 256),      # eight pipelines, 2 slots each, 1 mover per XCD
    ("dsv3-slice", 64, 64, 0, 256),
    ("dsv3-slice", 256, 32, 0, 256),
    ("dsv3-slice-zipf", 128, 32, 0, 256),
    ("dsv3-slice-zipf", 128, 32, 24, 256),
    ("mid-ragged", 128, 16, 0, 64),
]
CFG = {"dsv3-slice": SLICE, "dsv3-slice-zipf": SLICE_SKEW, "mid-ragged": MID_SMALL}


@pytest.mark.parametrize("name,mb,comm,slots,mib", CASES)
def test_persistent_equals_unfused(name, mb, comm, slots, mib):
    cfg = CFG[name]
    _say(f"[persistent] {name} minibatch={mb} comm_cus={comm} ring_slots={slots} ring={mib}MiB")
    inp, P, ref = _reference(cfg)
    ex = moe.Exec(mb, comm, slots, 0, 0)
    st = _run_persistent(P, ex, mib)
    assert st == 0
    _assert_same(P, ref)


def test_persistent_repeatable():
    import torch
    inp, P, ref = _reference(SLICE_SKEW)
    _say("[persistent] repeat x3")
    ex = moe.Exec(128, 32, 0, 0, 0)
    outs = []
    for _ in range(3):
        assert _run_persistent(P, ex, 256) == 0
        outs.append([t.clone() for t in P.y])
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a, b)


def test_persistent_watchdog_forced_from_host():
    """A 1 us wait budget expires on the first wait; every workgroup must still exit,
    the status reads MOE_ETIMEOUT, and the next normal call is correct again."""
    inp, P, ref = _reference(SLICE)
    _say("[persistent] forced watchdog expiry")
    st = _run_persistent(P, moe.Exec(128, 32, 0, 0, 1), 256)
    assert st == -5
    st = _run_persistent(P, moe.Exec(128, 32, 0, 0, 0), 256)
    assert st == 0
    _assert_same(P, ref)


@pytest.mark.parametrize("cfg", [configs.DSV3, configs.DSV3_SKEW], ids=["dsv3", "dsv3-zipf"])
def test_persistent_full_share(cfg):
    """The full DeepSeek-V3-shaped share (256 MiB ring, 32 movers), against the unfused
    path; the layout against the oracle."""
    _say(f"[persistent-full] {cfg.name}")
    inp, P, ref = _reference(cfg)
    idx, _ = O.route(inp.logits, cfg.k)
    lay = O.layout(idx, inp.expert_to_local, cfg.E_local)
    np.testing.assert_array_equal(ref["slot_of"].cpu().numpy(), lay["slot_of"])
    st = _run_persistent(P, moe.Exec(128, 32, 0, 0, 0), cfg.ring_mib)
    assert st == 0
    np.testing.assert_array_equal(P.slot_of.cpu().numpy(), lay["slot_of"])
    _assert_same(P, ref)
    cnt = lay["counts"][:cfg.E_local]
    _say(f"  N={lay['N']} hottest local/mean={cnt.max() / cnt.mean():.2f}")
