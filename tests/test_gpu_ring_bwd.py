"""GPU parity of moe_backward_ring (bf16): after moe_forward_persistent with the reverse ring,
the backward reads the token rows the ring still holds in place, pulls the others again, and
reads the expert outputs from recv.  Against moe_backward on staged rows (xe from the
unfused forward's gather, ye from its FFN): bit-identical, with the ring holding every row,
part of them, or not used at all (and the staging rows poisoned, so a held row read from
xe would show); against the fp64 backward oracle at the bars of test_gpu_bwd."""
import sys

import numpy as np
import pytest

from oracle import moe_oracle_bwd as B
from mixture_experts_layer_histogram_amd import configs, inputs, moe
from tests.test_gpu_bwd import TOL, _bf16_to_f64, _dl_scale, _row_rel

pytestmark = pytest.mark.gpu

WATCHDOG_US = 500_000
CASES = [
    # (name, dims, ring_slots, ring MiB)
    ("ring-all R1 T1024 d512 E8/8 k2 F384", dict(R=1, T=1024, d=512, E=8, E_local=8, k=2, F=384), 0, 64),
    ("ring-part R1 T1024 d512 E8/8 k2 F384", dict(R=1, T=1024, d=512, E=8, E_local=8, k=2, F=384), 16, 64),
    ("ring-remote R2 T256 d256 E16/8 k4 F256", dict(R=2, T=256, d=256, E=16, E_local=8, k=4, F=256), 16, 16),
    ("ring-dsv3-slice R4 T1024 d7168 E64/8 k8 F2048",
     dict(R=4, T=1024, d=7168, E=64, E_local=8, k=8, F=2048), 16, 256),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _grads(dp):
    return dict(dx=[t.clone() for t in dp.dx], dlogits=[t.clone() for t in dp.dlogits], dw1=dp.dw1.clone(),
                dw3=dp.dw3.clone(), dw2=dp.dw2.clone())


def _same(a, b):
    import torch
    for k_ in ("dw1", "dw3", "dw2"):
        assert torch.equal(a[k_], b[k_]), k_
    for k_ in ("dx", "dlogits"):
        for x, y in zip(a[k_], b[k_]):
            assert torch.equal(x, y), k_


@pytest.mark.parametrize("name,dims,slots,mib", CASES, ids=[c[0].split()[0] for c in CASES])
def test_backward_ring_equals_staged(name, dims, slots, mib):
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    cfg = configs.MoEConfig(name, dtype="bf16", **dims)
    inp = inputs.make_inputs(cfg, seed=0)
    dy_bits, dy = inputs.make_dy(cfg, seed=0)
    _say(f"[ring-bwd] {name}: staged forward + backward")
    dp = DeviceProblem(cfg, inp)
    dp.alloc_backward(dy_bits)
    dp.forward()
    dp.backward()
    torch.cuda.synchronize()
    assert dp.status() == 0
    ref = _grads(dp)
    ex = moe.Exec(cfg.minibatch, 16, slots, 0, WATCHDOG_US, 1)
    _say(f"[ring-bwd] {name}: reverse-ring forward (ring_slots={slots}, {mib} MiB), backward from the ring")
    dp.alloc_ring(mib, ex)
    for use_ring in (True, False):
        # recv holds the forward's outputs until the backward replaces them with dX rows
        dp.forward_persistent(ex)
        assert dp.status() == 0
        held = int((moe.read_resident(dp.ws, dp.shape, dp.placement) > 0).sum())
        dp.xe.view(torch.int16).fill_(-1)                 # NaN bits: a held row read from xe would show
        for t in dp.dx + dp.dlogits + [dp.dw1, dp.dw3, dp.dw2]:
            t.fill_(7.0)
        dp.backward_ring(use_ring=use_ring)
        torch.cuda.synchronize()
        _same(_grads(dp), ref)
    _say(f"  chunks held in the ring: {held}; both bit-identical to moe_backward")


def test_backward_ring_matches_oracle():
    """The ring backward (part of the rows held) against the fp64 backward oracle."""
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    name, dims, slots, mib = CASES[2]
    cfg = configs.MoEConfig(name, dtype="bf16", **dims)
    inp = inputs.make_inputs(cfg, seed=1)
    dy_bits, dy = inputs.make_dy(cfg, seed=1)
    dp = DeviceProblem(cfg, inp)
    dp.alloc_backward(dy_bits)
    ex = moe.Exec(cfg.minibatch, 16, slots, 0, WATCHDOG_US, 1)
    dp.alloc_ring(mib, ex)
    _say(f"[ring-bwd] {name}: reverse-ring forward + ring backward against the oracle")
    dp.forward_persistent(ex)
    assert dp.status() == 0
    assert (moe.read_resident(dp.ws, dp.shape, dp.placement) > 0).any()
    dp.backward_ring()
    torch.cuda.synchronize()
    ref = B.backward(inp.logits, inp.x_f32, inp.w1_f32, inp.w3_f32, inp.w2_f32, inp.expert_to_local,
                     cfg.E_local, cfg.k, dy, minibatch=cfg.minibatch)
    so = ref["slot_of"]
    has = (so >= 0).any(-1)
    dx = np.stack([_bf16_to_f64(t) for t in dp.dx])
    assert _row_rel(dx[has], ref["dx"][has]) <= TOL
    assert np.all(dx[~has] == 0.0)
    off = ref["offsets"]
    for key, got in (("dw1", dp.dw1), ("dw3", dp.dw3), ("dw2", dp.dw2)):
        g = _bf16_to_f64(got)
        for l in range(cfg.E_local):
            if off[l + 1] == off[l]:
                assert np.all(g[l] == 0.0)
            else:
                assert _row_rel(g[l], ref[key][l]) <= TOL, (key, l)
    dl = np.stack([t.cpu().numpy().astype(np.float64) for t in dp.dlogits])
    scale = _dl_scale(ref, dy)
    err = np.abs(dl - ref["dlogits"]).max(axis=-1)
    assert float((err[has] / np.maximum(scale[has], 1e-30)).max()) <= TOL
