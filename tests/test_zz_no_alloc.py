"""GPU test of moe_forward_persistent_noalloc (workspace and ring in the library's static
device array, no allocation in the call) against moe_forward_persistent on caller buffers:
recv (local-pair entries), y and the layout outputs bit-identical, status 0, on two calls in
a row -- the second with a smaller input, so nothing of the first call's array contents may
leak into it."""
import sys

import pytest

from mixture_experts_layer_histogram_amd import configs, inputs, moe

pytestmark = pytest.mark.gpu

BIG = configs.DSV3.scaled(name="dsv3-slice R4 T1024 d7168 E64/8 k8 F2048", R=4, T=1024, E=64, E_local=8)
SMALL = configs.DSV3.scaled(name="dsv3-small R2 T300 d7168 E64/8 k8 F2048", R=2, T=300, E=64, E_local=8,
                            load="skew")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _outputs(P):
    return ([t.clone() for t in P.y], [t.clone() for t in P.recv], P.slot_of.clone(), P.offsets.clone(),
            P.topk_idx.clone(), P.topk_w.clone(), P.pull_src.clone(), P.counts.clone())


def _case(cfg):
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    _say(f"[no-alloc] {cfg.name}")
    inp = inputs.make_inputs(cfg, seed=3)
    P = DeviceProblem(cfg, inp)
    ex = moe.Exec(128, 16, 0, 0, 500_000)
    # the existing entry point on caller buffers
    P.alloc_ring(cfg.ring_mib, ex)
    P.forward_persistent(ex)
    assert P.status() == 0
    ref = _outputs(P)
    # the no-allocation variant, outputs poisoned first
    for t in P.y:
        t.fill_(7.0)
    for t in P.recv:
        t.fill_(-3.0)
    for t in (P.slot_of, P.pull_src, P.topk_idx, P.counts, P.offsets):
        t.fill_(-9)
    P.topk_w.fill_(-1.0)
    status = torch.full((1,), 12345, dtype=torch.int32, device=P.device)
    moe.moe_forward_persistent_noalloc(P.shape, P.placement, ex, P.logits, P.x, P.w1, P.w3, P.w2, P.recv, P.y,
                                       P.topk_idx, P.topk_w, P.counts, P.offsets, P.pull_src, P.slot_of,
                                       status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = _outputs(P)
    for a, b in zip(got[0], ref[0]):
        assert torch.equal(a, b)
    so = ref[2]
    for r in range(cfg.R):
        m = so[r] >= 0
        assert torch.equal(got[1][r][m], ref[1][r][m])
    n = int(ref[3][-1].item())
    for i in (2, 3, 4, 5, 7):
        assert torch.equal(got[i], ref[i])
    assert torch.equal(got[6][:n], ref[6][:n])


def test_noalloc_two_calls_second_smaller():
    _case(BIG)
    _case(SMALL)


def test_noalloc_rejects_a_shape_beyond_the_array():
    """The full DeepSeek-V3 share fits (under 1 MiB of workspace); a shape whose workspace
    exceeds the array's workspace part is refused before any launch."""
    from mixture_experts_layer_histogram_amd.device import DeviceProblem   # noqa: F401
    s = moe.Shape(64, 65536, 7168, 256, 8, 2048, moe.MOE_BF16)
    import ctypes
    pl = moe.Placement(1 << 40, 32)
    assert moe.moe_persistent_workspace_bytes(s, pl) > moe.NOALLOC_WORKSPACE_BYTES
    rc = moe.lib().moe_forward_persistent_noalloc(ctypes.byref(s), ctypes.byref(pl), None, *([None] * 14), None)
    assert rc == -3
