"""HIP-graph capture of the forward: every entry point only enqueues kernels on the
caller's stream (no host round trip, no allocation, no memset), so one moe_forward call
can be captured once and replayed.  Each replay must equal the eager call bit for bit,
with eager work and synchronisations between the replays and the outputs overwritten
before each replay."""
import sys

import numpy as np
import pytest

from mixture_experts_layer_histogram_amd import configs, inputs

pytestmark = pytest.mark.gpu

CASES = {
    "bf16": configs.MoEConfig("graph-bf16 R2 T1100 d384 E16/8 k4 F320", R=2, T=1100, d=384, E=16, E_local=8, k=4,
                              F=320, dtype="bf16"),
    "fp32": configs.MoEConfig("graph-fp32 R2 T300 d96 E8/6 k3 F80", R=2, T=300, d=96, E=8, E_local=6, k=3, F=80,
                              dtype="f32"),
    "mxfp8": configs.MoEConfig("graph-mx R2 T1100 d384 E16/8 k4 F384", R=2, T=1100, d=384, E=16, E_local=8, k=4,
                               F=384, dtype="mxfp8"),
}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fused", [False, True], ids=["unfused", "fused"])
@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay_equals_eager(name, fused):
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    cfg = CASES[name]
    _say(f"[graph] {cfg.name} {'fused' if fused else 'unfused'}")
    inp = inputs.make_inputs(cfg, seed=11)
    P = DeviceProblem(cfg, inp)
    fwd = P.forward_fused if fused else P.forward
    fwd()
    assert P.status() == 0
    torch.cuda.synchronize()
    ref_y = [t.clone() for t in P.y]
    ref_so = P.slot_of.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()                            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fwd()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in P.y:
            t.fill_(float("nan"))
        P.slot_of.fill_(-7)
        if rep == 2:                     # eager work between replays
            fwd()
            torch.cuda.synchronize()
            for t in P.y:
                t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert P.status() == 0
        assert torch.equal(P.slot_of, ref_so)
        for a, b in zip(P.y, ref_y):
            assert torch.equal(a, b), f"replay {rep} differs"
    _say(f"  4 replays bit-identical, N={P.N()}")


@pytest.mark.parametrize("name", ["bf16", "mxfp8"])
def test_backward_graph_replay_equals_eager(name):
    """The whole backward (moe_backward, or moe_backward_mx after its once-per-update
    weight preparation) captured after an eager forward; replays equal the eager call."""
    import torch
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    cfg = CASES[name]
    _say(f"[graph-bwd] {cfg.name}")
    inp = inputs.make_inputs(cfg, seed=12)
    P = DeviceProblem(cfg, inp)
    P.forward()
    dy_bits, _ = inputs.make_dy(cfg, seed=12)
    P.alloc_backward(dy_bits)
    mx = cfg.dtype == "mxfp8"
    if mx:
        P.prepare_backward_mx()
    run = P.backward_mx if mx else P.backward
    run()
    assert P.status() == 0
    torch.cuda.synchronize()
    outs = lambda: P.dx + P.dlogits + [P.dw1, P.dw3, P.dw2]      # noqa: E731
    bits = lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)  # noqa: E731
    ref = [bits(t).clone() for t in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            t.fill_(7)
        if rep == 1:
            run()
            torch.cuda.synchronize()
            for t in outs():
                t.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        assert P.status() == 0
        for a, b in zip(outs(), ref):
            assert torch.equal(bits(a), b), f"replay {rep} differs"
    _say("  3 replays bit-identical")
