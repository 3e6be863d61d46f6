"""GPU parity: every C entry point against the CPU oracle on the same seeded inputs.

Bar: routing indices, counts, offsets, pull schedule and slot map bit-exact;
gates within 2e-6; dispatch and push copies bit-exact; outputs within the
row-relative tolerance (fp32 1e-4, bf16 2e-2); rows with no local expert exactly 0.
"""
import sys
import zlib

import numpy as np
import pytest

from oracle import moe_oracle as O
from mixture_experts_layer_histogram_amd import configs, inputs, moe

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _torch():
    import torch
    return torch


def _row_rel_err(yg, yr, has):
    num = np.abs(yg - yr).max(axis=-1)
    den = np.abs(yr).max(axis=-1)
    return float((num[has] / np.maximum(den[has], 1e-30)).max()) if has.any() else 0.0


# --------------------------------------------------------------------------- layout only
def _gpu_layout(logits, e2l, El, k, minibatch=128):
    torch = _torch()
    R, T, E = logits.shape
    dev = torch.device("cuda:0")
    shape = moe.Shape(R, T, 64, E, k, 64, moe.MOE_BF16)
    e2l_d = torch.from_numpy(np.ascontiguousarray(e2l, dtype=np.int32)).to(dev)
    pl = moe.Placement(e2l_d.data_ptr(), El)
    ex = moe.Exec(minibatch, 0, 0, 0, 0)
    nmax = moe.moe_max_pairs(shape, pl)
    lg = [torch.from_numpy(np.ascontiguousarray(logits[r])).to(dev) for r in range(R)]
    out = dict(topk_idx=torch.full((R, T, k), -7, dtype=torch.int32, device=dev),
               topk_w=torch.zeros((R, T, k), dtype=torch.float32, device=dev),
               counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
               offsets=torch.full((El + 1,), -7, dtype=torch.int32, device=dev),
               pull_src=torch.full((nmax, 2), -7, dtype=torch.int32, device=dev),
               slot_of=torch.full((R, T, k), -7, dtype=torch.int32, device=dev))
    ws = torch.empty(moe.moe_workspace_bytes(shape, pl, ex), dtype=torch.uint8, device=dev)
    moe.moe_layout(shape, pl, ex, lg, out["topk_idx"], out["topk_w"], out["counts"], out["offsets"],
                   out["pull_src"], out["slot_of"], ws)
    status = moe.moe_read_status(ws)
    host = {kk: v.cpu().numpy() for kk, v in out.items()}
    host["status"] = status
    host["ctrl"] = ws[:256].view(torch.int32).cpu().numpy()
    return host


def _check_layout(logits, e2l, El, k, got):
    idx, g = O.route(logits, k)
    lay = O.layout(idx, e2l, El)
    np.testing.assert_array_equal(got["topk_idx"], idx)
    np.testing.assert_allclose(got["topk_w"], g, rtol=0, atol=2e-6)
    np.testing.assert_array_equal(got["counts"], lay["counts"])
    np.testing.assert_array_equal(got["offsets"], lay["offsets"])
    N = lay["N"]
    np.testing.assert_array_equal(got["pull_src"][:N], lay["pull_src"])
    np.testing.assert_array_equal(got["slot_of"], lay["slot_of"])
    assert got["status"] == 0
    assert got["ctrl"][1] == N
    return lay


def _e2l_prefix(E, El):
    e2l = np.full(E, -1, dtype=np.int32)
    e2l[:El] = np.arange(El)
    return e2l


LAYOUT_CASES = {
    # name: (R, T, E, El, k, logits kind)
    "tiny": (1, 256, 8, 8, 2, "normal"),
    "mid": (1, 4096, 64, 64, 6, "normal"),
    "dsv3-full": (8, 4096, 256, 32, 8, "normal"),
    "ragged-T": (3, 1001, 256, 32, 8, "normal"),
    "k-equals-E": (2, 130, 16, 16, 16, "normal"),
    "E1-k1": (1, 77, 1, 1, 1, "normal"),
    "all-ties": (2, 300, 64, 8, 6, "ties"),
    "one-hot-expert": (2, 500, 32, 4, 3, "hot"),
    "quantised-ties": (4, 700, 128, 20, 8, "coarse"),
    "E1024": (1, 257, 1024, 100, 16, "normal"),
}


@pytest.mark.parametrize("name", list(LAYOUT_CASES))
def test_layout_parity(name):
    R, T, E, El, k, kind = LAYOUT_CASES[name]
    _say(f"[layout] {name} R={R} T={T} E={E} El={El} k={k}")
    logits = inputs.random_logits((R, T, E), seed=zlib.crc32(name.encode()) % 1000)
    if kind == "ties":
        logits[:] = 0.25
    elif kind == "hot":
        logits[..., 3] += 50.0          # expert 3 (local) is picked by every token
    elif kind == "coarse":
        logits = np.round(logits * 2) / 2   # many exact ties
    e2l = _e2l_prefix(E, El)
    got = _gpu_layout(logits, e2l, El, k)
    lay = _check_layout(logits, e2l, El, k, got)
    if kind == "hot":
        assert lay["counts"][3] == R * T


def test_layout_skewed_full_size():
    cfg = configs.DSV3_SKEW
    _say(f"[layout] {cfg.name}")
    e2l = _e2l_prefix(cfg.E, cfg.E_local)
    logits = inputs.skewed_logits(cfg, 0, e2l)
    got = _gpu_layout(logits, e2l, cfg.E_local, cfg.k)
    lay = _check_layout(logits, e2l, cfg.E_local, cfg.k, got)
    cnt = lay["counts"][:cfg.E_local]
    _say(f"  N={lay['N']} hottest local/mean={cnt.max() / cnt.mean():.2f}")


def test_layout_scattered_placement_and_zero_count_experts():
    R, T, E, El, k = 2, 640, 96, 24, 4
    rng = np.random.default_rng(5)
    e2l = np.full(E, -1, dtype=np.int32)
    e2l[rng.permutation(E)[:El]] = rng.permutation(El)
    logits = inputs.random_logits((R, T, E), seed=17)
    # make a few local experts unreachable (zero count)
    dead = np.flatnonzero(e2l >= 0)[:5]
    logits[..., dead] = -100.0
    got = _gpu_layout(logits, e2l, El, k)
    lay = _check_layout(logits, e2l, El, k, got)
    assert (lay["counts"][dead] == 0).all()


def test_layout_rejects_bad_placement_on_device():
    R, T, E, El, k = 1, 128, 16, 4, 2
    e2l = np.array([0, 1, 1, 3] + [-1] * 12, dtype=np.int32)      # local id 1 twice, 2 missing
    logits = inputs.random_logits((R, T, E), seed=3)
    got = _gpu_layout(logits, e2l, El, k)
    assert got["status"] == -1
    assert (got["offsets"] == 0).all()
    assert (got["slot_of"] == -1).all()
    assert got["ctrl"][1] == 0


# --------------------------------------------------------------------------- full path
def _problem(cfg, seed=0, never=None):
    """Seeded inputs on the device; experts listed in `never` get their logits lowered by
    100 so that no token selects them."""
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    inp = inputs.make_inputs(cfg, seed=seed)
    if never:
        inp.logits[..., list(never)] -= 100.0
    return inp, DeviceProblem(cfg, inp)


SLICE = configs.DSV3.scaled(name="dsv3-slice R4 T1024 d7168 E64/8 k8 F2048", R=4, T=1024, E=64, E_local=8)
SLICE_SKEW = SLICE.scaled(name="dsv3-slice-zipf", load="skew")
MID_SMALL = configs.MID.scaled(name="mid-ragged R2 T777 d2048 E64/64 k6 F1408", R=2, T=777)

FORWARD_CASES = {"tiny": configs.TINY, "mid": configs.MID, "mid-ragged": MID_SMALL, "dsv3-slice": SLICE,
                 "dsv3-slice-zipf": SLICE_SKEW}


# Degenerate and boundary shapes: (config, experts never selected)
EDGE_CASES = {
    # one expert, top-1: the layer is the plain SwiGLU FFN of every token; F = 192 leaves
    # a half-empty column tile in GEMM1 and d = 128 a half-empty one in GEMM2
    "E1-k1": (configs.MoEConfig("e1-k1 R1 T100 d128 E1 k1 F192", R=1, T=100, d=128, E=1, E_local=1, k=1,
                                F=192, dtype="bf16"), None),
    # k = E, all local: every token uses every expert
    "k-equals-E": (configs.MoEConfig("k=E R2 T130 d256 E16/16 k16 F256", R=2, T=130, d=256, E=16, E_local=16,
                                     k=16, F=256, dtype="bf16"), None),
    # a single token (2 rows in the whole GEMM)
    "single-token": (configs.MoEConfig("one-token R1 T1 d512 E8/8 k2 F256", R=1, T=1, d=512, E=8, E_local=8,
                                       k=2, F=256, dtype="bf16"), None),
    # one resident expert of 32: most tokens have no local pair
    "one-local-expert": (configs.MoEConfig("one-local R3 T200 d256 E32/1 k4 F128", R=3, T=200, d=256, E=32,
                                           E_local=1, k=4, F=128, dtype="bf16"), None),
    # no token selects a local expert: N = 0, empty GEMMs, y exactly zero everywhere
    "no-local-pairs": (configs.MoEConfig("no-local R2 T300 d256 E16/4 k4 F256", R=2, T=300, d=256, E=16,
                                         E_local=4, k=4, F=256, dtype="bf16"), (0, 1, 2, 3)),
    # fp32 with ragged d, F and T
    "fp32-ragged": (configs.MoEConfig("fp32-ragged R3 T333 d96 E8/6 k3 F80", R=3, T=333, d=96, E=8, E_local=6,
                                      k=3, F=80, dtype="f32"), None),
}


@pytest.mark.parametrize("name", list(FORWARD_CASES))
def test_forward_parity(name):
    cfg = FORWARD_CASES[name]
    _say(f"[forward] {cfg.name}")
    inp, P = _problem(cfg)
    _check_forward(cfg, inp, P)


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_forward_edge_cases(name):
    cfg, never = EDGE_CASES[name]
    _say(f"[forward-edge] {cfg.name}")
    inp, P = _problem(cfg, never=never)
    N = _check_forward(cfg, inp, P)
    if never:
        assert N == 0


def _check_forward(cfg, inp, P):
    torch = _torch()
    P.forward()
    assert P.status() == 0
    torch.cuda.synchronize()
    ref = O.forward(inp.logits, inp.x_f32, inp.w1_f32, inp.w3_f32, inp.w2_f32, inp.expert_to_local,
                    cfg.E_local, cfg.k)
    N = ref["N"]
    np.testing.assert_array_equal(P.topk_idx.cpu().numpy(), ref["idx"])
    np.testing.assert_allclose(P.topk_w.cpu().numpy(), ref["gates"], rtol=0, atol=2e-6)
    np.testing.assert_array_equal(P.offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(P.pull_src[:N].cpu().numpy(), ref["pull_src"])
    np.testing.assert_array_equal(P.slot_of.cpu().numpy(), ref["slot_of"])
    # dispatch: bit-exact rows
    xe = P.rows_f64(P.xe[:N])
    np.testing.assert_array_equal(xe, ref["xe"])
    # expert FFN on the dispatched rows
    ye = P.rows_f64(P.ye[:N])
    has_rows = np.ones(N, dtype=bool)
    err_ffn = _row_rel_err(ye, ref["ye"], has_rows)
    # push combine: recv[r][t][j] is ye[slot] bit for bit
    so = ref["slot_of"]
    ye_host = P.ye[:N].cpu()
    for r in range(cfg.R):
        rv = P.recv[r].cpu()
        sl = torch.from_numpy(so[r])
        mask = sl >= 0
        assert torch.equal(rv[mask], ye_host[sl[mask].long()])
    # merge
    y = np.stack([P.rows_f64(P.y[r]) for r in range(cfg.R)])
    has = (so >= 0).any(-1)
    err = _row_rel_err(y.reshape(-1, cfg.d), ref["y"].reshape(-1, cfg.d), has.reshape(-1))
    _say(f"  N={N} ffn_rel={err_ffn:.3e} y_rel={err:.3e}")
    assert err_ffn <= TOL[cfg.dtype]
    assert err <= TOL[cfg.dtype]
    assert (y[~has] == 0).all()
    return N


def test_forward_deterministic_and_stagewise_equals_fused_call():
    torch = _torch()
    cfg = SLICE_SKEW
    _say(f"[determinism] {cfg.name}")
    inp, P = _problem(cfg, seed=1)
    P.forward()
    y1 = [t.clone() for t in P.y]
    P.layout()
    P.dispatch()
    P.ffn()
    P.combine()
    torch.cuda.synchronize()
    for a, b in zip(y1, P.y):
        assert torch.equal(a, b)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [configs.DSV3, configs.DSV3_SKEW], ids=["dsv3", "dsv3-zipf"])
def test_forward_full_dsv3_sampled(cfg):
    """Full DeepSeek-V3-shaped share (uniform load, and Zipf(1.2) load whose hottest local
    expert holds ~10x the mean rows), the launch configuration the bench times; layout
    compared whole, outputs compared on sampled tokens computed one by one: 40 random tokens
    with a local pair, plus the tokens of the first, middle and last rows of the hottest local
    expert's first, middle and last 256-row tiles."""
    torch = _torch()
    _say(f"[forward-full] {cfg.name}")
    inp, P = _problem(cfg)
    P.forward()
    assert P.status() == 0
    torch.cuda.synchronize()
    idx, g = O.route(inp.logits, cfg.k)
    lay = O.layout(idx, inp.expert_to_local, cfg.E_local)
    np.testing.assert_array_equal(P.topk_idx.cpu().numpy(), idx)
    np.testing.assert_array_equal(P.offsets.cpu().numpy(), lay["offsets"])
    np.testing.assert_array_equal(P.slot_of.cpu().numpy(), lay["slot_of"])
    np.testing.assert_array_equal(P.pull_src[:lay["N"]].cpu().numpy(), lay["pull_src"])
    rng = np.random.default_rng(0)
    has = (lay["slot_of"] >= 0).any(-1)
    local_tok = np.argwhere(has)
    pick = [tuple(v) for v in local_tok[rng.choice(len(local_tok), 40, replace=False)]]
    off = lay["offsets"]
    cnt = np.diff(off)
    hot = int(np.argmax(cnt))
    tiles = (int(cnt[hot]) + 255) // 256
    for tile in sorted({0, tiles // 2, tiles - 1}):
        t0 = int(off[hot]) + 256 * tile
        t1 = min(t0 + 256, int(off[hot + 1]))
        for srow in sorted({t0, (t0 + t1) // 2, t1 - 1}):
            pick.append(tuple(int(v) for v in lay["pull_src"][srow]))
    worst = 0.0
    for r, t in pick:
        yr = O.token_output(inp.x_f32[r, t], idx[r, t], g[r, t], inp.expert_to_local, inp.w1_f32,
                            inp.w3_f32, inp.w2_f32)
        yg = P.y[r][t].float().cpu().numpy().astype(np.float64)
        worst = max(worst, float(np.abs(yg - yr).max() / np.abs(yr).max()))
    zr, zt = np.argwhere(~has)[0]
    assert (P.y[zr][zt].float().cpu().numpy() == 0).all()
    _say(f"  N={lay['N']} hottest local expert {hot}: {int(cnt[hot])} rows ({cnt[hot] / cnt.mean():.1f}x mean, "
         f"{tiles} row tiles); {len(pick)} sampled tokens y_rel={worst:.3e}")
    assert worst <= TOL["bf16"]
    # the fused multi-kernel configuration (pull and push fused into the GEMMs) and the
    # persistent megakernel the bench times: bit for bit the same y as the unfused path
    y_ref = [t.clone() for t in P.y]
    for t in P.y:
        t.fill_(float("nan"))
    P.forward_fused()
    assert P.status() == 0
    torch.cuda.synchronize()
    for a, b in zip(P.y, y_ref):
        assert torch.equal(a, b)
    for t in P.y:
        t.fill_(float("nan"))
    P.alloc_ring(cfg.ring_mib)
    P.forward_persistent(moe.Exec(cfg.minibatch, 16, 0, 0, 0))
    assert P.status() == 0
    torch.cuda.synchronize()
    for a, b in zip(P.y, y_ref):
        assert torch.equal(a, b)
    _say("  fused pull and push, and the persistent kernel: y bit-identical")


# --------------------------------------------------------------------------- metamorphic
# Relations the HIP path must satisfy bit for bit, whatever the oracle says: each output
# row's arithmetic (MFMA K order, fp32 merge in ascending j) does not depend on where the
# row lands in the expert segments or GEMM tiles.
META_CASES = {
    "bf16": configs.MoEConfig("meta-bf16 R2 T1100 d384 E16/8 k4 F320", R=2, T=1100, d=384, E=16, E_local=8, k=4,
                              F=320, dtype="bf16"),
    "fp32": configs.MoEConfig("meta-fp32 R2 T300 d96 E8/6 k3 F80", R=2, T=300, d=96, E=8, E_local=6, k=3, F=80,
                              dtype="f32"),
    # MXFP8: scaling W2 by 2^m moves each block's E8M0 scale by m and leaves the codes alone
    "mxfp8": configs.MoEConfig("meta-mx R2 T1100 d384 E16/8 k4 F384", R=2, T=1100, d=384, E=16, E_local=8, k=4,
                               F=384, dtype="mxfp8"),
}


def _run(cfg, inp):
    from mixture_experts_layer_histogram_amd.device import DeviceProblem
    torch = _torch()
    P = DeviceProblem(cfg, inp)
    P.forward()
    assert P.status() == 0
    torch.cuda.synchronize()
    return [P.y[r].float().cpu().numpy() for r in range(cfg.R)], P.N()


def _assert_no_topk_ties(logits, k):
    """The relations below change expert ids or token order; with an exact tie among a
    token's k + 1 largest logits the lower-id rule could pick or order differently."""
    top = -np.sort(-logits, axis=-1)[..., :min(k + 1, logits.shape[-1])]
    assert (np.diff(top, axis=-1) < 0).all()


def _replace(inp, **kw):
    import dataclasses
    return dataclasses.replace(inp, **kw)


def _scale_store(store, dtype, m):
    v = store if dtype == "f32" else inputs.bf16_bits_to_f32(store)
    s = (v.astype(np.float32) * np.float32(2.0 ** m)).astype(np.float32)
    return s if dtype == "f32" else inputs.f32_to_bf16_bits(s)


@pytest.mark.parametrize("name", list(META_CASES))
def test_forward_w2_power_of_two_scales_output_exactly(name):
    cfg = META_CASES[name]
    _say(f"[meta-w2-scale] {cfg.name}")
    inp = inputs.make_inputs(cfg, seed=5)
    y0, n0 = _run(cfg, inp)
    assert n0 > 0
    for m in (3, -2):
        yi, _ = _run(cfg, _replace(inp, w2_store=_scale_store(inp.w2_store, cfg.dtype, m)))
        for a, b in zip(y0, yi):
            np.testing.assert_array_equal(b, a * np.float32(2.0 ** m))


@pytest.mark.parametrize("name", list(META_CASES))
def test_forward_token_permutation_permutes_output(name):
    cfg = META_CASES[name]
    _say(f"[meta-token-perm] {cfg.name}")
    inp = inputs.make_inputs(cfg, seed=6)
    _assert_no_topk_ties(inp.logits, cfg.k)
    y0, _ = _run(cfg, inp)
    rng = np.random.default_rng(60)
    perm = np.stack([rng.permutation(cfg.T) for _ in range(cfg.R)])
    x_p = np.stack([inp.x_store[r][perm[r]] for r in range(cfg.R)])
    lg_p = np.stack([inp.logits[r][perm[r]] for r in range(cfg.R)])
    yp, _ = _run(cfg, _replace(inp, x_store=x_p, logits=lg_p))
    for r in range(cfg.R):
        np.testing.assert_array_equal(yp[r], y0[r][perm[r]])


@pytest.mark.parametrize("name", list(META_CASES))
def test_forward_expert_relabelling_leaves_output_unchanged(name):
    cfg = META_CASES[name]
    _say(f"[meta-relabel] {cfg.name}")
    inp = inputs.make_inputs(cfg, seed=7)
    _assert_no_topk_ties(inp.logits, cfg.k)
    y0, n0 = _run(cfg, inp)
    rng = np.random.default_rng(70)
    sigma = rng.permutation(cfg.E)              # old global id e -> new id sigma[e]
    pl = rng.permutation(cfg.E_local)           # old local id l -> new local id pl[l]
    logits = np.empty_like(inp.logits)
    logits[..., sigma] = inp.logits
    e2l = np.full(cfg.E, -1, dtype=np.int32)
    loc = inp.expert_to_local >= 0
    e2l[sigma[loc]] = pl[inp.expert_to_local[loc]]
    inv = np.argsort(pl)                        # new local id -> old local id
    w = {k: getattr(inp, k)[inv] for k in ("w1_store", "w3_store", "w2_store")}
    y1, n1 = _run(cfg, _replace(inp, logits=logits, expert_to_local=e2l, **w))
    assert n1 == n0
    for a, b in zip(y0, y1):
        np.testing.assert_array_equal(b, a)


# --------------------------------------------------------------------------- fused push
# moe_forward_fused / moe_expert_ffn_push: the push is fused into the down GEMM's epilogue
# and (fp32, bf16) the pull into the gate/up GEMM's row loads.
# The fused path must reproduce the unfused path (pinned to the oracle above) bit for bit:
# recv on every local-pair entry, and y everywhere.
def _fused_cases():
    from tests.test_gpu_mx import MX_CASES, MX_EDGE
    cases = dict(FORWARD_CASES)
    cases.update({f"edge-{k}": v[0] for k, v in EDGE_CASES.items()})
    cases.update(MX_CASES)
    cases.update({k: v[0] for k, v in MX_EDGE.items()})
    nevers = {f"edge-{k}": v[1] for k, v in EDGE_CASES.items()}
    nevers.update({k: v[1] for k, v in MX_EDGE.items()})
    return cases, nevers


FUSED_CASES, FUSED_NEVER = _fused_cases()


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_forward_fused_push_equals_unfused(name):
    torch = _torch()
    cfg = FUSED_CASES[name]
    _say(f"[fused] {cfg.name}")
    inp, P = _problem(cfg, seed=3, never=FUSED_NEVER.get(name))
    P.forward()
    assert P.status() == 0
    torch.cuda.synchronize()
    so = P.slot_of.clone()
    mask = [so[r] >= 0 for r in range(cfg.R)]
    ref_recv = [P.recv[r][mask[r]].clone() for r in range(cfg.R)]
    ref_y = [t.clone() for t in P.y]

    def clear():
        for r in range(cfg.R):
            P.recv[r].fill_(float("nan"))
            P.y[r].fill_(float("nan"))

    def check(tag):
        torch.cuda.synchronize()
        assert P.status() == 0
        for r in range(cfg.R):
            assert torch.equal(P.recv[r][mask[r]], ref_recv[r]), f"{tag}: recv rank {r}"
            assert torch.equal(P.y[r], ref_y[r]), f"{tag}: y rank {r}"

    clear()
    P.forward_fused()
    check("moe_forward_fused")
    clear()
    P.layout()
    P.dispatch()
    P.ffn_push()
    P.merge()
    check("staged calls, push fused")
    if cfg.dtype != "mxfp8":
        clear()
        P.xe.fill_(0)                     # the fused pull must not read xe
        P.layout()
        P.ffn_push(pull=True)
        P.merge()
        check("staged calls, pull and push fused")
    _say(f"  N={P.N()} bit-identical")
