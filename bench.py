"""Benchmark of one GPU's share of a MoE layer forward (HIP path on MI355X).

One step = one whole forward over one batch of synthetic inputs already resident
in HBM: top-k routing, sort-free layout, pull dispatch, grouped SwiGLU expert FFN,
push combine and the final weighted merge.  Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config dsv3]

With --backward a step is instead the whole backward of the share after one forward:
bf16 configs time moe_backward's three stages (pull reverse-combine, expert SwiGLU
backward with the weight-gradient GEMMs, push reverse-dispatch with the ordered sum and
the gate gradient); MXFP8 configs time moe_backward_prepare_mx (the weights re-quantised
along the backward's K, once per weight update) and moe_backward_mx.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_layer_histogram_amd import configs, inputs  # noqa: E402

METRIC = "MoE layer fwd tokens/s; grouped-GEMM % MFMA peak; gather/combine % HBM peak"
METRIC_BWD = "MoE layer bwd tokens/s; expert-backward GEMMs % MFMA peak; reverse pull/push % HBM peak"
PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_FP8_FLOPS = 5.0e15      # MI355X dense fp8 / MXFP8 MFMA
PEAK_F32_FLOPS = 157.3e12    # MI355X fp32 matrix
PEAK_HBM = 8.0e12            # MI355X HBM3E bytes/s
CSRC = os.path.join(ROOT, "mixture_experts_layer_histogram_amd", "csrc")
# per workload: committed traffic record, GEMM kernel name, and the sources the kernels are built from
TRAFFIC = {
    "dsv3/persistent": ("traffic_persistent_dsv3_bf16.json", "moe_persistent_kernel",
                        ("persistent.hip", "persist_sched.hpp", "gemm_tile.hpp", "gemm_mx_tile.hpp", "mx.hpp",
                         "common.hpp")),
    "dsv3_mx/persistent": ("traffic_persistent_dsv3_mxfp8.json", "moe_persistent_kernel",
                           ("persistent.hip", "persist_sched.hpp", "gemm_tile.hpp", "gemm_mx_tile.hpp", "mx.hpp",
                            "common.hpp")),
    "dsv3": ("traffic_grouped_gemm_dsv3_bf16.json", "grouped_gemm_bf16_kernel",
             ("gemm.hip", "gemm_tile.hpp", "common.hpp")),
    "dsv3_mx": ("traffic_grouped_gemm_dsv3_mxfp8.json", "grouped_gemm_mx_kernel",
                ("gemm_mx.hip", "gemm_mx_tile.hpp", "gemm_tile.hpp", "mx.hpp", "common.hpp")),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3", choices=sorted(configs.CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (bf16) instead of the forward; prints its own JSON line")
    ap.add_argument("--sweep-tokens", default="",
                    help="comma-separated tokens per rank: time the forward at each (one JSON line per value; "
                         "the minibatch-size curve of the unfused path)"),
    ap.add_argument("--cpu-sample-ranks", type=int, default=0, help="0 = all ranks (the whole step)")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure this GPU's ceilings instead of the layer: bf16 and MXFP8 MFMA issue rates, the "
                         "direct global->LDS fill bandwidth missing and hitting the L2, a 1 GiB device copy; "
                         "prints its own JSON line (add --sample-clocks for the clock during the MFMA runs)")
    ap.add_argument("--signal-latency", action="store_true",
                    help="time the inter-partition hand-off (flag round trip between workgroup pairs, same XCD and "
                         "across XCDs, L2-local and agent-scope) instead of the layer; prints its own JSON line")
    ap.add_argument("--sample-clocks", action="store_true",
                    help="sample the GPU's gfx clocks and socket power with amd-smi during the timed steps "
                         "(use enough --steps for a few seconds) and report their means")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused path (ye staged, separate push kernel) instead of the fused push")
    ap.add_argument("--graph", action="store_true",
                    help="after the timed steps, capture one forward in a HIP graph and time as many replays; "
                         "reported as 'graph' (value stays the eager figure)")
    ap.add_argument("--cold-cache", action="store_true",
                    help="after the timed steps, time as many again, each after writing a 1 GiB buffer "
                         "(evicts the 4 MB L2s and the 256 MB MALL); reported as 'cold'")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run three plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--persistent", action="store_true",
                    help="time the persistent megakernel path (layout, one persistent kernel for pull dispatch into "
                         "the ring, expert FFN and push combine, merge) instead of the fused multi-kernel path")
    ap.add_argument("--fused", action="store_true",
                    help="time the fused multi-kernel path (layout, FFN with the pull and push fused in, merge)")
    ap.add_argument("--no-compare", action="store_true",
                    help="persistent path: skip timing the fused multi-kernel path beside it")
    ap.add_argument("--comm-cus", type=int, default=8,
                    help="persistent path: data-movement workgroups (8, one per XCD pipeline: the best in the sweep with the reverse ring, whose movers only gather)")
    ap.add_argument("--minibatch", type=int, default=0, help="persistent path: rows per chunk (64, 128, 256)")
    ap.add_argument("--ring-mib", type=int, default=0, help="persistent path: ring size (default: the config's)")
    ap.add_argument("--ring-order", choices=("reverse", "forward"), default="reverse",
                    help="persistent path: 'reverse' (default) walks each pipeline's row tiles from last to first, "
                         "the down GEMM stores each output row straight to recv and the ring keeps the activations "
                         "the backward reads; 'forward' walks them in layout order and the data-movement "
                         "workgroups push the output rows from the ring to recv")
    ap.add_argument("--trace", action="store_true",
                    help="persistent path: after the timed steps, one traced call; per-role busy and wait summary")
    ap.add_argument("--trace-out", default="",
                    help="with --trace: also save the raw events (numpy .npy) to this path")
    ap.add_argument("--sweep-persistent", default="",
                    help="persistent path: 'C1,C2,...:M1,M2,...' -- time every comm_cus C x minibatch M "
                         "(one JSON line per point)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of "
                         "this --config into its committed traffic record, then exit")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.split("\n"))
    return "\n".join(ln for ln in lines if ln)


def gemm_source_sha(config) -> str:
    """Hash of the kernels' sources (comments and blank lines left out, so that a comment
    edit does not retire a counter record)."""
    h = hashlib.sha256()
    for f in TRAFFIC[config][2]:
        h.update(_code_only(open(os.path.join(CSRC, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def traffic_file(config):
    return os.path.join(ROOT, "profiles", TRAFFIC[config][0])


def traffic_bytes(config):
    """HBM bytes per FFN launch pair of this workload from the committed rocprofv3 counter
    runs, or None when there is none or the GEMM sources changed since they were taken."""
    if config not in TRAFFIC:
        return None
    try:
        rec = json.load(open(traffic_file(config)))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != gemm_source_sha(config):
        return None
    return rec.get("bytes_per_step")


CAL_BYTES = 1 << 30


class ClockSampler:
    """Polls `amd-smi metric -c -p` (a child process per sample) while the timed steps run:
    the sustained gfx clock under load sets the MFMA peak actually reachable (the published
    peaks assume 2.4 GHz)."""

    def __init__(self, period=0.25):
        import threading
        self.period, self.clk, self.pw, self.n = period, [], [], 0
        self.stop_ev = threading.Event()
        self.th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        import subprocess
        while not self.stop_ev.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                                   text=True, timeout=20)
                txt = r.stdout
            except (OSError, subprocess.SubprocessError):
                return
            c = [int(v) for v in re.findall(r'"gfx_\d+": \{\s*"clk": \{\s*"value": (\d+)', txt)]
            w = re.search(r'"socket_power": \{\s*"value": (\d+)', txt)
            if c and not self.stop_ev.is_set() and min(c) >= 1000:     # idle or ramping readings at the edges of the load
                self.clk.append(float(np.mean(c)))
                self.n += 1
                if w:
                    self.pw.append(float(w.group(1)))
            self.stop_ev.wait(self.period)

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *exc):
        self.stop_ev.set()
        self.th.join(timeout=30)

    def summary(self, peak):
        if not self.clk:
            return None
        mhz = float(np.mean(self.clk))
        return {"gfx_mhz_mean": mhz, "gfx_mhz_min": float(np.min(self.clk)), "gfx_mhz_max": float(np.max(self.clk)),
                "socket_w_mean": float(np.mean(self.pw)) if self.pw else None, "samples": self.n,
                "peak_at_mean_clock": peak * mhz / 2400.0 / 1e12, "peak_unit": "TFLOP/s"}


def _per_dispatch(csv_path, counter):
    import csv
    out = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter:
            out.append((r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))
    return out


def write_traffic(config, fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the workload's dominant kernels (the two
    FFN GEMM kernels, or the persistent kernel), each scaled by (known bytes / counter) of a
    plain 1 GiB device copy in the same run."""
    kname = TRAFFIC[config][1]
    persistent = config.endswith("/persistent")
    rec = {"workload": configs.CONFIGS[config.split("/")[0]].name, "kernel": kname,
           "source_sha": gemm_source_sha(config)}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _per_dispatch(path, counter)
        cal = [v for k, v in rows if "copyBuffer" in k and 0.5 * CAL_BYTES < v < 2.0 * CAL_BYTES]
        if not cal:
            raise SystemExit(f"no 1 GiB copy dispatch found in {path}")
        factor = CAL_BYTES / float(np.median(cal))
        if persistent:
            vals = [v for k, v in rows if kname in k]
            rec[name] = {"copy_factor": factor, "kernel_bytes": float(np.median(vals)) * factor}
        else:
            g = {}
            for mode in (0, 1):
                vals = [v for k, v in rows if re.search(rf"{kname}<{mode}[,>]", k)]
                g[mode] = float(np.median(vals)) * factor
            rec[name] = {"copy_factor": factor, "gemm1_bytes": g[0], "gemm2_bytes": g[1]}
    if persistent:
        rec["bytes_per_step"] = rec["fetch"]["kernel_bytes"] + rec["write"]["kernel_bytes"]
    else:
        rec["bytes_per_step"] = (rec["fetch"]["gemm1_bytes"] + rec["fetch"]["gemm2_bytes"] +
                                 rec["write"]["gemm1_bytes"] + rec["write"]["gemm2_bytes"])
    os.makedirs(os.path.dirname(traffic_file(config)), exist_ok=True)
    json.dump(rec, open(traffic_file(config), "w"), indent=1)
    print(json.dumps(rec))


def _oracle_mx_weights(cfg, inp):
    """Offline step of the MXFP8 oracle (untimed): every local expert's weights quantised."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import mx_oracle as MX
    jobs = [(i, l) for i in range(3) for l in range(cfg.E_local)]
    src = (inp.w1_f32, inp.w3_f32, inp.w2_f32)
    out = [[None] * cfg.E_local for _ in range(3)]

    def one(job):
        i, l = job
        out[i][l] = MX.quantize(np.asarray(src[i][l], dtype=np.float64))[2]
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(one, jobs))
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, ranks, threads=None):
    """The oracle as it stands, on a bounded sample: the first `ranks` source ranks of
    the same inputs through the share (all of them by default, i.e. the whole step).
    threads: cap of the BLAS thread pool (None = the library's default, all cores)."""
    from oracle import moe_oracle as O
    from oracle import mx_oracle as MX
    from contextlib import nullcontext
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    ranks = max(1, min(ranks, cfg.R))
    limit = threadpool_limits(limits=threads) if (threads and threadpool_limits) else nullcontext()
    with limit:
        if threadpool_info:
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        else:  # pragma: no cover
            cores = threads or os.cpu_count() or 1
        if cfg.dtype == "mxfp8":
            wq = _oracle_mx_weights(cfg, inp)
            t0 = time.perf_counter()
            MX.forward_q(inp.logits[:ranks], inp.x_f32[:ranks], *wq, inp.expert_to_local, cfg.E_local, cfg.k,
                         cfg.minibatch)
            what = ("fp64 NumPy quantised oracle (route, layout, pull with MX quantisation of x, SwiGLU experts "
                    "with h quantised, push, merge; weights quantised beforehand, untimed)")
        else:
            t0 = time.perf_counter()
            O.forward(inp.logits[:ranks], inp.x_f32[:ranks], inp.w1_f32, inp.w3_f32, inp.w2_f32,
                      inp.expert_to_local, cfg.E_local, cfg.k, cfg.minibatch)
            what = "fp64 NumPy oracle (route, layout, pull, SwiGLU experts, push, merge)"
        dt = time.perf_counter() - t0
    tokens = ranks * cfg.T / cfg.G
    frac = "the whole step" if ranks == cfg.R else f"{ranks}/{cfg.R} of the step"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"source ranks 0..{ranks - 1} of the same inputs ({frac}); {what}; {dt:.2f} s wall",
            "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def cpu_baseline_bwd(cfg, inp, dy, ranks):
    """The backward oracle as it stands (it recomputes its forward) on the first `ranks`
    source ranks of the same inputs."""
    from oracle import moe_oracle_bwd as B
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ranks = max(1, min(ranks, cfg.R))
    t0 = time.perf_counter()
    B.backward(inp.logits[:ranks], inp.x_f32[:ranks], inp.w1_f32, inp.w3_f32, inp.w2_f32, inp.expert_to_local,
               cfg.E_local, cfg.k, dy[:ranks], cfg.minibatch)
    dt = time.perf_counter() - t0
    tokens = ranks * cfg.T / cfg.G
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"source ranks 0..{ranks - 1} of {cfg.R} of the same inputs; fp64 NumPy backward oracle "
                      f"(its forward, pull reverse-combine, SwiGLU backward, weight gradients, push, gate "
                      f"gradients); {dt:.2f} s wall"}


def _oracle_mx_bwd_weights(cfg, inp):
    """The MXFP8 backward oracle's quantised weights (both orientations), per expert in
    threads: untimed setup, like the weights' offline quantisation on the GPU."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import mx_oracle_bwd as QB
    def one(l):
        return QB.weights_q([inp.w1_f32[l]], [inp.w3_f32[l]], [inp.w2_f32[l]], 1)
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(one, range(cfg.E_local)))
    return {key: [p[key][0] for p in parts] for key in parts[0]}


def cpu_baseline_bwd_mx(cfg, inp, dy, ranks):
    """The MXFP8 backward oracle as it stands on the first `ranks` source ranks (weights
    quantised beforehand, untimed)."""
    from oracle import mx_oracle_bwd as QB
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    ranks = max(1, min(ranks, cfg.R))
    W = _oracle_mx_bwd_weights(cfg, inp)
    t0 = time.perf_counter()
    QB.backward_q(inp.logits[:ranks], inp.x_f32[:ranks], inp.w1_f32, inp.w3_f32, inp.w2_f32, inp.expert_to_local,
                  cfg.E_local, cfg.k, dy[:ranks], cfg.minibatch, W=W)
    dt = time.perf_counter() - t0
    tokens = ranks * cfg.T / cfg.G
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"source ranks 0..{ranks - 1} of {cfg.R} of the same inputs; fp64 NumPy MXFP8 backward oracle "
                      f"(its quantised forward, pull reverse-combine, MX data-gradient GEMMs, weight gradients, push, "
                      f"gate gradients; weights quantised beforehand, untimed); {dt:.2f} s wall"}


def run_backward_mx(args, cfg, inp, P, stream, N):
    import torch
    dy_bits, dy = inputs.make_dy(cfg, seed=args.seed)
    P.alloc_backward(dy_bits)
    for _ in range(args.warmup):
        P.prepare_backward_mx()
        P.backward_mx()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        P.prepare_backward_mx()
        ev[i][1].record(stream)
        P.backward_mx()
        ev[i][2].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(["prepare", "backward"])}
    log(f"[bench] MXFP8 backward {args.steps} steps: {ms_step:.3f} ms/step; stages {stage_ms}")
    dfn = float(cfg.d) * cfg.F * N
    fl_mx, fl_bf = 10.0 * dfn, 6.0 * dfn          # dh, GEMM1 again, dX in MXFP8; three weight gradients in bf16
    peak = (fl_mx + fl_bf) / (fl_mx / PEAK_FP8_FLOPS + fl_bf / PEAK_BF16_FLOPS)
    t_b = stage_ms["backward"] * 1e-3
    tokens = cfg.R * cfg.T / cfg.G
    result = {
        "metric": METRIC_BWD, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens and incoming gradients, fan-in scaled random expert weights, "
                "router logits x@W_r)",
        "config": {"workload": cfg.name, "R": cfg.R, "T": cfg.T, "d": cfg.d, "E": cfg.E, "E_local": cfg.E_local,
                   "k": cfg.k, "F": cfg.F, "local_pairs": N,
                   "path": "MXFP8 backward after one forward: weight re-quantisation + moe_backward_mx"},
        "roofline": {"bound": "mfma", "kernel": "moe_backward_mx (10dFN MXFP8 data-gradient FLOP + 6dFN bf16 "
                                                 "weight-gradient FLOP; peak = that mix at 5.0 and 2.5 PFLOP/s)",
                     "achieved": (fl_mx + fl_bf) / t_b / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
                     "frac": (fl_mx + fl_bf) / t_b / peak, "traffic": None},
        "stages_ms": stage_ms,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU MXFP8 backward oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline_bwd_mx(cfg, inp, dy, args.cpu_sample_ranks or 1)
    print(json.dumps(result), flush=True)


def run_ring_backward(args, cfg, P, stream, N, ms_staged_backward):
    """The backward after the persistent forward with the reverse ring (moe_backward_ring):
    each step runs that forward, then the backward timed alone, once reading the token rows
    the ring still holds in place and once pulling every row again (ring unused).  Also the
    gather moe_backward would need first (moe_dispatch_pull of all N rows)."""
    import torch
    from mixture_experts_layer_histogram_amd import moe
    ex = moe.Exec(args.minibatch or cfg.minibatch, args.comm_cus, 0, 0, 0, 1)
    P.alloc_ring(args.ring_mib or cfg.ring_mib, ex)
    out = {"ring_mib": args.ring_mib or cfg.ring_mib, "rows": N}
    for use_ring in (True, False):
        for _ in range(max(1, args.warmup // 2)):
            P.forward_persistent(ex)
            P.backward_ring(use_ring=use_ring)
        torch.cuda.synchronize()
        times = []
        for _ in range(args.steps):
            P.forward_persistent(ex)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            P.backward_ring(use_ring=use_ring)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        out["ms_with_ring" if use_ring else "ms_without_ring"] = float(np.mean(times))
    if P.status() != 0:
        raise SystemExit("device status after the ring backward")
    res = moe.read_resident(P.ws, P.shape, P.placement)
    offs = P.offsets.cpu().numpy()
    counts = np.diff(offs[:cfg.E_local + 1])
    mtb = np.concatenate([[0], np.cumsum((counts + 255) // 256)])
    mb = ex.minibatch_rows
    held = 0
    for e in np.nonzero(res)[0]:
        m, h = divmod(int(e), 4)
        l = int(np.searchsorted(mtb, m, side="right") - 1)
        row0 = int(offs[l] + (m - mtb[l]) * 256)
        held += max(0, min(row0 + (h + 1) * mb, int(offs[l + 1]), row0 + 256) - (row0 + h * mb))
    # what moe_backward needs on top after this forward: every token row gathered into xe
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        P.dispatch()
    e1.record(stream)
    torch.cuda.synchronize()
    gather_ms = e0.elapsed_time(e1) / args.steps
    out.update({"rows_held": held, "rows_pulled_again": N - held,
                "bytes_pulled_again": (N - held) * cfg.d * 2,
                "moe_backward_plus_gather_ms": ms_staged_backward + gather_ms, "gather_all_rows_ms": gather_ms,
                "path": "moe_forward_persistent with reverse_ring (not timed), then moe_backward_ring: expert "
                        "outputs from recv, held token rows read in the ring, the rest pulled again"})
    log(f"[bench] ring backward: {out}")
    return out


def run_backward(args, cfg, inp, P, stream, N):
    import torch
    if cfg.dtype == "mxfp8":
        return run_backward_mx(args, cfg, inp, P, stream, N)
    if cfg.dtype != "bf16":
        raise SystemExit("--backward: the backward is built for bf16 and MXFP8 configs")
    dy_bits, dy = inputs.make_dy(cfg, seed=args.seed)
    P.alloc_backward(dy_bits)
    for _ in range(args.warmup):
        P.backward()
    torch.cuda.synchronize()
    names = ["pull_reverse", "ffn_backward", "push_reverse"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        P.combine_reverse()
        e[1].record(stream)
        P.ffn_backward()
        e[2].record(stream)
        P.dispatch_reverse()
        e[3].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_staged = t_start.elapsed_time(t_end) / args.steps
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    per_step = [ev[i][0].elapsed_time(ev[i][len(names)]) for i in range(args.steps)]
    log(f"[bench] backward, three stage calls, {args.steps} steps: {ms_staged:.3f} ms/step; stages {stage_ms}")
    # the single call (moe_backward), whose dX GEMM writes its rows straight to recv
    fev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    fev[0].record(stream)
    for i in range(args.steps):
        P.backward()
        fev[i + 1].record(stream)
    torch.cuda.synchronize()
    fused_step = [fev[i].elapsed_time(fev[i + 1]) for i in range(args.steps)]
    ms_fused = fev[0].elapsed_time(fev[args.steps]) / args.steps
    log(f"[bench] backward, moe_backward (dX push fused), {args.steps} steps: {ms_fused:.3f} ms/step")
    ms_step = ms_staged
    if not args.unfused:
        ms_step, per_step = ms_fused, fused_step
    row = cfg.d * 2
    # dh = dO W2 (2dFN), GEMM1 again (4dFN), dX (4dFN), dW1 + dW3 + dW2 (6dFN)
    flops = 16.0 * cfg.d * cfg.F * N
    t_ffn = stage_ms["ffn_backward"] * 1e-3
    pull_bytes = 3.0 * N * row + N * 12            # dy and ye rows in, dO out; schedule, gate, dg
    push_bytes = 2.0 * N * row + N * 12            # dX rows to recv, dg beside them
    merge_bytes = 1.0 * N * row + cfg.R * cfg.T * row
    gate_bytes = cfg.R * cfg.T * (cfg.k * 16 + cfg.E * 4)
    tokens = cfg.R * cfg.T / cfg.G
    result = {
        "metric": METRIC_BWD,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens and incoming gradients, fan-in scaled random expert weights, "
                "router logits x@W_r)",
        "config": {"workload": cfg.name, "R": cfg.R, "T": cfg.T, "d": cfg.d, "E": cfg.E, "E_local": cfg.E_local,
                   "k": cfg.k, "F": cfg.F, "local_pairs": N,
                   "path": ("backward after one forward: three stage calls on one stream" if args.unfused else
                            "backward after one forward: moe_backward, the push of dX fused into its GEMM")},
        "roofline": {"bound": "mfma", "kernel": "expert SwiGLU backward stage (dh, GEMM1+SwiGLU backward, dX, "
                                                 "dW1/dW3/dW2 GEMMs)",
                     "achieved": flops / t_ffn / 1e12, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": flops / t_ffn / PEAK_BF16_FLOPS, "traffic": None},
        "stages_ms": stage_ms,
        "step_ms": {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                    "staged_calls_mean": ms_staged},
        "ms_per_step_staged": ms_staged,
        "ms_per_step_fused": ms_fused,
        "stages_hbm_frac": {
            "pull_reverse": pull_bytes / (stage_ms["pull_reverse"] * 1e-3) / PEAK_HBM,
            "push_reverse": (push_bytes + merge_bytes + gate_bytes) / (stage_ms["push_reverse"] * 1e-3) / PEAK_HBM,
        },
    }
    result["ring_backward"] = run_ring_backward(args, cfg, P, stream, N, ms_fused)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU backward oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline_bwd(cfg, inp, dy, args.cpu_sample_ranks or 1)
    print(json.dumps(result), flush=True)


def run_signal_latency(args):
    """Round trip of a flag (and of a 64 KiB or 4 KiB payload) between two workgroups, the
    one-GPU analogue of the pages' push/pull signalling latency.  128 pairs run concurrently;
    a round is one flag plus one acknowledgement per pair.  Consumer forms: 0 L2-local
    (buffer_inv sc1), 1 agent-scope release/acquire, 2 workgroup-scope invalidate
    (buffer_inv sc0, shown stale), 3 no invalidate with sc1 loads (the persistent kernel's)."""
    import torch
    from mixture_experts_layer_histogram_amd import moe
    rounds = max(100, args.steps * 25)
    names = {0: "L2-local (buffer_inv sc1)", 1: "agent-scope release/acquire",
             2: "L2-local with buffer_inv sc0 (insufficient)", 3: "L2-local, sc1 loads, no invalidate"}
    res = []
    for words in (0, 1024, 16384):
        scratch = torch.empty(moe.moe_signal_probe_bytes(words), dtype=torch.uint8, device="cuda:0")
        for cross in (0, 1):
            for scope in (0, 1, 2, 3):
                if words == 0 and scope > 1:
                    continue
                moe.moe_signal_probe(cross, scope, words, 20, scratch, check=False)     # warm-up
                rc, us, stale, tmo, same = moe.moe_signal_probe(cross, scope, words, rounds, scratch, check=False)
                res.append({"payload_bytes": words * 4, "partners": "different XCDs" if cross else "same XCD",
                            "handoff": names[scope], "us_per_round_trip": us, "stale_words": stale, "timeouts": tmo,
                            "rc": rc, "pairs_on_one_xcd": same})
                log(f"[signal] payload {words * 4} B, {'cross' if cross else 'same'}-XCD, {names[scope]}: "
                    f"{us:.2f} us/round, stale {stale}, timeouts {tmo}")
    print(json.dumps({"metric": "inter-partition signal round trip (one GPU)", "unit": "us", "n_gpus": 1,
                      "rounds": rounds, "pairs": 128, "higher_is_better": False, "results": res}), flush=True)


def run_ceilings(args):
    """The ceilings the kernels' rooflines are read against, measured on this GPU through
    moe_ceiling_probe: MFMA issue rates with operands in registers (bf16 32x32x16, MXFP8
    32x32x64), the tiles' direct global->LDS fill pattern from HBM-resident and from
    L2-resident rows, and a 1 GiB device-to-device copy."""
    import torch
    from mixture_experts_layer_histogram_amd import moe
    scratch = torch.empty(moe.moe_ceiling_probe_bytes(), dtype=torch.uint8, device="cuda:0")
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda:0")
    src.view(torch.int32).random_(0, 1 << 30)
    torch.cuda.synchronize()
    out = {"metric": "hardware ceilings (one GPU)", "n_gpus": 1, "cus": torch.cuda.get_device_properties(0).multi_processor_count}
    reps_mfma = 100000
    for kind, name, peak in ((0, "mfma_bf16", 2500.0), (1, "mfma_mxfp8", 5000.0)):
        rc, work, ms = moe.moe_ceiling_probe(kind, reps_mfma, None, 0, scratch)
        tf = work / ms / 1e9
        out[name] = {"TFLOP/s": tf, "frac_of_nameplate": tf / peak, "ms": ms, "reps_per_wave": reps_mfma}
        log(f"[ceilings] {name}: {tf:.0f} TFLOP/s = {tf / peak:.3f} of {peak:.0f} ({ms:.1f} ms)")
        if args.sample_clocks:
            # back-to-back launches for a few seconds: the sustained rate and its clock
            clk = ClockSampler(0.1)
            tot_w = tot_ms = 0.0
            with clk:
                t_end = time.time() + 4.0
                while time.time() < t_end:
                    rc, work, ms = moe.moe_ceiling_probe(kind, reps_mfma, None, 0, scratch)
                    tot_w += work
                    tot_ms += ms
            out[name]["sustained_TFLOP/s"] = tot_w / tot_ms / 1e9
            out[name]["clock"] = clk.summary(peak * 1e12)
            log(f"[ceilings] {name} sustained over 4 s: {tot_w / tot_ms / 1e9:.0f} TFLOP/s; clock {out[name]['clock']}")
    for kind, name, reps in ((2, "lds_dma_fill_from_hbm", 2), (3, "lds_dma_fill_from_l2", 200)):
        rc, work, ms = moe.moe_ceiling_probe(kind, reps, src, src.numel(), scratch)
        tbs = work / ms / 1e9
        out[name] = {"TB/s": tbs, "bytes_per_cu_cycle_at_2.4GHz": work / (ms * 1e-3) / out["cus"] / 2.4e9, "ms": ms,
                     "bytes": work}
        log(f"[ceilings] {name}: {tbs:.2f} TB/s")
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst.copy_(src[:1 << 30])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src[:1 << 30])
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / 10
    out["device_copy_1GiB"] = {"TB/s (read + write)": 2 * (1 << 30) / ms / 1e9, "ms": ms,
                               "frac_of_8TBps": 2 * (1 << 30) / ms / 1e9 / 8.0}
    log(f"[ceilings] 1 GiB copy: {out['device_copy_1GiB']['TB/s (read + write)']:.2f} TB/s")
    print(json.dumps(out), flush=True)


def run_sweep(args, cfg, P, stream):
    """Forward time against tokens handed to the layer at once.  The problem's buffers are
    sized for T tokens per rank; each point lowers the shape's T in place (every call reads
    the first T rows of each rank's token and logit buffers) and times `args.steps` steps."""
    import torch
    fwd = P.forward_persistent if args.persistent else (P.forward if args.unfused else P.forward_fused)
    T_full = P.shape.T
    for t in [int(v) for v in args.sweep_tokens.split(",")]:
        if not 1 <= t <= T_full:
            raise SystemExit(f"--sweep-tokens: {t} outside 1..{T_full}")
        P.shape.T = t
        for _ in range(args.warmup):
            fwd()
        torch.cuda.synchronize()
        if P.status() != 0:
            raise SystemExit(f"device status {P.status()} at T={t}")
        n = P.N()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fwd()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        offs = P.offsets.cpu().numpy()
        tiles1 = int(sum((int(offs[l + 1] - offs[l]) + 255) // 256 for l in range(cfg.E_local))) * ((cfg.F + 127) // 128)
        line = {"metric": "MoE layer fwd ms per call vs tokens per call", "tokens_per_rank": t,
                "source_tokens": cfg.R * t, "local_pairs": n, "ms_per_call": ms,
                "us_per_source_token": ms * 1e3 / (cfg.R * t), "gemm1_tiles": tiles1,
                "gemm1_waves": tiles1 / 256.0, "workload": cfg.name,
                "path": "persistent" if args.persistent else ("unfused" if args.unfused else "fused pull and push")}
        print(json.dumps(line), flush=True)
        log(f"[sweep] T={t}: {ms:.3f} ms, N={n}, GEMM1 tiles {tiles1} ({tiles1 / 256:.2f} waves)")
    P.shape.T = T_full


def persistent_exec(args, cfg, comm=None, mb=None, trace=0):
    from mixture_experts_layer_histogram_amd import moe
    return moe.Exec(mb or args.minibatch or cfg.minibatch, args.comm_cus if comm is None else comm, 0, trace, 0,
                    1 if getattr(args, "ring_order", "reverse") == "reverse" else 0)


def trace_summary(ev, tpu, grid):
    """Per-role figures of one traced persistent call: span, busy and waiting fractions of
    the data-movement and compute workgroups, task counts, and the overlap of combine
    (pushes) with dispatch (gathers)."""
    import numpy as np
    t0 = int(ev["t_begin"].min())
    span = float(ev["t_end"].max() - t0)
    out = {"span_us": span / tpu, "events": int(len(ev))}
    starts = ev[ev["kind"] == 0]
    role_of = {int(w): int(r) for w, r in zip(starts["workgroup"], starts["index"])}
    for role, name, kinds in ((0, "data_movement", (1, 2)), (1, "compute", (3, 4))):
        wgs = [w for w, r in role_of.items() if r == role]
        sel = ev[np.isin(ev["kind"], kinds)]
        busy = float((sel["t_end"] - sel["t_begin"]).sum())
        wait = float(sel["t_wait"].sum())
        out[name] = {"workgroups": len(wgs), "tasks": int(len(sel)),
                     "busy_frac": busy / (span * max(1, len(wgs))),
                     "wait_frac": wait / (span * max(1, len(wgs)))}
    g, pu = ev[ev["kind"] == 1], ev[ev["kind"] == 2]
    if len(g) and len(pu):
        last_gather = float(g["t_end"].max() - t0)
        first_push = float(pu["t_begin"].min() - t0)
        pushes_before = int((pu["t_begin"] < g["t_end"].max()).sum())
        out["overlap"] = {"first_push_us": first_push / tpu, "last_gather_end_us": last_gather / tpu,
                          "pushes_started_before_last_gather": pushes_before, "pushes": int(len(pu))}
    ff = ev[np.isin(ev["kind"], (3, 4))]
    if len(ff):
        out["first_gemm_us"] = float(ff["t_begin"].min() - t0) / tpu
        out["last_gemm_end_us"] = float(ff["t_end"].max() - t0) / tpu
    # per task kind: mean / max duration and mean wait before it
    out["tasks"] = {}
    for k, name in ((1, "gather"), (2, "push"), (3, "gate_up"), (4, "down")):
        e = ev[ev["kind"] == k]
        if len(e):
            d = (e["t_end"] - e["t_begin"]) / tpu
            out["tasks"][name] = {"n": int(len(e)), "us_mean": float(d.mean()), "us_max": float(d.max()),
                                  "wait_us_mean": float((e["t_wait"] / tpu).mean())}
    # down tiles a workgroup ran for another pipeline (work stealing at the end of a launch)
    pipe_of = {int(w): int(q) for w, q in zip(starts["workgroup"], starts["pipeline"])}
    dn = ev[ev["kind"] == 4]
    out["stolen_down_tiles"] = int(sum(1 for w, q in zip(dn["workgroup"], dn["pipeline"])
                                       if pipe_of.get(int(w), int(q)) != int(q)))
    # per pipeline: row tiles, end of its last GEMM and of its last task
    out["pipelines"] = []
    for p in np.unique(ev["pipeline"]):
        e = ev[ev["pipeline"] == p]
        c = e[np.isin(e["kind"], (3, 4))]
        out["pipelines"].append({"pipeline": int(p), "workgroups": int((e["kind"] == 0).sum()),
                                 "row_tiles": int(len(np.unique(c["index"] // 256))) if len(c) else 0,
                                 "last_gemm_end_us": float(c["t_end"].max() - t0) / tpu if len(c) else 0.0,
                                 "end_us": float(e["t_end"].max() - t0) / tpu,
                                 "compute_wait_ms": float(c["t_wait"].sum()) / tpu / 1e3})
    # busy compute workgroups per 100 us of the span
    nb = int(np.ceil(span / tpu / 100.0)) + 1
    occ = np.zeros(nb)
    for b0, b1 in zip((ff["t_begin"] - t0) / tpu, (ff["t_end"] - t0) / tpu):
        for i in range(int(b0 // 100), min(nb, int(b1 // 100) + 1)):
            lo, hi = max(b0, i * 100.0), min(b1, (i + 1) * 100.0)
            if hi > lo:
                occ[i] += (hi - lo) / 100.0
    out["busy_compute_workgroups_per_100us"] = [round(float(v), 1) for v in occ]
    return out


def run_persistent_sweep(args, cfg, P, stream):
    """comm_cus x minibatch grid on the persistent kernel (layout once per minibatch)."""
    import torch
    from mixture_experts_layer_histogram_amd import moe
    comms, mbs = args.sweep_persistent.split(":")
    N = P.N()
    flops = 6.0 * cfg.d * cfg.F * N
    for mb in [int(v) for v in mbs.split(",")]:
        P.ex = moe.Exec(mb, 0, 0, 0, 0)
        P.layout()
        for comm in [int(v) for v in comms.split(",")]:
            ex = persistent_exec(args, cfg, comm=comm, mb=mb)
            P.alloc_ring(args.ring_mib or cfg.ring_mib, ex)
            for _ in range(args.warmup):
                P.persistent_dfc(ex)
            torch.cuda.synchronize()
            st = P.status()
            if st != 0:
                raise SystemExit(f"device status {st} at comm_cus={comm} minibatch={mb}")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                P.persistent_dfc(ex)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            line = {"metric": "persistent kernel ms (dispatch + FFN + combine)", "workload": cfg.name,
                    "comm_cus": comm, "minibatch": mb, "ring_mib": args.ring_mib or cfg.ring_mib, "ms": ms,
                    "ring_order": args.ring_order, "ffn_tflops": flops / (ms * 1e-3) / 1e12,
                    ("frac_fp8_peak" if cfg.dtype == "mxfp8" else "frac_bf16_peak"):
                        flops / (ms * 1e-3) / (PEAK_FP8_FLOPS if cfg.dtype == "mxfp8" else PEAK_BF16_FLOPS)}
            print(json.dumps(line), flush=True)
            log(f"[sweep-persistent] comm={comm} mb={mb}: {ms:.3f} ms")


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.config + ("/persistent" if args.persistent else ""), *args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the multi-GPU expert-parallel path is not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_layer_histogram_amd import moe
    from mixture_experts_layer_histogram_amd.device import DeviceProblem

    if args.signal_latency:
        run_signal_latency(args)
        return
    if args.ceilings:
        run_ceilings(args)
        return
    cfg = configs.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating inputs for {cfg.name}")
    t0 = time.time()
    inp = inputs.make_inputs(cfg, seed=args.seed)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s; uploading")
    P = DeviceProblem(cfg, inp, device=dev)
    stream = torch.cuda.current_stream()

    # the timed path: the persistent megakernel for bf16 (every step of the share, the CU
    # partition and the ring included) unless another is asked for; the fused multi-kernel path
    # for the other dtypes unless --persistent (the persistent kernel takes bf16 and MXFP8)
    if args.unfused:
        path = "unfused"
    elif args.fused:
        path = "fused"
    elif args.persistent or (cfg.dtype == "bf16" and not (args.backward or args.sweep_tokens)):
        path = "persistent"
    else:
        path = "fused"
    args.persistent = path == "persistent"
    if args.persistent or args.sweep_persistent:
        P.ex = moe.Exec(args.minibatch or cfg.minibatch, 0, 0, 0, 0)
        P.alloc_ring(args.ring_mib or cfg.ring_mib, persistent_exec(args, cfg))
        warm = P.forward_persistent
    else:
        warm = P.forward if (args.unfused or args.backward or args.sweep_tokens) else P.forward_fused
    for _ in range(args.warmup):
        warm()
    torch.cuda.synchronize()
    st = P.status()
    if st != 0:
        raise SystemExit(f"device status {st} after warmup")
    N = P.N()
    log(f"[bench] warmup done, N={N} local pairs")
    if args.backward:
        run_backward(args, cfg, inp, P, stream, N)
        return
    if args.sweep_tokens:
        run_sweep(args, cfg, P, stream)
        return
    if args.sweep_persistent:
        run_persistent_sweep(args, cfg, P, stream)
        return

    if args.persistent:
        # one persistent kernel for the pull into the ring, the expert FFN and the push
        names = ["layout", "ffn", "merge"]
        calls = [P.layout, P.persistent_dfc, P.merge]
        fwd = P.forward_persistent
    elif args.unfused:
        names = ["layout", "dispatch", "ffn", "combine"]
        calls = [P.layout, P.dispatch, P.ffn, P.combine]
        fwd = P.forward
    elif cfg.dtype == "mxfp8":
        # the push fused into the down GEMM: "ffn" writes each result row to its recv slot
        # (the gather stays: it quantises the rows)
        names = ["layout", "dispatch", "ffn", "merge"]
        calls = [P.layout, P.dispatch, P.ffn_push, P.merge]
        fwd = P.forward_fused
    else:
        # pull and push fused: "ffn" reads each pair's token row from x and writes its result
        # row to its recv slot
        names = ["layout", "ffn", "merge"]
        calls = [P.layout, lambda: P.ffn_push(pull=True), P.merge]
        fwd = P.forward_fused
    # The timed steps: each is one call of the path's own entry point (fwd), the way a caller
    # runs the layer, with an event between steps.  The stage split comes from a second pass of
    # the same number of steps whose stages are separate calls with events between them (those
    # extra host calls and events cost a few microseconds a step, so that pass is not the
    # timed one).
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    sampler = ClockSampler() if args.sample_clocks else None
    if sampler:
        sampler.__enter__()
    sev[0].record(stream)
    for i in range(args.steps):
        fwd()
        sev[i + 1].record(stream)
    torch.cuda.synchronize()
    if sampler:
        sampler.__exit__()
    total_ms = sev[0].elapsed_time(sev[args.steps])
    ms_step = total_ms / args.steps
    per_step = [sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        for c, call in enumerate(calls):
            call()
            e[c + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    staged_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][len(names)]) for i in range(args.steps)]))
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; stages {stage_ms} (staged calls {staged_ms:.3f} ms/step)")
    compare = None
    if args.persistent and not args.no_compare:
        # context: the fused multi-kernel path on the same inputs (pull fused into the gate/up
        # GEMM, push into the down GEMM; no CU partition, no ring, h staged at worst-case size)
        # (MXFP8: the gather quantises the rows, so it stays a kernel of its own; "FFN" is then
        # the gather and the two GEMMs)
        mx = cfg.dtype == "mxfp8"
        P.forward_fused()
        torch.cuda.synchronize()
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            cev[i][0].record(stream)
            P.layout()
            cev[i][1].record(stream)
            if mx:
                P.dispatch()
                P.ffn_push()
            else:
                P.ffn_push(pull=True)
            cev[i][2].record(stream)
            P.merge()
            cev[i][3].record(stream)
        torch.cuda.synchronize()
        cst = [cev[i][0].elapsed_time(cev[i][3]) for i in range(args.steps)]
        cffn = float(np.mean([cev[i][1].elapsed_time(cev[i][2]) for i in range(args.steps)]))
        cms = float(np.mean(cst))
        cpeak = PEAK_FP8_FLOPS if mx else PEAK_BF16_FLOPS
        compare = {"path": ("fused multi-kernel (layout, quantising gather, FFN with the push fused into the down "
                            "GEMM, merge; no CU partition, no ring, xe and h staged at worst-case size)" if mx else
                            "fused multi-kernel (layout, FFN with the pull fused into the gate/up GEMM and the push "
                            "into the down GEMM, merge; no CU partition, no ring, h staged at worst-case size)"),
                   "ms_per_step": cms, "tokens_per_s": cfg.R * cfg.T / cfg.G / (cms * 1e-3), "ffn_ms": cffn,
                   ("gather_ffn_frac_fp8_peak" if mx else "ffn_frac_bf16_peak"):
                       6.0 * cfg.d * cfg.F * N / (cffn * 1e-3) / cpeak}
        log(f"[bench] fused multi-kernel path for comparison: {cms:.3f} ms/step (FFN {cffn:.3f} ms)")
        # the pull and the push as kernels of their own (the unfused path's movers) on the same
        # inputs: the HBM fractions of gather and combine by themselves
        P.dispatch()
        P.ffn()
        P.combine()
        torch.cuda.synchronize()
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for i in range(args.steps):
            mev[i][0].record(stream)
            P.dispatch()
            mev[i][1].record(stream)
            P.ffn()
            mev[i][2].record(stream)
            P.combine()
            mev[i][3].record(stream)
        torch.cuda.synchronize()
        row_b = cfg.d * 2
        g_ms = float(np.mean([mev[i][0].elapsed_time(mev[i][1]) for i in range(args.steps)]))
        c_ms = float(np.mean([mev[i][2].elapsed_time(mev[i][3]) for i in range(args.steps)]))
        g_bytes = N * row_b + N * (cfg.d + cfg.d // 32) + N * 8 if mx else 2.0 * N * row_b + N * 8
        compare["standalone_movers"] = {
            "gather_ms": g_ms, "gather_hbm_frac": g_bytes / (g_ms * 1e-3) / PEAK_HBM,
            "push+merge_ms": c_ms,
            "push+merge_hbm_frac": (2.0 * N * row_b + N * row_b + cfg.R * cfg.T * row_b) / (c_ms * 1e-3) / PEAK_HBM}
        log(f"[bench] standalone movers: {compare['standalone_movers']}")
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fwd()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fwd()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = {"ms_per_step": gms, "tokens_per_s": cfg.R * cfg.T / cfg.G / (gms * 1e-3),
                 "note": "one moe_forward captured in a HIP graph, replayed back to back"}
        log(f"[bench] graph replay: {gms:.3f} ms/step")
    cold = None
    if args.cold_cache:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 255)
            e = cev[i]
            e[0].record(stream)
            for c, call in enumerate(calls):
                call()
                e[c + 1].record(stream)
        torch.cuda.synchronize()
        del flush
        cs = [cev[i][0].elapsed_time(cev[i][len(names)]) for i in range(args.steps)]
        cold = {"note": "each step after a 1 GiB buffer write; flush not timed",
                "ms_per_step": {"median": float(np.median(cs)), "min": float(np.min(cs)), "mean": float(np.mean(cs))},
                "stages_ms": {n: float(np.median([cev[i][j].elapsed_time(cev[i][j + 1]) for i in range(args.steps)]))
                              for j, n in enumerate(names)}}
        log(f"[bench] cold cache: {cold}")
    if args.copy_calibration:
        src = torch.empty(CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    counts = P.counts.cpu().numpy().astype(np.int64)
    local_counts = counts[np.asarray(inp.expert_to_local) >= 0]
    mean_load = cfg.R * cfg.T * cfg.k / cfg.E
    load = {"kind": cfg.load, "mean_pairs_per_expert": mean_load,
            "local_max_pairs": int(local_counts.max()) if local_counts.size else 0,
            "local_max_over_mean": float(local_counts.max() / mean_load) if local_counts.size else 0.0}
    esz = 4 if cfg.dtype == "f32" else 2
    row = cfg.d * esz
    flops = 6.0 * cfg.d * cfg.F * N
    peak = {"f32": PEAK_F32_FLOPS, "bf16": PEAK_BF16_FLOPS, "mxfp8": PEAK_FP8_FLOPS}[cfg.dtype]
    t_ffn = stage_ms["ffn"] * 1e-3
    if cfg.dtype == "mxfp8":     # bf16 row in, E4M3 codes + one scale byte per 32 out
        gather_bytes = N * row + N * (cfg.d + cfg.d // 32) + N * 8
    else:
        gather_bytes = 2.0 * N * row + N * 8
    push_bytes = 2.0 * N * row
    merge_bytes = 1.0 * N * row + cfg.R * cfg.T * row
    tokens = cfg.R * cfg.T / cfg.G
    value = tokens / (ms_step * 1e-3)
    traffic = traffic_bytes(args.config + "/persistent" if args.persistent else args.config)
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, fan-in scaled random expert weights, router logits x@W_r)",
        "config": {"workload": cfg.name, "R": cfg.R, "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "E_local": cfg.E_local, "k": cfg.k, "F": cfg.F, "local_pairs": N, "load": load,
                   "path": (("persistent megakernel, reverse ring (layout; one persistent kernel whose "
                             "data-movement workgroups pull token rows into the ring while its compute workgroups run "
                             "the grouped SwiGLU GEMMs, each pipeline walking its row tiles from last to first; the "
                             "down GEMM stores every output row straight to recv and the ring keeps the token and h "
                             "rows of its last chunks for the backward; merge)" if args.ring_order == "reverse" else
                             "persistent megakernel (layout; one persistent kernel whose data-movement "
                             "workgroups pull token rows into the ring and push finished rows to recv while its "
                             "compute workgroups run the grouped SwiGLU GEMMs; merge)") if args.persistent else
                            "unfused (layout, dispatch, ffn writing ye, push + merge kernels on one stream)"
                            if args.unfused else
                            ("fused push (layout, dispatch, ffn whose down GEMM writes each row to its recv slot, "
                             "merge; kernels on one stream)" if cfg.dtype == "mxfp8" else
                             "fused pull and push (layout, ffn whose gate/up GEMM reads each pair's token row from "
                             "its source buffer and whose down GEMM writes each row to its recv slot, merge; "
                             "kernels on one stream)"))},
        "roofline": {"bound": "mfma", "kernel": "grouped SwiGLU FFN (gate/up+SwiGLU, down GEMMs)",
                     "achieved": flops / t_ffn / 1e12, "peak": peak / 1e12, "unit": "TFLOP/s",
                     "frac": flops / t_ffn / peak, "traffic": traffic},
        "stages_ms": stage_ms,
        "step_ms": {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                    "staged_calls_mean": staged_ms},
        "stages_hbm_frac": {
            **({"dispatch": gather_bytes / (stage_ms["dispatch"] * 1e-3) / PEAK_HBM} if "dispatch" in stage_ms else {}),
            **({"combine+merge": (push_bytes + merge_bytes) / (stage_ms["combine"] * 1e-3) / PEAK_HBM}
               if args.unfused else {"merge": merge_bytes / (stage_ms["merge"] * 1e-3) / PEAK_HBM}),
        },
        "pairs_per_s": N / (ms_step * 1e-3),
        "source_tokens_per_s": cfg.R * cfg.T / (ms_step * 1e-3),
    }
    if args.persistent:
        pex = persistent_exec(args, cfg)
        result["config"].update({"ring_mib": args.ring_mib or cfg.ring_mib, "minibatch": pex.minibatch_rows,
                                 "comm_cus": pex.comm_cus, "ring_order": args.ring_order})
        if cfg.dtype == "mxfp8":
            result["config"]["path"] = (
                "persistent megakernel, MXFP8 (layout; one persistent kernel whose data-movement workgroups "
                "quantise token rows into the ring slots (E4M3 codes and E8M0 scale words) while its compute "
                "workgroups run the grouped SwiGLU GEMMs on the slots, writing h's codes and scales back into "
                "the slot; the down GEMM stores every output row straight to recv; "
                + ("each pipeline walks its row tiles from last to first; " if args.ring_order == "reverse" else "")
                + "merge)")
        result["roofline"]["kernel"] = ("persistent kernel (pull into the ring, gate/up+SwiGLU and down GEMMs, push"
                                        + (" by the down GEMM's row stores" if args.ring_order == "reverse"
                                           or cfg.dtype == "mxfp8" else "")
                                        + "), FLOPs of the GEMMs")
        # the movers' algorithmic bytes inside the persistent kernel: rows in and out of the ring
        result["stages_hbm_frac"]["dispatch+combine in the persistent kernel"] = (
            (gather_bytes + push_bytes) / t_ffn / PEAK_HBM)
        if args.trace:
            tex = persistent_exec(args, cfg, trace=1)
            wsb = moe.moe_persistent_workspace_bytes(P.shape, P.placement, tex)
            tws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
            moe.moe_forward_persistent(P.shape, P.placement, tex, P.logits, P.x, *P.weights(), P.ring,
                                       P.recv, P.y, P.topk_idx, P.topk_w, P.counts, P.offsets, P.pull_src,
                                       P.slot_of, tws, w_scales=P.w_scales)
            if moe.moe_read_status(tws) != 0:
                raise SystemExit("device status after the traced call")
            ev, tpu = moe.read_trace(tws, P.shape, P.placement, tex)
            if args.trace_out:
                np.save(args.trace_out, ev)
            result["trace"] = trace_summary(ev, tpu, P.cu_grid() if hasattr(P, "cu_grid") else 0)
            log(f"[bench] trace: {result['trace']}")
            del tws
    else:
        # the fused path: the pull and push bytes moved inside the FFN kernels, over the FFN time
        if not args.unfused and cfg.dtype != "mxfp8":
            result["stages_hbm_frac"]["dispatch+combine fused in the FFN"] = (gather_bytes + push_bytes) / t_ffn / PEAK_HBM
    if compare:
        result["fused_multi_kernel"] = compare
    if graph:
        result["graph"] = graph
    if cold:
        result["cold"] = cold
    if sampler:
        result["clocks"] = sampler.summary(peak)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample (all cores, then one thread on one rank)")
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_ranks or cfg.R)
        result["cpu_baseline_single_thread"] = cpu_baseline(cfg, inp, 1, threads=1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
