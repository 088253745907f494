"""Benchmark of the int4 grouped-GEMM MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch: lily_moe_route
(top-k, softmax, histogram, scan, scatter, block map) then the stages of
lily_moe_forward (lily_moe_ffn: gate/up + SwiGLU and down in one launch;
lily_moe_combine) for one MoE layer of
T = 2048 tokens (H 2048, F 512, 256 experts top-8 + 1 shared, int4 g64,
router logits N(0,1) plus a Zipf(1.1) log-bias per expert). Steps cycle
through several distinct layer weight sets (8 by default, 3.6 GB) so that
the weights stream from HBM instead of the on-package cache. Inputs are
resident in HBM before timing starts.

Prints ONE JSON line. ``value`` is MoE-layer tokens/s = T / (seconds per
step), timed with the wall clock between two device synchronisations.
A prefill run does 200 untimed warm-up steps (the clocks settle over the
first hundred or so), 50 untimed steps with HIP events around every stage
(``stages_ms``, and the choice of the dominant stage), then the 1000 timed
steps. ``roofline`` reports the dominant kernel: its algorithmic flops (or
bytes) per launch over its average duration from the HIP events recorded on
the launch stream around its launch in every timed step. ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload (about 10 s).

By default the run also measures the other configurations of the layer at
their stated sizes and reports them as extra keys (``extra``): one layer at
T = 512 (uniform routing, weight-streaming), and batch-1 decode through 40
distinct resident layers in one launch per step. ``--peaks`` measures the
device's achievable MFMA and HBM-read peaks instead (the calibration kernels
of include/lily_calib.h) and writes them to profiles/peaks.json, from which
``roofline.frac_of_measured`` is reported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer prefill tokens/s (T=2048, int4 g64); % of HBM / MFMA peak"
WORKLOAD = "prefill2048_zipf"
PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill2048_zipf.txt")
PEAKS_FILE = os.path.join(ROOT, "profiles", "peaks.json")
KERNEL_SOURCES = [os.path.join(ROOT, "int4_grouped_gemm_amd", "csrc", f)
                  for f in ("gemm_w4.hip", "gemm_common.hpp", "route.hip", "common.hpp", "topk.hpp",
                            "w4.hpp")]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "prefill512", "prefill8192", "decode40", "stack40"],
                    help="prefill2048_zipf (the headline), decode40 (T=1, 40-layer steps) or "
                         "stack40 (40 distinct layers, T=8192 in chunks of 2048, residual glue)")
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 1000 for a prefill layer, 50 for decode40 "
                         "and stack40)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 200 for a prefill layer, 10 for "
                         "decode40 and stack40)")
    ap.add_argument("--layers", type=int, default=None,
                    help="distinct layer weight sets (prefill: cycled, default 8; decode: "
                         "default 40, the stack's own depth)")
    ap.add_argument("--tile-m", type=int, default=128)
    ap.add_argument("--decode-path", default="stack", choices=["fused", "layer", "stack"],
                    help="decode40: lily_moe_decode_stack (the 40 layers and their residual "
                         "glue in one launch), lily_moe_decode (one launch per layer), or "
                         "route + forward")
    ap.add_argument("--router", action="store_true",
                    help="start each step from x: the router projection x.Wr^T (lily_moe_router) "
                         "computes the logits inside the timed step")
    ap.add_argument("--route-host", action="store_true",
                    help="ablation: route with lily_moe_route_host (histogram, scan, scatter and "
                         "block map on the host after a stream synchronisation)")
    ap.add_argument("--separate-gemms", action="store_true",
                    help="time gate/up and down as two launches (lily_moe_gate_up, "
                         "lily_moe_down) instead of lily_moe_ffn")
    ap.add_argument("--unfused", action="store_true",
                    help="ablation: lily_moe_dequant (bf16 weights of the used experts to HBM) "
                         "then lily_moe_forward_bf16 (the same GEMMs on bf16 tiles); tile_m 32 "
                         "or 64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline only: skip the T=512 and decode40 measurements")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of layer 0 the CPU oracle computes for the baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (twice) so that "
                         "profiler byte counters can be scaled against a known size")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the achievable MFMA and HBM-read peaks and the clock; with "
                         "--write-peaks, record them in profiles/peaks.json")
    ap.add_argument("--write-peaks", action="store_true")
    args = ap.parse_args()
    layer_step = args.workload not in ("decode40", "stack40")
    if args.steps is None:
        args.steps = 1000 if layer_step else 50
    if args.warmup is None:
        args.warmup = 200 if layer_step else 10
    return args


def stage_work(cfg, P):
    """Algorithmic work per launch of each stage (flops for GEMMs, bytes
    for the memory-bound stages)."""
    rows = P + cfg.T
    return {
        "router": ("mfma", 2.0 * cfg.T * cfg.H * cfg.E),
        "route": ("hbm", cfg.T * cfg.E * 4 + P * 4 * 4 + cfg.T * cfg.k * 4),
        "gate_up": ("mfma", 2.0 * rows * cfg.H * 2 * cfg.F),
        "down": ("mfma", 2.0 * rows * cfg.F * cfg.H),
        "ffn": ("mfma", 2.0 * rows * cfg.H * 3 * cfg.F),
        "combine": ("hbm", rows * cfg.H * 4 + cfg.T * cfg.H * 2 + P * 8),
        # unfused twin: the packed weights of every expert read (upper bound:
        # only used ones are) and their bf16 written; then both GEMMs
        "dequant": ("hbm", (cfg.E + 1) * 3 * cfg.H * cfg.F * (0.5625 + 2.0)),
        "forward_bf16": ("mfma", 2.0 * rows * cfg.H * 3 * cfg.F),
    }


def expert_bytes(cfg) -> float:
    """Packed bytes of one expert's three matrices (4.5 bits per weight)."""
    return 3 * cfg.H * cfg.F * (0.5 + 4.0 / 64)


def measured_peaks():
    """The achievable peaks recorded by --peaks, or None."""
    if not os.path.exists(PEAKS_FILE):
        return None
    try:
        return json.load(open(PEAKS_FILE))
    except (OSError, ValueError):
        return None


def frac_of_measured(bound, achieved):
    pk = measured_peaks()
    if not pk:
        return None
    ref = pk.get("mfma_bf16_tflops") if bound == "mfma" else pk.get("hbm_read_gbs")
    return round(achieved / ref, 4) if ref else None


def upload_layers(L, S, cfg, layers, dev):
    """Draws the weights of the given layers on the host cores (a thread pool:
    the generator releases the GIL for the bulk of the work) and uploads
    them packed, in order."""
    import concurrent.futures as cf
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    out = []
    with cf.ThreadPoolExecutor(n) as ex:
        for i, lw in enumerate(ex.map(lambda l: S.layer_weights(cfg, l), layers)):
            out.append(L.weights_from_host(lw, dev))
            if i % 10 == 9:
                print(f"# {i + 1} layers uploaded", file=sys.stderr, flush=True)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the layer is a single-GPU kernel path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.peaks:
        return main_peaks(args)
    if args.workload == "decode40":
        res = run_decode(args, args.layers or 40, args.steps, args.warmup, args.decode_path)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_decode()
        print(json.dumps(res), flush=True)
        return
    if args.workload == "stack40":
        return main_stack(args)
    return main_prefill(args)


def copy_calibration(dev):
    """Two plain device copies of 256 MiB after the timed region: the
    reference that FETCH_SIZE / WRITE_SIZE counter passes are scaled by."""
    import torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def check_give_up(L, sched, what):
    """Exit non-zero if a bounded device-wide wait gave up during the timed
    steps (sched[30], which no call clears): the outputs, and so the timing,
    are not valid (the workgroups were not all resident, or a device fault)."""
    if int(sched[L.SCHED_GIVE_UP].item()) != 0:
        print(f"{what}: a bounded device-wide wait gave up (sched[30] set): outputs and timing "
              "are not valid", file=sys.stderr)
        sys.exit(3)


def main_prefill(args):
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[args.workload]
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, args.tile_m)
    P = cfg.T * cfg.k
    n_sets = args.layers or 8

    # ---- inputs, resident in HBM before timing
    t_gen = time.time()
    weights = upload_layers(L, S, cfg, range(n_sets), dev)
    logits, routers = [], []
    for layer in range(n_sets):
        if args.router:
            routers.append(torch.from_numpy(S.router_weights(cfg, layer).view(np.int16)).to(dev))
            logits.append(torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev))
        else:
            logits.append(torch.from_numpy(S.router_logits(cfg, layer)).to(dev))
    x = torch.from_numpy(S.activations(cfg).view(np.int16)).to(dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    if args.unfused and args.tile_m not in (32, 64):
        sys.exit("--unfused needs --tile-m 32 or 64")
    bf16w = L.alloc_bf16_weights(d, dev) if args.unfused else None
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    stages = (("router",) if args.router else ()) + (
        ("route", "dequant", "forward_bf16") if args.unfused else
        ("route", "gate_up", "down", "combine") if args.separate_gemms else
        ("route", "ffn", "combine"))

    def step(i, ev=None, only=None):
        """One layer step; ev: events recorded around every stage's call, or
        (only = a stage index) around that call alone."""
        layer = i % n_sets
        w = weights[layer]
        calls = []
        if args.router:
            calls.append(lambda: L.lily_moe_router(d, routers[layer], x, logits[layer], stream))
        route = L.lily_moe_route_host if args.route_host else L.lily_moe_route
        calls.append(lambda: route(d, logits[layer], routing, stream))
        if args.unfused:
            calls += [lambda: L.lily_moe_dequant(d, w, routing, bf16w, stream),
                      lambda: L.lily_moe_forward_bf16(d, bf16w, x, routing, out, ws,
                                                      stream=stream)]
        elif args.separate_gemms:
            calls += [lambda: L.lily_moe_gate_up(d, w, x, routing, ws, stream),
                      lambda: L.lily_moe_down(d, w, routing, ws, stream),
                      lambda: L.lily_moe_combine(d, routing, ws, out, stream)]
        else:
            calls += [lambda: L.lily_moe_ffn(d, w, x, routing, ws, stream),
                      lambda: L.lily_moe_combine(d, routing, ws, out, stream)]
        for j, call in enumerate(calls):
            if ev is not None and only is None:
                ev[j].record(stream)
            elif ev is not None and j == only:
                ev[0].record(stream)
            call()
            if ev is not None and j == only:
                ev[1].record(stream)
        if ev is not None and only is None:
            ev[len(calls)].record(stream)

    # Untimed warmup (the clocks and the weight sets' first touches settle
    # over the first hundred steps or so), then one untimed pass with events
    # around every stage for the stage breakdown and the dominant stage.
    for i in range(args.warmup):
        step(i)
    n_split = 50
    split_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
                for _ in range(n_split)]
    for i in range(n_split):
        step(args.warmup + i, split_ev[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in split_ev]))
                for j, s in enumerate(stages)}
    dom = max(stages, key=lambda s: stage_ms[s])
    dom_j = stages.index(dom)

    # The timed steps: events only around the dominant stage's launch, on
    # the stream it runs on, for its roofline.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(2):  # the first steps after the event pass
        step(args.warmup + n_split + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + n_split + 2 + i, events[i], dom_j)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    check_give_up(L, routing.sched, "prefill")

    if args.copy_calibration:
        copy_calibration(dev)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = cfg.T / ((t1 - t0) / args.steps)
    dom_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events]))

    work = stage_work(cfg, P)
    bound, amount = work[dom]
    if bound == "mfma":
        achieved = amount / (dom_ms * 1e-3) / 1e12
        peak, unit = PEAK_MFMA_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = amount / (dom_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.loads([ln for ln in open(TRAFFIC_FILE) if ln.startswith("{")][0])
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("stage") == dom \
                and tr.get("tile_m") == args.tile_m and tr.get("workload") == args.workload \
                and not args.router:
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "kernel_ms": round(dom_ms, 4),
                "frac_of_measured": frac_of_measured(bound, achieved)}

    # whole-layer fractions: useful flops and the weight bytes one layer must read
    counts = routing.counts.cpu().numpy()
    used = int((counts > 0).sum()) + 1
    w_bytes = used * expert_bytes(cfg)
    layer_flops = 2.0 * 3 * cfg.H * cfg.F * (P + cfg.T)
    step_s = ms_per_step * 1e-3

    result = {
        "metric": METRIC if args.workload == WORKLOAD else
                  f"MoE-layer prefill tokens/s (T={cfg.T}, int4 g64); % of HBM / MFMA peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "T": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E,
            "topk": cfg.k,
            "shared_experts": 1, "group": 64, "tile_m": args.tile_m,
            "layer_weight_sets": n_sets,
            "logits": "router projection x.Wr^T in the step" if args.router
                      else "given (router_logits)",
            "routing": "logits N(0,1) + per-expert Zipf(1.1) log-bias" if cfg.zipf
                       else "logits N(0,1)",
            "weights": "int4 q~U{0..15}, bf16 scale~U(0.005,0.02), bf16 bias~N(0,0.01)",
            "route": "host-synchronised (lily_moe_route_host)" if args.route_host
                     else "GPU-resident (lily_moe_route)",
            "dequant": "unfused: bf16 weights through HBM (lily_moe_dequant + "
                       "lily_moe_forward_bf16)" if args.unfused
                       else "fused into the grouped GEMM",
        },
        "layer": {
            "mfma_frac": round(layer_flops / step_s / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
            "hbm_weight_frac": round(w_bytes / step_s / 1e9 / PEAK_HBM_GBS, 4),
            "experts_touched": used,
        },
        "stages_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "roofline": roofline,
    }
    del weights, logits, routers, ws, routing, out, bf16w
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        # The oracle on the same steps: route + forward of the layer weight
        # sets in the GPU's order, until about ten seconds of CPU work (the
        # inputs' generation is not timed).
        import oracle
        xs = S.activations(cfg)
        ntok = min(args.cpu_tokens, cfg.T)
        cpu_s, layers_done = 0.0, 0
        while layers_done < n_sets and cpu_s < 10.0:
            lw = S.layer_weights(cfg, layers_done)
            lg = S.router_logits(cfg, layers_done)
            c0 = time.perf_counter()
            rr = oracle.route(lg, cfg.k, args.tile_m)
            oracle.forward(xs, rr["topk_ids"], rr["topk_w"], oracle.getter_from_layer(lw),
                           cfg.H, cfg.F, cfg.E, tokens=list(range(ntok)))
            cpu_s += time.perf_counter() - c0
            layers_done += 1
        result["cpu_baseline"] = {
            "value": round(ntok * layers_done / cpu_s, 2), "unit": "tokens/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{layers_done} layer steps (weight sets 0..{layers_done - 1}), each the "
                      f"route of all {cfg.T} tokens + forward of {ntok} tokens (dequant of the "
                      f"experts they use included), {cpu_s:.1f} s",
        }

    if args.workload == WORKLOAD and not (args.no_extra or args.router or args.route_host
                                          or args.unfused):
        result["extra"] = {
            "prefill512": run_prefill_rate(S.CONFIGS["prefill512"], 8, 1000, 200),
            "decode40": run_decode(args, 40, 50, 20, "stack", brief=True),
        }
    print(json.dumps(result), flush=True)


def run_prefill_rate(cfg, n_sets, steps, warmup, tile_m=128):
    """Route + forward of one layer per step, cycling n_sets weight sets: the
    layer's tokens/s and the fraction of HBM peak at which it streams the
    weights of the experts it touches."""
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    dev = torch.device("cuda:0")
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    weights = upload_layers(L, S, cfg, range(n_sets), dev)
    logits = [torch.from_numpy(S.router_logits(cfg, layer)).to(dev) for layer in range(n_sets)]
    x = torch.from_numpy(S.activations(cfg).view(np.int16)).to(dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        L.lily_moe_route(d, logits[i % n_sets], routing, stream)
        L.lily_moe_forward(d, weights[i % n_sets], x, routing, out, ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    s = (time.perf_counter() - t0) / steps
    used = int((routing.counts.cpu().numpy() > 0).sum()) + 1
    gbs = used * expert_bytes(cfg) / s / 1e9
    res = {"T": cfg.T, "tokens_per_s": round(cfg.T / s, 1), "us_per_layer": round(s * 1e6, 2),
           "weight_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "experts_touched": used, "layer_weight_sets": n_sets, "tile_m": tile_m}
    del weights, ws, routing
    torch.cuda.empty_cache()
    return res


def run_decode(args, n_layers_distinct, steps, warmup, path, brief=False):
    """Batch-1 decode: one step = the 40 MoE layers of the stack at T = 1.
    The stack holds n_layers_distinct distinct resident weight sets (40: every
    layer its own). Each of the 256 steps has its own activations and router
    logits per layer; all inputs are resident before timing. Exits with an
    error if a decode barrier gave up (routing.sched[30]): its outputs, and so
    the timing, would be invalid."""
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS["decode40"]
    n_layers = cfg.layers
    d = L.dims(1, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    t_gen = time.time()
    weights = upload_layers(L, S, cfg, range(n_layers_distinct), dev)
    n_steps = warmup + steps
    logits = torch.from_numpy(np.stack([np.stack([S.router_logits(cfg, layer, step % cfg.steps)
                                                  for layer in range(n_layers)])
                                        for step in range(n_steps)])).to(dev)
    xs = torch.from_numpy(np.stack([S.activations(cfg, step % cfg.steps).view(np.int16)
                                    for step in range(n_steps)])).to(dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((1, cfg.H), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    layer_w = [weights[layer % n_layers_distinct] for layer in range(n_layers)]
    if path == "stack":
        table = L.layer_table(layer_w, dev)
        r_st = torch.empty(cfg.H, dtype=torch.float32, device=dev)
        outs_st = torch.empty((n_layers, cfg.H), dtype=torch.int16, device=dev)
        ids_st = torch.empty((n_layers, cfg.k), dtype=torch.int32, device=dev)
        w_st = torch.empty((n_layers, cfg.k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print(f"# decode inputs ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    def step(i):
        if path == "stack":
            L.lily_moe_decode_stack(d, n_layers, table, logits[i], xs[i], r_st, outs_st, ids_st,
                                    w_st, routing.sched, ws, 1e-6, stream)
            return
        for layer in range(n_layers):
            if path == "fused":
                L.lily_moe_decode(d, layer_w[layer], logits[i, layer], xs[i], routing, out, ws,
                                  stream)
            else:
                L.lily_moe_route(d, logits[i, layer], routing, stream)
                L.lily_moe_forward(d, layer_w[layer], xs[i], routing, out, ws, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if getattr(args, "copy_calibration", False) and not brief:
        copy_calibration(dev)
    check_give_up(L, routing.sched, "decode")
    ms_per_step = (t1 - t0) * 1e3 / steps
    us_per_layer = ms_per_step * 1e3 / n_layers
    # weight bytes a layer must read: the k routed experts and the shared one
    layer_bytes = (cfg.k + 1) * expert_bytes(cfg)
    gbs = layer_bytes / (us_per_layer * 1e-6) / 1e9
    del weights, ws, routing, logits, xs, layer_w
    if path == "stack":
        del table
    torch.cuda.empty_cache()
    paths = {"fused": "lily_moe_decode, one launch per layer",
             "layer": "lily_moe_route + lily_moe_forward (tile_m 32)",
             "stack": "lily_moe_decode_stack: 40 layers and the residual glue in one launch"}
    if brief:
        return {"us_per_layer": round(us_per_layer, 3), "ms_per_step": round(ms_per_step, 4),
                "weight_gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "distinct_layers": n_layers_distinct, "path": paths[path]}
    return {
        "metric": "MoE-layer decode time per layer (T=1, 40-layer step, int4 g64); % of HBM peak",
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode40", "T": 1, "H": cfg.H, "F": cfg.F, "E": cfg.E,
                   "topk": cfg.k, "layers_per_step": n_layers,
                   "distinct_layers": n_layers_distinct, "path": paths[path]},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "whole layer", "frac_of_measured": frac_of_measured("hbm", gbs)},
    }


def expert_getter(S, cfg, layer):
    """Oracle expert getter that draws each requested expert's matrices from
    its own seeded stream (only the experts a sample routes to)."""
    cache = {}

    def get(tensor, e):
        key = (tensor, e)
        if key not in cache:
            cache[key] = S.expert_matrix(cfg, layer, e, tensor)
        return cache[key]

    return get, cache


def oracle_chain_sample(cfg, samples, tile_m):
    """The oracle's layer chain (route, forward, residual glue) for sampled
    tokens: samples = [(chunk or step, token indices)]. Returns the seconds
    spent in oracle calls (weight generation excluded) and the count of
    (token, layer) pairs."""
    import numpy as np

    import oracle
    from synth import inputs as S

    x0 = np.concatenate([S.activations(cfg, c)[np.asarray(toks)] for c, toks in samples])
    r = ((x0.astype(np.uint32) << 16).view(np.float32)).copy()
    x = oracle.residual_norm(r, None, 1e-6)
    spent = 0.0
    for layer in range(cfg.layers):
        lgs = np.concatenate([S.router_logits(cfg, layer, c)[np.asarray(toks)]
                              for c, toks in samples])
        rr = oracle.route(lgs, cfg.k, tile_m)
        get, cache = expert_getter(S, cfg, layer)
        for e in set(np.unique(rr["topk_ids"]).tolist()) | {cfg.E}:  # draw outside the timing
            for t in range(3):
                get(t, e)
        c0 = time.perf_counter()
        rr = oracle.route(lgs, cfg.k, tile_m)
        _, out = oracle.forward(x, rr["topk_ids"], rr["topk_w"], get, cfg.H, cfg.F, cfg.E)
        x = oracle.residual_norm(r, out, 1e-6)
        spent += time.perf_counter() - c0
        del cache
    return spent, len(x0) * cfg.layers


def cpu_baseline_decode():
    import oracle
    from synth import inputs as S
    cfg = S.CONFIGS["decode40"]
    steps = list(range(16))
    spent, n = oracle_chain_sample(cfg, [(s, [0]) for s in steps], 32)
    return {"value": round(spent * 1e6 / n, 1), "unit": "us/layer", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"sampled: decode steps 0-15 of 256 through all {cfg.layers} layers "
                      f"(route, forward, residual glue per layer; weight generation excluded), "
                      f"{spent:.1f} s"}


def main_stack(args):
    """Prefill through a stack of 40 distinct MoE layers (18.2 GB of int4
    weights resident): T = 8192 tokens in 4 chunks of 2048, chunk-major; each
    chunk runs layer after layer (route + forward), chained by the residual
    glue (r += out; next input bf16(r / rms(r))). One step = the whole stack
    for all 8192 tokens. Router logits per (layer, chunk) are given."""
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS["stack40_T8192"]
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, args.tile_m)
    t_gen = time.time()
    weights = upload_layers(L, S, cfg, range(cfg.layers), dev)
    logits = [[torch.from_numpy(S.router_logits(cfg, layer, c)).to(dev) for c in range(cfg.chunks)]
              for layer in range(cfg.layers)]
    x0 = [torch.from_numpy(S.activations(cfg, c).view(np.int16)).to(dev) for c in range(cfg.chunks)]
    r0 = [torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev) for _ in range(cfg.chunks)]
    for c in range(cfg.chunks):  # r0 = fp32(x0): bf16 bits shifted into the high half
        r0[c].view(torch.int32).copy_(x0[c].to(torch.int32).bitwise_left_shift(16))
    r = torch.empty_like(r0[0])
    x = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step():
        for c in range(cfg.chunks):
            r.copy_(r0[c])
            L.lily_residual_norm(cfg.T, cfg.H, r, None, x, 1e-6, stream)
            for layer in range(cfg.layers):
                L.lily_moe_route(d, logits[layer][c], routing, stream)
                L.lily_moe_forward(d, weights[layer], x, routing, out, ws, stream=stream)
                L.lily_residual_norm(cfg.T, cfg.H, r, out, x, 1e-6, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    check_give_up(L, routing.sched, "stack")
    s_step = (t1 - t0) / args.steps
    n_tok = cfg.T * cfg.chunks
    layer_flops = 2.0 * 3 * cfg.H * cfg.F * (cfg.k + 1) * n_tok * cfg.layers
    # every chunk-layer touches (nearly) all experts: their weights are read once per chunk
    w_bytes = (cfg.E + 1) * expert_bytes(cfg) * cfg.chunks * cfg.layers
    result = {
        "metric": "MoE-layer prefill tokens/s per layer (40-layer stack, T=8192 in chunks of "
                  "2048, int4 g64); % of HBM / MFMA peak",
        "value": round(n_tok * cfg.layers / s_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(s_step * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "stack40", "layers": cfg.layers, "tokens": n_tok,
                   "chunk_tokens": cfg.T, "H": cfg.H, "F": cfg.F, "E": cfg.E, "topk": cfg.k,
                   "tile_m": args.tile_m, "glue": "r += out; x = bf16(r / rms(r))",
                   "weights_resident_gb": round(cfg.layers * (cfg.E + 1) * expert_bytes(cfg) /
                                                1e9, 2)},
        "layer": {"mfma_frac": round(layer_flops / s_step / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                  "hbm_weight_frac": round(w_bytes / s_step / 1e9 / PEAK_HBM_GBS, 4),
                  "prefill_tokens_per_s_whole_stack": round(n_tok / s_step, 1)},
    }
    del weights, logits, ws, routing
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        rng = np.random.default_rng(40)
        samples = [(c, sorted(rng.choice(cfg.T, 16, replace=False).tolist()))
                   for c in range(cfg.chunks)]
        spent, n = oracle_chain_sample(cfg, samples, args.tile_m)
        result["cpu_baseline"] = {
            "value": round(n / spent, 2), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"sampled: 64 tokens (16 per chunk) through all {cfg.layers} layers "
                      f"(route, forward, residual glue; weight generation excluded), "
                      f"{spent:.1f} s; value = token-layers per second"}
    print(json.dumps(result), flush=True)


def main_peaks(args):
    """Achievable peaks of this device: MFMA throughput on random operands
    at 1 and 2 wavefronts per SIMD (with the shader clock from s_memtime
    against the 100 MHz s_memrealtime), the int4 -> bf16 weight rebuild rate
    on the VALU at 1, 2 and 4 wavefronts per SIMD, and HBM streaming reads of
    4 GiB with plain and LDS-DMA loads (timed with HIP events, median of 5)."""
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L

    L.load()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps=5):
        ms = []
        for _ in range(reps + 1):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ms[1:]))

    res = {"device_cus": cus, "mfma": {}, "read": {}}
    iters = 20000
    for waves in (4, 8):  # 1 and 2 wavefronts per SIMD
        sink = torch.empty(cus * waves * 64, dtype=torch.float32, device=dev)
        times = torch.zeros((cus * waves, 2), dtype=torch.int64, device=dev)
        ms = timed(lambda: L.lily_calib_mfma(cus, waves, iters, sink, times, stream))
        t = times.cpu().numpy().astype(np.float64)
        ghz = float(np.median(t[:, 0] / (t[:, 1] * 10.0)))
        flops = cus * waves * iters * 8 * 32768.0
        res["mfma"][f"{waves // 4}_wave_per_simd"] = {
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "clock_ghz": round(ghz, 3),
            "ms": round(ms, 3)}
    res["dequant"] = {}
    for waves in (4, 8, 16):  # 1, 2 and 4 wavefronts per SIMD
        sink = torch.empty(cus * waves * 64, dtype=torch.int32, device=dev)
        times = torch.zeros((cus * waves, 2), dtype=torch.int64, device=dev)
        ms = timed(lambda: L.lily_calib_dequant(cus, waves, 4000, sink, times, stream))
        t = times.cpu().numpy().astype(np.float64)
        weights = cus * waves * 64 * 4000 * 64.0
        res["dequant"][f"{waves // 4}_wave_per_simd"] = {
            "t_weights_per_s": round(weights / (ms * 1e-3) / 1e12, 2),
            "clock_ghz": round(float(np.median(t[:, 0] / (t[:, 1] * 10.0))), 3), "ms": round(ms, 3)}
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    for grid_mult in (4, 8):
        grid = cus * grid_mult
        sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
        for dma in (False, True):
            ms = timed(lambda: L.lily_calib_read(src, nbytes, grid, dma, sink, stream))
            res["read"][f"{'lds_dma' if dma else 'plain'}_wg_per_cu_{grid_mult}"] = round(
                nbytes / (ms * 1e-3) / 1e9, 1)
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    res["copy_gbs_read_plus_write"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
    del src, dst
    res["mfma_bf16_tflops"] = max(v["tflops"] for v in res["mfma"].values())
    res["hbm_read_gbs"] = max(res["read"].values())
    res["published"] = {"mfma_bf16_tflops": PEAK_MFMA_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    if args.write_peaks:
        with open(PEAKS_FILE, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
