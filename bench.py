"""Benchmark of the int4 grouped-GEMM MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch: lily_moe_route
(top-k, softmax, histogram, scan, scatter, block map) then the three stages
of lily_moe_forward (gate/up + SwiGLU, down, combine) for one MoE layer of
T = 2048 tokens (H 2048, F 512, 256 experts top-8 + 1 shared, int4 g64,
router logits N(0,1) plus a Zipf(1.1) log-bias per expert). Steps cycle
through several distinct layer weight sets (8 by default, 3.6 GB) so that
the weights stream from HBM instead of the on-package cache. Inputs are
resident in HBM before timing starts.

Prints ONE JSON line. ``value`` is MoE-layer tokens/s = T / (seconds per
step), timed with the wall clock between two device synchronisations.
``roofline`` reports the dominant kernel: its algorithmic flops (or bytes)
per launch over its average duration from HIP events recorded on the launch
stream around every launch in the timed region. ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload.
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
KERNEL_SOURCES = [os.path.join(ROOT, "int4_grouped_gemm_amd", "csrc", f)
                  for f in ("gemm_w4.hip", "route.hip", "common.hpp", "topk.hpp", "w4.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "prefill512", "prefill8192", "decode40", "stack40"],
                    help="prefill2048_zipf (the headline), decode40 (T=1, 40-layer steps) or "
                         "stack40 (40 distinct layers, T=8192 in chunks of 2048, residual glue)")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer weight sets cycled")
    ap.add_argument("--tile-m", type=int, default=128)
    ap.add_argument("--decode-path", default="fused", choices=["fused", "layer", "stack"],
                    help="decode40: lily_moe_decode (one launch per layer), route + forward, or "
                         "lily_moe_decode_stack (the 40 layers and their residual glue in one "
                         "launch)")
    ap.add_argument("--router", action="store_true",
                    help="start each step from x: the router projection x.Wr^T (lily_moe_router) "
                         "computes the logits inside the timed step")
    ap.add_argument("--route-host", action="store_true",
                    help="ablation: route with lily_moe_route_host (histogram, scan, scatter and "
                         "block map on the host after a stream synchronisation)")
    ap.add_argument("--unfused", action="store_true",
                    help="ablation: lily_moe_dequant (bf16 weights of the used experts to HBM) "
                         "then lily_moe_forward_bf16 (the same GEMMs on bf16 tiles); tile_m 32 "
                         "or 64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of layer 0 the CPU oracle computes for the baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 256 MiB device copy (twice) so that "
                         "profiler byte counters can be scaled against a known size")
    return ap.parse_args()


def stage_work(cfg, P):
    """Algorithmic work per launch of each stage (flops for GEMMs, bytes
    for the memory-bound stages)."""
    rows = P + cfg.T
    return {
        "router": ("mfma", 2.0 * cfg.T * cfg.H * cfg.E),
        "route": ("hbm", cfg.T * cfg.E * 4 + P * 4 * 4 + cfg.T * cfg.k * 4),
        "gate_up": ("mfma", 2.0 * rows * cfg.H * 2 * cfg.F),
        "down": ("mfma", 2.0 * rows * cfg.F * cfg.H),
        "combine": ("hbm", rows * cfg.H * 4 + cfg.T * cfg.H * 2 + P * 8),
        # unfused twin: the packed weights of every expert read (upper bound:
        # only used ones are) and their bf16 written; then both GEMMs
        "dequant": ("hbm", (cfg.E + 1) * 3 * cfg.H * cfg.F * (0.5625 + 2.0)),
        "forward_bf16": ("mfma", 2.0 * rows * cfg.H * 3 * cfg.F),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the layer is a single-GPU kernel path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "decode40":
        return main_decode(args)
    if args.workload == "stack40":
        return main_stack(args)

    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[args.workload]
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, args.tile_m)
    P = cfg.T * cfg.k

    # ---- inputs, resident in HBM before timing
    t_gen = time.time()
    weights, logits, routers = [], [], []
    for layer in range(args.layers):
        weights.append(L.weights_from_host(S.layer_weights(cfg, layer), dev))
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
        ("route", "gate_up", "down", "combine"))

    def step(i, ev=None):
        layer = i % args.layers
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
        else:
            calls += [lambda: L.lily_moe_gate_up(d, w, x, routing, ws, stream),
                      lambda: L.lily_moe_down(d, w, routing, ws, stream),
                      lambda: L.lily_moe_combine(d, routing, ws, out, stream)]
        for j, call in enumerate(calls):
            if ev is not None:
                ev[j].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

    for i in range(args.warmup):
        step(i)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = cfg.T / ((t1 - t0) / args.steps)
    stage_ms = {s: float(np.mean([ev[j].elapsed_time(ev[j + 1]) for ev in events]))
                for j, s in enumerate(stages)}

    work = stage_work(cfg, P)
    dom = max(stages, key=lambda s: stage_ms[s])
    bound, amount = work[dom]
    if bound == "mfma":
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e12
        peak, unit = PEAK_MFMA_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.loads([ln for ln in open(TRAFFIC_FILE) if ln.startswith("{")][0])
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("stage") == dom \
                and tr.get("tile_m") == args.tile_m and tr.get("workload") == args.workload \
                and not args.router:
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom}

    # whole-layer fractions: useful flops and the weight bytes one layer must read
    counts = routing.counts.cpu().numpy()
    used = int((counts > 0).sum()) + 1
    w_bytes = used * 3 * cfg.H * cfg.F * (0.5 + 4.0 / 64)
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
            "layer_weight_sets": args.layers,
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

    if not args.no_cpu_baseline:
        import oracle
        from oracle import build as _ob  # noqa: F401  (oracle is built by __graft_entry__.build)
        lw = S.layer_weights(cfg, 0)
        lg = S.router_logits(cfg, 0)
        xs = S.activations(cfg)
        ntok = min(args.cpu_tokens, cfg.T)
        c0 = time.perf_counter()
        rr = oracle.route(lg, cfg.k, args.tile_m)
        oracle.forward(xs, rr["topk_ids"], rr["topk_w"], oracle.getter_from_layer(lw),
                       cfg.H, cfg.F, cfg.E, tokens=list(range(ntok)))
        c1 = time.perf_counter()
        result["cpu_baseline"] = {
            "value": round(ntok / (c1 - c0), 2), "unit": "tokens/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"route of all {cfg.T} tokens + forward of {ntok} tokens of layer 0 "
                      f"(dequant of the experts they use included), {c1 - c0:.1f} s",
        }
    print(json.dumps(result), flush=True)


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
    weights = []
    for layer in range(cfg.layers):
        weights.append(L.weights_from_host(S.layer_weights(cfg, layer), dev))
        if layer % 10 == 9:
            print(f"# {layer + 1} layers uploaded", file=sys.stderr, flush=True)
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
    s_step = (t1 - t0) / args.steps
    n_tok = cfg.T * cfg.chunks
    layer_flops = 2.0 * 3 * cfg.H * cfg.F * (cfg.k + 1) * n_tok * cfg.layers
    # every chunk-layer touches (nearly) all experts: their weights are read once per chunk
    w_bytes = (cfg.E + 1) * 3 * cfg.H * cfg.F * (0.5 + 4.0 / 64) * cfg.chunks * cfg.layers
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
                   "weights_resident_gb": round(cfg.layers * (cfg.E + 1) * 3 * cfg.H * cfg.F *
                                                (0.5 + 4.0 / 64) / 1e9, 2)},
        "layer": {"mfma_frac": round(layer_flops / s_step / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                  "hbm_weight_frac": round(w_bytes / s_step / 1e9 / PEAK_HBM_GBS, 4),
                  "prefill_tokens_per_s_whole_stack": round(n_tok / s_step, 1)},
    }
    print(json.dumps(result), flush=True)


def main_decode(args):
    """Batch-1 decode: one step = 40 MoE layers at T = 1 (route + forward per
    layer). The 40 layers cycle through --layers distinct weight sets (8 by
    default, 3.6 GB), so every layer's weights stream from HBM. Each step and
    layer has its own router logits; all inputs are resident before timing."""
    import numpy as np
    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS["decode40"]
    n_layers = cfg.layers
    d = L.dims(1, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    weights = [L.weights_from_host(S.layer_weights(cfg, layer), dev) for layer in range(args.layers)]
    n_steps = args.warmup + args.steps
    logits = torch.from_numpy(np.stack([np.stack([S.router_logits(cfg, layer, step % cfg.steps)
                                                  for layer in range(n_layers)])
                                        for step in range(n_steps)])).to(dev)
    xs = torch.from_numpy(np.stack([S.activations(cfg, step % cfg.steps).view(np.int16)
                                    for step in range(n_steps)])).to(dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((1, cfg.H), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()

    if args.decode_path == "stack":
        table = L.layer_table([weights[layer % args.layers] for layer in range(n_layers)], dev)
        r_st = torch.empty(cfg.H, dtype=torch.float32, device=dev)
        outs_st = torch.empty((n_layers, cfg.H), dtype=torch.int16, device=dev)
        ids_st = torch.empty((n_layers, cfg.k), dtype=torch.int32, device=dev)
        w_st = torch.empty((n_layers, cfg.k), dtype=torch.float32, device=dev)

    def step(i):
        if args.decode_path == "stack":
            L.lily_moe_decode_stack(d, n_layers, table, logits[i], xs[i], r_st, outs_st, ids_st,
                                    w_st, routing.sched, ws, 1e-6, stream)
            return
        for layer in range(n_layers):
            w = weights[layer % args.layers]
            if args.decode_path == "fused":
                L.lily_moe_decode(d, w, logits[i, layer], xs[i], routing, out, ws, stream)
            else:
                L.lily_moe_route(d, logits[i, layer], routing, stream)
                L.lily_moe_forward(d, w, xs[i], routing, out, ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    us_per_layer = ms_per_step * 1e3 / n_layers
    # weight bytes a layer must read: the k routed experts and the shared one
    layer_bytes = (cfg.k + 1) * 3 * cfg.H * cfg.F * (0.5 + 4.0 / 64)
    gbs = layer_bytes / (us_per_layer * 1e-6) / 1e9
    result = {
        "metric": "MoE-layer decode time per layer (T=1, 40-layer step, int4 g64); % of HBM peak",
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode40", "T": 1, "H": cfg.H, "F": cfg.F, "E": cfg.E,
                   "topk": cfg.k, "layers_per_step": n_layers, "layer_weight_sets": args.layers,
                   "path": {"fused": "lily_moe_decode, one launch per layer",
                            "layer": "lily_moe_route + lily_moe_forward (tile_m 32)",
                            "stack": "lily_moe_decode_stack: 40 layers and the residual glue "
                                     "in one launch"}[args.decode_path]},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "whole layer"},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
