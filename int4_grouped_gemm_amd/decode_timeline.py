"""Phase timeline of the whole-step decode kernel from its trace.

Runs batch-1 decode steps through 40 distinct resident layers in one
lily_moe_decode_stack launch each, through the tracing build of the library
(liblily_moe_trace.so, see include/lily_trace.h), on seeded synthetic inputs,
and summarises the phase trace of several launches: the layer period and
where inside a layer the time goes, per workgroup and over the slowest one.

    python -m int4_grouped_gemm_amd.decode_timeline [--launches 8] [--warmup 20]

Times are in microseconds of the 100 MHz wall clock the kernel reads.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICK_US = 0.01
POINTS = ("layer start", "previous output gathered, r updated", "x staged (norm done)",
          "phase A part sums ready", "h words stored", "h gathered (all compute waves)")


def summarise(traces, n_layers: int) -> str:
    lo, hi = 5, n_layers - 4  # layers away from the launch's ramp-up and drain
    t = np.stack([tr[:, :n_layers, :6].astype(np.int64) for tr in traces]) * TICK_US
    start = t[..., 0].max(axis=1)                       # [launch, layer]: the latest start
    lines = [f"launches {len(traces)}, workgroups {t.shape[1]}, layers {n_layers} "
             f"(statistics over layers {lo}..{hi - 1})"]
    period = np.diff(start[:, lo:hi + 1], axis=1)
    lines.append(f"layer period (latest start to latest start): median {np.median(period):.2f} us")
    lines.append("each point relative to the latest start of its layer: median over "
                 "workgroups / latest workgroup (us)")
    for i, name in enumerate(POINTS):
        rel = t[:, :, lo:hi, i] - start[:, None, lo:hi]
        lines.append(f"  {i} {name:38s} {np.median(rel):6.2f} / {np.median(rel.max(axis=1)):6.2f}")
    lines.append("phases (median over workgroups and layers, us):")
    names = ("gather previous output + r", "norm + x staging", "phase A (after x staged)",
             "h assembly + stores", "h exchange (gather by the compute waves)")
    for i, name in enumerate(names):
        d = t[:, :, lo:hi, i + 1] - t[:, :, lo:hi, i]
        lines.append(f"  {name:42s} {np.median(d):6.2f} (p90 {np.percentile(d, 90):.2f})")
    d = t[:, :, lo + 1:hi + 1, 0] - t[:, :, lo:hi, 5]
    lines.append(f"  {'phase B + output exchange to next start':42s} {np.median(d):6.2f} "
                 f"(p90 {np.percentile(d, 90):.2f})")
    return "\n".join(lines)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--launches", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=20)
    args = ap.parse_args()

    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load_trace()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS["decode40"]
    n_layers = cfg.layers
    d = L.dims(1, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    weights = [L.weights_from_host(S.layer_weights(cfg, layer), dev) for layer in range(n_layers)]
    table = L.layer_table(weights, dev)
    steps = args.warmup + args.launches
    logits = torch.from_numpy(np.stack([np.stack([S.router_logits(cfg, layer, s % cfg.steps)
                                                  for layer in range(n_layers)])
                                        for s in range(steps)])).to(dev)
    xs = torch.from_numpy(np.stack([S.activations(cfg, s % cfg.steps).view(np.int16)
                                    for s in range(steps)])).to(dev)
    ws = L.alloc_workspace(d, dev)
    sched = torch.zeros(L.LILY_SCHED_INTS, dtype=torch.int32, device=dev)
    r = torch.empty(cfg.H, dtype=torch.float32, device=dev)
    outs = torch.empty((n_layers, cfg.H), dtype=torch.int16, device=dev)
    ids = torch.empty((n_layers, cfg.k), dtype=torch.int32, device=dev)
    wts = torch.empty((n_layers, cfg.k), dtype=torch.float32, device=dev)
    traces = []
    for s in range(steps):
        L.lily_moe_decode_stack(d, n_layers, table, logits[s], xs[s], r, outs, ids, wts, sched, ws)
        if s >= args.warmup:
            traces.append(L.lily_trace_decode_stack())
    if int(sched[L.SCHED_GIVE_UP].item()) != 0:
        sys.exit("a bounded device-wide wait gave up: the trace is not valid")
    print(f"moe_decode_stack_kernel phase trace: decode40 (T=1, {n_layers} distinct layers), "
          f"{args.warmup} warm-up launches")
    print(summarise(traces, n_layers))


if __name__ == "__main__":
    main()
