"""Timeline of the one-launch expert FFN (moe_w4_ffn) from its item trace.

Runs MoE layer steps (route, lily_moe_ffn, combine) through the tracing build
of the library (liblily_moe_trace.so, see include/lily_trace.h) on seeded
synthetic inputs, after a warm-up that brings the clocks to their steady
state, and summarises the item trace of several launches: how long the
items of each kind took, how busy the workgroups were over the launch, when
each work queue ran dry, and what ran in the launch's tail.

    python -m int4_grouped_gemm_amd.ffn_timeline [--workload prefill2048_zipf]
        [--tile-m 128] [--warmup 300] [--launches 8]

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

TICK_US = 0.01  # s_memrealtime runs at 100 MHz
QUEUES = 8      # work queues, one per XCD: workgroup w takes items from queue w % 8


def items_of(tr: np.ndarray):
    """The launch's workgroups and items from one trace [n][33][4]: (grid,
    t0, list of (wg, start, end, down, mia, n0, block, wait)), times in us
    from the launch's first item."""
    grid = int(tr[0, -1, 3])
    tr = tr[:grid].astype(np.int64)
    t0 = tr[:, 0, 0].min()
    out = []
    for w in range(grid):
        n = min(int(tr[w, -1, 2]), tr.shape[1] - 1)
        for i in range(n):
            st, en, info, wait = tr[w, i]
            out.append((w, (st - t0) * TICK_US, (en - t0) * TICK_US, int((info >> 8) & 1),
                        int(info & 0xFF), int((info >> 16) & 0xFFFF), int(info >> 32),
                        wait * TICK_US))
    return grid, out


def summarise(traces) -> str:
    lines = []
    spans, busy_frac, ends_all, tail = [], [], [], []
    dur = {}
    per_q = np.zeros((QUEUES, 2))
    for tr in traces:
        grid, its = items_of(tr)
        span = max(e for _, _, e, *_ in its)
        spans.append(span)
        busy = sum(e - s for _, s, e, *_ in its)
        busy_frac.append(busy / (span * grid))
        ends = np.zeros(grid)
        for w, s, e, down, mia, *_ in its:
            ends[w] = max(ends[w], e)
            dur.setdefault(("down" if down else "gate_up", mia), []).append(e - s)
            per_q[w % QUEUES, 0] += e - s
        ends_all.append(ends)
        for q in range(QUEUES):
            per_q[q, 1] += np.median(ends[q::QUEUES])
        tail += [(down, mia) for _, s, e, down, mia, *_ in its if e > np.percentile(ends, 10)]
    n = len(traces)
    lines.append(f"launches {n}, workgroups {len(ends_all[0])}; span (first item start to last "
                 f"item end) median {np.median(spans):.1f} us")
    lines.append(f"workgroup time busy in items: {np.mean(busy_frac):.3f} of span x workgroups")
    e = np.concatenate(ends_all)
    lines.append("workgroup last item end p10/50/90/max: " +
                 " ".join(f"{v:.1f}" for v in np.percentile(e, [10, 50, 90, 100])) + " us")
    lines.append("item durations (us), by kind and 32-row sub-tiles holding rows (mia):")
    for k in sorted(dur):
        v = np.array(dur[k])
        lines.append(f"  {k[0]:7s} mia {k[1]}: {len(v) / n:6.0f} per launch, p10/50/90 "
                     f"{np.percentile(v, 10):.1f} / {np.median(v):.1f} / {np.percentile(v, 90):.1f}")
    lines.append("per queue (workgroups w % 8): busy workgroup-us per launch, median workgroup end:")
    for q in range(QUEUES):
        lines.append(f"  queue {q}: {per_q[q, 0] / n:8.0f}  {per_q[q, 1] / n:6.1f} us")
    waits = [[wt for _, _, _, down, _, _, _, wt in items_of(tr)[1] if down] for tr in traces]
    tot = np.mean([sum(w) for w in waits])
    frac = np.mean([np.mean(np.array(w) > 1.0) for w in waits])
    lines.append(f"down items' wait for their block's gate/up tiles: {tot:.0f} workgroup-us per "
                 f"launch in all, {100 * frac:.1f}% of the down items waited more than 1 us")
    from collections import Counter
    c = Counter(tail)
    lines.append("items running after the first 10% of workgroups ran dry (per launch): " +
                 ", ".join(f"{'down' if d else 'gate_up'} mia {m}: {k / n:.0f}"
                           for (d, m), k in sorted(c.items())))
    return "\n".join(lines)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="prefill2048_zipf",
                    choices=["prefill512", "prefill2048_zipf", "prefill8192"])
    ap.add_argument("--tile-m", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--launches", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer weight sets, cycled")
    args = ap.parse_args()

    import torch

    import int4_grouped_gemm_amd as L
    from synth import inputs as S

    L.load_trace()
    dev = torch.device("cuda:0")
    cfg = S.CONFIGS[args.workload]
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, args.tile_m)
    weights = [L.weights_from_host(S.layer_weights(cfg, layer), dev) for layer in range(args.layers)]
    logits = [torch.from_numpy(S.router_logits(cfg, layer)).to(dev) for layer in range(args.layers)]
    x = torch.from_numpy(S.activations(cfg).view(np.int16)).to(dev)
    routing = L.alloc_routing(d, dev)
    ws = L.alloc_workspace(d, dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.int16, device=dev)

    def step(i):
        layer = i % args.layers
        L.lily_moe_route(d, logits[layer], routing)
        L.lily_moe_ffn(d, weights[layer], x, routing, ws)
        L.lily_moe_combine(d, routing, ws, out)

    for i in range(args.warmup):
        step(i)
    traces = []
    for i in range(args.launches):
        step(args.warmup + i)
        traces.append(L.lily_trace_ffn_items())
    if int(routing.sched[L.SCHED_GIVE_UP].item()) != 0:
        sys.exit("a bounded device-wide wait gave up: the trace is not valid")
    print(f"moe_w4_ffn<{args.tile_m}> item trace: {args.workload} (T={cfg.T}), "
          f"{args.layers} layer weight sets cycled, {args.warmup} warm-up steps")
    print(summarise(traces))


if __name__ == "__main__":
    main()
