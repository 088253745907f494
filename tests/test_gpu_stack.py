"""GPU parity for the layer-stack workloads: 40 distinct MoE layers chained by
the residual stream (r <- r + out; next input = bf16(r / rms(r))), for
T = 8192 prefill in 4 chunks of 2048 tokens, and for batch-1 decode steps.

The GPU runs every token of every chunk through all layers; the oracle runs
its own chain for a sample of tokens (each token's path through the stack is
independent of the other tokens given the router logits, so the sample is
exact). Routing is compared bit-exact for every (layer, chunk); layer outputs
of the sampled tokens are compared at every layer to the tolerance
|gpu - ref| <= 1e-2 (|ref| + RMS(ref)), with ref the oracle's fp32 sum and
RMS over the sampled rows of each chunk (decode: over the step's one row).
Layers are processed one at a time (generate,
upload, run all chunks, free), which gives the same results as chunk-major
order because the tokens are independent.
"""
import numpy as np
import pytest
import torch

import int4_grouped_gemm_amd as L
import oracle
from synth import inputs as S

import gpu_layer as G

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _flush(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def run_chain(cfg, chunks, sample, tile_m=128, n_layers=None, fused_decode=False):
    """chunks: list of chunk indices (prefill chunk or decode step); sample:
    token indices inside each chunk that the oracle follows. fused_decode:
    run each layer with lily_moe_decode instead of route + forward."""
    dev = torch.device("cuda")
    n_layers = n_layers or cfg.layers
    T = cfg.T
    d = L.dims(T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    ws = L.alloc_workspace(d, dev)
    rt = L.alloc_routing(d, dev)
    out = torch.empty((T, cfg.H), dtype=torch.int16, device=dev)
    # GPU state per chunk: residual r (fp32) and the next layer input x (bf16)
    gpu_r, gpu_x = [], []
    for c in chunks:
        x0 = S.activations(cfg, c)
        r = torch.from_numpy(G.bf16_bits_to_f64(x0).astype(np.float32)).to(dev)
        x = torch.empty((T, cfg.H), dtype=torch.int16, device=dev)
        L.lily_residual_norm(T, cfg.H, r, None, x, EPS)
        gpu_r.append(r)
        gpu_x.append(x)
    # oracle state for the sampled tokens of every chunk, stacked
    ora_r = np.concatenate([G.bf16_bits_to_f64(S.activations(cfg, c)[sample]).astype(np.float32)
                            for c in chunks])
    ora_x = oracle.residual_norm(ora_r, None, EPS)
    worst = 0.0
    for layer in range(n_layers):
        lw = S.layer_weights(cfg, layer)
        w = L.weights_from_host(lw, dev)
        ids_s, wts_s, got = [], [], []
        for ci, c in enumerate(chunks):
            lg = S.router_logits(cfg, layer, c)
            ref_r = oracle.route(lg, cfg.k, tile_m)
            if fused_decode:
                L.lily_moe_decode(d, w, torch.from_numpy(lg).to(dev), gpu_x[ci], rt, out, ws)
            else:
                L.lily_moe_route(d, torch.from_numpy(lg).to(dev), rt)
                L.lily_moe_forward(d, w, gpu_x[ci], rt, out, ws)
            L.lily_residual_norm(T, cfg.H, gpu_r[ci], out, gpu_x[ci], EPS)
            torch.cuda.synchronize()
            if fused_decode:
                assert np.array_equal(rt.topk_ids.cpu().numpy(), ref_r["topk_ids"])
                assert not np.any(rt.sched.cpu().numpy())
            else:
                G.compare_routing(G.routing_to_host(rt), ref_r, tile_m)
            ids_s.append(ref_r["topk_ids"][sample])
            wts_s.append(ref_r["topk_w"][sample])
            got.append(G.from_dev_bits(out)[sample])
        acc, out_o = oracle.forward(ora_x, np.concatenate(ids_s), np.concatenate(wts_s),
                                    oracle.getter_from_layer(lw), cfg.H, cfg.F, cfg.E)
        # the tolerance's RMS is over one layer call's output: per chunk (or
        # decode step), not pooled over several
        n_s = len(sample)
        got_all = np.concatenate(got)
        err = max(G.output_error(got_all[i * n_s:(i + 1) * n_s], acc[i * n_s:(i + 1) * n_s])
                  for i in range(len(chunks)))
        worst = max(worst, err)
        if layer % 8 == 0 or layer == n_layers - 1:
            _flush(f"  layer {layer:2d}: normalised error {err:.4f}")
        assert err <= 1.0, f"layer {layer}: normalised error {err}"
        ora_x = oracle.residual_norm(ora_r, out_o, EPS)
        del w
    return worst


def test_stack40_T8192_chunked():
    cfg = S.CONFIGS["stack40_T8192"]
    _flush(f"stack: {cfg.layers} layers, T={cfg.total_tokens} in {cfg.chunks} chunks of {cfg.T}")
    sample = [0, 1, 517, 1024, 1500, 2046, 2047, 777]
    worst = run_chain(cfg, list(range(cfg.chunks)), sample)
    _flush(f"  worst normalised error over 40 layers: {worst:.4f}")


@pytest.mark.parametrize("fused", [False, True], ids=["route_forward", "fused_decode"])
def test_decode40_steps(fused):
    cfg = S.CONFIGS["decode40"]
    steps = [0, 1, 128, 255]
    _flush(f"decode: {cfg.layers} layers, T=1, steps {steps} of {cfg.steps}, fused={fused}")
    worst = run_chain(cfg, steps, [0], fused_decode=fused)
    _flush(f"  worst normalised error over 40 layers: {worst:.4f}")


@pytest.mark.parametrize("step", [0, 255])
def test_decode_stack_one_launch(step):
    """lily_moe_decode_stack (all layers of a decode step in one launch)
    against the oracle's chain of the same layers: routing exact, every
    layer's output within the tolerance; against the per-layer launches
    (lily_moe_decode + lily_residual_norm): routing identical and outputs
    identical bit for bit, final residual included; run twice
    bit-identically; barrier counters left zero."""
    cfg = S.CONFIGS["decode40"]
    n_layers = 16
    dev = torch.device("cuda")
    _flush(f"decode stack: {n_layers} layers, T=1, step {step}")
    d = L.dims(1, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    lws = [S.layer_weights(cfg, layer) for layer in range(n_layers)]
    ws_ = [L.weights_from_host(lw, dev) for lw in lws]
    table = L.layer_table(ws_, dev)
    lg = np.stack([S.router_logits(cfg, layer, step) for layer in range(n_layers)])
    x0 = S.activations(cfg, step)
    lgd = torch.from_numpy(lg).to(dev)
    x0d = torch.from_numpy(x0.view(np.int16)).to(dev)
    ws = L.alloc_workspace(d, dev)
    sched = torch.zeros(L.LILY_SCHED_INTS, dtype=torch.int32, device=dev)

    def run():
        r = torch.full((cfg.H,), float("nan"), dtype=torch.float32, device=dev)
        outs = torch.full((n_layers, cfg.H), -1, dtype=torch.int16, device=dev)
        ids = torch.full((n_layers, cfg.k), -1, dtype=torch.int32, device=dev)
        wts = torch.zeros((n_layers, cfg.k), dtype=torch.float32, device=dev)
        L.lily_moe_decode_stack(d, n_layers, table, lgd, x0d, r, outs, ids, wts, sched, ws, EPS)
        torch.cuda.synchronize()
        return r.cpu().numpy(), outs.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy()

    r_s, outs_s, ids_s, wts_s = run()
    assert not np.any(sched.cpu().numpy()), "barrier counters and error flag must be zero"
    again = run()
    assert np.array_equal(again[1], outs_s) and np.array_equal(again[0], r_s), \
        "decode stack is not deterministic"

    # per-layer launches
    rt = L.alloc_routing(d, dev)
    r = torch.from_numpy(G.bf16_bits_to_f64(x0).astype(np.float32)).to(dev)
    x = torch.empty((1, cfg.H), dtype=torch.int16, device=dev)
    out = torch.empty((1, cfg.H), dtype=torch.int16, device=dev)
    L.lily_residual_norm(1, cfg.H, r, None, x, EPS)
    chain = []
    for layer in range(n_layers):
        L.lily_moe_decode(d, ws_[layer], lgd[layer], x, rt, out, ws)
        L.lily_residual_norm(1, cfg.H, r, out, x, EPS)
        torch.cuda.synchronize()
        assert np.array_equal(rt.topk_ids.cpu().numpy()[0], ids_s[layer]), f"layer {layer} ids"
        assert np.array_equal(rt.topk_w.cpu().numpy()[0], wts_s[layer]), f"layer {layer} weights"
        chain.append(out.cpu().numpy()[0].copy())
    same = sum(np.array_equal(c, o) for c, o in zip(chain, outs_s))
    _flush(f"  layers bit-identical to the per-layer launches: {same} of {n_layers}")
    assert same == n_layers, "the one-launch stack must equal the per-layer launches bit for bit"
    assert np.array_equal(r.cpu().numpy().reshape(-1).view(np.uint32),
                          r_s.reshape(-1).view(np.uint32)), \
        "final residual differs from the per-layer chain's"

    # the oracle's chain
    ora_r = G.bf16_bits_to_f64(x0).astype(np.float32).reshape(1, cfg.H)
    ora_x = oracle.residual_norm(ora_r, None, EPS)
    worst = 0.0
    for layer in range(n_layers):
        ref_r = oracle.route(lg[layer], cfg.k, 32)
        assert np.array_equal(ref_r["topk_ids"][0], ids_s[layer]), f"layer {layer} ids vs oracle"
        assert np.max(np.abs(ref_r["topk_w"][0] - wts_s[layer])) <= 2e-6
        acc, out_o = oracle.forward(ora_x, ref_r["topk_ids"], ref_r["topk_w"],
                                    oracle.getter_from_layer(lws[layer]), cfg.H, cfg.F, cfg.E)
        err = G.output_error(outs_s[layer][None, :].view(np.uint16), acc)
        worst = max(worst, err)
        assert err <= 1.0, f"layer {layer}: normalised error {err}"
        ora_x = oracle.residual_norm(ora_r, out_o, EPS)
    _flush(f"  worst normalised error over {n_layers} layers: {worst:.4f}")


def test_decode_stack_trace():
    """The tracing build's lily_moe_decode_stack writes the same outputs and
    final residual as the library, bit for bit, and its phase trace runs in
    order: per workgroup and layer the lead wavefront's points 0-5 do not go
    back in time, and a layer starts after the previous one's h was gathered."""
    cfg = S.CONFIGS["decode40"]
    n_layers = 8
    dev = torch.device("cuda")
    _flush(f"decode stack trace: {n_layers} layers")
    d = L.dims(1, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    ws_ = [L.weights_from_host(S.layer_weights(cfg, layer), dev) for layer in range(n_layers)]
    table = L.layer_table(ws_, dev)
    lgd = torch.from_numpy(np.stack([S.router_logits(cfg, layer, 0)
                                     for layer in range(n_layers)])).to(dev)
    x0d = torch.from_numpy(S.activations(cfg, 0).view(np.int16)).to(dev)
    ws = L.alloc_workspace(d, dev)
    sched = torch.zeros(L.LILY_SCHED_INTS, dtype=torch.int32, device=dev)

    def run():
        r = torch.full((cfg.H,), float("nan"), dtype=torch.float32, device=dev)
        outs = torch.full((n_layers, cfg.H), -1, dtype=torch.int16, device=dev)
        ids = torch.full((n_layers, cfg.k), -1, dtype=torch.int32, device=dev)
        wts = torch.zeros((n_layers, cfg.k), dtype=torch.float32, device=dev)
        L.lily_moe_decode_stack(d, n_layers, table, lgd, x0d, r, outs, ids, wts, sched, ws, EPS)
        torch.cuda.synchronize()
        return r.cpu().numpy(), outs.cpu().numpy()

    r_p, outs_p = run()
    prod = L.load()
    try:
        L.load_trace()
        r_t, outs_t = run()
        tr = L.lily_trace_decode_stack().astype(np.int64)
    finally:
        L._lib = prod
    assert np.array_equal(outs_t, outs_p), "the tracing build's layer outputs differ"
    assert np.array_equal(r_t.view(np.uint32), r_p.view(np.uint32)), "its final residual differs"
    assert not np.any(sched.cpu().numpy()), "barrier counters and error flag must be zero"
    t = tr[:, :n_layers, :6]
    assert np.all(np.diff(t, axis=2) >= 0), "a lead point precedes the one before it"
    assert np.all(t[:, 1:, 0] >= t[:, :-1, 5]), "a layer starts before the previous one ended"
