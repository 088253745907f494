"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing must be bit-exact (ids, histogram, scan, scatter, block map; the
softmax weights within 2e-6). Layer outputs must satisfy
|gpu - ref| <= 1e-2 * (|ref| + RMS(ref)) per element, where ref is the
oracle's fp32 sum before the final bf16 rounding.
"""
import numpy as np
import pytest
import torch

import int4_grouped_gemm_amd as L
import oracle
from synth import inputs as S

import gpu_layer as G

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


# ------------------------------------------------------------------- routing

ROUTE_CASES = [
    # (name, T, E, k, tile_m, source)
    ("tiny", 32, 16, 2, 8, "tiny"),
    ("prefill512", 512, 256, 8, 64, "prefill512"),
    ("zipf2048_m32", 2048, 256, 8, 32, "prefill2048_zipf"),
    ("zipf2048_m64", 2048, 256, 8, 64, "prefill2048_zipf"),
    ("zipf2048_m128", 2048, 256, 8, 128, "prefill2048_zipf"),
    ("decode_T1", 1, 256, 8, 64, "decode40"),
    ("fused_edge_T64", 64, 256, 8, 64, "prefill512"),
    ("split_edge_T65", 65, 256, 8, 64, "prefill512"),
    ("m1", 100, 256, 8, 1, "prefill512"),
    ("k_equals_E", 40, 16, 16, 4, "tiny"),
    ("E1_k1", 70, 1, 1, 16, None),
    ("E512_k64", 300, 512, 64, 64, None),
    ("odd_T", 777, 256, 8, 128, "prefill2048_zipf"),
    # route_finish runs one workgroup per part of >= 128 tokens (at most 64 parts)
    ("parts_T129_last_1", 129, 256, 8, 64, "prefill512"),
    ("parts_T8192_64", 8192, 256, 8, 128, "prefill8192"),
    ("parts_T8193_size129", 8193, 256, 8, 128, None),
    ("parts_E512_k64", 1000, 512, 64, 64, None),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: c[0])
def test_route_bit_exact(case):
    name, T, E, k, M, src = case
    _flush(f"route case {name}: T={T} E={E} k={k} M={M}")
    if src is None:
        lg = np.random.default_rng([T, E, k]).standard_normal((T, E)).astype(np.float32)
    else:
        cfg = S.CONFIGS[src]
        lg = S.router_logits(cfg, T=T) if cfg.E == E else None
        assert lg is not None
    d = L.dims(T, 256, 128, E, k, M)
    ref = oracle.route(lg, k, M)
    gpu = G.routing_to_host(G.route_gpu(d, lg))
    G.compare_routing(gpu, ref, M)


def test_route_ties_and_signed_zero():
    T, E, k = 96, 64, 4
    lg = np.zeros((T, E), np.float32)
    lg[::2] = -0.0
    lg[1::3, 5] = 1.0
    lg[2::5, 60] = 1.0
    lg[::7] = np.round(np.random.default_rng(1).standard_normal((len(lg[::7]), E)))
    d = L.dims(T, 256, 128, E, k, 16)
    G.compare_routing(G.routing_to_host(G.route_gpu(d, lg)), oracle.route(lg, k, 16), 16)


def test_route_deterministic():
    cfg = S.CONFIGS["prefill2048_zipf"]
    lg = S.router_logits(cfg)
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, 64)
    a = G.routing_to_host(G.route_gpu(d, lg))
    b = G.routing_to_host(G.route_gpu(d, lg))
    for key in L.ROUTING_FIELDS:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("case", [c for c in ROUTE_CASES if c[0] in
                                  ("tiny", "prefill512", "zipf2048_m128", "decode_T1", "m1",
                                   "E512_k64", "odd_T")], ids=lambda c: c[0])
def test_route_host_twin(case):
    """lily_moe_route_host (the CPU-synchronised twin) writes the oracle's
    routing bit for bit, the same as lily_moe_route, and the forward after
    it gives the forward after the GPU route bit for bit."""
    name, T, E, k, M, src = case
    _flush(f"route_host case {name}: T={T} E={E} k={k} M={M}")
    if src is None:
        lg = np.random.default_rng([T, E, k]).standard_normal((T, E)).astype(np.float32)
    else:
        lg = S.router_logits(S.CONFIGS[src], T=T)
    d = L.dims(T, 256, 128, E, k, M)
    r = L.alloc_routing(d)
    r.sched.fill_(7)  # the twin must clear the GEMM counters itself,
    r.sched[L.SCHED_GIVE_UP] = 0  # but no call clears the give-up flag
    L.lily_moe_route_host(d, torch.from_numpy(lg).cuda(), r)
    torch.cuda.synchronize()
    G.compare_routing(G.routing_to_host(r), oracle.route(lg, k, M), M)
    gpu = G.routing_to_host(G.route_gpu(d, lg))
    host = G.routing_to_host(r)
    for key in L.ROUTING_FIELDS:
        assert np.array_equal(gpu[key], host[key]), key


@pytest.mark.parametrize("host", [False, True], ids=["gpu_route", "host_route"])
def test_give_up_flag_sticky(host):
    """sched[30], the give-up flag of the bounded device-wide waits, survives
    both routes (which clear every counter around it) and the GEMMs: only the
    caller clears it, so a give-up in any step of a run stays visible."""
    _flush(f"give-up flag sticky, host route {host}")
    d = L.dims(64, 256, 128, 16, 2, 32)
    lg = np.random.default_rng(5).standard_normal((64, 16)).astype(np.float32)
    r = L.alloc_routing(d)
    r.sched[L.SCHED_GIVE_UP] = 1
    (L.lily_moe_route_host if host else L.lily_moe_route)(d, torch.from_numpy(lg).cuda(), r)
    torch.cuda.synchronize()
    sched = r.sched.cpu().numpy()
    assert sched[L.SCHED_GIVE_UP] == 1, "a route cleared the give-up flag"
    assert not np.any(np.delete(sched, L.SCHED_GIVE_UP)), "counters left non-zero"


def test_route_host_twin_forward():
    cfg = S.CONFIGS["prefill512"]
    lw = S.layer_weights(cfg, 0)
    x = S.activations(cfg, 0)
    lg = S.router_logits(cfg, 0, 0)
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, 64)
    w = L.weights_from_host(lw)
    xd = G.to_dev_bits(x)
    a = G.from_dev_bits(G.forward_gpu(d, w, xd, G.route_gpu(d, lg)))
    r = L.alloc_routing(d)
    L.lily_moe_route_host(d, torch.from_numpy(lg).cuda(), r)
    b = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
    assert np.array_equal(a, b), "forward after the host route differs"


@pytest.mark.parametrize("name,tile_m", [("tiny", 32), ("tiny", 64), ("prefill512", 64),
                                         ("prefill2048_zipf", 64), ("prefill2048_zipf", 32)])
def test_unfused_twin(name, tile_m):
    """lily_moe_dequant + lily_moe_forward_bf16 (the unfused twin): the bf16
    weights it writes equal the oracle's dequantisation bit for bit; experts
    without rows are left untouched; and its output is bit-identical to the
    fused lily_moe_forward (same weights, same products in the same order)."""
    cfg = S.CONFIGS[name]
    _flush(f"unfused twin {name} tile_m={tile_m}")
    lw = S.layer_weights(cfg, 0)
    x = S.activations(cfg, 0)
    lg = S.router_logits(cfg, 0, 0)
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    w = L.weights_from_host(lw)
    xd = G.to_dev_bits(x)
    r = G.route_gpu(d, lg)
    fused = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
    bw = L.alloc_bf16_weights(d)
    for name_ in L.WEIGHT_FIELDS:
        getattr(bw, name_).fill_(0x7FC1)  # a NaN pattern: untouched entries stay so
    L.lily_moe_dequant(d, w, r, bw)
    torch.cuda.synchronize()
    counts = r.counts.cpu().numpy()
    used = np.flatnonzero(counts)
    unused = np.flatnonzero(counts == 0)
    for t, (routed, shared) in enumerate([(bw.gate, bw.sh_gate), (bw.up, bw.sh_up),
                                          (bw.down, bw.sh_down)]):
        get = oracle.getter_from_layer(lw)
        for e in ([int(used[0]), int(used[-1])] if len(used) else []):
            want = oracle.dequant(*get(t, e))
            assert np.array_equal(routed[e].cpu().numpy().view(np.uint16), want), (t, e)
        want = oracle.dequant(*get(t, cfg.E))
        assert np.array_equal(shared[0].cpu().numpy().view(np.uint16), want), (t, "shared")
        if len(unused):
            assert np.all(routed[int(unused[0])].cpu().numpy() == 0x7FC1), (t, "unused touched")
    ws = L.alloc_workspace(d)
    ws.fill_(0xFF)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device="cuda")
    L.lily_moe_forward_bf16(d, bw, xd, r, out, ws)
    torch.cuda.synchronize()
    got = G.from_dev_bits(out)
    assert np.array_equal(got, fused), "unfused twin differs from the fused forward"
    assert not np.any(r.sched.cpu().numpy()), "GEMMs must leave their queue counters zero"


# ------------------------------------------------------------------- forward

def _layer_case(cfg, tile_m, tokens=None, layer=0, seed=0):
    lw = S.layer_weights(cfg, layer, seed)
    x = S.activations(cfg, 0, seed)
    lg = S.router_logits(cfg, layer, 0, seed)
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    w = L.weights_from_host(lw)
    xd = G.to_dev_bits(x)
    r = G.route_gpu(d, lg)
    ref_r = oracle.route(lg, cfg.k, tile_m)
    G.compare_routing(G.routing_to_host(r), ref_r, tile_m)
    out = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
    assert not np.any(r.sched.cpu().numpy()), "GEMMs must leave their queue counters zero"
    acc, _ = oracle.forward(x, ref_r["topk_ids"], ref_r["topk_w"], oracle.getter_from_layer(lw),
                            cfg.H, cfg.F, cfg.E, tokens=tokens)
    got = out if tokens is None else out[np.asarray(tokens)]
    return got, acc, (d, w, xd, r)


@pytest.mark.parametrize("tile_m", [16, 32, 64, 128])
def test_forward_tiny(tile_m):
    _flush(f"forward tiny tile_m={tile_m}")
    got, acc, _ = _layer_case(S.CONFIGS["tiny"], tile_m)
    err = G.output_error(got, acc)
    assert err <= 1.0, f"normalised error {err}"


@pytest.mark.parametrize("tile_m", [16, 32, 64, 128])
def test_forward_prefill512(tile_m):
    _flush(f"forward prefill512 tile_m={tile_m}")
    got, acc, _ = _layer_case(S.CONFIGS["prefill512"], tile_m)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"


@pytest.mark.parametrize("tile_m", [16, 64, 128])
def test_forward_zipf2048_all_tokens(tile_m):
    _flush(f"forward prefill2048_zipf, all tokens, tile_m={tile_m}")
    got, acc, (d, w, xd, r) = _layer_case(S.CONFIGS["prefill2048_zipf"], tile_m)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"
    # run-to-run determinism with a poisoned workspace
    again = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
    assert np.array_equal(again, got), "forward is not deterministic"


@pytest.mark.parametrize("layer", range(1, 8))
def test_forward_zipf2048_layer_sets(layer):
    """The other seven Zipf layer weight sets that bench.py cycles, at its
    tile height (128): routing bit-exact, and sampled tokens (part edges and
    the ends included) within the tolerance."""
    cfg = S.CONFIGS["prefill2048_zipf"]
    rng = np.random.default_rng(2048 + layer)
    tokens = sorted(set([0, 127, 128, 1023, 1024, 2047] + rng.choice(cfg.T, 122, replace=False).tolist()))
    _flush(f"forward prefill2048_zipf layer set {layer}, {len(tokens)} sampled tokens")
    got, acc, _ = _layer_case(cfg, 128, tokens=tokens, layer=layer)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"


def test_forward_prefill8192_sampled():
    """One T = 8192 layer call (64 route parts): routing bit-exact, and the
    outputs of sampled tokens (part edges included) within the tolerance."""
    cfg = S.CONFIGS["prefill8192"]
    rng = np.random.default_rng(8192)
    tokens = sorted(set([0, 1, 127, 128, 129, 4095, 4096, 8190, 8191] +
                        rng.choice(cfg.T, 55, replace=False).tolist()))
    _flush(f"forward prefill8192, {len(tokens)} sampled tokens")
    got, acc, _ = _layer_case(cfg, 128, tokens=tokens)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"


# ------------------------------------------------------------------- packing

def _pack_reference(q: np.ndarray, scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """The packed layout as the header states it, built with numpy."""
    n, N, K2 = q.shape
    G_ = K2 // 32
    qb = q.reshape(n, N // 128, 128, G_, 2, 16).transpose(0, 1, 3, 4, 2, 5)  # e s g h r byte
    qb = qb.reshape(n, N // 128, G_, 4096)
    sb = scale.view(np.uint8).reshape(n, N // 128, 128, G_, 2).transpose(0, 1, 3, 2, 4)
    bb = bias.view(np.uint8).reshape(n, N // 128, 128, G_, 2).transpose(0, 1, 3, 2, 4)
    blk = np.concatenate([qb, sb.reshape(n, N // 128, G_, 256), bb.reshape(n, N // 128, G_, 256)],
                         axis=-1)
    return np.ascontiguousarray(blk).reshape(-1)


@pytest.mark.parametrize("shape", [(1, 128, 64), (3, 256, 192), (2, 384, 512)])
def test_pack_layout(shape):
    n, N, K = shape
    rng = np.random.default_rng(list(shape))
    q = rng.integers(0, 256, (n, N, K // 2), dtype=np.uint8)
    sc = rng.integers(0, 65536, (n, N, K // 64), dtype=np.uint16)
    bi = rng.integers(0, 65536, (n, N, K // 64), dtype=np.uint16)
    plain = L.W4(torch.from_numpy(q).cuda(), torch.from_numpy(sc.view(np.int16)).cuda(),
                 torch.from_numpy(bi.view(np.int16)).cuda())
    packed = L.pack_w4(plain, n, N, K)
    torch.cuda.synchronize()
    assert packed.numel() == n * N * K * 9 // 16
    assert np.array_equal(packed.cpu().numpy(), _pack_reference(q, sc, bi))


def test_gemm_queue_counters_reset():
    """Two gate/up launches on one routing with no route call between them:
    each launch leaves its counters zero, so the second computes the same h."""
    cfg = S.CONFIGS["prefill512"]
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, 128)
    w = L.weights_from_host(S.layer_weights(cfg, 0))
    xd = G.to_dev_bits(S.activations(cfg))
    r = G.route_gpu(d, S.router_logits(cfg))
    ws = L.alloc_workspace(d)
    h, y = L.workspace_views(d, ws)
    L.lily_moe_gate_up(d, w, xd, r, ws)
    torch.cuda.synchronize()
    first = h.clone()
    assert not np.any(r.sched.cpu().numpy())
    h.fill_(0)
    L.lily_moe_gate_up(d, w, xd, r, ws)
    L.lily_moe_down(d, w, r, ws)
    L.lily_moe_down(d, w, r, ws)
    torch.cuda.synchronize()
    assert torch.equal(first, h)
    assert not np.any(r.sched.cpu().numpy())


@pytest.mark.parametrize("name,tile_m", [("prefill2048_zipf", 128), ("prefill512", 128),
                                         ("prefill512", 64), ("prefill2048_zipf", 32), ("tiny", 32)])
def test_ffn_one_launch(name, tile_m):
    """lily_moe_ffn (gate/up and down in one launch where neither splits K,
    a down tile waiting for its block's gate/up tiles) writes the same h and y
    bit for bit as lily_moe_gate_up then lily_moe_down, three times in a row
    on one routing (its queue counters and block tallies are left zero, and
    no wait gave up)."""
    cfg = S.CONFIGS[name]
    _flush(f"one-launch ffn {name} tile_m={tile_m}")
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    w = L.weights_from_host(S.layer_weights(cfg, 0))
    xd = G.to_dev_bits(S.activations(cfg))
    r = G.route_gpu(d, S.router_logits(cfg))
    ws = L.alloc_workspace(d)
    h, y = L.workspace_views(d, ws)
    L.lily_moe_gate_up(d, w, xd, r, ws)
    L.lily_moe_down(d, w, r, ws)
    torch.cuda.synchronize()
    want_h, want_y = h.clone(), y.clone()
    for _ in range(3):
        h.fill_(0)
        y.fill_(0)
        L.lily_moe_ffn(d, w, xd, r, ws)
        torch.cuda.synchronize()
        assert torch.equal(h, want_h), "h differs from the two launches"
        assert torch.equal(y, want_y), "y differs from the two launches"
        assert not np.any(r.sched.cpu().numpy()), "counters, tallies and the give-up flag stay zero"


@pytest.mark.parametrize("name,tile_m", [("prefill512", 128), ("tiny", 32)])
def test_ffn_item_trace(name, tile_m):
    """The tracing build (liblily_moe_trace.so) writes the same h and y as
    the library, bit for bit, and its item trace accounts for every work
    item of the launch exactly once: each block's gate/up and down n-tiles,
    with start <= end and waits on down items only."""
    cfg = S.CONFIGS[name]
    _flush(f"ffn item trace {name} tile_m={tile_m}")
    d = L.dims(cfg.T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    w = L.weights_from_host(S.layer_weights(cfg, 0))
    xd = G.to_dev_bits(S.activations(cfg))
    r = G.route_gpu(d, S.router_logits(cfg))
    ws = L.alloc_workspace(d)
    h, y = L.workspace_views(d, ws)
    L.lily_moe_ffn(d, w, xd, r, ws)
    torch.cuda.synchronize()
    want_h, want_y = h.clone(), y.clone()
    h.fill_(0)
    y.fill_(0)
    prod = L.load()
    try:
        L.load_trace()
        L.lily_moe_ffn(d, w, xd, r, ws)
        tr = L.lily_trace_ffn_items()
    finally:
        L._lib = prod
    assert torch.equal(h, want_h) and torch.equal(y, want_y), "the tracing build's h or y differs"
    assert not np.any(r.sched.cpu().numpy()), "counters, tallies and the give-up flag stay zero"
    grid = int(tr[0, -1, 3])
    assert 1 <= grid <= tr.shape[0]
    n_blocks = int(r.num_blocks.cpu()[0]) + (cfg.T + tile_m - 1) // tile_m
    nt_gu, nt_dn = cfg.F // 128, cfg.H // 256
    seen = []
    for wg in range(grid):
        n = int(tr[wg, -1, 2])
        assert n <= L.TRACE_SLOTS, "more items than the trace records"
        assert tr[wg, -1, 0] <= tr[wg, -1, 1]
        for st, en, info, wait in tr[wg, :n].astype(np.int64):
            down = int((info >> 8) & 1)
            assert st <= en and (down or wait == 0)
            seen.append((down, int(info >> 32), int((info >> 16) & 0xFFFF)))
    want = sorted([(0, b, 128 * t) for b in range(n_blocks) for t in range(nt_gu)] +
                  [(1, b, 256 * t) for b in range(n_blocks) for t in range(nt_dn)])
    assert sorted(seen) == want, "the trace does not hold every item exactly once"


# ------------------------------------------------------------------- split K

@pytest.mark.parametrize("T,tile_m", [(1, 32), (1, 128), (4, 32), (8, 64), (3, 128)])
def test_forward_small_T_split_k(T, tile_m):
    """Few tokens: the GEMMs spread each tile's K over several workgroups and
    the last to finish adds the fp32 partials in chunk order. All tokens
    against the oracle, twice (deterministic), then twice more on the same
    routing (the tile counters are left zero)."""
    cfg = S.CONFIGS["prefill512"]
    _flush(f"small T: T={T} tile_m={tile_m}")
    lw = S.layer_weights(cfg, 0)
    x = S.activations(cfg, 0, T=T)
    lg = S.router_logits(cfg, 0, 0, T=T)
    d = L.dims(T, cfg.H, cfg.F, cfg.E, cfg.k, tile_m)
    w = L.weights_from_host(lw)
    r = G.route_gpu(d, lg)
    ref_r = oracle.route(lg, cfg.k, tile_m)
    G.compare_routing(G.routing_to_host(r), ref_r, tile_m)
    xd = G.to_dev_bits(x)
    got = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
    acc, _ = oracle.forward(x, ref_r["topk_ids"], ref_r["topk_w"], oracle.getter_from_layer(lw),
                            cfg.H, cfg.F, cfg.E)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"
    for _ in range(2):
        again = G.from_dev_bits(G.forward_gpu(d, w, xd, r))
        assert np.array_equal(again, got), "split-K forward is not deterministic"
    assert not np.any(r.sched.cpu().numpy()), "tile counters must be left zero"


# ------------------------------------------------------------------- fused decode

@pytest.mark.parametrize("name,T", [("decode40", 1), ("prefill512", 2), ("prefill512", 4),
                                    ("prefill2048_zipf", 3)])
def test_decode_fused(name, T):
    """lily_moe_decode (route and forward in one launch) against
    the oracle: top-k ids exact, weights within 2e-6, outputs within the
    tolerance; run twice bit-identically; barrier counters left zero."""
    cfg = S.CONFIGS[name]
    _flush(f"fused decode {name} T={T}")
    lw = S.layer_weights(cfg, 0)
    x = S.activations(cfg, 0, T=T)
    lg = S.router_logits(cfg, 0, 0, T=T)
    d = L.dims(T, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    w = L.weights_from_host(lw)
    r = L.alloc_routing(d)
    ws = L.alloc_workspace(d)
    ws.fill_(0xFF)
    lgd = torch.from_numpy(lg).cuda()
    xd = G.to_dev_bits(x)
    out = torch.full((T, cfg.H), -1, dtype=torch.int16, device="cuda")
    L.lily_moe_decode(d, w, lgd, xd, r, out, ws)
    torch.cuda.synchronize()
    ref_r = oracle.route(lg, cfg.k, 32)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref_r["topk_ids"])
    assert np.max(np.abs(r.topk_w.cpu().numpy() - ref_r["topk_w"])) <= 2e-6
    got = G.from_dev_bits(out)
    acc, _ = oracle.forward(x, ref_r["topk_ids"], ref_r["topk_w"], oracle.getter_from_layer(lw),
                            cfg.H, cfg.F, cfg.E)
    err = G.output_error(got, acc)
    _flush(f"  normalised error {err:.4f}")
    assert err <= 1.0, f"normalised error {err}"
    again = torch.full_like(out, -1)
    L.lily_moe_decode(d, w, lgd, xd, r, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(again, out), "fused decode is not deterministic"
    assert not np.any(r.sched.cpu().numpy()), "barrier counters and error flag must be zero"


# ------------------------------------------------------------------- router

@pytest.mark.parametrize("name,T", [("tiny", 32), ("tiny", 7), ("prefill512", 512),
                                    ("prefill512", 77), ("decode40", 1),
                                    ("prefill2048_zipf", 2048)])
def test_router_projection(name, T):
    """lily_moe_router against the oracle: every logit within the fp32
    summation bound 2 H 2^-24 sum|x w| of the double-precision reference; the
    route of the GPU logits bit-exact with the oracle's route of the same
    logits; and every expert the GPU logits select is a valid choice under the
    reference logits (no unselected expert beats it by more than the bound)."""
    cfg = S.CONFIGS[name]
    _flush(f"router {name} T={T}")
    x = S.activations(cfg, 0, T=T)
    w = S.router_weights(cfg)
    ref, absdot = oracle.router(x, w)
    d = L.dims(T, cfg.H, cfg.F, cfg.E, cfg.k, 32)
    lg = torch.full((T, cfg.E), float("nan"), dtype=torch.float32, device="cuda")
    L.lily_moe_router(d, G.to_dev_bits(w), G.to_dev_bits(x), lg)
    torch.cuda.synchronize()
    got = lg.cpu().numpy()
    bound = 2.0 * cfg.H * 2.0 ** -24 * absdot.astype(np.float64) + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    _flush(f"  max error / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound), "router logits outside the fp32 summation bound"
    # the route of the GPU logits
    gpu_r = G.routing_to_host(G.route_gpu(d, got))
    G.compare_routing(gpu_r, oracle.route(got, cfg.k, 32), 32)
    # validity of the selection under the reference logits
    sel = gpu_r["topk_ids"].astype(np.int64)
    chosen = np.take_along_axis(ref, sel, axis=1)
    mask = np.ones_like(ref, dtype=bool)
    np.put_along_axis(mask, sel, False, axis=1)
    best_other = np.where(mask, ref, -np.inf).max(axis=1)
    slack = 2.0 * bound.max(axis=1)
    assert np.all(chosen.min(axis=1) >= best_other - slack), "a selected expert is not in the top-k"
