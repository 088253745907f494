"""Checks that pin the CPU oracle to values that do not come from the oracle.

Each ``pin_*`` function takes an oracle library (``oracle.load(path)``) and
raises ``AssertionError`` when the oracle disagrees with a closed form, an
invariant, a hand-worked fixture or an independent float64 formulation. The
oracle's own tests run them on the real oracle; the mutant tests run them on
copies of the oracle with a planted mistake and expect at least one to fail.

Independent arithmetic used here: float64 numpy for sums and products, and
torch's CPU float32 -> bfloat16 conversion (round to nearest even) for bf16
rounding. Neither the oracle's nor the input generator's bf16 routine is used.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
from synth import inputs as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ independent helpers

def bf16_round64(a) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE, by torch) -> float64."""
    t = torch.from_numpy(np.asarray(a, dtype=np.float64).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def bits_to_f64(b) -> np.ndarray:
    t = torch.from_numpy(np.asarray(b, dtype=np.uint16).astype(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def f64_to_bits(a) -> np.ndarray:
    t = torch.from_numpy(np.asarray(a, dtype=np.float64).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] values; element 2i in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0x0F
    out[..., 1::2] = q >> 4
    return out


def pack_nibbles(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.uint8)
    return (v[..., 0::2] | (v[..., 1::2] << 4)).astype(np.uint8)


def dequant64(q, scale, bias) -> np.ndarray:
    """Independent dequantisation: exact s*q+b in float64, then fp32, then bf16."""
    v = unpack_nibbles(q).astype(np.float64)
    N, K = v.shape
    s = np.repeat(bits_to_f64(scale), S.GROUP, axis=1)[:, :K]
    b = np.repeat(bits_to_f64(bias), S.GROUP, axis=1)[:, :K]
    return bf16_round64(s * v + b)


def silu64(z):
    return z / (1.0 + np.exp(-z))


def norm_err(got, ref) -> float:
    """max |got - ref| / (|ref| + RMS(ref))."""
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + rms)))


# -------------------------------------------------------------------- dequant pins

def pin_dequant_closed_form(lib, n_rows=640, seed=1):
    """All 256 byte values (both nibbles) x >= 10^4 (scale, bias) pairs drawn
    from the workload distributions plus edge values, against exact float64."""
    g = np.random.default_rng(seed)
    K = 256  # 4 groups per row
    q = np.tile(np.arange(256, dtype=np.uint8), (n_rows, K // 2 // 256 + 1))[:, :K // 2]
    q = np.ascontiguousarray(np.roll(q, g.integers(0, 256), axis=1))
    s = f64_to_bits(g.uniform(0.005, 0.02, (n_rows, K // 64)))
    b = f64_to_bits(g.normal(0, 0.01, (n_rows, K // 64)))
    # edge values: scale 0 (w == bias), bias 0 (exact product), wide magnitudes
    s[0, :] = 0
    b[1, :] = 0
    s[2, :] = f64_to_bits([1.0, 2.0 ** -20, 3.5, 0.0078125])
    b[2, :] = f64_to_bits([-7.5, 1e-3, 2.0 ** 10, -0.0])
    w = bits_to_f64(oracle.dequant(q, s, b, lib=lib))
    ref = dequant64(q, s, b)
    assert np.array_equal(w, ref), f"dequant mismatch at {np.argwhere(w != ref)[:5]}"
    assert np.all(w[0].reshape(-1, 64) == bits_to_f64(b[0])[:, None]), "scale 0 must give bias"
    v1 = unpack_nibbles(q[1:2])[0]
    pow2 = np.isin(v1, (0, 1, 2, 4, 8))
    assert np.array_equal(w[1][pow2], (bits_to_f64(s[1]).repeat(64) * v1)[pow2]), \
        "bias 0 with q a power of two must give the exact product"


def pin_dequant_golden(lib):
    d = json.load(open(os.path.join(GOLDEN, "dequant_handworked.json")))
    for c in d["cases"]:
        q = np.full((1, 32), c["byte"], np.uint8)
        s = np.full((1, 1), c["scale"], np.uint16)
        b = np.full((1, 1), c["bias"], np.uint16)
        w = oracle.dequant(q, s, b, lib=lib)
        assert w[0, 0] == c["expect"][0] and w[0, 1] == c["expect"][1], \
            (c["derivation"], hex(w[0, 0]), hex(w[0, 1]))


def pin_nibble_order(lib):
    """scale 1, bias 0 makes w == q: the oracle must read element 2i from the
    low nibble. Also checks that pack/unpack round-trip."""
    g = np.random.default_rng(7)
    v = g.integers(0, 16, (8, 128), dtype=np.uint8)
    q = pack_nibbles(v)
    assert np.array_equal(unpack_nibbles(q), v)
    one = np.full((8, 2), 0x3F80, np.uint16)
    zero = np.zeros((8, 2), np.uint16)
    w = bits_to_f64(oracle.dequant(q, one, zero, lib=lib))
    assert np.array_equal(w, v.astype(np.float64)), "nibble order"


def pin_group_axis(lib):
    """Groups run along K: a distinct scale per 64-column group and per row."""
    N, K = 4, 256
    q = pack_nibbles(np.ones((N, K), np.uint8))  # q = 1 everywhere -> w = s + 0
    s = f64_to_bits(np.arange(1, N * K // 64 + 1, dtype=np.float64).reshape(N, K // 64))
    w = bits_to_f64(oracle.dequant(q, s, np.zeros_like(s), lib=lib))
    exp = np.repeat(bits_to_f64(s), 64, axis=1)
    assert np.array_equal(w, exp), "group axis / group index"


# ---------------------------------------------------------------------- route pins

def brute_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Full sort by (-logit, expert); -0.0 compares equal to +0.0."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int64)
    e = np.arange(E)
    for t in range(T):
        order = np.lexsort((e, -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


def softmax64(v):
    v = np.asarray(v, np.float64)
    z = np.exp(v - v.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def check_route_invariants(r: dict, T: int, E: int, k: int, M: int):
    ids = r["topk_ids"].astype(np.int64)
    P = T * k
    counts, offsets = r["counts"], r["offsets"]
    sp, pr = r["sorted_pairs"].astype(np.int64), r["pair_rows"].astype(np.int64)
    assert counts.sum() == P, "histogram must sum to T*k"
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E)), "histogram"
    assert offsets[0] == 0 and offsets[E] == P and np.all(np.diff(offsets) == counts), "scan"
    assert np.array_equal(np.sort(sp), np.arange(P)), "scatter must be a permutation"
    assert np.array_equal(pr[sp], np.arange(P)), "pair_rows must invert sorted_pairs"
    assert np.array_equal(np.bincount(sp // k, minlength=T), np.full(T, k)), "k rows per token"
    assert np.array_equal(sp, np.argsort(ids.ravel(), kind="stable")), "stable scatter order"
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(ids.ravel()[seg] == e), "segment expert"
        assert np.all(np.diff(seg // k) >= 0), "ascending tokens in a segment"
    # block map tiles every segment exactly once, in ascending expert order
    be, b0 = r["block_expert"], r["block_row0"]
    exp_e, exp_r = [], []
    for e in range(E):
        for r0 in range(offsets[e], offsets[e + 1], M):
            exp_e.append(e)
            exp_r.append(r0)
    assert int(r["num_blocks"][0]) == len(exp_e), "num_blocks"
    assert np.array_equal(be, exp_e) and np.array_equal(b0, exp_r), "block map"
    assert len(exp_e) <= oracle.max_blocks_for(T, E, k, M), "block map capacity"


def pin_route_brute_force(lib):
    for name, M in (("tiny", 8), ("prefill512", 32), ("prefill2048_zipf", 64)):
        cfg = S.CONFIGS[name]
        lg = S.router_logits(cfg)
        r = oracle.route(lg, cfg.k, M, lib=lib)
        assert np.array_equal(r["topk_ids"], brute_topk(lg, cfg.k)), f"top-k ({name})"
        sel = np.take_along_axis(lg, r["topk_ids"].astype(np.int64), axis=1)
        assert np.max(np.abs(r["topk_w"] - softmax64(sel))) <= 2e-6, f"softmax ({name})"
        check_route_invariants(r, cfg.T, cfg.E, cfg.k, M)


def pin_route_ties(lib):
    # all equal: experts 0..k-1, weight 1/k
    for k in (1, 3, 8):
        lg = np.zeros((2, 16), np.float32)
        r = oracle.route(lg, k, 4, lib=lib)
        assert np.array_equal(r["topk_ids"], np.tile(np.arange(k), (2, 1))), "all-equal tie"
        assert np.all(r["topk_w"] == np.float32(1.0) / np.float32(k)), "all-equal weights"
    # -0.0 ties +0.0: the lower index wins whichever sign it carries
    lg = np.full((2, 8), -5.0, np.float32)
    lg[0, 2], lg[0, 5] = -0.0, 0.0
    lg[1, 2], lg[1, 5] = 0.0, -0.0
    r = oracle.route(lg, 1, 1, lib=lib)
    assert list(r["topk_ids"][:, 0]) == [2, 2], "signed-zero tie"
    # equal pair straddling the k-th place
    lg = np.array([[0.0, 3.0, 1.0, 2.0, 1.0, -1.0]], np.float32)
    r = oracle.route(lg, 3, 2, lib=lib)
    assert list(r["topk_ids"][0]) == [1, 3, 2], "tie at the k-th place"
    # large logits: the softmax must not overflow (the largest is subtracted)
    lg = (np.random.default_rng(5).standard_normal((4, 32)) + 200.0).astype(np.float32)
    r = oracle.route(lg, 8, 4, lib=lib)
    sel = np.take_along_axis(lg, r["topk_ids"].astype(np.int64), axis=1)
    assert np.all(np.isfinite(r["topk_w"])), "softmax overflow"
    assert np.max(np.abs(r["topk_w"] - softmax64(sel))) <= 2e-6, "softmax at large logits"
    # k = 1: weight exactly 1
    lg = S.router_logits(S.CONFIGS["tiny"])
    r = oracle.route(lg, 1, 4, lib=lib)
    assert np.all(r["topk_w"] == 1.0), "k=1 weight"
    assert np.array_equal(r["topk_ids"][:, 0], np.argmax(lg, axis=1)), "k=1 is argmax"
    # k = E: plain softmax over all logits
    r = oracle.route(lg, lg.shape[1], 4, lib=lib)
    sm = softmax64(lg)
    got = np.zeros_like(sm)
    np.put_along_axis(got, r["topk_ids"].astype(np.int64), r["topk_w"], axis=1)
    assert np.max(np.abs(got - sm)) <= 1e-6, "k=E softmax"
    assert np.all(np.diff(np.take_along_axis(lg, r["topk_ids"].astype(np.int64), 1), axis=1) <= 0)


def pin_route_golden(lib):
    d = json.load(open(os.path.join(GOLDEN, "route_handworked.json")))
    lg = np.array(d["logits"], np.float32)
    lg[1, 0] = -0.0  # JSON keeps the sign, but make it explicit
    for M, bm in d["block_map"].items():
        r = oracle.route(lg, d["k"], int(M), lib=lib)
        for key in ("topk_ids", "counts", "offsets", "sorted_pairs", "pair_rows"):
            assert np.array_equal(r[key], np.array(d[key])), f"golden {key}"
        assert np.max(np.abs(r["topk_w"] - np.array(d["topk_w"]))) <= 2e-6, "golden topk_w"
        assert list(r["block_expert"]) == bm["block_expert"], f"golden block_expert M={M}"
        assert list(r["block_row0"]) == bm["block_row0"], f"golden block_row0 M={M}"


# -------------------------------------------------------------------- forward pins

def dense_layer64(x_bits, ids, w, lw, E):
    """Every expert on every token in float64 with bf16 rounding at the
    dequantised weights and at h, then out = sum_e G[t,e] FFN_e(x) + FFN_sh(x)
    with a dense gate matrix G (the routing weight or 0)."""
    x = bits_to_f64(x_bits)
    T = x.shape[0]
    G = np.zeros((T, E + 1))
    for t in range(T):
        for j in range(ids.shape[1]):
            G[t, ids[t, j]] += w[t, j]
    G[:, E] = 1.0
    out = np.zeros((T, lw.down.q.shape[1]))
    for e in range(E + 1):
        src = (lw.sh_gate, lw.sh_up, lw.sh_down) if e == E else (lw.gate, lw.up, lw.down)
        i = 0 if e == E else e
        Wg = dequant64(src[0].q[i], src[0].scale[i], src[0].bias[i])
        Wu = dequant64(src[1].q[i], src[1].scale[i], src[1].bias[i])
        Wd = dequant64(src[2].q[i], src[2].scale[i], src[2].bias[i])
        h = bf16_round64(silu64(x @ Wg.T) * (x @ Wu.T))
        out += G[:, e:e + 1] * (h @ Wd.T)
    return out


def pin_forward_dense(lib):
    cfg = S.CONFIGS["tiny"]
    lw = S.layer_weights(cfg)
    x = S.activations(cfg)
    r = oracle.route(S.router_logits(cfg), cfg.k, 8, lib=lib)
    acc, out = oracle.forward(x, r["topk_ids"], r["topk_w"], oracle.getter_from_layer(lw),
                              cfg.H, cfg.F, cfg.E, lib=lib)
    ref = dense_layer64(x, r["topk_ids"], r["topk_w"], lw, cfg.E)
    assert norm_err(acc, ref) <= 1e-3, f"dense float64 formulation: {norm_err(acc, ref)}"
    assert np.array_equal(out, f64_to_bits(acc.astype(np.float64))), "final bf16 rounding"
    # a token subset gives the same rows
    sub = [5, 0, 31]
    acc2, _ = oracle.forward(x, r["topk_ids"], r["topk_w"], oracle.getter_from_layer(lw),
                             cfg.H, cfg.F, cfg.E, tokens=sub, lib=lib)
    assert np.array_equal(acc2, acc[sub]), "token subset"


def _const_layer(H, F, E, gate_v, up_v, down_v, s_gate, s_up, s_down):
    """Every expert (and the shared one) with the same nibbles and scales, bias 0."""
    def w4(vals, s, n):
        N, K = vals.shape
        q = np.broadcast_to(pack_nibbles(vals), (n, N, K // 2)).copy()
        sc = np.full((n, N, K // 64), f64_to_bits([s])[0], np.uint16)
        return S.W4(q, sc, np.zeros_like(sc))
    return S.LayerWeights(gate=w4(gate_v, s_gate, E), up=w4(up_v, s_up, E),
                          down=w4(down_v, s_down, E), sh_gate=w4(gate_v, s_gate, 1),
                          sh_up=w4(up_v, s_up, 1), sh_down=w4(down_v, s_down, 1))


def pin_forward_h_rounding(lib):
    """Closed form that exposes the bf16 rounding of h: gate/up weights q/16
    and x on a 1/8 grid make g and u exact; down weights are all 1, so
    y_n = sum_f h_f; E = 1, k = 1 and a shared expert equal to the routed one
    give acc = 2 * sum_f bf16(silu(g_f) * u_f)."""
    g = np.random.default_rng(11)
    H = F = 64
    T = 6
    gv = g.integers(0, 16, (F, H), dtype=np.uint8)
    uv = g.integers(0, 16, (F, H), dtype=np.uint8)
    dv = np.ones((H, F), np.uint8)
    lw = _const_layer(H, F, 1, gv, uv, dv, 1.0 / 256, 1.0 / 256, 1.0)
    xv = g.integers(-8, 9, (T, H)) / 8.0
    x = f64_to_bits(xv)
    gg = xv @ (gv.astype(np.float64) / 256).T
    uu = xv @ (uv.astype(np.float64) / 256).T
    v = silu64(gg) * uu
    # bf16 rounding of v must not sit within fp32 noise of a rounding boundary
    h = bf16_round64(v)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    acc, _ = oracle.forward(x, ids, wts, oracle.getter_from_layer(lw), H, F, 1, lib=lib)
    exp = 2.0 * h.sum(axis=1)
    assert np.max(np.abs(acc[:, 0] - exp) / np.abs(exp)) <= 1e-6, "h must be rounded to bf16"
    assert np.all(acc == acc[:, :1]), "all outputs equal for all-ones down weights"


def pin_forward_special_cases(lib):
    cfg = S.CONFIGS["tiny"]
    lw = S.layer_weights(cfg)
    r = oracle.route(S.router_logits(cfg), cfg.k, 8, lib=lib)
    # x = 0 -> out = 0 exactly
    x0 = np.zeros((cfg.T, cfg.H), np.uint16)
    acc, out = oracle.forward(x0, r["topk_ids"], r["topk_w"], oracle.getter_from_layer(lw),
                              cfg.H, cfg.F, cfg.E, lib=lib)
    assert np.all(acc == 0) and np.all(out == 0), "x = 0"
    # identical experts: out = 2 FFN(x) independent of routing
    def rep(w, n):
        return S.W4(*(np.broadcast_to(a[:1], (n,) + a.shape[1:]).copy()
                      for a in (w.q, w.scale, w.bias)))
    same = S.LayerWeights(gate=rep(lw.sh_gate, cfg.E), up=rep(lw.sh_up, cfg.E),
                          down=rep(lw.sh_down, cfg.E), sh_gate=lw.sh_gate, sh_up=lw.sh_up,
                          sh_down=lw.sh_down)
    x = S.activations(cfg)
    acc, _ = oracle.forward(x, r["topk_ids"], r["topk_w"], oracle.getter_from_layer(same),
                            cfg.H, cfg.F, cfg.E, lib=lib)
    ids1 = np.zeros((cfg.T, 1), np.int32)
    acc1, _ = oracle.forward(x, ids1, np.ones((cfg.T, 1), np.float32),
                             oracle.getter_from_layer(same), cfg.H, cfg.F, cfg.E, lib=lib)
    assert norm_err(acc, acc1) <= 1e-5, "identical experts: routing must not matter"
    # E = 1, k = 1, T = 1: a single SwiGLU GEMV pair in float64
    x1 = x[:1]
    one = np.zeros((1, 1), np.int32)
    lw1 = S.LayerWeights(*(S.W4(m.q[:1], m.scale[:1], m.bias[:1])
                           for m in (lw.gate, lw.up, lw.down)),
                         lw.sh_gate, lw.sh_up, lw.sh_down)
    acc, _ = oracle.forward(x1, one, np.ones((1, 1), np.float32),
                            oracle.getter_from_layer(lw1), cfg.H, cfg.F, 1, lib=lib)
    xs = bits_to_f64(x1)
    ref = 0
    for src, i in (((lw.sh_gate, lw.sh_up, lw.sh_down), 0), ((lw.gate, lw.up, lw.down), 0)):
        Wg, Wu, Wd = (dequant64(m.q[i], m.scale[i], m.bias[i]) for m in src)
        ref = ref + bf16_round64(silu64(xs @ Wg.T) * (xs @ Wu.T)) @ Wd.T
    assert norm_err(acc, ref) <= 1e-5, "single-token GEMV"


def pin_router(lib):
    """Router projection against a float64 numpy matmul of the widened bf16
    inputs (a different summation, so at most 1 ulp of the final fp32
    rounding apart), on non-square shapes so a transposed index shows; a
    one-hot x picks a column of Wr exactly."""
    rng = np.random.default_rng(7)
    T, H, E = 5, 192, 7
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = S.f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.1))
    lg, ad = oracle.router(x, w, lib=lib)
    xf = S.bf16_bits_to_f32(x).astype(np.float64)
    wf = S.bf16_bits_to_f32(w).astype(np.float64)
    ref = (xf @ wf.T).astype(np.float32)
    assert np.all(np.abs(lg - ref) <= np.spacing(np.abs(ref))), "router logits"
    mag = (np.abs(xf) @ np.abs(wf).T).astype(np.float32)
    assert np.all(np.abs(ad - mag) <= np.spacing(mag)), "router |x w| sums"
    # one-hot rows: token t selects column h_t of every router row
    cols = np.array([0, 3, 64, 130, 191])
    onehot = np.zeros((T, H), np.uint16)
    onehot[np.arange(T), cols] = S.f32_to_bf16_bits(np.ones(T, np.float32))
    lg1, _ = oracle.router(onehot, w, lib=lib)
    assert np.array_equal(lg1, wf[:, cols].T.astype(np.float32)), "one-hot router row"


def pin_residual_norm(lib):
    g = np.random.default_rng(3)
    T, H = 4, 256
    r = g.normal(0, 50, (T, H)).astype(np.float32)
    r0 = r.copy()
    o = f64_to_bits(g.normal(0, 10, (T, H)))
    xn = oracle.residual_norm(r, o, 1e-6, lib=lib)
    rr = r0.astype(np.float64) + bits_to_f64(o)
    assert np.max(np.abs(r - rr)) <= 1e-4, "residual add"
    ref = rr / np.sqrt((rr * rr).mean(axis=1, keepdims=True) + 1e-6)
    got = bits_to_f64(xn)
    assert np.max(np.abs(got - ref) / np.abs(ref)) <= 2.0 ** -8, "unit RMSNorm"
    c = np.full((1, H), -3.0, np.float32)
    assert np.all(bits_to_f64(oracle.residual_norm(c, None, 1e-6, lib=lib)) == -1.0)


ALL_PINS = [pin_dequant_closed_form, pin_dequant_golden, pin_nibble_order, pin_group_axis,
            pin_route_brute_force, pin_route_ties, pin_route_golden, pin_forward_dense,
            pin_forward_h_rounding, pin_forward_special_cases, pin_router, pin_residual_norm]
