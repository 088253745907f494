"""lily_moe_decode_noalloc (scratch in the library's static device array)
against lily_moe_decode (caller workspace and routing buffers): the same
routing and the same outputs on two calls in a row, the second with fewer
tokens than the first, and outputs within the layer's tolerance of the
oracle."""
import numpy as np
import pytest
import torch

import int4_grouped_gemm_amd as L
import oracle
from synth import inputs as S

import gpu_layer as G

pytestmark = pytest.mark.gpu


def test_decode_noalloc_matches_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    cfg = S.CONFIGS["prefill512"]  # H 2048, F 512, E 256, top-8 + shared
    lw = S.layer_weights(cfg, 0)
    w = L.weights_from_host(lw)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for call, T in enumerate((4, 1)):
        print(f"decode_noalloc call {call}: T = {T}", flush=True)
        d = L.dims(T, cfg.H, cfg.F, cfg.E, cfg.k, 32)
        x = S.activations(cfg, 7, T=T)
        lg = S.router_logits(cfg, 0, 7, T=T)
        xd, lgd = G.to_dev_bits(x), torch.from_numpy(lg).cuda()
        # the existing entry point, with caller-owned workspace and routing
        r = L.alloc_routing(d)
        ws = L.alloc_workspace(d)
        out_a = torch.full((T, cfg.H), -1, dtype=torch.int16, device="cuda")
        L.lily_moe_decode(d, w, lgd, xd, r, out_a, ws)
        # the one that allocates nothing
        ids = torch.full((T, cfg.k), -1, dtype=torch.int32, device="cuda")
        wts = torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device="cuda")
        out_b = torch.full((T, cfg.H), -1, dtype=torch.int16, device="cuda")
        L.lily_moe_decode_noalloc(d, w, lgd, xd, ids, wts, out_b, status)
        torch.cuda.synchronize()
        assert status.item() == 0, "barrier wait gave up"
        assert not np.any(r.sched.cpu().numpy()), "lily_moe_decode left its counters non-zero"
        assert np.array_equal(ids.cpu().numpy(), r.topk_ids.cpu().numpy())
        assert np.array_equal(wts.cpu().numpy().view(np.uint32),
                              r.topk_w.cpu().numpy().view(np.uint32))
        got = G.from_dev_bits(out_b)
        assert np.array_equal(got, G.from_dev_bits(out_a)), "outputs differ from lily_moe_decode"
        ref = oracle.route(lg, cfg.k, 32)
        assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
        acc, _ = oracle.forward(x, ref["topk_ids"], ref["topk_w"], oracle.getter_from_layer(lw),
                                cfg.H, cfg.F, cfg.E)
        err = G.output_error(got, acc)
        print(f"  normalised error vs the oracle {err:.4f}", flush=True)
        assert err <= 1.0


def test_decode_noalloc_rejects():
    """Host checks before anything is enqueued."""
    L.load()
    lib = L.load()
    import ctypes
    fake = 0x7F0000000000
    d = L.dims(5, 2048, 512, 256, 8, 32)
    wt = L.LilyMoeWeights(*[fake + 4096 * i for i in range(6)])
    rc = lib.lily_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(wt), fake, fake, fake, fake,
                                     fake, None, None)
    assert rc == L.LILY_ERR_UNSUPPORTED and "T = 5" in lib.lily_last_error().decode()
    d = L.dims(1, 2048, 512, 256, 8, 32)
    rc = lib.lily_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(wt), fake, fake, None, fake,
                                     fake, None, None)
    assert rc == L.LILY_ERR_INVALID_ARG and "topk_ids" in lib.lily_last_error().decode()
    rc = lib.lily_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(wt), fake, fake, fake, fake,
                                     fake, fake + 2, None)
    assert rc == L.LILY_ERR_INVALID_ARG and "status" in lib.lily_last_error().decode()
