"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects bad arguments with the documented codes before
anything is enqueued (no GPU needed: no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

import int4_grouped_gemm_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lily_moe.h", "lily_calib.h", "lily_trace.h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from int4_grouped_gemm_amd import build
        build.build()
    return L.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(lily_\w+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.path.basename(h) for h in HEADERS) == \
        sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


FAKE = 0x7F0000000000  # 16-byte aligned; never dereferenced on these paths


def good_dims(**kw):
    d = dict(T=64, H=256, F=128, E=16, topk=2, group=64, tile_m=64)
    d.update(kw)
    return L.LilyMoeDims(**d)


def routing(fake=FAKE, **over):
    vals = {n: fake + 4096 * i for i, n in enumerate(L.ROUTING_FIELDS)}
    vals.update(over)
    return L.LilyMoeRouting(**vals)


def weights(**over):
    w = {n: FAKE + 4096 * i for i, n in enumerate(L.WEIGHT_FIELDS)}
    w.update(over)
    return L.LilyMoeWeights(**w)


def call_route(lib, d, logits=FAKE, r=None):
    r = r or routing()
    return lib.lily_moe_route(ctypes.byref(d), logits, ctypes.byref(r), None)


def call_forward(lib, d, w=None, x=FAKE, r=None, out=FAKE, ws=FAKE, nbytes=1 << 40):
    w = w or weights()
    r = r or routing()
    return lib.lily_moe_forward(ctypes.byref(d), ctypes.byref(w), x, ctypes.byref(r), out, ws,
                                nbytes, None)


def test_size_queries(lib):
    d = good_dims(T=2048, H=2048, F=512, E=256, topk=8, tile_m=64)
    assert lib.lily_moe_max_blocks(ctypes.byref(d)) == 2048 * 8 // 64 + 256
    rows = 2048 * 9
    assert lib.lily_moe_workspace_bytes(ctypes.byref(d)) == rows * 512 * 2 + rows * 2048 * 4
    d = good_dims(T=1, E=256, topk=8, tile_m=64)
    assert lib.lily_moe_max_blocks(ctypes.byref(d)) == 1 + 8
    bad = good_dims(T=0)
    assert lib.lily_moe_max_blocks(ctypes.byref(bad)) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_moe_workspace_bytes(ctypes.byref(bad)) == 0


@pytest.mark.parametrize("kw,code,text", [
    (dict(T=0), L.LILY_ERR_INVALID_ARG, "T = 0"),
    (dict(E=0), L.LILY_ERR_INVALID_ARG, "E = 0"),
    (dict(topk=0), L.LILY_ERR_INVALID_ARG, "topk"),
    (dict(topk=17), L.LILY_ERR_INVALID_ARG, "topk"),
    (dict(group=32), L.LILY_ERR_INVALID_ARG, "group"),
    (dict(H=100), L.LILY_ERR_INVALID_ARG, "H = 100"),
    (dict(F=0), L.LILY_ERR_INVALID_ARG, "F = 0"),
    (dict(tile_m=0), L.LILY_ERR_INVALID_ARG, "tile_m"),
    (dict(E=600, topk=8), L.LILY_ERR_UNSUPPORTED, "E = 600"),
    (dict(E=128, topk=65), L.LILY_ERR_UNSUPPORTED, "topk = 65"),
])
def test_route_rejects_bad_dims(lib, kw, code, text):
    assert call_route(lib, good_dims(**kw)) == code
    assert text in lib.lily_last_error().decode()


def test_route_rejects_pointers(lib):
    assert call_route(lib, good_dims(), logits=None) == L.LILY_ERR_INVALID_ARG
    assert "logits" in lib.lily_last_error().decode()
    assert call_route(lib, good_dims(), logits=FAKE + 4) == L.LILY_ERR_INVALID_ARG
    assert "aligned" in lib.lily_last_error().decode()
    for n in L.ROUTING_FIELDS:
        assert call_route(lib, good_dims(), r=routing(**{n: None})) == L.LILY_ERR_INVALID_ARG
        assert n in lib.lily_last_error().decode()
    assert lib.lily_moe_route(ctypes.byref(good_dims()), FAKE, None, None) == \
        L.LILY_ERR_INVALID_ARG
    assert lib.lily_moe_route(None, FAKE, ctypes.byref(routing()), None) == L.LILY_ERR_INVALID_ARG


def test_unfused_twin_rejects(lib):
    d = good_dims(tile_m=128)
    rc = lib.lily_moe_forward_bf16(ctypes.byref(d), ctypes.byref(weights()), FAKE,
                                   ctypes.byref(routing()), FAKE, FAKE, 1 << 40, None)
    assert rc == L.LILY_ERR_UNSUPPORTED and "tile_m" in lib.lily_last_error().decode()
    rc = lib.lily_moe_dequant(ctypes.byref(good_dims()), ctypes.byref(weights()),
                              ctypes.byref(routing()), None, None)
    assert rc == L.LILY_ERR_INVALID_ARG and "bf16" in lib.lily_last_error().decode()
    rc = lib.lily_moe_dequant(ctypes.byref(good_dims()), ctypes.byref(weights()),
                              ctypes.byref(routing()), ctypes.byref(weights(down=None)), None)
    assert rc == L.LILY_ERR_INVALID_ARG and "down" in lib.lily_last_error().decode()


def test_decode_stack_rejects(lib):
    """lily_moe_decode_stack validates pointers, eps and sizes before any
    device work."""
    def call(d, n_layers=4, logits=FAKE, eps=1e-6):
        return lib.lily_moe_decode_stack(ctypes.byref(d), n_layers, FAKE, logits, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, FAKE, ctypes.c_float(eps), FAKE, 1 << 40, None)
    ok = good_dims(T=1, H=512, F=256)
    assert call(ok, logits=None) == L.LILY_ERR_INVALID_ARG
    assert "logits" in lib.lily_last_error().decode()
    assert call(ok, eps=-1.0) == L.LILY_ERR_INVALID_ARG and "eps" in lib.lily_last_error().decode()
    assert call(ok, n_layers=0) == L.LILY_ERR_INVALID_ARG
    assert "n_layers" in lib.lily_last_error().decode()
    assert call(good_dims(T=2, H=512, F=256)) == L.LILY_ERR_UNSUPPORTED
    assert "T = 2" in lib.lily_last_error().decode()
    assert call(good_dims(T=1, H=4096, F=256)) == L.LILY_ERR_UNSUPPORTED
    assert "H = 4096" in lib.lily_last_error().decode()
    assert call(good_dims(T=1, H=512, F=128)) == L.LILY_ERR_UNSUPPORTED
    assert "F = 128" in lib.lily_last_error().decode()
    assert call(ok, n_layers=2000) == L.LILY_ERR_UNSUPPORTED  # n_layers * topk beyond the LDS table


def test_route_host_rejects(lib):
    """The host-synchronised twin validates like lily_moe_route, before any
    device work."""
    d = good_dims()
    assert lib.lily_moe_route_host(ctypes.byref(d), None, ctypes.byref(routing()), None) == \
        L.LILY_ERR_INVALID_ARG
    assert "logits" in lib.lily_last_error().decode()
    for n in L.ROUTING_FIELDS:
        assert lib.lily_moe_route_host(ctypes.byref(d), FAKE, ctypes.byref(routing(**{n: None})),
                                       None) == L.LILY_ERR_INVALID_ARG
        assert n in lib.lily_last_error().decode()
    assert lib.lily_moe_route_host(ctypes.byref(good_dims(E=513)), FAKE, ctypes.byref(routing()),
                                   None) == L.LILY_ERR_UNSUPPORTED


def test_forward_rejects(lib):
    assert call_forward(lib, good_dims(tile_m=48)) == L.LILY_ERR_UNSUPPORTED
    assert call_forward(lib, good_dims(H=192)) == L.LILY_ERR_UNSUPPORTED
    assert call_forward(lib, good_dims(F=192)) == L.LILY_ERR_UNSUPPORTED
    assert call_forward(lib, good_dims(), x=None) == L.LILY_ERR_INVALID_ARG
    assert call_forward(lib, good_dims(), out=FAKE + 2) == L.LILY_ERR_INVALID_ARG
    assert call_forward(lib, good_dims(), ws=None) == L.LILY_ERR_INVALID_ARG
    for n in L.WEIGHT_FIELDS:
        w = weights(**{n: None})
        assert call_forward(lib, good_dims(), w=w) == L.LILY_ERR_INVALID_ARG
        assert n in lib.lily_last_error().decode()
        w = weights(**{n: FAKE + 8})
        assert call_forward(lib, good_dims(), w=w) == L.LILY_ERR_INVALID_ARG
        assert "aligned" in lib.lily_last_error().decode()
    d = good_dims()
    need = lib.lily_moe_workspace_bytes(ctypes.byref(d))
    assert call_forward(lib, d, nbytes=need - 1) == L.LILY_ERR_WORKSPACE
    assert str(need) in lib.lily_last_error().decode()
    assert lib.lily_moe_forward(ctypes.byref(d), None, FAKE, ctypes.byref(routing()), FAKE, FAKE,
                                need, None) == L.LILY_ERR_INVALID_ARG


def test_forward_rejects_32bit_offsets(lib):
    """Shapes whose A rows the GEMMs cannot reach with 32-bit byte offsets are
    rejected on the host before any launch (x [T, H] or h [T (k + 1), F] of
    4 GiB or more)."""
    big_x = good_dims(T=1 << 20, H=2048, F=512, E=256, topk=8, tile_m=128)
    assert call_forward(lib, big_x) == L.LILY_ERR_UNSUPPORTED
    assert "x [T = 1048576" in lib.lily_last_error().decode()
    just_x = good_dims(T=(1 << 20) - 1, H=2048, F=128, E=256, topk=1, tile_m=128)
    rc = call_forward(lib, just_x, nbytes=0)  # passes the shape checks, fails on the workspace
    assert rc == L.LILY_ERR_WORKSPACE, lib.lily_last_error().decode()
    big_h = good_dims(T=466_034, H=256, F=512, E=256, topk=8, tile_m=128)  # 9 T * 1024 >= 2^32
    assert call_forward(lib, big_h) == L.LILY_ERR_UNSUPPORTED
    assert "h [T * (topk + 1) = 4194306" in lib.lily_last_error().decode()
    ok_h = good_dims(T=466_033, H=256, F=512, E=256, topk=8, tile_m=128)
    rc = call_forward(lib, ok_h, nbytes=0)  # passes the shape checks, fails on the workspace
    assert rc == L.LILY_ERR_WORKSPACE, lib.lily_last_error().decode()
    for fn in (lib.lily_moe_gate_up,):
        assert fn(ctypes.byref(big_x), ctypes.byref(weights()), FAKE, ctypes.byref(routing()), FAKE,
                  1 << 40, None) == L.LILY_ERR_UNSUPPORTED
    assert lib.lily_moe_down(ctypes.byref(big_h), ctypes.byref(weights()), ctypes.byref(routing()),
                             FAKE, 1 << 40, None) == L.LILY_ERR_UNSUPPORTED
    assert lib.lily_moe_forward_bf16(ctypes.byref(big_x), ctypes.byref(weights()), FAKE,
                                     ctypes.byref(routing()), FAKE, FAKE, 1 << 40,
                                     None) == L.LILY_ERR_UNSUPPORTED


def test_calib_rejects(lib):
    assert lib.lily_calib_mfma(0, 4, 100, FAKE, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_mfma(256, 4, 101, FAKE, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_mfma(256, 4, 100, None, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_dequant(0, 4, 100, FAKE, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_dequant(256, 17, 100, FAKE, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_dequant(256, 4, 0, FAKE, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_dequant(256, 4, 100, FAKE, None, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_read(FAKE, 1000, 256, 0, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_read(FAKE + 4, 1024, 256, 1, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_calib_read(None, 1024, 256, 1, FAKE, None) == L.LILY_ERR_INVALID_ARG


def test_residual_norm_rejects(lib):
    assert lib.lily_residual_norm(0, 256, FAKE, FAKE, FAKE, 1e-6, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_residual_norm(4, 250, FAKE, FAKE, FAKE, 1e-6, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_residual_norm(4, 256, None, FAKE, FAKE, 1e-6, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_residual_norm(4, 256, FAKE, FAKE, FAKE, -1.0, None) == L.LILY_ERR_INVALID_ARG


def test_binding_raises(lib):
    with pytest.raises(L.LilyError) as ei:
        L.lily_moe_max_blocks(good_dims(topk=99))
    assert ei.value.code == L.LILY_ERR_INVALID_ARG


def test_packed_bytes(lib):
    assert lib.lily_w4_packed_bytes(256, 512, 2048, 64) == 256 * 512 * 2048 * 9 // 16
    assert lib.lily_w4_packed_bytes(1, 128, 64, 64) == 4608
    for bad in [(0, 128, 64, 64), (1, 100, 64, 64), (1, 128, 96, 64), (1, 128, 64, 32),
                (1, -128, 64, 64)]:
        assert lib.lily_w4_packed_bytes(*bad) == 0, bad


def test_pack_rejects(lib):
    w = L.LilyW4(FAKE, FAKE + 256, FAKE + 512)
    pack = lib.lily_w4_pack
    assert pack(ctypes.byref(w), 1, 100, 64, 64, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert "multiple of 128" in lib.lily_last_error().decode()
    assert pack(None, 1, 128, 64, 64, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert pack(ctypes.byref(w), 1, 128, 64, 64, None, None) == L.LILY_ERR_INVALID_ARG
    assert "packed" in lib.lily_last_error().decode()
    bad = L.LilyW4(FAKE, FAKE + 2, FAKE)
    assert pack(ctypes.byref(bad), 1, 128, 64, 64, FAKE, None) == L.LILY_ERR_INVALID_ARG
    assert "scale" in lib.lily_last_error().decode()


def test_decode_rejects(lib):
    d = good_dims(T=5, H=512, F=128)
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights()), FAKE, FAKE,
                             ctypes.byref(routing()), FAKE, FAKE, 1 << 40, None)
    assert rc == L.LILY_ERR_UNSUPPORTED and "T = 5" in lib.lily_last_error().decode()
    d = good_dims(T=1, H=256, F=128)
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights()), FAKE, FAKE,
                             ctypes.byref(routing()), FAKE, FAKE, 1 << 40, None)
    assert rc == L.LILY_ERR_UNSUPPORTED and "H = 256" in lib.lily_last_error().decode()
    d = good_dims(T=1, H=512, F=128)
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights()), FAKE, FAKE,
                             ctypes.byref(routing()), FAKE, FAKE, 1 << 40, None)
    assert rc == L.LILY_ERR_UNSUPPORTED and "F = 128" in lib.lily_last_error().decode()
    d = good_dims(T=1, H=512, F=256)
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights()), None, FAKE,
                             ctypes.byref(routing()), FAKE, FAKE, 1 << 40, None)
    assert rc == L.LILY_ERR_INVALID_ARG and "logits" in lib.lily_last_error().decode()
    need = lib.lily_moe_workspace_bytes(ctypes.byref(d))
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights()), FAKE, FAKE,
                             ctypes.byref(routing()), FAKE, FAKE, need - 1, None)
    assert rc == L.LILY_ERR_WORKSPACE


def test_trace_only_in_the_tracing_build(lib):
    """The traces are the tracing build's: the ordinary library reports them
    as unsupported, the tracing build exports the same symbols and rejects a
    NULL destination before any device call."""
    buf = (ctypes.c_ulonglong * 4)()
    assert lib.lily_trace_ffn_items(buf, 1, None) == L.LILY_ERR_UNSUPPORTED
    assert "built without" in lib.lily_last_error().decode()
    if not os.path.exists(L.TRACE_LIB_PATH):
        from int4_grouped_gemm_amd import build
        build.build()
    tl = L.load(L.TRACE_LIB_PATH)
    for n in declared_functions():
        assert hasattr(tl, n), f"{n} not exported by the tracing build"
    assert tl.lily_trace_ffn_items(None, 1, None) == L.LILY_ERR_INVALID_ARG
    assert tl.lily_trace_ffn_items(buf, 0, None) == L.LILY_ERR_INVALID_ARG
    assert lib.lily_trace_decode_stack(buf, 1, None) == L.LILY_ERR_UNSUPPORTED
    assert tl.lily_trace_decode_stack(None, 1, None) == L.LILY_ERR_INVALID_ARG
    assert tl.lily_trace_decode_stack(buf, 0, None) == L.LILY_ERR_INVALID_ARG
