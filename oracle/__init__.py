"""Python side of the CPU oracle (ctypes over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package's smoke check
and by the benchmark's CPU-baseline leg, never by the GPU path. The library
is built from ``oracle.c`` with gcc (``oracle/build.py``); it shares no code
with the HIP sources.
"""
from __future__ import annotations

import ctypes
import os
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_f32p = ctypes.POINTER(ctypes.c_float)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)


class W4Set(ctypes.Structure):
    _fields_ = [("q", ctypes.POINTER(ctypes.c_void_p)),
                ("scale", ctypes.POINTER(ctypes.c_void_p)),
                ("bias", ctypes.POINTER(ctypes.c_void_p))]


_LIBS = {}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (building first if needed) an oracle library."""
    path = path or LIB_PATH
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise FileNotFoundError(path)
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_route.argtypes = [ctypes.c_int] * 4 + [_c_f32p, _c_i32p, _c_f32p, _c_i32p, _c_i32p,
                                                      _c_i32p, _c_i32p, _c_i32p, _c_i32p, _c_i32p]
    lib.oracle_dequant.restype = ctypes.c_int
    lib.oracle_dequant.argtypes = [_c_u8p, _c_u16p, _c_u16p, ctypes.c_int, ctypes.c_int, _c_u16p]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [ctypes.c_int] * 4 + [
        _c_u16p, _c_i32p, _c_f32p, _c_i32p, ctypes.c_int, W4Set, W4Set, W4Set, _c_f32p, _c_u16p,
        ctypes.c_int]
    lib.oracle_residual_norm.restype = ctypes.c_int
    lib.oracle_residual_norm.argtypes = [ctypes.c_int, ctypes.c_int, _c_f32p, _c_u16p, _c_u16p,
                                         ctypes.c_float]
    lib.oracle_router.restype = ctypes.c_int
    lib.oracle_router.argtypes = [ctypes.c_int] * 3 + [_c_u16p, _c_u16p, _c_f32p, _c_f32p]
    lib.oracle_float_to_bf16.restype = ctypes.c_uint16
    lib.oracle_float_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    _LIBS[path] = lib
    return lib


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


class OracleError(RuntimeError):
    pass


def route(logits: np.ndarray, k: int, tile_m: int, lib: Optional[ctypes.CDLL] = None) -> dict:
    """Routing arrays of one layer: top-k ids and weights, histogram, scan,
    stable scatter and block map (block map trimmed to ``num_blocks``)."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    P = T * k
    max_blocks = max_blocks_for(T, E, k, tile_m)
    out = dict(
        topk_ids=np.zeros((T, k), np.int32), topk_w=np.zeros((T, k), np.float32),
        counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
        sorted_pairs=np.zeros(P, np.int32), pair_rows=np.zeros(P, np.int32),
        block_expert=np.zeros(max_blocks, np.int32), block_row0=np.zeros(max_blocks, np.int32),
        num_blocks=np.zeros(1, np.int32))
    rc = lib.oracle_route(T, E, k, tile_m, _p(logits, _c_f32p), _p(out["topk_ids"], _c_i32p),
                          _p(out["topk_w"], _c_f32p), _p(out["counts"], _c_i32p),
                          _p(out["offsets"], _c_i32p), _p(out["sorted_pairs"], _c_i32p),
                          _p(out["pair_rows"], _c_i32p), _p(out["block_expert"], _c_i32p),
                          _p(out["block_row0"], _c_i32p), _p(out["num_blocks"], _c_i32p))
    if rc != 0:
        raise OracleError(f"oracle_route failed: {rc}")
    nb = int(out["num_blocks"][0])
    out["block_expert"] = out["block_expert"][:nb].copy()
    out["block_row0"] = out["block_row0"][:nb].copy()
    return out


def router(x: np.ndarray, w: np.ndarray, lib: Optional[ctypes.CDLL] = None):
    """Router projection of bf16 x [T, H] by bf16 Wr [E, H]: (logits, absdot),
    float32 [T, E] each; absdot = sum |x w| bounds fp32 summation error."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    T, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    logits = np.zeros((T, E), np.float32)
    absdot = np.zeros((T, E), np.float32)
    rc = lib.oracle_router(T, H, E, _p(x, _c_u16p), _p(w, _c_u16p), _p(logits, _c_f32p),
                           _p(absdot, _c_f32p))
    if rc != 0:
        raise OracleError(f"oracle_router failed: {rc}")
    return logits, absdot


def max_blocks_for(T: int, E: int, k: int, tile_m: int) -> int:
    """Capacity of the block map: every expert adds at most one partial block."""
    P = T * k
    return -(-P // tile_m) + min(E, P)


def dequant(q: np.ndarray, scale: np.ndarray, bias: np.ndarray,
            lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """bf16 bit patterns [N, K] of an int4 matrix."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    bias = np.ascontiguousarray(bias, dtype=np.uint16)
    N, K2 = q.shape
    w = np.zeros((N, 2 * K2), np.uint16)
    rc = lib.oracle_dequant(_p(q, _c_u8p), _p(scale, _c_u16p), _p(bias, _c_u16p), N, 2 * K2,
                            _p(w, _c_u16p))
    if rc != 0:
        raise OracleError(f"oracle_dequant failed: {rc}")
    return w


# An expert getter returns (q, scale, bias) of one matrix of one expert, or
# None when that expert is not available. tensor: 0 gate, 1 up, 2 down;
# expert == E means the shared expert.
ExpertGetter = Callable[[int, int], Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]]]


def getter_from_layer(lw) -> ExpertGetter:
    """Expert getter over a ``synth.LayerWeights`` (stacked arrays)."""
    E = lw.gate.q.shape[0]
    routed = (lw.gate, lw.up, lw.down)
    shared = (lw.sh_gate, lw.sh_up, lw.sh_down)

    def get(tensor: int, e: int):
        w = shared[tensor] if e == E else routed[tensor]
        i = 0 if e == E else e
        return w.q[i], w.scale[i], w.bias[i]

    return get


def forward(x: np.ndarray, topk_ids: np.ndarray, topk_w: np.ndarray, get: ExpertGetter,
            H: int, F: int, E: int, tokens: Optional[Sequence[int]] = None,
            threads: Optional[int] = None, lib: Optional[ctypes.CDLL] = None
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Layer output (fp32 sum before rounding, bf16 bits) for ``tokens``."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    topk_ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = topk_ids.shape
    if tokens is None:
        tok = None
        n_tok = T
        used = set(np.unique(topk_ids).tolist())
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n_tok = len(tok)
        used = set(np.unique(topk_ids[tok]).tolist()) if n_tok else set()
    used.add(E)
    keep = []  # keep arrays alive across the call
    sets = []
    for tensor in range(3):
        arrs = [(ctypes.c_void_p * (E + 1))() for _ in range(3)]
        for e in used:
            m = get(tensor, e)
            if m is None:
                raise OracleError(f"weights of expert {e} (tensor {tensor}) not provided")
            for f, a in enumerate(m):
                a = np.ascontiguousarray(a)
                keep.append(a)
                arrs[f][e] = a.ctypes.data
        keep.append(arrs)
        sets.append(W4Set(ctypes.cast(arrs[0], ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(arrs[1], ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(arrs[2], ctypes.POINTER(ctypes.c_void_p))))
    acc = np.zeros((n_tok, H), np.float32)
    out = np.zeros((n_tok, H), np.uint16)
    rc = lib.oracle_forward(H, F, E, k, _p(x, _c_u16p), _p(topk_ids, _c_i32p),
                            _p(topk_w, _c_f32p), None if tok is None else _p(tok, _c_i32p), n_tok,
                            sets[0], sets[1], sets[2], _p(acc, _c_f32p), _p(out, _c_u16p),
                            int(threads or 0))
    if rc != 0:
        raise OracleError(f"oracle_forward failed: {rc}")
    return acc, out


def residual_norm(r: np.ndarray, out_bf16: Optional[np.ndarray], eps: float = 1e-6,
                  lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """r += out (in place, fp32); returns bf16 bits of r / rms(r)."""
    lib = lib or load()
    assert r.dtype == np.float32 and r.flags["C_CONTIGUOUS"]
    T, H = r.shape
    xn = np.zeros((T, H), np.uint16)
    ob = None if out_bf16 is None else np.ascontiguousarray(out_bf16, dtype=np.uint16)
    rc = lib.oracle_residual_norm(T, H, _p(r, _c_f32p), None if ob is None else _p(ob, _c_u16p),
                                  _p(xn, _c_u16p), eps)
    if rc != 0:
        raise OracleError(f"oracle_residual_norm failed: {rc}")
    return xn


def float_to_bf16(f: float, lib: Optional[ctypes.CDLL] = None) -> int:
    lib = lib or load()
    return int(lib.oracle_float_to_bf16(f))


def threads(lib: Optional[ctypes.CDLL] = None) -> int:
    lib = lib or load()
    return int(lib.oracle_threads())
