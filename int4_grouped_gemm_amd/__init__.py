"""Python binding of ``liblily_moe.so``: the int4 grouped-GEMM MoE layer on MI355X.

The functions below carry the C ABI's names (``include/lily_moe.h``) and do
argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch provides device memory and streams. There is no fallback:
if the library has not been built, loading it raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblily_moe.so")
TRACE_LIB_PATH = os.path.join(HERE, "liblily_moe_trace.so")  # the same, with the FFN item trace

LILY_OK = 0
LILY_ERR_INVALID_ARG = -1
LILY_ERR_UNSUPPORTED = -2
LILY_ERR_WORKSPACE = -3
LILY_ERR_HIP = -4

EXPORTS = ("lily_moe_max_blocks", "lily_moe_workspace_bytes", "lily_w4_packed_bytes",
           "lily_w4_pack", "lily_moe_router", "lily_moe_route", "lily_moe_route_host",
           "lily_moe_forward", "lily_moe_dequant", "lily_moe_forward_bf16", "lily_moe_gate_up",
           "lily_moe_down", "lily_moe_ffn", "lily_moe_combine", "lily_moe_decode", "lily_moe_decode_noalloc",
           "lily_moe_decode_stack",
           "lily_residual_norm",
           "lily_last_error",
           # include/lily_calib.h
           "lily_calib_mfma", "lily_calib_dequant", "lily_calib_read",
           # include/lily_trace.h
           "lily_trace_ffn_items", "lily_trace_decode_stack")
LILY_SCHED_INTS = 1632 + 64 * 512 + 1
SCHED_GIVE_UP = 30  # sched[30]: sticky flag, set when a bounded device-wide wait gave up
WEIGHT_FIELDS = ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")


class LilyMoeDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("F", ctypes.c_int32),
                ("E", ctypes.c_int32), ("topk", ctypes.c_int32), ("group", ctypes.c_int32),
                ("tile_m", ctypes.c_int32)]


class LilyW4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class LilyMoeWeights(ctypes.Structure):
    """Packed weight stacks (device pointers written by lily_w4_pack)."""
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


ROUTING_FIELDS = ("topk_ids", "topk_w", "counts", "offsets", "sorted_pairs", "pair_rows",
                  "block_expert", "block_row0", "num_blocks", "block_order", "sched",
                  "block_info")


class LilyMoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ROUTING_FIELDS]


class LilyError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"lily error {code}: {text}")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the HIP library. Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -c 'import __graft_entry__ as g;"
                           f" g.build()'` (or int4_grouped_gemm_amd/build.py)")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER
    lib.lily_moe_max_blocks.restype = ctypes.c_int32
    lib.lily_moe_max_blocks.argtypes = [P(LilyMoeDims)]
    lib.lily_moe_workspace_bytes.restype = ctypes.c_size_t
    lib.lily_moe_workspace_bytes.argtypes = [P(LilyMoeDims)]
    lib.lily_w4_packed_bytes.restype = ctypes.c_size_t
    lib.lily_w4_packed_bytes.argtypes = [ctypes.c_int32] * 4
    lib.lily_w4_pack.restype = ctypes.c_int
    lib.lily_w4_pack.argtypes = [P(LilyW4), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_moe_router.restype = ctypes.c_int
    lib.lily_moe_router.argtypes = [P(LilyMoeDims), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_moe_route.restype = ctypes.c_int
    lib.lily_moe_route.argtypes = [P(LilyMoeDims), ctypes.c_void_p, P(LilyMoeRouting),
                                   ctypes.c_void_p]
    lib.lily_moe_route_host.restype = ctypes.c_int
    lib.lily_moe_route_host.argtypes = [P(LilyMoeDims), ctypes.c_void_p, P(LilyMoeRouting),
                                        ctypes.c_void_p]
    lib.lily_moe_forward.restype = ctypes.c_int
    lib.lily_moe_forward.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                     P(LilyMoeRouting), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
    lib.lily_moe_dequant.restype = ctypes.c_int
    lib.lily_moe_dequant.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), P(LilyMoeRouting),
                                     P(LilyMoeWeights), ctypes.c_void_p]
    lib.lily_moe_forward_bf16.restype = ctypes.c_int
    lib.lily_moe_forward_bf16.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                          P(LilyMoeRouting), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
    lib.lily_moe_gate_up.restype = ctypes.c_int
    lib.lily_moe_gate_up.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                     P(LilyMoeRouting), ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    lib.lily_moe_down.restype = ctypes.c_int
    lib.lily_moe_down.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), P(LilyMoeRouting),
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.lily_moe_ffn.restype = ctypes.c_int
    lib.lily_moe_ffn.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                 P(LilyMoeRouting), ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    lib.lily_moe_combine.restype = ctypes.c_int
    lib.lily_moe_combine.argtypes = [P(LilyMoeDims), P(LilyMoeRouting), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_moe_decode.restype = ctypes.c_int
    lib.lily_moe_decode.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                    ctypes.c_void_p, P(LilyMoeRouting), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.lily_moe_decode_stack.restype = ctypes.c_int
    lib.lily_moe_decode_stack.argtypes = [P(LilyMoeDims), ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
    lib.lily_residual_norm.restype = ctypes.c_int
    lib.lily_residual_norm.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                       ctypes.c_void_p]
    lib.lily_last_error.restype = ctypes.c_char_p
    lib.lily_last_error.argtypes = []
    lib.lily_moe_decode_noalloc.restype = ctypes.c_int
    lib.lily_moe_decode_noalloc.argtypes = [P(LilyMoeDims), P(LilyMoeWeights), ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_calib_mfma.restype = ctypes.c_int
    lib.lily_calib_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_calib_dequant.restype = ctypes.c_int
    lib.lily_calib_dequant.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_calib_read.restype = ctypes.c_int
    lib.lily_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.lily_trace_ffn_items.restype = ctypes.c_int
    lib.lily_trace_ffn_items.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.lily_trace_decode_stack.restype = ctypes.c_int
    lib.lily_trace_decode_stack.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    if path is None:
        _lib = lib
    return lib


# ----------------------------------------------------------------- marshalling

def dims(T: int, H: int, F: int, E: int, topk: int, tile_m: int = 64,
         group: int = 64) -> LilyMoeDims:
    return LilyMoeDims(T, H, F, E, topk, group, tile_m)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, lib: ctypes.CDLL) -> None:
    if rc != LILY_OK:
        raise LilyError(rc, lib.lily_last_error().decode())


@dataclasses.dataclass
class W4:
    """One stacked int4 matrix set on the device in the plain layout (uint8 q,
    int16 bf16 bits); the input of lily_w4_pack."""

    q: torch.Tensor
    scale: torch.Tensor
    bias: torch.Tensor

    def c(self) -> LilyW4:
        return LilyW4(_ptr(self.q), _ptr(self.scale), _ptr(self.bias))


@dataclasses.dataclass
class Weights:
    """The six packed matrix stacks of one layer (uint8 device tensors)."""

    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    sh_gate: torch.Tensor
    sh_up: torch.Tensor
    sh_down: torch.Tensor

    def c(self) -> LilyMoeWeights:
        # device pointers do not change while the tensors live: build once
        if getattr(self, "_c", None) is None:
            self._c = LilyMoeWeights(*(_ptr(getattr(self, n)) for n in WEIGHT_FIELDS))
        return self._c


@dataclasses.dataclass
class Routing:
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pairs: torch.Tensor
    pair_rows: torch.Tensor
    block_expert: torch.Tensor
    block_row0: torch.Tensor
    num_blocks: torch.Tensor
    block_order: torch.Tensor
    sched: torch.Tensor
    block_info: torch.Tensor

    def c(self) -> LilyMoeRouting:
        if getattr(self, "_c", None) is None:
            self._c = LilyMoeRouting(*(_ptr(getattr(self, n)) for n in ROUTING_FIELDS))
        return self._c


def lily_moe_max_blocks(d: LilyMoeDims) -> int:
    lib = load()
    n = lib.lily_moe_max_blocks(ctypes.byref(d))
    _check(min(n, 0), lib)
    return n


def lily_moe_workspace_bytes(d: LilyMoeDims) -> int:
    lib = load()
    n = lib.lily_moe_workspace_bytes(ctypes.byref(d))
    if n == 0:
        raise LilyError(LILY_ERR_INVALID_ARG, lib.lily_last_error().decode())
    return n


def lily_w4_packed_bytes(n: int, N: int, K: int, group: int = 64) -> int:
    lib = load()
    b = lib.lily_w4_packed_bytes(n, N, K, group)
    if b == 0:
        raise LilyError(LILY_ERR_INVALID_ARG, lib.lily_last_error().decode())
    return b


def lily_w4_pack(w: W4, n: int, N: int, K: int, packed, group: int = 64, stream=None) -> None:
    lib = load()
    rc = lib.lily_w4_pack(ctypes.byref(w.c()), n, N, K, group, _ptr(packed), _stream(stream))
    _check(rc, lib)


def lily_moe_router(d: LilyMoeDims, w_router, x, logits, stream=None) -> None:
    """logits fp32 [T, E] = x [T, H] (bf16 bits) times w_router [E, H] (bf16 bits)^T."""
    lib = load()
    rc = lib.lily_moe_router(ctypes.byref(d), _ptr(w_router), _ptr(x), _ptr(logits),
                             _stream(stream))
    _check(rc, lib)


def lily_moe_route(d: LilyMoeDims, logits, routing: Routing, stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_route(ctypes.byref(d), _ptr(logits), ctypes.byref(routing.c()),
                            _stream(stream))
    _check(rc, lib)


def lily_moe_route_host(d: LilyMoeDims, logits, routing: Routing, stream=None) -> None:
    """The CPU-synchronised twin of lily_moe_route (blocks the calling thread)."""
    lib = load()
    rc = lib.lily_moe_route_host(ctypes.byref(d), _ptr(logits), ctypes.byref(routing.c()),
                                 _stream(stream))
    _check(rc, lib)


def lily_moe_forward(d: LilyMoeDims, weights: Weights, x, routing: Routing, out, workspace,
                     workspace_bytes: Optional[int] = None, stream=None) -> None:
    lib = load()
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    rc = lib.lily_moe_forward(ctypes.byref(d), ctypes.byref(weights.c()), _ptr(x),
                              ctypes.byref(routing.c()), _ptr(out), _ptr(workspace),
                              workspace_bytes, _stream(stream))
    _check(rc, lib)


def _ws_bytes(workspace) -> int:
    return workspace.numel() * workspace.element_size()


def lily_moe_dequant(d: LilyMoeDims, packed: Weights, routing: Routing, bf16: Weights,
                     stream=None) -> None:
    """Unfused twin, step 1: bf16 weights of the experts with rows (and the
    shared expert) into the stacks of ``bf16`` (see alloc_bf16_weights)."""
    lib = load()
    rc = lib.lily_moe_dequant(ctypes.byref(d), ctypes.byref(packed.c()), ctypes.byref(routing.c()),
                              ctypes.byref(bf16.c()), _stream(stream))
    _check(rc, lib)


def lily_moe_forward_bf16(d: LilyMoeDims, bf16: Weights, x, routing: Routing, out, workspace,
                          workspace_bytes: Optional[int] = None, stream=None) -> None:
    """Unfused twin, step 2: the forward reading the bf16 stacks."""
    lib = load()
    nbytes = _ws_bytes(workspace) if workspace_bytes is None else workspace_bytes
    rc = lib.lily_moe_forward_bf16(ctypes.byref(d), ctypes.byref(bf16.c()), _ptr(x),
                                   ctypes.byref(routing.c()), _ptr(out), _ptr(workspace), nbytes,
                                   _stream(stream))
    _check(rc, lib)


def alloc_bf16_weights(d: LilyMoeDims, device="cuda") -> Weights:
    """Caller-owned bf16 [n][N][K] stacks for lily_moe_dequant (bf16 bits as
    int16): gate and up [E][F][H], down [E][H][F], the shared ones n = 1."""
    E, H, F = d.E, d.H, d.F
    e16 = dict(dtype=torch.int16, device=device)
    return Weights(gate=torch.empty((E, F, H), **e16), up=torch.empty((E, F, H), **e16),
                   down=torch.empty((E, H, F), **e16), sh_gate=torch.empty((1, F, H), **e16),
                   sh_up=torch.empty((1, F, H), **e16), sh_down=torch.empty((1, H, F), **e16))


def lily_moe_gate_up(d: LilyMoeDims, weights: Weights, x, routing: Routing, workspace,
                     stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_gate_up(ctypes.byref(d), ctypes.byref(weights.c()), _ptr(x),
                              ctypes.byref(routing.c()), _ptr(workspace), _ws_bytes(workspace),
                              _stream(stream))
    _check(rc, lib)


def lily_moe_down(d: LilyMoeDims, weights: Weights, routing: Routing, workspace,
                  stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_down(ctypes.byref(d), ctypes.byref(weights.c()), ctypes.byref(routing.c()),
                           _ptr(workspace), _ws_bytes(workspace), _stream(stream))
    _check(rc, lib)


def lily_moe_ffn(d: LilyMoeDims, weights: Weights, x, routing: Routing, workspace,
                 stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_ffn(ctypes.byref(d), ctypes.byref(weights.c()), _ptr(x),
                          ctypes.byref(routing.c()), _ptr(workspace), _ws_bytes(workspace),
                          _stream(stream))
    _check(rc, lib)


def lily_moe_combine(d: LilyMoeDims, routing: Routing, workspace, out, stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_combine(ctypes.byref(d), ctypes.byref(routing.c()), _ptr(workspace),
                              _ws_bytes(workspace), _ptr(out), _stream(stream))
    _check(rc, lib)


def lily_moe_decode(d: LilyMoeDims, weights: Weights, logits, x, routing: Routing, out, workspace,
                    stream=None) -> None:
    """Route + forward of a few tokens (T <= 4) in one launch."""
    lib = load()
    rc = lib.lily_moe_decode(ctypes.byref(d), ctypes.byref(weights.c()), _ptr(logits), _ptr(x),
                             ctypes.byref(routing.c()), _ptr(out), _ptr(workspace),
                             _ws_bytes(workspace), _stream(stream))
    _check(rc, lib)


def lily_moe_decode_noalloc(d: LilyMoeDims, weights: Weights, logits, x, topk_ids, topk_w, out,
                            status=None, stream=None) -> None:
    lib = load()
    rc = lib.lily_moe_decode_noalloc(ctypes.byref(d), ctypes.byref(weights.c()), _ptr(logits),
                                     _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(out),
                                     _ptr(status), _stream(stream))
    _check(rc, lib)


def layer_table(weights: list, device="cuda") -> torch.Tensor:
    """Device array of lily_moe_weights (six pointers per layer) for
    lily_moe_decode_stack; the Weights objects must outlive it."""
    rows = [[getattr(w, n).data_ptr() for n in WEIGHT_FIELDS] for w in weights]
    return torch.tensor(rows, dtype=torch.int64).to(device)


def lily_moe_decode_stack(d: LilyMoeDims, n_layers: int, layers, logits, x0, r, outs, topk_ids,
                          topk_w, sched, workspace, eps: float = 1e-6, stream=None) -> None:
    """T = 1 decode through n_layers MoE layers in one launch (see the header)."""
    lib = load()
    rc = lib.lily_moe_decode_stack(ctypes.byref(d), n_layers, _ptr(layers), _ptr(logits), _ptr(x0),
                                   _ptr(r), _ptr(outs), _ptr(topk_ids), _ptr(topk_w), _ptr(sched),
                                   eps, _ptr(workspace), _ws_bytes(workspace), _stream(stream))
    _check(rc, lib)


def lily_residual_norm(T: int, H: int, r, out, x_next, eps: float = 1e-6, stream=None) -> None:
    lib = load()
    rc = lib.lily_residual_norm(T, H, _ptr(r), _ptr(out), _ptr(x_next), eps, _stream(stream))
    _check(rc, lib)


def lily_last_error() -> str:
    return load().lily_last_error().decode()


def lily_calib_mfma(grid: int, waves_per_cu: int, iters: int, sink, times, stream=None) -> None:
    lib = load()
    _check(lib.lily_calib_mfma(grid, waves_per_cu, iters, _ptr(sink), _ptr(times),
                               _stream(stream)), lib)


def lily_calib_dequant(grid: int, waves_per_cu: int, iters: int, sink, times, stream=None) -> None:
    lib = load()
    _check(lib.lily_calib_dequant(grid, waves_per_cu, iters, _ptr(sink), _ptr(times),
                                  _stream(stream)), lib)


def lily_calib_read(src, nbytes: int, grid: int, dma: bool, sink, stream=None) -> None:
    lib = load()
    _check(lib.lily_calib_read(_ptr(src), nbytes, grid, 1 if dma else 0, _ptr(sink),
                               _stream(stream)), lib)


def load_trace() -> ctypes.CDLL:
    """Make the tracing build (liblily_moe_trace.so) the library that every
    call of this module goes through; call it before any other call."""
    global _lib
    _lib = load(TRACE_LIB_PATH)
    return _lib


TRACE_SLOTS = 32  # item rows per workgroup in the FFN trace; row 32 is the launch row


def lily_trace_ffn_items(max_wgs: int = 1024, stream=None) -> np.ndarray:
    """The item trace of the last lily_moe_ffn launch (tracing build only):
    uint64 [n][33][4], as lily_trace.h describes."""
    lib = load()
    buf = np.zeros((max_wgs, TRACE_SLOTS + 1, 4), dtype=np.uint64)
    n = lib.lily_trace_ffn_items(buf.ctypes.data_as(ctypes.c_void_p), max_wgs, _stream(stream))
    _check(min(n, 0), lib)
    return buf[:n]


def lily_trace_decode_stack(max_wgs: int = 256, stream=None) -> np.ndarray:
    """The phase trace of the last lily_moe_decode_stack launch (tracing build
    only): uint64 [n][64][8], as lily_trace.h describes."""
    lib = load()
    buf = np.zeros((max_wgs, 64, 8), dtype=np.uint64)
    n = lib.lily_trace_decode_stack(buf.ctypes.data_as(ctypes.c_void_p), max_wgs, _stream(stream))
    _check(min(n, 0), lib)
    return buf[:n]


# ----------------------------------------------------------------- allocation

def alloc_routing(d: LilyMoeDims, device="cuda") -> Routing:
    """Device buffers for one layer's routing (the library allocates nothing)."""
    T, E, k = d.T, d.E, d.topk
    P = T * k
    mb = lily_moe_max_blocks(d)
    i32 = dict(dtype=torch.int32, device=device)
    return Routing(topk_ids=torch.empty((T, k), **i32),
                   topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
                   counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                   sorted_pairs=torch.empty(P, **i32), pair_rows=torch.empty(P, **i32),
                   block_expert=torch.empty(mb, **i32), block_row0=torch.empty(mb, **i32),
                   num_blocks=torch.empty(1, **i32), block_order=torch.empty(mb, **i32),
                   sched=torch.zeros(LILY_SCHED_INTS, **i32),
                   block_info=torch.empty((mb, 4), **i32))


def alloc_workspace(d: LilyMoeDims, device="cuda") -> torch.Tensor:
    return torch.empty(lily_moe_workspace_bytes(d), dtype=torch.uint8, device=device)


def workspace_views(d: LilyMoeDims, ws: torch.Tensor):
    """(h, y) views of a forward workspace, laid out as the library uses it:
    h bf16 bits [P + T, F] at offset 0, y fp32 [P + T, H] at the next
    256-byte boundary (the split-K partials, when present, follow y)."""
    rows = d.T * d.topk + d.T
    hb = rows * d.F * 2
    y0 = (hb + 255) // 256 * 256
    h = ws[:hb].view(torch.int16).view(rows, d.F)
    y = ws[y0:y0 + rows * d.H * 4].view(torch.float32).view(rows, d.H)
    return h, y


def pack_w4(w: W4, n: int, N: int, K: int, stream=None) -> torch.Tensor:
    """Packed copy (uint8 device tensor) of a plain-layout matrix stack."""
    out = torch.empty(lily_w4_packed_bytes(n, N, K), dtype=torch.uint8, device=w.q.device)
    lily_w4_pack(w, n, N, K, out, stream=stream)
    return out


def weights_from_host(lw, device="cuda") -> Weights:
    """Upload a ``synth.LayerWeights`` (numpy, plain layout) and pack it on the
    device; the plain copies are freed once packed."""
    packed = {}
    for name in WEIGHT_FIELDS:
        m = getattr(lw, name)
        n, N, K2 = m.q.shape
        plain = W4(torch.from_numpy(m.q).to(device),
                   torch.from_numpy(m.scale.view("int16")).to(device),
                   torch.from_numpy(m.bias.view("int16")).to(device))
        packed[name] = pack_w4(plain, n, N, 2 * K2)
        torch.cuda.current_stream(packed[name].device).synchronize()
        del plain
    return Weights(**packed)
