"""Helpers for the GPU tests: upload seeded inputs and run the layer through
the C ABI (``int4_grouped_gemm_amd``), and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import int4_grouped_gemm_amd as L

ROUTE_KEYS = ("topk_ids", "counts", "offsets", "sorted_pairs", "pair_rows")


def to_dev_bits(a: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> int16 tensor on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def from_dev_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def route_gpu(d: L.LilyMoeDims, logits: np.ndarray, device="cuda"):
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(device)
    r = L.alloc_routing(d, device)
    L.lily_moe_route(d, lg, r)
    torch.cuda.synchronize()
    return r


def routing_to_host(r: L.Routing) -> dict:
    out = {n: getattr(r, n).cpu().numpy() for n in L.ROUTING_FIELDS}
    nb = int(out["num_blocks"][0])
    for key in ("block_expert", "block_row0", "block_order", "block_info"):
        out[key] = out[key][:nb]
    return out


def expected_block_order(ref: dict, tile_m: int) -> np.ndarray:
    """The GEMM schedule the header documents, from a block map: the full
    blocks in block order, then the partial blocks (each expert's last) by
    descending class ceil(4 rows / tile_m), ties in expert order."""
    nb = int(ref["num_blocks"][0])
    be = np.asarray(ref["block_expert"][:nb])
    rows = np.minimum(tile_m, np.asarray(ref["offsets"])[be + 1] - np.asarray(ref["block_row0"][:nb]))
    full = [b for b in range(nb) if rows[b] == tile_m]
    part = sorted((b for b in range(nb) if rows[b] < tile_m),
                  key=lambda b: (-((4 * int(rows[b]) + tile_m - 1) // tile_m), int(be[b])))
    return np.array(full + part, np.int32)


def compare_routing(gpu: dict, ref: dict, tile_m: int = None) -> None:
    for k in ROUTE_KEYS:
        assert np.array_equal(gpu[k], ref[k]), f"routing {k} differs at " \
            f"{np.argwhere(np.asarray(gpu[k]) != np.asarray(ref[k]))[:5].tolist()}"
    assert int(gpu["num_blocks"][0]) == int(ref["num_blocks"][0]), "num_blocks"
    assert np.array_equal(gpu["block_expert"], ref["block_expert"]), "block_expert"
    assert np.array_equal(gpu["block_row0"], ref["block_row0"]), "block_row0"
    assert np.max(np.abs(gpu["topk_w"] - ref["topk_w"])) <= 2e-6, "topk_w"
    if tile_m is not None:
        want = expected_block_order(ref, tile_m)
        assert np.array_equal(gpu["block_order"], want), "block_order"
        be, br0 = np.asarray(ref["block_expert"]), np.asarray(ref["block_row0"])
        rows = np.minimum(tile_m, np.asarray(ref["offsets"])[be[want] + 1] - br0[want])
        info = np.stack([be[want], br0[want], rows, want], axis=1).astype(np.int32)
        assert np.array_equal(gpu["block_info"].reshape(-1, 4), info.reshape(-1, 4)), "block_info"
        assert not np.any(gpu["sched"]), "route must leave the GEMM queue counters zero"


def forward_gpu(d: L.LilyMoeDims, w: L.Weights, x: torch.Tensor, r: L.Routing,
                poison: bool = True, device="cuda") -> torch.Tensor:
    ws = L.alloc_workspace(d, device)
    if poison:  # NaN in every byte pattern: reads of unwritten workspace show up
        ws.fill_(0xFF)
    out = torch.empty((d.T, d.H), dtype=torch.int16, device=device)
    out.fill_(-1)
    L.lily_moe_forward(d, w, x, r, out, ws)
    torch.cuda.synchronize()
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def output_error(gpu_bits: np.ndarray, ref_acc: np.ndarray) -> float:
    """max over elements of |gpu - ref| / (1e-2 * (|ref| + RMS(ref))): <= 1 passes."""
    g = bf16_bits_to_f64(gpu_bits)
    ref = ref_acc.astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref) / (1e-2 * (np.abs(ref) + rms))))
