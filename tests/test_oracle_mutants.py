"""The pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/oracle.c``, plants one mistake by a textual edit
(on the CPU, in a temporary directory), builds the copy with gcc and runs the
pins of ``pins.py`` on it. At least one pin must fail. Every planted mistake
keeps memory accesses in bounds.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pins

MUTANTS = {
    "nibble_order": ("(kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
                     "(kk % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "group_index": ("int g = kk / GROUP;", "int g = kk / GROUP / 2;"),
    "scale_bias_swapped": ("fmaf(s, (float)nib, b)", "fmaf(b, (float)nib, s)"),
    "weight_not_rounded": ("    return round_bf16(w);\n}", "    return w;\n}"),
    "bf16_ties_not_even": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
                           "if (rest >= 0x8000u) keep += 1u;"),
    "bf16_truncates": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
                       "(void)rest;"),
    "tie_to_higher_index": ("return ea < eb;", "return ea > eb;"),
    "softmax_not_normalised": ("topk_w[(size_t)t * k + j] = ex[j] / sum;",
                               "topk_w[(size_t)t * k + j] = ex[j];"),
    "softmax_without_max": ("ex[j] = expf(l[topk_ids[(size_t)t * k + j]] - lmax);",
                            "ex[j] = expf(l[topk_ids[(size_t)t * k + j]] - lmax * 0.5f);"),
    "softmax_over_all_experts": ("            sum += ex[j];\n",
                                 "            sum += ex[j];\n            if (j == k - 1)\n"
                                 "                for (int e2 = 0; e2 < E; ++e2)\n"
                                 "                    if (!taken[e2]) sum += expf(l[e2] - lmax);\n"),
    "scatter_unstable": ("    for (int p = 0; p < P; ++p) {\n        int e = topk_ids[p];\n        int row",
                         "    for (int p = P - 1; p >= 0; --p) {\n        int e = topk_ids[p];\n        int row"),
    "block_row_relative": ("block_row0[nb] = r0;", "block_row0[nb] = r0 - offsets[e];"),
    "h_not_rounded": ("hbuf[f] = round_bf16(silu(g) * u);", "hbuf[f] = silu(g) * u;"),
    "silu_sign": ("return z / (1.0f + expf(-z));", "return z / (1.0f + expf(z));"),
    "gate_up_swapped": ("hbuf[f] = round_bf16(silu(g) * u);", "hbuf[f] = round_bf16(silu(u) * g);"),
    "shared_expert_dropped": ("for (int n = 0; n < H; ++n) acc[n] = y[n];",
                              "for (int n = 0; n < H; ++n) acc[n] = 0.0f * y[n];"),
    "down_transposed": ("acc = acc + hbuf[f] * wd[(size_t)n * F + f];",
                        "acc = acc + hbuf[f] * wd[(size_t)f * H + n];"),
    "routing_weight_slot": ("float w = topk_w[(size_t)t * k + j];",
                            "float w = topk_w[(size_t)t * k];"),
    "final_not_rounded_rne": ("out_bf16[(size_t)i * H + n] = float_to_bf16(acc[n]);",
                              "out_bf16[(size_t)i * H + n] = (uint16_t)(((union {float f; uint32_t u;}){acc[n]}).u >> 16);"),
    "router_weight_transposed": ("(double)bf16_to_float(w[(size_t)e * H + h]);",
                                 "(double)bf16_to_float(w[(size_t)h * E + e]);"),
    "router_abs_signed": ("mag += fabs(p);", "mag += p;"),
    "router_float_sum": ("            double acc = 0.0, mag = 0.0;",
                         "            float acc = 0.0f; double mag = 0.0;"),
    "rmsnorm_mean": ("float inv = 1.0f / sqrtf(ss / (float)H + eps);",
                     "float inv = 1.0f / sqrtf(ss + eps);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src.replace(old, new))
    so = obuild.build(str(path), str(tmp_path / f"liboracle_{name}.so"))
    lib = oracle.load(so)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError) as e:  # noqa: PERF203
            failed.append((pin.__name__, str(e)[:80]))
            break
    assert failed, f"no pin caught the planted mistake {name!r}"
