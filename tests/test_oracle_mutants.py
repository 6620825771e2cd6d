"""CPU: plant one plausible mistake at a time in a copy of the oracle's C
source, build it, and check that at least one pin fails.  This shows the pins
are strong enough to catch a dropped term, a wrong sign or index, a transposed
operand, a wrong rounding rule or a swapped scale -- the kinds of mistake an
oracle written from prose could contain.  The real oracle is never modified."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import pins
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("bf16_ties_away", "lower > 0x8000u ||", "lower >= 0x8000u ||"),
    ("bf16_truncate", "upper += 1u;", "upper += 0u;"),
    ("e4m3_ties_away", "double r = nearbyint(n);", "double r = floor(n + 0.5);"),
    ("e4m3_truncate", "double r = nearbyint(n);", "double r = floor(n);"),
    ("e4m3_decode_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("e4m3_subnormal_spacing", "quantum = ldexp(1.0, -9);", "quantum = ldexp(1.0, -10);"),
    ("e4m3_no_saturation", "if (a >= 464.0) return (uint8_t)(sign | 0x7E);",
     "if (a >= 464.0) return (uint8_t)(sign | 0x7F);"),
    ("e4m3_lost_sign", "uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = v < 0 ? 0x80 : 0x00;"),
    ("rank_map_modulo", "is_token_in_rank[t * R + e / El] = 1;", "is_token_in_rank[t * R + e % R] = 1;"),
    ("rank_count_from_experts", "num_tokens_per_rank[r] += is_token_in_rank[t * R + r];",
     "num_tokens_per_rank[r] += is_token_in_rank[t * R + r] + (t == 0);"),
    ("pos_off_by_one", "int32_t rank_in_expert = ce[e]++;", "int32_t rank_in_expert = ++ce[e] - (e == 0);"),
    ("expert_offsets_inclusive", "expert_offsets[e + 1] = expert_offsets[e] + num_tokens_per_expert[e];",
     "expert_offsets[e + 1] = expert_offsets[e] + num_tokens_per_expert[e] + (e == 1);"),
    ("send_order_reversed", "sp = rank_offsets[r] + cr[r]++;",
     "sp = rank_offsets[r + 1] - 1 - cr[r]++;"),
    ("ll_slot_without_source", "(int64_t)s0 * M + rank_in_expert", "rank_in_expert"),
    ("ll_window_ignored", "if (rank_in_expert < M) pl =", "if (rank_in_expert < M + 1000000) pl ="),
    ("quant_scale_swapped", "float s = 448.0f / ap;", "float s = ap / 448.0f;"),
    ("quant_no_floor", "float ap = a > 1e-4f ? a : 1e-4f;", "float ap = a;"),
    ("quant_amax_signed", "float v = fabsf(orc_bf16_to_f32(x[b * 128 + i]));",
     "float v = orc_bf16_to_f32(x[b * 128 + i]);"),
    ("quant_stored_scale_inverse", "scales[b] = sinv;", "scales[b] = s;"),
    ("quant_block_shift", "float prod = orc_bf16_to_f32(x[b * 128 + i]) * s;",
     "float prod = orc_bf16_to_f32(x[b * 128 + (i + 1) % 128]) * s;"),
    ("combine_weights_transposed", "float prod = w[t * k + j] * orc_bf16_to_f32(y",
     "float prod = w[(j * T + t) % (T * k)] * orc_bf16_to_f32(y"),
    ("combine_wrong_sign", "acc = acc + prod;", "acc = acc - prod;"),
    ("combine_dropped_term", "for (int j = 0; j < k; j++) {\n                int32_t p = pos[t * k + j];\n"
     "                if (p < 0) continue;",
     "for (int j = 1; j < k; j++) {\n                int32_t p = pos[t * k + j];\n"
     "                if (p < 0) continue;"),
    ("combine_start_not_zero", "float acc = 0.0f;\n            for (int j = 0; j < k; j++) {\n"
     "                int32_t p = pos[t * k + j];\n                if (p < 0)",
     "float acc = 1e-3f;\n            for (int j = 0; j < k; j++) {\n"
     "                int32_t p = pos[t * k + j];\n                if (p < 0)"),
    ("dispatch_bwd_dropped_term", "if (p >= 0) acc = acc + orc_bf16_to_f32(g[",
     "if (p >= 0 && j > 0) acc = acc + orc_bf16_to_f32(g["),
    ("dispatch_bwd_wrong_sign", "acc = acc + orc_bf16_to_f32(g[", "acc = acc - orc_bf16_to_f32(g["),
    ("dispatch_bwd_token_row", "orc_bf16_to_f32(g[(int64_t)p * H + h])", "orc_bf16_to_f32(g[(int64_t)t * H + h])"),
    ("dispatch_bwd_start_not_zero", "float acc = 0.0f;\n            for (int j = 0; j < k; j++) {\n"
     "                int32_t p = pos[t * k + j];\n                if (p >= 0)",
     "float acc = 1e-3f;\n            for (int j = 0; j < k; j++) {\n"
     "                int32_t p = pos[t * k + j];\n                if (p >= 0)"),
    ("combine_bwd_no_weight", "float prod = w[t * k + j] * gv;", "float prod = gv;"),
    ("combine_bwd_weight_transposed", "float prod = w[t * k + j] * gv;",
     "float prod = w[(j * T + t) % (T * k)] * gv;"),
    ("combine_bwd_grad_y_truncated", "grad_y[(int64_t)p * H + h] = orc_f32_to_bf16(prod);",
     "grad_y[(int64_t)p * H + h] = (uint16_t)(f32_bits(prod) >> 16);"),
    ("combine_bwd_grad_w_weighted", "dot += (double)gv * (double)orc_bf16_to_f32(y[",
     "dot += (double)prod * (double)orc_bf16_to_f32(y["),
    ("combine_bwd_grad_w_shifted", "(double)orc_bf16_to_f32(y[(int64_t)p * H + h]);",
     "(double)orc_bf16_to_f32(y[(int64_t)p * H + (h + 1) % H]);"),
    ("combine_bwd_grad_w_float", "double dot = 0.0;", "float dot = 0.0f;"),
    ("combine_bwd_empty_slot", "grad_w[t * k + j] = 0.0;", "grad_w[t * k + j] = -1.0;"),
    ("dispatch_wrong_source", "const uint16_t* xr = x + (int64_t)src[i] * H;",
     "const uint16_t* xr = x + (int64_t)src[n - 1 - i] * H;"),
]


def _mutant_module(tmpdir, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not unique: %s" % name
    src = os.path.join(tmpdir, "mut_%s.c" % name)
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    import oracle.build as ob
    lib = ob.build(src=src, lib=os.path.join(tmpdir, "libmut_%s.so" % name))
    spec = importlib.util.spec_from_file_location(
        "oracle_mutant_" + name, os.path.join(ROOT, "oracle", "__init__.py"),
        submodule_search_locations=[os.path.join(ROOT, "oracle")])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    mod._lib = mod._bind(lib)
    return mod


def run_all_pins(orc):
    """A compact pass over every pin family; raises AssertionError on the
    first disagreement."""
    pins.check_e4m3_decode(orc)
    pins.check_e4m3_encode(orc)
    pins.check_bf16_codec(orc)
    rng = np.random.Generator(np.random.PCG64(2))
    idx = W.route_uniform(rng, 70, 32, 4)
    pins.check_layout_and_positions(orc, idx, 32, 4)
    pins.check_layout_and_positions(orc, W.with_empty_slots(idx, 0.25), 32, 4, M=80, s0=2)
    pins.check_tiny_brute(orc, W.make("tiny")["topk_idx"], 8, 2)
    pins.check_layout_and_positions(orc, pins.repeated_expert_routing(40, 4, 8, rng), 8, 2, M=40, s0=1)
    f = np.zeros((3, 256), np.float32)
    f[1] = np.linspace(-3, 1, 256)
    f[2] = np.exp2(np.arange(256) % 30 - 25.0)
    xb = np.concatenate([W.make("decode", T=8)["x"][:, :256], W.to_bf16_bits(f)])
    pins.check_quant_invariants(orc, xb)
    d = W.make("skewed", T=64)
    c = d["cfg"]
    for q in (0, 1):
        pins.check_dispatch_rows(orc, d["x"][:, :256] if q else d["x"], d["topk_idx"], c["E"], c["R"], q)
    lay = orc.layout(d["topk_idx"], c["E"], c["R"])
    pp = orc.positions(d["topk_idx"], c["E"], c["R"], lay)
    y = W.expert_outputs(d, pp["n_pairs"])
    pins.check_combine(orc, y, d["topk_weights"], pp["pos"])
    pins.check_identity_roundtrip(orc, d["x"], d["topk_idx"], d["topk_weights"], c["E"], c["R"])
    g = W.grad_rows(d, pp["n_pairs"])
    pins.check_dispatch_backward_bound(orc, g, pp["pos"])
    pins.check_dispatch_backward_adjoint(orc, W.with_empty_slots(idx, 0.25), 32, 4, rng)
    go = W.grad_rows(d, 64)
    pins.check_combine_backward_bounds(orc, go, d["topk_weights"], y, pp["pos"])
    pins.check_combine_backward_closed_form(orc, rng)
    pins.check_backward_finite_differences(orc, rng)


def test_real_oracle_passes_compact_pins(orc):
    run_all_pins(orc)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    mod = _mutant_module(str(tmp_path), name, old, new)
    with pytest.raises(AssertionError):
        run_all_pins(mod)
