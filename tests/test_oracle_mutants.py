"""The oracle's pins are strong enough: each plausible mistake planted in a copy
of the oracle (on the CPU) makes at least one pin fail, and the unmodified copy
passes them all."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import test_oracle_fp16 as t16
import test_oracle_q4 as t4
import test_oracle_q8 as t8
import test_oracle_q8w as t8w
import test_oracle_attn as tat
import test_oracle_pinned as tpn

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "q4_oracle.c")

MUTANTS = [
    ("nibble_halves_swapped",
     "return j < 16 ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);",
     "return j < 16 ? (qs[j] >> 4) : (qs[j - 16] & 0x0f);"),
    ("offset_dropped", "s += (q4_nibble(q4_block, j) - 8) * (int32_t)q[j];",
     "s += (q4_nibble(q4_block, j)) * (int32_t)q[j];"),
    ("offset_sign", "s += (q4_nibble(q4_block, j) - 8) * (int32_t)q[j];",
     "s += (8 - q4_nibble(q4_block, j)) * (int32_t)q[j];"),
    ("round_half_even", "float r = roundf(v);", "float r = nearbyintf(v);"),
    ("round_floor_plus_half", "float r = roundf(v);", "float r = floorf(v + 0.5f);"),
    ("divide_by_fp16_scale", "float v = x[j] / d;",
     "float v = x[j] / q4o_fp16_to_f32(q4o_f32_to_fp16(d));"),
    ("multiply_by_reciprocal", "float v = x[j] / d;", "float v = x[j] * (1.0f / d);"),
    ("scale_from_signed_max", "float a = fabsf(x[j]);", "float a = x[j];"),
    ("scale_255", "float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    ("fp16_encode_truncates", "double r = nearbyint(k);", "double r = floor(k);"),
    ("fp16_encode_ties_away", "double r = nearbyint(k);", "double r = round(k);"),
    ("fp16_subnormal_decode", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("scale_product_drops_dx", "double p = dw * dx;", "double p = dw;"),
    ("accumulate_sign", "acc += t;", "acc -= t;"),
    ("scale_big_endian", "return (uint16_t)(p[0] | (p[1] << 8));",
     "return (uint16_t)(p[1] | (p[0] << 8));"),
    ("activation_row_ignored",
     "gemv_one(w + r * nb * Q4_BLOCK_BYTES, xq8 + (int64_t)t * nb * Q8_BLOCK_BYTES, nb,",
     "gemv_one(w + r * nb * Q4_BLOCK_BYTES, xq8, nb,"),
    ("last_block_dropped", "for (int64_t b = 0; b < nb; ++b) {\n        const uint8_t* wb",
     "for (int64_t b = 0; b + 1 < nb; ++b) {\n        const uint8_t* wb"),
    ("q8w_weights_unsigned", "const int8_t* w = (const int8_t*)(w_block + 2);",
     "const uint8_t* w = (const uint8_t*)(w_block + 2);"),
    ("q8w_scale_drops_dx", "*\n                           (double)q4o_fp16_to_f32(load_u16_le(xb));",
     "*\n                           1.0;"),
    ("q8w_token_ignored",
     "const uint8_t* xb = xq8 + ((int64_t)t * nb + b) * Q8_BLOCK_BYTES;\n                double p",
     "const uint8_t* xb = xq8 + ((int64_t)0 * nb + b) * Q8_BLOCK_BYTES;\n                double p"),
    ("requant_last_tie_wins", "if (fabsf(x[j]) > amax) {", "if (fabsf(x[j]) >= amax) {"),
    ("requant_unsigned_max", "float d = vmax / -8.0f;", "float d = amax / 8.0f;"),
    ("requant_exact_division", "float v = x[j] * id + 8.5f;", "float v = x[j] / d + 8.5f;"),
    ("requant_round_plus_8", "float v = x[j] * id + 8.5f;", "float v = x[j] * id + 8.0f;"),
    ("requant_no_clamp", "nib[j] = n > 15 ? 15 : n;", "nib[j] = n & 15;"),
    ("requant_halves_swapped", "(uint8_t)(nib[j] | (nib[j + 16] << 4));",
     "(uint8_t)(nib[j + 16] | (nib[j] << 4));"),
    ("attn_group_modulo", "int g = h / group;", "int g = h % n_kv;"),
    ("attn_no_max_subtraction", "denom += exp(scale * dot - smax);", "denom += exp(scale * dot);"),
    ("attn_scale_dropped", "double sc = scale * dot;", "double sc = dot;"),
    ("attn_unnormalized", "double p = exp(scale * dot - smax) / denom;", "double p = exp(scale * dot - smax);"),
    ("pinned_one_chain", "if (k < 4)\n                    chain_a", "if (1)\n                    chain_a"),
    ("pinned_even_odd_chains", "if (k < 4)\n                    chain_a", "if (k % 2 == 0)\n                    chain_a"),
    ("pinned_segments_of_8", "(c + 1 - c0) % 16 == 0", "(c + 1 - c0) % 8 == 0"),
    ("pinned_no_segments", "if (c + 1 == c1 || (c + 1 - c0) % 16 == 0)", "if (c + 1 == c1)"),
    ("pinned_split_rounds_up", "const int64_t c0 = s * nc / ks, c1 = (s + 1) * nc / ks;",
     "const int64_t c0 = (s * nc + ks - 1) / ks, c1 = ((s + 1) * nc + ks - 1) / ks;"),
    ("pinned_four_splits_early", "nc <= 8 ? 1 : (nc <= 16 ? 2 : 4)", "nc <= 8 ? 1 : 4"),
    ("pinned_two_splits_late", "nc <= 8 ? 1 : (nc <= 16 ? 2 : 4)", "nc <= 8 ? 1 : (nc <= 32 ? 2 : 4)"),
    ("pinned_splits_pairwise", "y = s == 0 ? total : y + total;", "y = s == 0 ? total : (s == 3 ? y + total : (s == 2 ? total : y + total));"),
    ("pinned_drops_partial_chunk", "for (int64_t k = 0; k < 8 && c * 8 + k < nb; ++k) {",
     "for (int64_t k = 0; k < 8 && c * 8 + k < nb - 1; ++k) {"),
    ("rms_sequential", "p[l] = fmaf(x[i], x[i], p[l]);", "p[0] = fmaf(x[i], x[i], p[0]);"),
    ("rms_lane_stride_64", "const int64_t i = c * 256 + 4 * l + k;", "const int64_t i = c * 256 + l + 64 * k;"),
    ("rms_reverse_tree", "for (int d = 32; d >= 1; d /= 2) {", "for (int d = 1; d <= 32; d *= 2) {"),
    ("rms_epsilon", "sqrtf(ss / (float)n + 1e-6f)", "sqrtf(ss / (float)n + 1e-5f)"),
    ("rms_no_mean", "sqrtf(ss / (float)n + 1e-6f)", "sqrtf(ss + 1e-6f)"),
    ("chain_o_reads_k", "chain_gemv(lw[3], E, E, q, xq, o);", "chain_gemv(lw[3], E, E, k, xq, o);"),
    ("chain_no_attention_residual", "h1[i] = h[i] + o[i];", "h1[i] = o[i];"),
    ("chain_gate_only", "prod[i] = g[i] * u[i];", "prod[i] = g[i];"),
    ("chain_qkv_unnormed", "q4o_rmsnorm(h, E, nrm);\n        chain_gemv(lw[0], E, E, nrm, xq, q);",
     "memcpy(nrm, h, (size_t)E * sizeof(float));\n        chain_gemv(lw[0], E, E, nrm, xq, q);"),
    ("chain_mlp_reads_h", "q4o_rmsnorm(h1, E, nrm);", "q4o_rmsnorm(h, E, nrm);"),
    ("chain_mlp_residual_from_h", "h2[i] = h1[i] + dn[i];", "h2[i] = h[i] + dn[i];"),
    ("chain_head_unnormed", "q4o_rmsnorm(h, E, nrm);\n    chain_gemv(w[7 * layers], V, E, nrm, xq, logits);",
     "chain_gemv(w[7 * layers], V, E, h, xq, logits);"),
]


def _pins(o, b):
    """Run the oracle's pins; return the names of those that fail."""
    checks = [("fp16_exhaustive", lambda: t16.test_fp16_decode_exhaustive(o)),
              ("fp16_ties", lambda: t16.test_fp16_encode_every_tie_and_neighbour(o)),
              ("fp16_specials", lambda: t16.test_fp16_encode_specials(o)),
              ("q8_properties", lambda: t8.test_q8_0_properties_random(o)),
              ("q8_near_ties", lambda: t8.test_q8_0_near_ties(o)),
              ("sum_fold_brute", lambda: t4.test_block_sums_fold_identity_and_brute_force(o)),
              ("gemv_golden", lambda: t4.test_gemv_golden_small(o)),
              ("gemv_zero", lambda: t4.test_gemv_all_eight_nibbles_is_exact_zero(o)),
              ("gemv_one_hot", lambda: t4.test_gemv_one_hot_activation_closed_form(o)),
              ("gemv_brute_a", lambda: t4.test_gemv_matches_fp64_bruteforce(o, b, 17, 288, 8)),
              ("gemv_brute_b", lambda: t4.test_gemv_matches_fp64_bruteforce(o, b, 70, 96, 1)),
              ("q8w_golden", lambda: t8w.test_q8w_gemv_golden(o)),
              ("q8w_sums_brute", lambda: t8w.test_q8w_block_sums_brute_force(o)),
              ("q8w_brute", lambda: t8w.test_q8w_gemv_matches_fp64_bruteforce(o, b, 17, 288, 8)),
              ("q8w_unit", lambda: t8w.test_q8w_gemv_unit_weights_closed_form(o)),
              ("requant_round_trip", lambda: t8w.test_requant_round_trips_q4_0_blocks(o)),
              ("requant_nearest", lambda: t8w.test_requant_rounds_to_nearest_level(o)),
              ("attn_golden", lambda: tat.test_attn_golden(o)),
              ("attn_one_position", lambda: tat.test_attn_single_position_returns_v(o)),
              ("attn_equal_keys", lambda: tat.test_attn_equal_keys_average_values(o)),
              ("attn_dominant", lambda: tat.test_attn_one_dominant_key_closed_form(o)),
              ("attn_large", lambda: tat.test_attn_large_scores_stay_finite(o)),
              ("attn_gqa", lambda: tat.test_attn_gqa_groups(o)),
              ("attn_brute", lambda: tat.test_attn_matches_bruteforce(o, 7, 12, 2, 128)),
              ("pinned_exact", lambda: tpn.test_pinned_exact_with_unit_scales(o, 9, 4608, 1)),
              ("pinned_bound", lambda: tpn.test_pinned_within_fp32_bound_of_fp64(o, 40, 800, 3)),
              ("rms_golden", lambda: tpn.test_rmsnorm_order_golden(o)),
              ("rms_closed_form", lambda: tpn.test_rmsnorm_constant_vector_closed_form(o, 3.0, 128)),
              ("rms_closed_form_small", lambda: tpn.test_rmsnorm_constant_vector_closed_form(o, 1e-4, 3584)),
              ("chain_unquantized", lambda: tpn.test_chain_matches_unquantized_fp64(o, b)),
              ("chain_one_gemv", lambda: tpn.test_chain_without_residual_branches_is_one_gemv(o))]
    checks += [(f"pinned_golden_{c['name']}", (lambda c=c: tpn.test_pinned_order_golden(o, c)))
               for c in tpn.CASES]
    checks += [(f"q8_golden_{c['name']}", (lambda c=c: t8.test_q8_0_golden_blocks(o, c)))
               for c in t8.CASES]
    checks += [(f"q4_golden_{c['name']}", (lambda c=c: t4.test_q4_0_golden_decode(o, c)))
               for c in t4.Q4_CASES]
    checks += [(f"sum_golden_{c['name']}", (lambda c=c: t4.test_block_sum_golden(o, c)))
               for c in t4.SUM_CASES]
    checks += [(f"requant_golden_{c['name']}", (lambda c=c: t8w.test_requant_golden(o, c)))
               for c in t8w.RQ_CASES]
    failed = []
    with np.errstate(all="ignore"):
        for name, fn in checks:
            try:
                fn()
            except AssertionError:
                failed.append(name)
    return failed


def _build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation site for {name} not unique"
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                    str(so), str(c), "-lm"], check=True)
    return str(so)


def test_unmodified_copy_passes_all_pins(oracle, bruteforce, tmp_path):
    so = _build_variant(tmp_path, "control", None, None)
    with oracle.using(so):
        assert _pins(oracle, bruteforce) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(oracle, bruteforce, tmp_path, name, old, new):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    so = _build_variant(tmp_path, name, old, new)
    with oracle.using(so):
        failed = _pins(oracle, bruteforce)
    assert failed, f"mutant {name} survived every pin"
