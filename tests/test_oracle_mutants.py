"""Plant plausible mistakes in copies of the oracle source (on the CPU) and check that
the pins catch every one. A mutant that no pin catches would mean the oracle could
carry that mistake unnoticed."""
import os
import tempfile

import pytest

import oracle
import oracle_pins as P

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "qsa_oracle.c")).read()

# (name, text in the oracle source, replacement). Leaving the sink out of the running
# maximum is not listed: softmax is shift-invariant, so that change is an equivalent
# mutant (it only matters once exp overflows, where both results round to zero).
MUTANTS = [
    ("page_from_slot", "p / c->page_size]", "p % c->page_size]"),
    ("slot_from_page", "int64_t slot = p % c->page_size;", "int64_t slot = p / c->page_size;"),
    ("kv_head_dropped", "* c->num_kv_heads + g)", "* c->num_kv_heads + 0)"),
    ("layer_dropped", "(plane * c->num_layers + layer)", "(plane * c->num_layers + 0)"),
    ("page_stride_ignored", "c->page_stride == -1 ? packed : c->page_stride", "packed"),
    ("scale_dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("exp_sign_flipped", "double w = exp(s[j] - m);", "double w = exp(m - s[j]);"),
    ("value_is_key", "out[d] += w * V[j * D + d];", "out[d] += w * K[j * D + d];"),
    ("q_reversed", "qv[d] = elem(q, dt, (r * Hq + h) * D + d);",
     "qv[d] = elem(q, dt, (r * Hq + h) * D + (D - 1 - d));"),
    ("v_from_k_plane", "gather_row(&c, b, p, 1, layer_idx, g, V + j * D)",
     "gather_row(&c, b, p, 0, layer_idx, g, V + j * D)"),
    ("counts_ignored", "int64_t n = counts[r] < W ? counts[r] : W;", "int64_t n = W;"),
    ("counts_off_by_one", "int64_t n = counts[r] < W ? counts[r] : W;",
     "int64_t n = counts[r] < W ? counts[r] - 1 : W;"),
    ("causal_clip_off_by_one", "if (p > pos)", "if (p >= pos)"),
    ("window_off_by_one", "pos - window + 1 > 0 ? pos - window + 1 : 0", "pos - window > 0 ? pos - window : 0"),
    ("sink_dropped", "double z = exp(sink - m);", "double z = 0.0;"),
    ("unused_slot_zero_skipped", "if (e >= 0)", "if (e > 0)"),
    ("bf16_shift", "(uint32_t)h << 16", "(uint32_t)h << 15"),
    ("e4m3_bias", "ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 9)"),
    ("e4m3_subnormal", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("normalise_dropped", "out[d] /= z;", "out[d] /= 1.0;"),
    ("max_not_subtracted_consistently", "z += w;", "z += w * 1.0000001;"),
    ("dense_causal_off_by_one", "int64_t hi = causal ? t : len - 1;", "int64_t hi = causal ? t - 1 : len - 1;"),
    ("dense_mask_ignored", "int64_t hi = causal ? t : len - 1;", "int64_t hi = len - 1;"),
    ("dense_window_off_by_one", "t - window + 1 > 0 ? t - window + 1 : 0", "t - window > 0 ? t - window : 0"),
    ("dense_other_sequence", "K[j * D + d] = elem(k, dt, ((start + lo + j) * Hkv + g) * D + d);",
     "K[j * D + d] = elem(k, dt, ((lo + j) * Hkv + g) * D + d);"),
    ("dense_kv_head_dropped", "V[j * D + d] = elem(v, dt, ((start + lo + j) * Hkv + g) * D + d);",
     "V[j * D + d] = elem(v, dt, ((start + lo + j) * Hkv + 0) * D + d);"),
    ("compress_sum_not_mean", "x[d] /= (double)ratio;", "x[d] /= 1.0;"),
    ("compress_partial_group_kept", "key_counts[b] / ratio : 0", "(key_counts[b] + ratio - 1) / ratio : 0"),
    ("compress_eps_dropped", "sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)D)"),
    ("compress_rms_divisor", "sqrt(ss / (double)D + (double)eps)", "sqrt(ss / (double)(D - 1) + (double)eps)"),
    ("compress_gamma_dropped", "x[d] = elem(gamma, dt, d) * x[d] * inv;", "x[d] = x[d] * inv;"),
    ("compress_rotation_sign", "o[2 * i] = cs * x[2 * i] - sn * x[2 * i + 1];",
     "o[2 * i] = cs * x[2 * i] + sn * x[2 * i + 1];"),
    ("compress_rotation_position_is_block", "int64_t p = j * ratio;", "int64_t p = j;"),
    ("compress_rotation_past_rotary_dim", "2 * i + 1 < rotary_dim; ++i)", "2 * i + 1 < D; ++i)"),
    ("compress_cos_sin_swapped", "double cs = elem(freqs, fdt, p * rotary_dim + 2 * i);",
     "double cs = elem(freqs, fdt, p * rotary_dim + 2 * i + 1);"),
    ("select_ties_reversed", "return x->j < y->j ? -1 : x->j > y->j;", "return x->j > y->j ? -1 : x->j < y->j;"),
    ("select_candidates_off_by_one", "int64_t nfull = (pos + 1) / ratio;", "int64_t nfull = pos / ratio;"),
    ("select_tail_short", "for (int64_t p = nfull * ratio; p <= pos; ++p)", "for (int64_t p = nfull * ratio; p < pos; ++p)"),
    ("select_not_ascending", "qsort(kept, (size_t)k, sizeof(int64_t), cmp_i64);", "(void)cmp_i64;"),
    ("select_lowest_scores", "sc[j].s = s;", "sc[j].s = -s;"),
    ("select_wrong_sequence", "elem(block_keys, dt, (b * max_blocks + j) * D + d)", "elem(block_keys, dt, j * D + d)"),
    ("compress_last_block_dropped", "for (int64_t j = 0; j < max_blocks; ++j) {",
     "for (int64_t j = 0; j < max_blocks - 1; ++j) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    assert SRC.count(old) >= 1, "mutation site vanished: " + old
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(SRC.replace(old, new))
    lib = oracle.load(oracle.compile_source(str(src), str(tmp_path / ("mut_%s.so" % name))))
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            return
    pytest.fail("no pin caught the planted mistake " + name)
