"""Planted mistakes: each pin set must reject a wrong oracle (CPU only).

Every case copies attn_oracle.c, plants one plausible slip (a dropped term,
a wrong sign or index, a mis-masked key, a wrong head map), compiles the copy
with the same flags, binds it with ``oracle.from_library`` and runs the pins
of test_oracle_fwd.py / test_oracle_bwd.py against it.  At least one pin must
fail for every mutant; the unmodified source must pass them all.
"""
import os
import shutil

import pytest

import oracle
import test_oracle_blockmask as pm
import test_oracle_bwd as pb
import test_oracle_fwd as pf
import test_oracle_varlen as pv

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

# (name, text to replace, replacement, expected number of occurrences)
MUTANTS = [
    ("exp_sign", "double w = exp(scores[j] - m);", "double w = exp(scores[j] + m);", 1),
    ("drop_normalise", "for (int c = 0; c < dv; ++c) orow[c] /= l;", "", 1),
    ("drop_scale", "scores[j] = scale * dot(qi, Kh + j * dk, dk);",
     "scores[j] = dot(qi, Kh + j * dk, dk);", 1),
    ("causal_excludes_diagonal", "const int64_t n = i + 1 + off;", "const int64_t n = i + off;", 1),
    ("causal_one_extra_key", "const int64_t n = i + 1 + off;", "const int64_t n = i + 2 + off;", 1),
    ("gqa_modulo_map", "const int64_t g = h / group;", "const int64_t g = h % Hkv;", 8),
    ("key_index_slip", "scores[j] = scale * dot(qi, Kh + j * dk, dk);",
     "scores[j] = scale * dot(qi, Kh + j, dk);", 1),
    ("value_transposed", "const double* vj = Vh + j * dv;", "const double* vj = Vh + j;", 1),
    ("lse_drops_max", "*lse = m + log(l);", "*lse = log(l);", 1),
    ("merge_no_rescale", "ua[c] = fa * ua[c] + fb * u_blk[c];", "ua[c] = ua[c] + fb * u_blk[c];", 1),
    ("merge_wrong_max", "const double m_new = (m_a > m_b) ? m_a : m_b;",
     "const double m_new = (m_a > m_b) ? m_b : m_a;", 1),
    ("bwd_ds_sign", "const double ds = p * (dp - dsum[r]);", "const double ds = p * (dp + dsum[r]);", 2),
    ("bwd_dk_no_scale", "for (int c = 0; c < dk; ++c) dkj[c] *= scale;", "", 1),
    ("bwd_dq_no_scale", "for (int c = 0; c < dk; ++c) dqi[c] *= scale;", "", 1),
    ("bwd_dv_uses_ds", "for (int c = 0; c < dv; ++c) dvj[c] += p * doi[c];",
     "for (int c = 0; c < dv; ++c) dvj[c] += ds * doi[c];", 1),
    ("bwd_dsum_drops", "dsum[r] = dot(dout + r * dv, obuf + r * dv, dv);", "dsum[r] = 0.0;", 1),
    ("bottom_right_offset_sign", "const int64_t off = (int64_t)Nk - Nq;",
     "const int64_t off = (int64_t)Nq - Nk;", 1),
    ("bwd_dk_skips_group", "for (int64_t hh = 0; hh < group; ++hh) {",
     "for (int64_t hh = 0; hh < 1; ++hh) {", 1),
    ("blockmask_inverted", "if (!mrow[j / bn]) continue;", "if (mrow[j / bn]) continue;", 1),
    ("blockmask_head_zero", "const int64_t hm = (mask_heads == 1) ? 0 : h;",
     "const int64_t hm = 0;", 1),
    ("blockmask_ignores_causal", "if (causal && j > i) continue;", "", 1),
    ("varlen_sequence_boundary", "while (cu[s + 1] <= t) ++s;", "while (cu[s + 1] < t) ++s;", 1),
    ("varlen_global_position", "visible_keys(i, len, causal)", "visible_keys(t, len, causal)", 1),
    ("varlen_kv_offset_dropped", "const double* Kh = k + (g * T + start) * dk;",
     "const double* Kh = k + (g * T) * dk;", 1),
]


def run_pins(om):
    """Run the pin set against oracle `om`; return the names of pins that failed."""
    pins = [
        ("worked_example_page_check", lambda: pf.test_worked_example_page_check(om)),
        ("worked_example_library", lambda: pf.test_worked_example_vs_library_softmax(om)),
        ("single_key", lambda: pf.test_single_key_returns_its_value(om)),
        ("two_keys", lambda: pf.test_two_keys_is_a_sigmoid_mix(om)),
        ("uniform_causal", lambda: pf.test_uniform_weights_closed_form(om, True, "zero_q")),
        ("uniform", lambda: pf.test_uniform_weights_closed_form(om, False, "zero_scale")),
        ("probabilities", lambda: pf.test_identity_values_expose_probabilities(om, False)),
        ("probabilities_causal", lambda: pf.test_identity_values_expose_probabilities(om, True)),
        ("gqa", lambda: pf.test_gqa_equals_mha_with_repeated_kv(om, True)),
        ("heads", lambda: pf.test_batches_and_heads_are_independent(om, True)),
        ("blockwise", lambda: pf.test_blockwise_equals_dense(om, True, 13, 7, 3, 2)),
        ("blockwise_nc", lambda: pf.test_blockwise_equals_dense(om, False, 7, 13, 2, 3)),
        ("blockwise_extreme", lambda: pf.test_blockwise_survives_extreme_logits(om, False)),
        ("bottom_right", lambda: pf.test_bottom_right_is_top_left_on_the_suffix(om, 3, 9)),
        ("bottom_right_long", lambda: pf.test_bottom_right_is_top_left_on_the_suffix(om, 12, 5)),
        ("fd", lambda: pb.test_gradients_match_central_differences(om, True, pb.SHAPES[3])),
        ("autograd", lambda: pb.test_gradients_match_torch_autograd(
            om, True, (1, 3, 1, 9, 12, 5, 7))),
        ("sums", lambda: pb.test_gradient_sum_identities(om, False)),
        ("blockmask_full", lambda: pm.test_full_mask_is_the_dense_forward(om, True, 13, 4, 3)),
        ("blockmask_scipy", lambda: pm.test_matches_scipy_on_the_expanded_mask(om, False, 1)),
        ("blockmask_heads", lambda: pm.test_per_head_masks_act_head_by_head(om)),
        ("varlen_scipy", lambda: pv.test_matches_scipy_with_a_document_mask(om, True, [5, 1, 9])),
        ("varlen_single", lambda: pv.test_single_sequence_is_the_dense_forward(om, True)),
    ]
    failed = []
    for name, fn in pins:
        try:
            fn()
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    return failed


def build_variant(tmp_path, name, old, new, count):
    src = open(SRC).read()
    assert src.count(old) == count, f"{name}: pattern found {src.count(old)} times"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    oracle.compile_source(str(path), str(lib))
    return oracle.from_library(str(lib))


def test_unmodified_copy_passes_every_pin(tmp_path):
    lib = tmp_path / "libclean.so"
    shutil.copy(SRC, tmp_path / "clean.c")
    oracle.compile_source(str(tmp_path / "clean.c"), str(lib))
    assert run_pins(oracle.from_library(str(lib))) == []


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, count):
    om = build_variant(tmp_path, name, old, new, count)
    failed = run_pins(om)
    assert failed, f"mutant {name} passed every pin"
