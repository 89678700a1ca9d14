"""Mutation tests: plant each mistake the explainer's CPU-lab section asks about into a
copy of the oracle (dropping alpha on the old numerator, dropping the scale, turning the
causal <= into <), and a few plausible backward and mask/bias-variant mistakes, rebuild
it, and require at least one pin to fail."""
import os

import pytest

import oracle as oracle_pkg
import oracle_checks as oc

MUTANTS = {
    "drop_alpha_on_numerator": ("o_row[c] = alpha * o_row[c] + pv;", "o_row[c] = o_row[c] + pv;"),
    "drop_scale": ("double s = p->scale * acc;", "double s = acc;"),
    "causal_strict": ("p->causal && !(j <= diag)", "p->causal && !(j < diag)"),
    # backward: the scale left out of dQ, D left out of dS, dS in place of P for dV,
    # dK with the wrong sign
    "bwd_drop_scale_dq": ("dq[q_index(&P, b, i, h, c)] = scale * acc;",
                          "dq[q_index(&P, b, i, h, c)] = acc;"),
    "bwd_ds_without_D": ("ds[j] = prob[j] * (dp - dsum_i);", "ds[j] = prob[j] * dp;"),
    "bwd_dv_uses_ds": ("dv[x] += prob[j] * doc;", "dv[x] += ds[j] * doc;"),
    "bwd_dk_sign": ("dk[x] += scale * ds[j] * qc;", "dk[x] -= scale * ds[j] * qc;"),
    # mask and bias variants: window bounds off by one or mirrored, ALiBi with the wrong
    # sign, without the absolute value or with the kv head's slope, the soft cap without
    # its outer factor or applied before the scale
    "window_left_inclusive": ("j < diag - p->window_left", "j <= diag - p->window_left"),
    "window_right_mirrored": ("j > diag + p->window_right", "j > diag - p->window_right"),
    "alibi_sign": ("s -= p->alibi[", "s += p->alibi["),
    "alibi_no_abs": ("* fabs(dist);", "* dist;"),
    "alibi_kv_head_slope": ("p->alibi[(int64_t)b * p->Hq + h]",
                            "p->alibi[(int64_t)b * p->Hq + kv_head(p, h)]"),
    "softcap_no_outer_factor": ("s = p->softcap * tanh(s / p->softcap);",
                                "s = tanh(s / p->softcap);"),
    "softcap_before_scale": ("double s = p->scale * acc;\n  if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);",
                             "double s = acc;\n  if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);\n  s *= p->scale;"),
    # FP8: exponent bias 8, ties away from zero, the scale of the fnuz format (max 240),
    # 64-row scale blocks when dequantizing, a missing butterfly stage, swapped butterfly
    "e4m3_bias_8": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_ties_away": ("(err == best_err && (c & 1) == 0)", "(err == best_err && 0)"),
    "fp8_scale_240": ("amax / 448.0f", "amax / 240.0f"),
    "fp8_dequant_block_64": ("scales[((int64_t)b * H + h) * nblk + r / 128]",
                             "scales[((int64_t)b * H + h) * nblk + r / 64 % nblk]"),
    "fwht_missing_stage": ("for (int h = 1; h < d; h *= 2)", "for (int h = 2; h < d; h *= 2)"),
    "fwht_swapped_pair": ("y[i] = a + b;\n          y[i + h] = a - b;",
                          "y[i] = a - b;\n          y[i + h] = a + b;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle_pkg.SOURCE).read()
    assert src.count(old) == 1, f"anchor for {name} not found exactly once"
    mut_src = tmp_path / f"oracle_{name}.c"
    mut_src.write_text(src.replace(old, new))
    lib = str(tmp_path / f"liboracle_{name}.so")
    oracle_pkg.build(src=str(mut_src), out=lib)
    failed = oc.failing_checks(oracle_pkg.Oracle(lib))
    assert failed, f"mutant {name} passed every check"


def test_unmutated_oracle_passes_all(oracle):
    assert oc.failing_checks(oracle) == []
