"""Planted mistakes in the oracle (CPU only): each mutant is a copy of oracle.c with one
plausible error (a dropped term, a wrong sign or index, a transposed operand), built
into a temporary library.  Every mutant must fail at least one pin of oracle_pins.py,
which shows the pins tie each part of the oracle down."""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins as P

# (name, old text, new text, occurrence index of `old` to replace)
MUTANTS = [
    ("fwd_pad_sign", "i64 ih = oh * sh - ph + kh;", "i64 ih = oh * sh + ph + kh;", 0),
    ("fwd_kh_kw_swapped", "const double* wp = w + ((oc * KH + kh) * KW + kw) * IC;",
     "const double* wp = w + ((oc * KH + kw) * KW + kh) * IC;", 0),
    ("fwd_bias_dropped", "double acc = b ? b[oc] : 0.0;", "double acc = 0.0;", 0),
    ("fwd_stride_ignored_w", "i64 iw = ow * sw - pw + kw;", "i64 iw = ow - pw + kw;", 0),
    ("fwd_upper_bound", "if (ih < 0 || ih >= H) continue;", "if (ih < 0 || ih > H) continue;", 0),
    ("extent_ceil", "return span / s + 1;", "return (span + s - 1) / s + 1;", 0),
    ("bn_unbiased_var", "double v = q / (double)M;", "double v = q / (double)(M - 1);", 0),
    ("bn_eps_outside_sqrt", "inv_std[c] = 1.0 / sqrt(v + eps);", "inv_std[c] = 1.0 / (sqrt(v) + eps);", 0),
    ("bn_momentum_swapped", "running_mean[c] = (1.0 - momentum) * running_mean[c] + momentum * mu;",
     "running_mean[c] = momentum * running_mean[c] + (1.0 - momentum) * mu;", 0),
    ("bn_running_var_uses_mean", "running_var[c] = (1.0 - momentum) * running_var[c] + momentum * v;",
     "running_var[c] = (1.0 - momentum) * running_var[c] + momentum * mu;", 0),
    ("apply_beta_dropped", "a = gamma[c] * ((a - mean[c]) * inv_std[c]) + beta[c];",
     "a = gamma[c] * ((a - mean[c]) * inv_std[c]);", 0),
    ("tanh_slope", "double t = tanh(a); return 1.0 - t * t;", "double t = tanh(a); return 1.0 - t;", 0),
    ("sigmoid_sign", "case ACT_SIGMOID: return 1.0 / (1.0 + exp(-a));",
     "case ACT_SIGMOID: return 1.0 / (1.0 + exp(a));", 0),
    ("relu_slope_at_negative", "case ACT_RELU: return a > 0.0 ? 1.0 : 0.0;",
     "case ACT_RELU: return a > 0.0 ? 1.0 : 0.1;", 0),
    ("bnbwd_term_dropped", "dz[i] = is / (double)M * ((double)M * dzh - s1 - zh * s2);",
     "dz[i] = is / (double)M * ((double)M * dzh - s1);", 0),
    ("bnbwd_sign", "dz[i] = is / (double)M * ((double)M * dzh - s1 - zh * s2);",
     "dz[i] = is / (double)M * ((double)M * dzh + s1 - zh * s2);", 0),
    ("bnbwd_gamma_missing", "double dzh = dno * g;", "double dzh = dno;", 0),
    ("bnbwd_dgamma_no_zhat", "sg += dno * zh;", "sg += dno;", 0),
    ("bnbwd_mask_at_z", "double dno = act_slope(act, a) * dy[i];", "double dno = act_slope(act, z[i]) * dy[i];", 0),
    ("bnbwd_dz_mask_at_z", "double dzh = act_slope(act, a) * dy[i] * g;", "double dzh = act_slope(act, z[i]) * dy[i] * g;",
     0),
    ("bneval_mask_at_z", "double dno = act_slope(act, a) * dy[i];", "double dno = act_slope(act, z[i]) * dy[i];", 1),
    ("dx_flipped_kernel", "const double* wp = w + ((oc * KH + kh) * KW + kw) * IC;",
     "const double* wp = w + ((oc * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)) * IC;", 1),
    ("dx_pad_sign", "i64 ih = oh * sh - ph + kh;", "i64 ih = oh * sh + ph - kh;", 1),
    ("dx_at_stride_check", "if (th < 0 || th % sh != 0 || th / sh >= OH) continue;",
     "if (th < 0 || th / sh >= OH) continue;", 0),
    ("dw_row_offset", "double* rp = row + (kh * KW + kw) * IC;", "double* rp = row + (kw * KW + kh) * IC;", 0),
    ("dw_bias_dropped_term", "bsum += g;", "bsum += g * g;", 0),
    ("dw_at_tap_sign", "i64 ih = oh * sh - ph + kh;", "i64 ih = oh * sh - ph - kh;", 3),
    ("bias_grad_square", "for (i64 m = 0; m < M; ++m) s += dz[m * C + c];",
     "for (i64 m = 0; m < M; ++m) s += dz[m * C + c] * dz[m * C + c];", 0),
    ("bneval_eps_dropped", "inv_std[c] = 1.0 / sqrt(running_var[c] + eps);",
     "inv_std[c] = 1.0 / sqrt(running_var[c]);", 0),
    ("bneval_inv_std_missing", "dz[i] = dno * g * is;", "dz[i] = dno * g;", 0),
    ("bneval_dgamma_no_zhat", "sg += dno * zh;", "sg += dno;", 1),
    ("outform_tanh", "else if (act == ACT_TANH) s = 1.0 - v * v;", "else if (act == ACT_TANH) s = 1.0 - v;", 0),
    ("outform_sigmoid", "else if (act == ACT_SIGMOID) s = v * (1.0 - v);", "else if (act == ACT_SIGMOID) s = v * (1.0 + v);", 0),
    ("outform_relu_mask", "if (act == ACT_RELU) s = v > 0.0 ? 1.0 : 0.0;", "if (act == ACT_RELU) s = v >= 0.0 ? 1.0 : 0.0;", 0),
    ("gelu_value_cubic_dropped", "(a + GELU_K1 * a * a * a)", "(a)", 0),
    ("gelu_slope_cubic_factor", "(1.0 + 3.0 * GELU_K1 * a * a)", "(1.0 + GELU_K1 * a * a)", 0),
    ("gelu_slope_half_dropped", "return 0.5 * (1.0 + t) + 0.5 * a", "return (1.0 + t) + 0.5 * a", 0),
    ("gelu_slope_sech_sign", "0.5 * a * (1.0 - t * t) * du", "0.5 * a * (1.0 + t * t) * du", 0),
    ("gn_count_all_channels", "const double cnt = (double)(S * cg);", "const double cnt = (double)(S * C);", 0),
    ("gn_var_unbiased", "double v = q / cnt;", "double v = q / (cnt - 1.0);", 0),
    ("gn_group_of_channel", "i64 i = (n * S + p) * C + c, st = n * G + c / cg;",
     "i64 i = (n * S + p) * C + c, st = n * G + c % G;", 0),
    ("gn_apply_beta_dropped", "double a = gamma[c] * ((z[i] - mean[st]) * inv_std[st]) + beta[c];",
     "double a = gamma[c] * ((z[i] - mean[st]) * inv_std[st]);", 0),
    ("gn_bwd_count", "const double cnt = (double)(S * cg);", "const double cnt = (double)S;", 1),
    ("gn_bwd_term_dropped", "dz[i] = is / cnt * (cnt * dzh - s1 - zh * s2);", "dz[i] = is / cnt * (cnt * dzh - s1);", 0),
    ("gn_bwd_gamma_dropped", "double dzh = act_slope(act, gamma[c] * zh + beta[c]) * dy[i] * gamma[c];",
     "double dzh = act_slope(act, gamma[c] * zh + beta[c]) * dy[i];", 0),
    ("gn_bwd_dgamma_no_zhat", "sg += dno * zh;\n                sb += dno;", "sg += dno;\n                sb += dno;", 0),
    ("gn_bwd_mask_at_z", "double dno = act_slope(act, gamma[c] * zh + beta[c]) * dy[i];",
     "double dno = act_slope(act, z[i]) * dy[i];", 0),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"mutation anchor not found: {old!r} #{n}"
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, nth):
    src = open(obuild.SRC).read()
    mutated = _replace_nth(src, old, new, nth)
    assert mutated != src
    c_path = os.path.join(tmp_path, "oracle_mutant.c")
    so_path = os.path.join(tmp_path, "liboracle_mutant.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", so_path, c_path, "-lm"], check=True)
    failed = []
    with oracle.using(so_path):
        for pin in P.ALL_PINS:
            try:
                pin()
            except Exception:  # a wrong value, or a wrong shape the pin trips over
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
