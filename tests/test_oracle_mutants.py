"""Planted mistakes in the oracle must each fail at least one pin (no GPU).

Each mutant is a copy of oracle/convt_oracle.c with one textual change (a
plausible mistake: flipped kernel, wrong padding sign, transposed weight
operand, dropped bias, ...), compiled into a temporary directory with gcc.
The real oracle is never modified.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "flip_kernel": ("(double)wc[co_l * k_sp + (kd * KH + kh) * KW + kw]",
                    "(double)wc[co_l * k_sp + ((KD - 1 - kd) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)]"),
    "pad_sign_w": ("iw * P->s[2] - P->p[2] + kw * P->d[2]", "iw * P->s[2] + P->p[2] + kw * P->d[2]"),
    "stride_dilation_swapped": ("iw * P->s[2] - P->p[2] + kw * P->d[2]",
                                "iw * P->d[2] - P->p[2] + kw * P->s[2]"),
    "dilation_dropped": ("iw * P->s[2] - P->p[2] + kw * P->d[2]", "iw * P->s[2] - P->p[2] + kw"),
    "depth_axis_pad_dropped": ("id * P->s[0] - P->p[0] + kd * P->d[0]", "id * P->s[0] + kd * P->d[0]"),
    "closed_form_half_pad": ("return (L_in - 1) * s - 2 * p + d * (K - 1) + op + 1;",
                             "return (L_in - 1) * s - p + d * (K - 1) + op + 1;"),
    "closed_form_no_outpad": ("return (L_in - 1) * s - 2 * p + d * (K - 1) + op + 1;",
                              "return (L_in - 1) * s - 2 * p + d * (K - 1) + 1;"),
    "bias_dropped": ("double b = J->bias ? (double)J->bias[g * Cog + co_l] : 0.0;", "double b = 0.0;"),
    "bias_wrong_channel": ("double b = J->bias ? (double)J->bias[g * Cog + co_l] : 0.0;",
                           "double b = J->bias ? (double)J->bias[co_l] : 0.0;"),
    "group_input_channel": ("const int64_t ci = g * Cig + ci_l;\n        const float *xc = J->x",
                            "const int64_t ci = ci_l;\n        const float *xc = J->x"),
    "weight_transposed": ("const double wv = (double)wc[co_l * k_sp + (kd * KH + kh) * KW + kw];",
                          "const double wv = (double)J->w[((g * Cog + co_l) * Cig + ci_l) * k_sp"
                          " + (kd * KH + kh) * KW + kw];"),
    "epilogue_plain_hardswish": ("return t * hardswish(t);", "return hardswish(t);"),
    "epilogue_no_upper_clamp": ("if (r > 6.0) r = 6.0;", ""),
    "epilogue_add_dropped": ("            if (J->add) t += (double)J->add[yi];\n", ""),
    # selectable epilogue
    "hardswish_scale": ("return t * r / 6.0;", "return t * r / 3.0;"),
    "act_modes_swapped": ("if (act == 1) return hardswish(t);", "if (act == 1) return times_hardswish(t);"),
    "act_before_add": ("            if (J->add) t += (double)J->add[yi];\n            J->y[yi] = activate(t, J->act);",
                       "            t = activate(t, J->act);\n            if (J->add) t += (double)J->add[yi];\n"
                       "            J->y[yi] = t;"),
    "points_act_dropped": ("        out[t] = activate(acc, act);", "        out[t] = acc;"),
    # channels last
    "channels_last_x_stride": ("const int64_t xs = J->layout ? P->C_in : 1;", "const int64_t xs = 1;"),
    "channels_last_y_index": ("return layout ? (n * sp + e) * C + c : (n * C + c) * sp + e;",
                              "return layout ? (n * sp + e) * C + (C - 1 - c) : (n * C + c) * sp + e;"),
    "points_channels_last_decoded_first": (
        "        if (layout) { co = e % C_out; e /= C_out; }\n        o[2] = e % P.L_out[2]; e /= P.L_out[2];\n"
        "        o[1] = e % P.L_out[1]; e /= P.L_out[1];\n        o[0] = e % P.L_out[0]; e /= P.L_out[0];\n"
        "        if (!layout) { co = e % C_out; e /= C_out; }",
        "        o[2] = e % P.L_out[2]; e /= P.L_out[2];\n        o[1] = e % P.L_out[1]; e /= P.L_out[1];\n"
        "        o[0] = e % P.L_out[0]; e /= P.L_out[0];\n        co = e % C_out; e /= C_out;"),
    "points_pad_sign": ("if (i * s - p + k * d == o)", "if (i * s + p + k * d == o)"),
    # input gradient
    "bwd_pad_sign_w": ("iw * P->s[2] + kw * P->d[2] - P->p[2]", "iw * P->s[2] + kw * P->d[2] + P->p[2]"),
    "bwd_flip_kernel": ("(double)wci[((co_l * KD + kd) * KH + kh) * KW + kw]",
                        "(double)wci[((co_l * KD + (KD - 1 - kd)) * KH + (KH - 1 - kh)) * KW + (KW - 1 - kw)]"),
    "bwd_group_output_channel": ("J->dy + (n * P->C_out + g * Cog + co_l) * out_sp",
                                 "J->dy + (n * P->C_out + co_l) * out_sp"),
    "bwd_stride_dilation_swapped": ("ih * P->s[1] + kh * P->d[1] - P->p[1]",
                                    "ih * P->d[1] + kh * P->s[1] - P->p[1]"),
    # weight and bias gradients
    "wgrad_pad_sign_w": ("kw * P->d[2] + iw * P->s[2] - P->p[2]", "kw * P->d[2] + iw * P->s[2] + P->p[2]"),
    "wgrad_group_output_channel": ("J->dy + (n * P->C_out + (g * Cog + co_l)) * out_sp;",
                                   "J->dy + (n * P->C_out + (co_l)) * out_sp;"),
    "wgrad_batch_dropped": ("for (int64_t n = 0; n < P->N; ++n) {", "for (int64_t n = 0; n < 1; ++n) {"),
    "bgrad_first_sample_only": ("for (int64_t n = 0; n < N; ++n)\n", "for (int64_t n = 0; n < 1; ++n)\n"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = os.path.join(tmp_path, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(mpath, os.path.join(tmp_path, "libmutant.so"), extra_flags=["-w"])
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # any pin that does not pass counts
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
