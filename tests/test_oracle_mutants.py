"""Plant plausible mistakes in a copy of the oracle; each must trip a pin.

Each mutant is a textual edit of ``oracle/z1_oracle.c`` compiled with the
oracle's own gcc flags into a temporary library.  A mutant that passes every
pin would mean the pins cannot tell that mistake from the correct oracle.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "plan_extra_to_rank_eq_rho": [("len[i] = q + (rank < rho ? 1 : 0);",
                                   "len[i] = q + (rank <= rho ? 1 : 0);")],
    "plan_start_max": [("start[i] = (int64_t)rank * q + (rank < rho ? rank : rho);",
                        "start[i] = (int64_t)rank * q + (rank < rho ? rho : rank);")],
    "plan_extra_to_last_ranks": [
        ("len[i] = q + (rank < rho ? 1 : 0);",
         "len[i] = q + (dp_size - 1 - rank < rho ? 1 : 0);"),
        ("start[i] = (int64_t)rank * q + (rank < rho ? rank : rho);",
         "start[i] = (int64_t)rank * q + (rank > dp_size - rho ? rank - (dp_size - rho) : 0);")],
    "flat_extra_to_last": [("int64_t lo = (int64_t)rank * q + (rank < rho ? rank : rho);",
                            "int64_t lo = (int64_t)rank * q + (rank > rho ? rank - rho : 0);"),
                           ("int64_t hi = lo + q + (rank < rho ? 1 : 0);",
                            "int64_t hi = lo + q + (rank >= dp_size - rho ? 1 : 0);")],
    "flat_off_by_one": [("int64_t b = hi < base + numel[i] ? hi : base + numel[i];",
                         "int64_t b = hi <= base + numel[i] ? hi : base + numel[i] - 1;")],
    "dim0_floor_rows": [("int64_t per = (rows[i] + dp_size - 1) / dp_size;",
                         "int64_t per = rows[i] / dp_size;")],
    "seg_lr_scale_ignored": [("const double lr = hp->lr * (n_seg > 0 ? lr_scale[j] : 1.0);",
                              "const double lr = hp->lr;")],
    "seg_wd_scale_ignored": [("const double wd = hp->weight_decay * (n_seg > 0 ? wd_scale[j] : 1.0);",
                              "const double wd = hp->weight_decay;")],
    "lr_warmup_off_by_one": [("return lr_max * (double)t / (double)warmup;",
                              "return lr_max * (double)(t - 1) / (double)warmup;")],
    "lr_cosine_sign": [("(1.0 + cos(M_PI * tau))", "(1.0 - cos(M_PI * tau))")],
    "lr_linear_wrong_end": [("return lr_max + (lr_min - lr_max) * tau;", "return lr_max - lr_max * tau;")],
    "pack_divide_by_dp_minus_1": [("out[o++] = divide ? x / (float)dp_size : x;",
                                   "out[o++] = divide ? x / (float)(dp_size > 1 ? dp_size - 1 : 1) : x;")],
    "pack_multiply_reciprocal": [("out[o++] = divide ? x / (float)dp_size : x;",
                                  "out[o++] = divide ? x * (1.0f / (float)dp_size) : x;")],
    "pack_wrong_base": [("                out[o++] = divide ? x / (float)dp_size : x;\n            }\n            base += numel[i];",
                         "                out[o++] = divide ? x / (float)dp_size : x;\n            }\n            base += ln;")],
    "rne_ties_away": [("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)")],
    "rne_truncate": [("kept += 1u;", "kept += 0u;")],
    "rne_nan_not_quieted": [("| 0x0040u", "| 0x0000u"),
                            ("(u & 0x007FFFFFu) != 0)", "(u & 0x007FFFFFu) != 0 && 0)")],
    "acc_in_double": [("float a = bf16_to_f32(g[e]);", "double a = bf16_to_f32(g[e]);")],
    "acc_drops_first": [("float a = bf16_to_f32(g[e]);", "float a = 0.0f;")],
    "acc_drops_last": [("for (int32_t k = 1; k < K; ++k)", "for (int32_t k = 1; k < K - 1; ++k)")],
    "norm_no_square": [("double x = a * a;", "double x = a;")],
    "norm_in_float": [("double t = s + x;", "double t = (float)(s + x);")],
    "norm_uncompensated": [("return isfinite(s) ? s + err : s;", "return s;")],
    "clip_no_eps": [("double c = clip / (sqrt(S) + 1e-6);", "double c = clip / sqrt(S);")],
    "clip_no_min": [("return c >= 1.0 ? 1.0 : c;", "return c;")],
    "norm_inf_becomes_nan": [("return isfinite(s) ? s + err : s;", "return s + err;")],
    "clip_nan_means_no_clip": [("return c >= 1.0 ? 1.0 : c;", "return c < 1.0 ? c : 1.0;")],
    "clip_uses_S": [("double c = clip / (sqrt(S) + 1e-6);", "double c = clip / (S + 1e-6);")],
    "adamw_decay_without_lr": [("(1.0 - lr * wd)", "(1.0 - wd)")],
    "adamw_decay_after_update": [
        ("pe = pe * (1.0 - lr * wd);", ""),
        ("pe = pe - lr * mhat / (sqrt(vhat) + hp->eps);",
         "pe = (pe - lr * mhat / (sqrt(vhat) + hp->eps)) * (1.0 - lr * wd);")],
    "adamw_l2_not_decoupled": [("pe = pe * (1.0 - lr * wd);", "g = g + wd * pe;")],
    "adamw_beta_swap_m": [("me = hp->beta1 * me + (1.0 - hp->beta1) * g;",
                           "me = hp->beta2 * me + (1.0 - hp->beta2) * g;")],
    "adamw_beta_swap_v": [("ve = hp->beta2 * ve + (1.0 - hp->beta2) * g * g;",
                           "ve = hp->beta1 * ve + (1.0 - hp->beta1) * g * g;")],
    "adamw_eps_inside_sqrt": [("(sqrt(vhat) + hp->eps)", "sqrt(vhat + hp->eps)")],
    "adamw_no_bias_correction_v": [("double vhat = ve / bc2;", "double vhat = ve;")],
    "adamw_no_bias_correction_m": [("double mhat = me / bc1;", "double mhat = me;")],
    "adamw_bias_power_off_by_one": [("pow(hp->beta1, t)", "pow(hp->beta1, t + 1.0)")],
    "adamw_update_sign": [("pe = pe - lr * mhat", "pe = pe + lr * mhat")],
    "adamw_ignores_clip": [("double g = c * (double)acc[e];", "double g = (double)acc[e];")],
    "adamw_weight_from_old_master": [("w[e] = z1o_bf16_rne(p[e]);",
                                      "w[e] = z1o_bf16_rne((float)(double)acc[e] * 0.0f + p[e] * 0.999f);")],
    "adamw_bias2_power_off_by_one": [("pow(hp->beta2, t)", "pow(hp->beta2, t + 1.0)")],
    "adamw_t_from_zero": [("const double t = (double)hp->step;",
                           "const double t = (double)(hp->step - 1);")],
    "adamw_v_not_squared": [("(1.0 - hp->beta2) * g * g;", "(1.0 - hp->beta2) * g;")],
    "adamw_v_unclipped": [("(1.0 - hp->beta2) * g * g;",
                           "(1.0 - hp->beta2) * (double)acc[e] * (double)acc[e];")],
    "acc_mean_not_sum": [("acc[e] = a;", "acc[e] = a / (float)K;")],
    "lr_decay_from_zero": [("int64_t d = t - (warmup > 0 ? warmup : 0);", "int64_t d = t;")],
    "rne_saturates": [("kept += 1u;", "kept += ((kept & 0x7FFFu) == 0x7F7Fu) ? 0u : 1u;")],
    "rne_inf_becomes_nan": [("if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)",
                             "if ((u & 0x7F800000u) == 0x7F800000u)")],
    "clip_eps_inside_sqrt": [("double c = clip / (sqrt(S) + 1e-6);",
                              "double c = clip / sqrt(S + 1e-6);")],
    "norm_square_in_float": [("double x = a * a;", "double x = (double)((float)a * (float)a);")],
    # fp32 stores of the new state rounded toward minus infinity, not to nearest
    "master_store_floor": [("p[e] = (float)pe;",
                            "p[e] = (float)pe; if ((double)p[e] > pe) p[e] = nextafterf(p[e], -INFINITY);")],
    "m_store_floor": [("m[e] = (float)me;",
                       "m[e] = (float)me; if ((double)m[e] > me) m[e] = nextafterf(m[e], -INFINITY);")],
    "v_store_floor": [("v[e] = (float)ve;",
                       "v[e] = (float)ve; if ((double)v[e] > ve) v[e] = nextafterf(v[e], -INFINITY);")],
    "clip_g_in_float": [("double g = c * (double)acc[e];",
                         "double g = (double)(float)(c * (double)acc[e]);")],
    "bias_corrections_in_float": [
        ("const double bc1 = 1.0 - pow(hp->beta1, t);",
         "const double bc1 = (double)(1.0f - powf((float)hp->beta1, (float)t));"),
        ("const double bc2 = 1.0 - pow(hp->beta2, t);",
         "const double bc2 = (double)(1.0f - powf((float)hp->beta2, (float)t));")],
    "acc_reverse_order": [("float a = bf16_to_f32(g[e]);",
                           "float a = bf16_to_f32(g[(int64_t)(K - 1) * L + e]);"),
                          ("float gk = bf16_to_f32(g[(int64_t)k * L + e]);",
                           "float gk = bf16_to_f32(g[(int64_t)(K - 1 - k) * L + e]);")],
    "lr_warmup_plus_one": [("return lr_max * (double)t / (double)warmup;",
                            "return lr_max * (double)t / (double)(warmup + 1);")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SOURCE).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor must occur exactly once: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    lib = oracle.build(str(path), str(tmp_path / f"lib{name}.so"))
    o = oracle.Oracle(lib)
    caught = []
    for check in pins.ALL:
        try:
            check(o)
        except (AssertionError, ValueError) as e:
            caught.append(check.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
