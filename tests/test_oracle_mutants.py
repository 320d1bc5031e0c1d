"""The pins are strong enough: each plausible slip planted in a copy of the
oracle's C source (a dropped term, a wrong sign, a swapped index, a transposed
operand, the state read after instead of before its update) makes at least one
pin fail.  A slip in an expression that the source writes more than once (the
decay of a token, the head's static decay logit) is planted at every place it
is written.  Mutants are built from a temporary copy on the CPU; the oracle
itself is never modified."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P

MUTANTS = {
    "rwkv4_decay_sign": ("double decay = exp(-(double)w[c]);",
                         "double decay = exp((double)w[c]);"),
    "rwkv4_no_bonus": ("double cur = exp(bonus + kt);", "double cur = exp(kt);"),
    "rwkv4_no_decay_num": ("num = decay * num + ek * vt;", "num = num + ek * vt;"),
    "rwkv4_den_drops_k": ("den = decay * den + ek;", "den = decay * den + 1.0;"),
    "rwkv4_den_drops_current": ("y[idx] = (num + cur * vt) / (den + cur);",
                                "y[idx] = (num + cur * vt) / (den + 1.0);"),
    "rwkv4_output_after_update": (
        "y[idx] = (num + cur * vt) / (den + cur);",
        "y[idx] = (decay * num + exp(kt) * vt + cur * vt) / "
        "(decay * den + exp(kt) + cur);"),
    "matrix_decay_sign": ("wt[i] = exp(-exp((double)xt[i]));",
                          "wt[i] = exp(-exp(-(double)xt[i]));"),
    "matrix_bonus_drops_u": (
        "ruk += (double)rt[i] * (double)uh[i] * (double)kt[i];",
        "ruk += (double)rt[i] * (double)kt[i];"),
    "matrix_state_transposed_in_output": ("acc += (double)rt[i] * S[i * N + j];",
                                          "acc += (double)rt[i] * S[j * N + i];"),
    "matrix_decay_on_value_channel": ("S[i * N + j] = wt[i] * S[i * N + j]",
                                      "S[i * N + j] = wt[j] * S[i * N + j]"),
    "matrix_outer_product_transposed": (
        "+ (double)kt[i] * (double)vt[j];", "+ (double)kt[j] * (double)vt[i];"),
    "matrix_bonus_times_k": ("o[base + j] = acc + ruk * (double)vt[j];",
                             "o[base + j] = acc + ruk * (double)kt[j];"),
    "matrix_output_after_update": (
        "acc += (double)rt[i] * S[i * N + j];",
        "acc += (double)rt[i] * (wt[i] * S[i * N + j] + (double)kt[i] * (double)vt[j]);"),
    "matrix_static_decay_wrong_head": (
        "const float *xt = x_per_token ? x + base : x + h * N;",
        "const float *xt = x_per_token ? x + base : x + ((h + 1) % H) * N;"),
    "matrix_state_in_ignores_batch": ("S[i] = s_in ? s_in[(b * H + h) * N * N + i] : 0.0;",
                                      "S[i] = s_in ? s_in[h * N * N + i] : 0.0;"),
    # backward
    "bwd_dr_drops_bonus": ("d_r[base + i] = ar + (double)uh[i] * (double)kt[i] * dbeta;",
                           "d_r[base + i] = ar;"),
    "bwd_dk_bonus_uses_k": ("d_k[base + i] = ak + (double)uh[i] * (double)rt[i] * dbeta;",
                            "d_k[base + i] = ak + (double)uh[i] * (double)kt[i] * dbeta;"),
    "bwd_dv_drops_beta": ("d_v[base + j] = av + beta * dot[j];", "d_v[base + j] = av;"),
    "bwd_dx_sign": ("double dx = aw * wt[i] * (-exp((double)xt[i]));",
                    "double dx = aw * wt[i] * exp((double)xt[i]);"),
    "bwd_dx_drops_w": ("double dx = aw * wt[i] * (-exp((double)xt[i]));",
                       "double dx = aw * (-exp((double)xt[i]));"),
    "bwd_dS_not_decayed": ("dS[i * N + j] = wt[i] * dS[i * N + j] + (double)rt[i] * dot[j];",
                           "dS[i * N + j] = dS[i * N + j] + (double)rt[i] * dot[j];"),
    "bwd_dS_outer_transposed": (
        "dS[i * N + j] = wt[i] * dS[i * N + j] + (double)rt[i] * dot[j];",
        "dS[i * N + j] = wt[i] * dS[i * N + j] + (double)rt[j] * dot[i];"),
    "bwd_dw_drops_state": ("aw += dS[i * N + j] * Sp[i * N + j];", "aw += dS[i * N + j];"),
    "bwd_dr_reads_gradient_state": ("ar += dot[j] * Sp[i * N + j];",
                                    "ar += dot[j] * dS[i * N + j];"),
    "bwd_dv_transposed": ("av += dS[i * N + j] * (double)kt[i];",
                          "av += dS[j * N + i] * (double)kt[i];"),
    "bwd_du_drops_r": ("pu[unit * N + i] += (double)rt[i] * (double)kt[i] * dbeta;",
                       "pu[unit * N + i] += (double)kt[i] * dbeta;"),
    "bwd_checkpoint_only_first": ("if (t % CK == 0)\n", "if (t == 0)\n"),
    "ng_unbiased_variance": ("var /= (double)N;", "var /= (double)(N - 1);"),
    "ng_drops_eps": ("double rstd = 1.0 / sqrt(var + eps);", "double rstd = 1.0 / sqrt(var);"),
    "ng_sigmoid_gate": ("double silu = gi / (1.0 + exp(-gi));", "double silu = 1.0 / (1.0 + exp(-gi));"),
    "ng_no_centering": ("double n = (ou[i] - mean) * rstd", "double n = ou[i] * rstd"),
    "ng_bias_wrong_head": ("(double)ln_b[h * N + i];", "(double)ln_b[((h + 1) % H) * N + i];"),
    # decay producer
    "dl_shift_sign": ("dx[i] = prev - (double)xt[i];", "dx[i] = (double)xt[i] - prev;"),
    "dl_lerp_drops_mu": ("y[i] = (double)xt[i] + dx[i] * (double)mu_x[i];",
                         "y[i] = (double)xt[i];"),
    "dl_ignores_shift_row": ("(shift ? (double)shift[b * D + i] : 0.0)", "(shift ? 0.0 : 0.0)"),
    "dl_first_shift_late": ("double prev = t > 0 ?", "double prev = t > 1 ?"),
    "dl_mix_drops_lam": ("double m = (double)lam[i];", "double m = 0.0;"),
    "dl_mix_not_scaled_by_dx": ("z[i] = (double)xt[i] + dx[i] * m;", "z[i] = (double)xt[i] + m;"),
    "dl_mix_lora_drops_hidden": ("m += h1[j] * (double)B1[j * D + i];", "m += (double)B1[j * D + i];"),
    "dl_mix_lora_rank_permuted": ("s += y[i] * (double)A1[i * R1 + j];",
                                  "s += y[i] * (double)A1[i * R1 + (R1 - 1 - j)];"),
    "dl_omega_lora_reads_lerp": ("s += z[i] * (double)A2[i * R2 + j];",
                                 "s += y[i] * (double)A2[i * R2 + j];"),
    "dl_omega_lora_no_activation": ("h2[j] = act ? tanh(s) : s;", "h2[j] = s;"),
    "dl_omega_lora_channel_reversed": ("s += h2[j] * (double)B2[j * D + i];",
                                       "s += h2[j] * (double)B2[j * D + (D - 1 - i)];"),
    "bwd_ignores_final_state_gradient": (
        "dS[i] = d_sT ? d_sT[(b * H + h) * NN + i] : 0.0;", "dS[i] = 0.0;"),
}

PINS = [
    (P.test_rwkv4_bruteforce_workload1, {}),
    (P.test_rwkv4_bruteforce_with_history, {}),
    (P.test_rwkv4_constant_inputs_closed_form, {}),
    (P.test_rwkv4_first_token_is_v, {}),
    (P.test_rwkv4_golden_hand_example, {}),
    (P.test_matrix_bruteforce, {"per_token": False}),
    (P.test_matrix_bruteforce, {"per_token": True}),
    (P.test_matrix_golden_hand_example, {}),
    (P.test_matrix_geometric_closed_form, {}),
    (P.test_matrix_no_decay_is_causal_linear_attention, {}),
    (P.test_matrix_full_decay_keeps_only_last_token, {}),
    (P.test_matrix_single_token, {}),
    (P.test_matrix_bwd_finite_differences, {"per_token": False, "T": 5}),
    (P.test_matrix_bwd_finite_differences, {"per_token": True, "T": 70}),
    (P.test_matrix_bwd_no_decay_is_linear_attention_backward, {}),
    (P.test_matrix_bwd_eagle_decay_gradient_is_finch_summed, {}),
    (P.test_norm_gate_is_group_norm_times_silu, {}),
    (P.test_norm_gate_normalises_each_head, {}),
    (P.test_norm_gate_affine_and_gate_structure, {}),
    (P.test_decay_lora_without_offset_is_omega, {}),
    (P.test_decay_lora_constant_sequence, {}),
    (P.test_decay_lora_full_and_no_shift, {}),
    (P.test_decay_lora_mix_lora_structure, {}),
    (P.test_decay_lora_tanh_saturates, {}),
    (P.test_decay_lora_split_and_channel_locality, {}),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation site not found: {old}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(str(path), lib_path)
    lib = oracle.load(lib_path)
    caught = []
    for fn, kw in PINS:
        try:
            fn(lib, **kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_source_passes_every_pin(tmp_path):
    lib_path = str(tmp_path / "libclean.so")
    oracle.build(oracle.SOURCE, lib_path)
    lib = oracle.load(lib_path)
    for fn, kw in PINS:
        fn(lib, **kw)
