"""Mutation check of the pins: plausible mistakes planted in a copy of the
oracle's C source (a flipped sign, a dropped term, a transposed index, a
shifted window, a wrong head map, ...) must each make at least one pin fail.

In the spirit of the rewind test on "perf(qwen): full-context MTP draft
prefill and replay-free rewind" (Tests), which was confirmed to fail when
the rerun or the trim is removed.  Mistakes are planted only in a throwaway
CPU build of the oracle."""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "correction_sign": ("double u = beta * (v[j] - a * p);", "double u = beta * (v[j] + a * p);"),
    "drop_decay_in_update": ("= a * hh[(size_t)i * DV + j] + k[i] * u;",
                             "= hh[(size_t)i * DV + j] + k[i] * u;"),
    "drop_decay_in_correction": ("(v[j] - a * p)", "(v[j] - p)"),
    "drop_beta": ("double u = beta * (v[j] - a * p);", "double u = (v[j] - a * p);"),
    "transposed_state_read": ("p += hh[(size_t)i * DV + j] * k[i];",
                              "p += hh[(size_t)j * DV + i] * k[i];"),
    "output_before_update": ("for (int i = 0; i < DK; ++i) r += hh[(size_t)i * DV + j] * q[i];",
                             "for (int i = 0; i < DK; ++i) r += (hh[(size_t)i * DV + j] - k[i] * u) * q[i];"),
    "output_reads_k": ("r += hh[(size_t)i * DV + j] * q[i];", "r += hh[(size_t)i * DV + j] * k[i];"),
    "gqa_modulo_map": ("int m = hv / group;", "int m = hv % d->HK;"),
    "q_k_swapped": ("const double* qsrc = y + (size_t)m * DK;",
                    "const double* qsrc = y + (size_t)d->HK * DK + (size_t)m * DK;"),
    "conv_taps_reversed": ("acc += w_l[(size_t)c * d->KCONV + j] *",
                           "acc += w_l[(size_t)c * d->KCONV + (d->KCONV - 1 - j)] *"),
    "no_silu": ("acc = acc / (1.0 + exp(-acc));", "acc = acc;"),
    "l2_without_sqrt": ("double nq = sqrt(sq + d->l2_eps), nk = sqrt(sk + d->l2_eps);",
                        "double nq = (sq + d->l2_eps), nk = (sk + d->l2_eps);"),
    "gate_not_exponentiated": ("double a = exp(g_t[hv]);", "double a = 1.0 + g_t[hv];"),
    "candidate_slot_off_by_one": ("(c0 + t + 1) % d->S", "(c0 + t) % d->S"),
    "commit_window_off_by_one": ("window_row(d, cs, xl, kp + r)", "window_row(d, cs, xl, kp + r - 1)"),
    "commit_slot_not_advanced": ("cur[l * d->B + b] = (c0 + kp) % d->S;",
                                 "cur[l * d->B + b] = (c0 + kp - 1) % d->S;"),
    "inactive_keep_not_reported": ("if (!act && keep != 0) e |= 4;", "(void)act;"),
    "verify_ignores_active": ("if (!row_active(active, b)) continue;\n            int c0 = cur ? cur[l * d->B + b] : 0;\n            if (c0 < 0 || c0 >= d->S) { err |= 2; continue; }\n            memcpy(h,",
                              "int c0 = cur ? cur[l * d->B + b] : 0;\n            if (c0 < 0 || c0 >= d->S) { err |= 2; continue; }\n            memcpy(h,"),
    "rewind_one_token_short": ("for (int t = 0; t < kp; ++t) {", "for (int t = 0; t + 1 < kp; ++t) {"),
    "accept_compares_same_position": ("== target[(size_t)b * T + (k - 1)]) k++;",
                                      "== target[(size_t)b * T + k]) k++;"),
    "rmsnorm_sum_not_mean": ("const double r = 1.0 / sqrt(ss / DV + eps);",
                             "const double r = 1.0 / sqrt(ss + eps);"),
    "rmsnorm_gate_without_silu": ("* (zz / (1.0 + exp(-zz)));", "* zz;"),
    "rmsnorm_weight_by_head": ("w[(size_t)l * DV + j]", "w[(size_t)l * DV + (h % DV)]"),
    "accept_next_one_late": ("if (next) next[b] = target[(size_t)b * T + (k - 1)];",
                             "if (next) next[b] = target[(size_t)b * T + (k < T ? k : k - 1)];"),
}


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation %s no longer applies" % name
    path = tmp_path / ("m_%s.c" % name)
    path.write_text(src.replace(old, new))
    so = tmp_path / ("m_%s.so" % name)
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-std=c99", "-shared", "-fPIC",
                           "-o", str(so), str(path), "-lm"])
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(tmp_path, name):
    so = _build(tmp_path, name, *MUTANTS[name])
    caught = []
    with oracle.library(so):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(oracle)
            except AssertionError:
                caught.append(pin.__name__)
    assert caught, "no pin catches the mutation %s" % name
