"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/ssu_ref.c with one plausible mistake (a dropped
term, a wrong sign, a wrong index or operand, a wrong rounding), built with gcc
into a temporary library and run through every pin on the CPU. Every mistake
keeps all memory accesses in bounds. A mutant that no pin notices would mean
the pins leave that part of the oracle unchecked.
"""
import os

import pytest

import oracle
from oracle.build import SRC, build_oracle

from .oracle_pins import PINS

# (name, text in ssu_ref.c, replacement)
MUTANTS = [
    ("update_sign", "Sp[n] * a + (delta * xp)", "Sp[n] * a - (delta * xp)"),
    ("drop_decay", "Sp[n] = Sp[n] * a + ", "Sp[n] = Sp[n] + "),
    ("drop_input_term", "Sp[n] = Sp[n] * a + (delta * xp) * ref_bf16_value(Br[n * g->B_n]);",
     "Sp[n] = Sp[n] * a;"),
    ("drop_delta_in_input", "(delta * xp) * ref_bf16_value(Br", "(xp) * ref_bf16_value(Br"),
    ("B_for_C_in_update", "ref_bf16_value(Br[n * g->B_n])", "ref_bf16_value(Cr[n * g->C_n])"),
    ("C_for_B_in_output", "Sp[n] * ref_bf16_value(Cr[n * g->C_n])", "Sp[n] * ref_bf16_value(Br[n * g->B_n])"),
    ("drop_skip_D", "    y += Dv * xp;\n", "\n"),
    ("skip_uses_B", "y += Dv * xp;", "y += Dv * ref_bf16_value(Br[p % N * g->B_n]);"),
    ("decay_sign", "*a = exp(A * d);", "*a = exp(-A * d);"),
    ("decay_uses_u", "*a = exp(A * d);", "*a = exp(A * u);"),
    ("drop_bias", "double u = dt + dt_bias;", "double u = dt;"),
    ("softplus_sign", "log1p(exp(-fabs(u)))", "log1p(exp(fabs(u)))"),
    ("softplus_naive", "return fmax(u, 0.0) + log1p(exp(-fabs(u)));", "return log(1.0 + exp(u));"),
    ("softplus_shifted_form", "return fmax(u, 0.0) + log1p(exp(-fabs(u)));", "return u + log1p(exp(-u));"),
    ("softplus_ignored", "double d = softplus ? ssu_ref_softplus(u) : u;", "double d = u;"),
    ("group_map", "(((int64_t)h * G) / H)", "(h % G)"),
    ("slot_is_request", "g->state + slot * g->st_slot", "g->state + (int64_t)b * g->st_slot"),
    ("head_ignored", "+ (int64_t)h * g->st_head;", ";"),
    ("x_row_index", "xr[p * g->x_p]", "xr[(P - 1 - p) * g->x_p]"),
    ("output_old_state", "const double term = Sp[n] * ref_bf16_value",
     "const double term = (double)pool[(int64_t)p * g->st_row + n] * ref_bf16_value"),
    ("no_write_back", "pool[(int64_t)p * g->st_row + n] = (float)v;", "(void)v;"),
    ("bf16_truncate", "w += 0x7FFFu + lsb;", "w += 0u * lsb;"),
    ("bf16_ties_away", "w += 0x7FFFu + lsb;", "w += 0x8000u + 0u * lsb;"),
    ("tau_signed", "tau += fabs(term);", "tau += term;"),
    ("no_carry_between_tokens", "for (int32_t t = 0; t < K; ++t) {",
     "for (int32_t t = 0; t < K; ++t) {\n"
     "                for (int32_t q = 0; q < P * N; ++q) S[q] = (double)pool[(q / N) * g->st_row + q % N];"),
    ("skip_check_off", "if (slot < 0 || slot >= g->pool_slots)\n                continue;",
     "if (slot < 0 || slot >= g->pool_slots)\n                slot = 0;"),
    ("dups_allowed", "if (seen[s]) {", "if (0 && seen[s]) {"),
    ("copy_direction", "memcpy(t[k].base + d * t[k].block_stride, t[k].base + s * t[k].block_stride,",
     "memcpy(t[k].base + s * t[k].block_stride, t[k].base + d * t[k].block_stride,"),
    ("copy_stride_ignored", "t[k].base + s * t[k].block_stride,", "t[k].base + s * t[k].block_bytes,"),
    ("copy_skip_off",
     "const int64_t s = src[r], d = dst[r];\n"
     "            if (s < 0 || s >= t[k].nblocks || d < 0 || d >= t[k].nblocks || s == d)\n"
     "                continue;",
     "int64_t s = src[r], d = dst[r];\n"
     "            if (s == d) continue;\n"
     "            if (s < 0 || s >= t[k].nblocks) s = 0;\n"
     "            if (d < 0 || d >= t[k].nblocks) d = 0;"),
    ("copy_overlap_allowed", "            if (src[q] == dst[r] && src[q] != dst[q])\n                return 3;\n", ""),
    # selective scan over a sequence
    ("scan_update_sign", "h[n] = h[n] * a + beta;", "h[n] = h[n] * a - beta;"),
    ("scan_drop_decay", "h[n] = h[n] * a + beta;", "h[n] = h[n] + beta;"),
    ("scan_step_not_on_u", "(Delta * ut) * ref_io_value(Bt", "(ut) * ref_io_value(Bt"),
    ("scan_C_for_B", "ref_io_value(Bt[n * g->B_n], io)", "ref_io_value(Ct[n * g->C_n], io)"),
    ("scan_B_for_C", "const double c = ref_io_value(Ct[n * g->C_n], io);",
     "const double c = ref_io_value(Bt[n * g->B_n], io);"),
    ("scan_drop_D", "y += Dv * ut;", "y += 0.0 * Dv * ut;"),
    ("scan_D_on_step", "y += Dv * ut;", "y += Dv * Delta;"),
    ("scan_decay_sign", "exp(An * Delta)", "exp(-An * Delta)"),
    ("scan_decay_raw_step", "exp(An * Delta)", "exp(An * v)"),
    ("scan_drop_bias", "io) + bias;", "io);"),
    ("scan_softplus_ignored", "g->delta_softplus ? ssu_ref_softplus(v) : v", "v"),
    ("scan_group_map", "(((int64_t)d * G) / Dm)", "(d % G)"),
    ("scan_A_wrong_state", "Ar[n * g->A_n]", "Ar[((n + 1) % N) * g->A_n]"),
    ("scan_A_channel_ignored", "const float *Ar = g->A + d * g->A_d;", "const float *Ar = g->A;"),
    ("scan_initial_state_ignored", "h[n] = (double)st[n];", "h[n] = 0.0 * st[n];"),
    ("scan_no_write_back", "st[n] = (float)h[n];", "(void)st;"),
    ("scan_output_before_input", "y += h[n] * c;", "y += (h[n] - beta) * c;"),
    ("scan_step_order_reversed", "d * g->dl_d + t * g->dl_t]", "d * g->dl_d + (L - 1 - t) * g->dl_t]"),
    ("scan_B_lagged", "grp * g->B_g + t * g->B_t", "grp * g->B_g + (t > 0 ? t - 1 : 0) * g->B_t"),
    ("scan_out_always_bf16", "io ? ssu_ref_f16_rne(yf) : ssu_ref_bf16_rne(yf)", "ssu_ref_bf16_rne(yf)"),
    ("scan_error_scale_no_carry", "E[n] = a * E[n] +", "E[n] = 0.0 * E[n] +"),
    # error scales inflated or mis-formed (each loosens or skews the scan's tolerance)
    ("scan_E_times4", "E[n] = a * E[n] + (1.0 + fabs(An * Delta)) * a * Mprev + M[n];",
     "E[n] = 4.0 * (a * E[n] + (1.0 + fabs(An * Delta)) * a * Mprev + M[n]);"),
    ("scan_err_out_times4", "g->err_ref[si] = E[n];", "g->err_ref[si] = 4.0 * E[n];"),
    ("scan_E_new_term_times4", "* a * Mprev + M[n];", "* a * Mprev + 4.0 * M[n];"),
    ("scan_E_decay_term_times4", "(1.0 + fabs(An * Delta)) * a * Mprev", "4.0 * (1.0 + fabs(An * Delta)) * a * Mprev"),
    ("scan_E_no_step_term", "(1.0 + fabs(An * Delta)) * a * Mprev", "(1.0) * a * Mprev"),
    ("scan_E_initial_times4", "M[n] = E[n] = fabs(h[n]);", "M[n] = fabs(h[n]);\n                E[n] = 4.0 * M[n];"),
    ("scan_M_signed_input", "M[n] = a * M[n] + fabs(beta);", "M[n] = a * M[n] + beta;"),
    ("scan_M_no_decay", "M[n] = a * M[n] + fabs(beta);", "M[n] = M[n] + fabs(beta);"),
    ("scan_rho_times16", "rho += fabs(c) * E[n];", "rho += 16.0 * fabs(c) * E[n];"),
    ("scan_rho_signed_C", "rho += fabs(c) * E[n];", "rho += c * E[n];"),
    ("scan_tau_times16", "tau += fabs(h[n] * c);", "tau += 16.0 * fabs(h[n] * c);"),
    ("scan_tau_signed", "tau += fabs(h[n] * c);", "tau += h[n] * c;"),
    ("scan_tau_no_D", "tau += fabs(Dv * ut);", "tau += 0.0 * Dv * ut;"),
    ("f16_exponent_bias", "e - 25", "e - 24"),
    ("f16_subnormal_zero", "v = ldexp((double)m, -24);", "v = 0.0 * m;"),
    ("f16_implicit_bit", "(m | 0x400)", "(m)"),
    ("f16_round_truncate", "rint(ldexp(a, 10 - E))", "floor(ldexp(a, 10 - E))"),
    ("f16_subnormal_truncate", "(uint16_t)rint(ldexp(a, 24))", "(uint16_t)floor(ldexp(a, 24))"),
    ("f16_overflow_saturates", "if (E + 15 >= 31)\n        return (uint16_t)(sign | 0x7C00u);",
     "if (E + 15 >= 31)\n        return (uint16_t)(sign | 0x7BFFu);"),
]


def _caught(o):
    names = []
    for pin in PINS:
        try:
            pin(o)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            names.append(pin.__name__)
    return names


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    if name == "skip_check_off":
        # 'slot' is const in the original; the mutant needs a mutable copy
        src = src.replace("const int64_t slot = g->idx[b];", "int64_t slot = g->idx[b];")
        # keep the mutant in bounds: slot 0 exists whenever pool_slots > 0
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    msrc = tmp_path / f"ssu_ref_{name}.c"
    msrc.write_text(src.replace(old, new, 1))
    lib = build_oracle(src=str(msrc), out=str(tmp_path / f"libssu_ref_{name}.so"),
                       extra_flags=["-Wno-unused-variable", "-Wno-unused-parameter",
                                    "-Wno-unused-but-set-variable"], quiet=True)
    caught = _caught(oracle.Oracle(lib))
    print(f"{name}: caught by {caught}")
    assert caught, f"mutant {name} passes every pin"
    os.remove(lib)
