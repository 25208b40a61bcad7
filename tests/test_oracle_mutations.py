"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them: a pin that no mistake can trip pins nothing."""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = open(oracle._SRC).read()

# (name, original text, planted mistake)
MUTATIONS = [
    ("drop_D_term", "y[bt * D + d] = yv + delta * xv;", "y[bt * D + d] = yv;"),
    ("readout_before_update",
     "          h[n] = a * h[n] + bb;\n          yv += Cm[bt * N + n] * h[n];",
     "          yv += Cm[bt * N + n] * h[n];\n          h[n] = a * h[n] + bb;"),
    ("exp_sign", "double a = exp(Dt * Abar);", "double a = exp(-Dt * Abar);"),
    ("softplus_sign", "log1p(exp(-fabs(z)))", "log1p(exp(fabs(z)))"),
    ("softplus_drop_relu", "return (z > 0.0 ? z : 0.0) + log1p", "return log1p"),
    ("bias_unmixed", "beta += g[j] * dt_bias", "beta += dt_bias"),
    ("D_unmixed", "delta += g[j] * Dskip", "delta += Dskip"),
    ("A_first_gate_only", "Abar += g[j] * A[", "Abar += g[0] * A["),
    ("A_transposed", "Abar += g[j] * A[((int64_t)e[j] * D + d) * N + n];",
     "Abar += g[j] * A[((int64_t)e[j] * N + n) * D + d];"),
    ("injection_no_delta", "double bb = input_coeff(Dt, Abar, zoh) * Bm[bt * N + n] * xv;",
     "double bb = Bm[bt * N + n] * xv;"),
    ("zoh_divides_by_delta", "return z == 0.0 ? Dt : expm1(z) / Abar;",
     "return z == 0.0 ? Dt : expm1(z) / Dt;"),
    ("zoh_exp_for_expm1", "return z == 0.0 ? Dt : expm1(z) / Abar;",
     "return z == 0.0 ? Dt : exp(z) / Abar;"),
    ("zoh_ignored", "  if (!zoh) return Dt;\n", "  return Dt;\n"),
    ("B_C_swapped", "yv += Cm[bt * N + n] * h[n];", "yv += Bm[bt * N + n] * h[n];"),
    ("h0_ignored", "h[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;\n      for (int t = 0; t < L; ++t) {\n        int64_t bt = (int64_t)b * L + t;\n        const int32_t* e",
     "h[n] = 0.0;\n      for (int t = 0; t < L; ++t) {\n        int64_t bt = (int64_t)b * L + t;\n        const int32_t* e"),
    ("route_tie_to_higher", "if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("route_softmax_all", "for (int j = 0; j < k; ++j) z += exp(l[idx[t * k + j]] - m);",
     "for (int j = 0; j < E; ++j) z += exp(l[j] - m);"),
    ("route_absdot_signed", "sa += fabs(p);", "sa += p;"),
    ("separate_wrong_expert_A", "double Ae = A[((int64_t)e * D + d) * N + n];",
     "double Ae = A[((int64_t)0 * D + d) * N + n];"),
    ("separate_ungated", "yv += gate[bt * k + j] * ye;", "yv += ye;"),
    ("separate_bias_of_slot0", "softplus(dt_raw[bt * D + d] + dt_bias[(int64_t)e * D + d]);",
     "softplus(dt_raw[bt * D + d] + dt_bias[(int64_t)idx[bt * k] * D + d]);"),
    ("separate_decays_all",
     "          ye += Dskip[(int64_t)e * D + d] * xv;",
     "          for (int o = 0; o < E; ++o) if (o != e) for (int n = 0; n < N; ++n) H[o * N + n] *= 0.5;\n          ye += Dskip[(int64_t)e * D + d] * xv;"),
    ("slots_expert_of_slot0", "const int64_t ed = (int64_t)idx[bt * k + j] * D + d;",
     "const int64_t ed = (int64_t)idx[bt * k + 0] * D + d;"),
    ("slots_gate_in_state", "input_coeff(Dt, Aj, zoh)", "gate[bt * k + j] * input_coeff(Dt, Aj, zoh)"),
    ("slots_no_Dskip", "(yj + Dskip[ed] * xv)", "(yj)"),
    ("slots_readout_before_update",
     "            H[j * N + n] = exp(Dt * Aj) * H[j * N + n] +\n                           input_coeff(Dt, Aj, zoh) * Bm[bt * N + n] * xv;\n            yj += Cm[bt * N + n] * H[j * N + n];",
     "            yj += Cm[bt * N + n] * H[j * N + n];\n            H[j * N + n] = exp(Dt * Aj) * H[j * N + n] +\n                           input_coeff(Dt, Aj, zoh) * Bm[bt * N + n] * xv;"),
    ("slots_h0_layout", "h0[(((int64_t)b * k + j) * D + d) * N + n]",
     "h0[(((int64_t)b * D + d) * k + j) * N + n]"),
    ("slots_reset_on_switch", "H[j * N + n] = exp(Dt * Aj) * H[j * N + n] +",
     "H[j * N + n] = (t > 0 && idx[bt * k + j] != idx[(bt - 1) * k + j] ? 0.0 : exp(Dt * Aj) * H[j * N + n]) +"),
    ("all_only_selected_advance", "        /* every expert advances */\n        for (int e = 0; e < E; ++e) {\n",
     "        for (int e = 0; e < E; ++e) {\n          int sel = 0;\n          for (int j = 0; j < k; ++j) sel |= idx[bt * k + j] == e;\n          if (!sel) { out[e] = 0.0; continue; }\n"),
    ("all_ungated", "yv += gate[bt * k + j] * out[idx[bt * k + j]];", "yv += out[idx[bt * k + j]];"),
    ("all_output_of_slot0", "yv += gate[bt * k + j] * out[idx[bt * k + j]];",
     "yv += gate[bt * k + j] * out[idx[bt * k]];"),
    ("all_bias_of_expert0", "const double step = softplus(dt_raw[bt * D + d] + dt_bias[ed]);",
     "const double step = softplus(dt_raw[bt * D + d] + dt_bias[d]);"),
    ("all_no_Dskip", "double acc = Dskip[ed] * u;", "double acc = 0.0;"),
    ("all_h0_layout", "S[e * N + n] = h0 ? h0[(((int64_t)b * E + e) * D + d) * N + n] : 0.0;",
     "S[e * N + n] = h0 ? h0[(((int64_t)b * D + d) * E + e) * N + n] : 0.0;"),
    ("all_readout_before_update",
     "            S[e * N + n] = exp(step * an) * S[e * N + n] +\n                           input_coeff(step, an, zoh) * Bm[bt * N + n] * u;\n            acc += Cm[bt * N + n] * S[e * N + n];",
     "            acc += Cm[bt * N + n] * S[e * N + n];\n            S[e * N + n] = exp(step * an) * S[e * N + n] +\n                           input_coeff(step, an, zoh) * Bm[bt * N + n] * u;"),
    ("mamba_wrong_A_index", "double An = A[(int64_t)d * N + n];", "double An = A[(int64_t)n];"),
    ("mamba_no_D", "double out = Dskip[d] * u;", "double out = 0.0;"),
    ("step_routes_first_token_only", "ref_route(B, D, E, k, x, Wr, idx, gate, NULL, NULL);",
     "ref_route(1, D, E, k, x, Wr, idx, gate, NULL, NULL);\n    for (int64_t i = k; i < (int64_t)B * k; ++i) { idx[i] = idx[i % k]; gate[i] = gate[i % k]; }"),
    ("streams_injection_ungated", "inj += g[j] * Bs[", "inj += Bs["),
    ("streams_readout_ungated", "c += g[j] * Cs[", "c += Cs["),
    ("streams_readout_slot0", "c += g[j] * Cs[(bt * k + j) * N + n];",
     "c += g[j] * Cs[(bt * k + 0) * N + n];"),
    ("streams_X_transposed", "X[(bt * k + j) * D + d]", "X[(bt * D + d) * k + j]"),
    ("streams_X_slot0", "X[(bt * k + j) * D + d]", "X[(bt * k) * D + d]"),
    ("streams_B_slot0", "inj += g[j] * Bs[(bt * k + j) * N + n]", "inj += g[j] * Bs[(bt * k) * N + n]"),
    ("streams_injection_no_delta", "h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;",
     "h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + inj;"),
    ("streams_A_transposed", "h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;",
     "h[n] = exp(Dt * A[(int64_t)n * D + d]) * h[n] + Dt * inj;"),
    ("streams_exp_sign", "h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;",
     "h[n] = exp(-Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;"),
    ("streams_readout_before_update",
     "          h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;\n          yv += c * h[n];",
     "          yv += c * h[n];\n          h[n] = exp(Dt * A[(int64_t)d * N + n]) * h[n] + Dt * inj;"),
    ("streams_bias_ignored",
     "const double* g = gate + bt * k;\n        double Dt = softplus(dt_raw[bt * D + d] + dt_bias[d]);",
     "const double* g = gate + bt * k;\n        double Dt = softplus(dt_raw[bt * D + d]);"),
    ("streams_h0_ignored",
     "h[n] = h0 ? h0[((int64_t)b * D + d) * N + n] : 0.0;\n      for (int t = 0; t < L; ++t) {\n        int64_t bt = (int64_t)b * L + t;\n        const double* g",
     "h[n] = 0.0;\n      for (int t = 0; t < L; ++t) {\n        int64_t bt = (int64_t)b * L + t;\n        const double* g"),
    ("bwd_no_decay_of_adjoint", "          for (int n = 0; n < N; ++n) lam[n] *= aa[(int64_t)t * N + n];\n",
     ""),
    ("bwd_sigmoid_sign", "double sig = 1.0 / (1.0 + exp(-zz[t]));", "double sig = 1.0 / (1.0 + exp(zz[t]));"),
    ("bwd_dC_previous_state", "+= g_dy * ht;", "+= g_dy * hp;"),
    ("bwd_dB_no_delta", "+= lam[n] * Dt[t] * xv;", "+= lam[n] * xv;"),
    ("bwd_dgate_no_A_term", "Dskip[(int64_t)e * D + d] * ddelta + s;", "Dskip[(int64_t)e * D + d] * ddelta;"),
    ("bwd_dA_ungated", "dA[((int64_t)e * D + d) * N + n] += gj * dAbar[n];",
     "dA[((int64_t)e * D + d) * N + n] += dAbar[n];"),
    ("bwd_dx_no_D_term", "double dxv = delta * g_dy, dDt = 0.0;", "double dxv = 0.0, dDt = 0.0;"),
    ("bwd_dDelta_no_injection", "(a * Ab[(int64_t)t * N + n] * hp + Bm[bt * N + n] * xv)",
     "(a * Ab[(int64_t)t * N + n] * hp)"),
    ("bwd_adjoint_from_next_C", "lam[n] += Cm[bt * N + n] * g_dy;",
     "lam[n] += Cm[(t + 1 < L ? bt + 1 : bt) * N + n] * g_dy;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new, tmp_path):
    assert SRC.count(old) == 1, "mutation anchor for %s not unique/present" % name
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(SRC.replace(old, new))
    so = str(tmp_path / ("libmut_%s.so" % name))
    oracle.build(force=True, src=str(src), out=so)
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, "no pin caught mutation %s" % name
