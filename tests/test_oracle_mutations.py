"""Planted mistakes in a copy of the oracle must fail at least one pin.

Each case copies oracle/la_oracle.c, applies one textual mutation of the kind
a transcription of the pages could plausibly contain (a dropped term, a wrong
sign, a wrong or transposed operand, an off-by-one mask), builds it with gcc
into a temporary directory, swaps it in for the real oracle and runs the pin
tests.  Everything happens on the CPU; the real oracle is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")

MUTATIONS = {
    "phi drops the +1": ("x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x : exp(x)"),
    "phi' wrong for x<=0": ("x > 0.0 ? 1.0 : exp(x)", "x > 0.0 ? 1.0 : 1.0"),
    "state update uses phi(Q)": ("S[d * M + m] += pk[d] * v[m];", "S[d * M + m] += pq[d] * v[m];"),
    "normaliser uses phi(Q)": ("        Z[d] += pk[d];\n      }\n      double dn", "        Z[d] += pq[d];\n      }\n      double dn"),
    "parallel form sees one future token": ("for (long j = 0; j <= i; ++j) {\n        double a",
                                             "for (long j = 0; j <= i + (i + 1 < N); ++j) {\n        double a"),
    "denominator gradient sign": ("G[i * Mb + M] = -dot / den[i];", "G[i * Mb + M] = dot / den[i];"),
    "chain rule uses phi not phi'": ("dQ[(bh * N + i) * D + d] = dP[i * D + d] * dfeat(q[i * D + d], fm);",
                                     "dQ[(bh * N + i) * D + d] = dP[i * D + d] * feat(q[i * D + d], fm);"),
    "eq. 15 transposed operand": ("acc += R[c * Mb + m] * Kf[i * C + c];", "acc += R[c * Mb + m] * P[i * C + c];"),
    "eq. 14 reverse sum of wrong factor": ("R[c * Mb + m] += P[i * C + c] * G[i * Mb + m];",
                                           "R[c * Mb + m] += Kf[i * C + c] * G[i * Mb + m];"),
    "eq. 13 forward sum off by one": ("    for (long c = 0; c < C; ++c) {\n      double acc = 0.0;\n      for (long m = 0; m < Mb; ++m) acc += S[c * Mb + m] * G[i * Mb + m];\n      dP[i * C + c] = acc;\n    }\n  }",
                                      "    for (long c = 0; c < C; ++c) {\n      double acc = 0.0;\n      for (long m = 0; m < Mb; ++m) acc += S[c * Mb + m] * G[i * Mb + m] * (i > 0);\n      dP[i * C + c] = acc;\n    }\n  }"),
    "non-causal drops phi on keys": ("double pk = feat(k[d], fm);\n        for", "double pk = k[d];\n        for"),
    "decode normaliser ignores keys": ("      z[d] = a * z[d] + pk;", "      z[d] = a * z[d] + 1.0;"),
    "non-causal backward denominator sign": ("double c = -dot / den;", "double c = dot / den;"),
    "non-causal reverse sum of phi(K)": ("for (long m = 0; m < M; ++m) R[d * M + m] += pq[d] * g[m];",
                                         "for (long m = 0; m < M; ++m) R[d * M + m] += feat(k[i * D + d], fm) * g[m];"),
    "non-causal value gradient uses phi(Q)": ("for (long d = 0; d < D; ++d) acc += R[d * M + m] * feat(k[j * D + d], fm);",
                                              "for (long d = 0; d < D; ++d) acc += R[d * M + m] * feat(q[j * D + d], fm);"),
    "final-state gradient not carried": ("if (RN) memcpy(R, RN, (size_t)(C * Mb) * sizeof(double));",
                                         "if (RN) memset(R, 0, (size_t)(C * Mb) * sizeof(double));"),
    "initial-state gradient misses token 1": (
        "if (R0) memcpy(R0, R, (size_t)(C * Mb) * sizeof(double));",
        "if (R0) for (long e = 0; e < C * Mb; ++e) R0[e] = R[e] - (N > 0 ? P[e / Mb] * G[e % Mb] : 0.0);"),
    "decay applied after the update": ("S[d * M + m] = a * S[d * M + m] + pk[d] * v[m];",
                                       "S[d * M + m] = a * (S[d * M + m] + pk[d] * v[m]);"),
    "normaliser not decayed": ("Z[d] = a * Z[d] + pk[d];", "Z[d] = Z[d] + pk[d];"),
    "decay gradient misses a_t": ("dlogA[bh * N + i] = a * ip;", "dlogA[bh * N + i] = ip;"),
    "decay gradient uses the current state": ("ip += R[e] * prev[e];", "ip += R[e] * cur[e];"),
    "reverse state not decayed": ("for (long e = 0; e < SB; ++e) R[e] *= a;", "(void)a;"),
    "feature mode still applies elu + 1": ("static double feat(double x, long fm) { return fm ? x : orc_phi(x); }",
                                          "static double feat(double x, long fm) { return orc_phi(x); }"),
    "poly2 features drop the constant": ("    f[0] = 1.0;\n", "    f[0] = 0.0;\n"),
    "poly2 gradient misses the transposed term": (
        "acc += (g[1 + Din + a * Din + b] + g[1 + Din + b * Din + a]) * x[b];",
        "acc += 2.0 * g[1 + Din + a * Din + b] * x[b];"),
    "random features miss the norm term": ("Phi[r * C + c] = exp(t - 0.5 * nx) * sc;", "Phi[r * C + c] = exp(t) * sc;"),
    "random-feature gradient misses -x": ("dX[r * Din + d] += gphi * (w[c * Din + d] - x[d]);",
                                          "dX[r * Din + d] += gphi * w[c * Din + d];"),
    "initial state ignored in backward": ("acc += (Z0 ? Z0[bh * D + d] : 0.0) * G[i * Mb + M];",
                                          "acc += 0.0 * G[i * Mb + M];"),
}

PIN_CALLS = [
    P.test_phi_closed_forms,
    P.test_dphi_finite_difference,
    P.test_worked_example_forward,
    P.test_worked_example_backward,
    lambda: P.test_recurrent_equals_bruteforce_eq8((2, 3, 17, 5, 3)),
    lambda: P.test_parallel_form_equals_recurrent((2, 3, 17, 5, 3)),
    lambda: P.test_noncausal_equals_bruteforce((2, 3, 17, 5, 3)),
    P.test_final_state_definition,
    P.test_constant_values_give_constant_output,
    P.test_first_row_is_first_value,
    P.test_zero_queries_and_keys_give_running_mean,
    P.test_decode_steps_equal_bruteforce,
    lambda: P.test_backward_finite_differences(3, 3, False),
    lambda: P.test_backward_finite_differences(4, 8, True),
    P.test_numerator_gradient_finite_differences,
    P.test_euler_identities,
    lambda: P.test_noncausal_backward_finite_differences(3, 3),
    lambda: P.test_noncausal_backward_equals_autograd((2, 3, 17, 5, 3)),
    P.test_noncausal_backward_last_row_is_causal,
    P.test_noncausal_backward_constant_values,
    lambda: P.test_state_gradient_finite_differences(3, 3),
    lambda: P.test_state_gradient_equals_autograd((2, 3, 17, 5, 3)),
    P.test_state_gradient_chains_across_a_split,
    P.test_state_gradient_without_output_gradient,
    lambda: P.test_decay_forward_equals_bruteforce((2, 3, 17, 5, 3), True),
    P.test_decay_of_one_is_the_base_method,
    lambda: P.test_decay_backward_equals_autograd((2, 3, 17, 5, 3)),
    P.test_decay_backward_finite_differences,
    P.test_decay_decode_equals_forward,
    P.test_decay_log_gradient_identity,
    P.test_poly2_features_give_the_polynomial_kernel,
    P.test_performer_features_are_unbiased_for_exp,
    lambda: P.test_feature_vjp_finite_differences("poly2"),
    lambda: P.test_feature_vjp_finite_differences("performer"),
    lambda: P.test_feature_mode_with_poly2_is_the_polynomial_attention(True),
    P.test_feature_mode_with_elu_features_is_the_method,
]


def _count_failures():
    failed = 0
    for call in PIN_CALLS:
        try:
            call()
        except (AssertionError, ZeroDivisionError, FloatingPointError, ValueError):
            failed += 1
    return failed


def test_pins_pass_on_real_oracle():
    assert _count_failures() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} must match exactly once"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-o", str(so), str(mutated), "-lm"], check=True)
    lib = oracle._configure(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    assert _count_failures() > 0, f"no pin caught the planted mistake {name!r}"
