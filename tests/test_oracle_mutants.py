"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a one-line change of oracle/la_oracle.c of the kind a careless
re-derivation could make (a dropped term, a wrong sign, a wrong index, an
exclusive instead of inclusive prefix, a transposed state, a wrong branch of
phi).  The mutant is compiled with gcc into a temporary folder and the pin
suite is run against it; the real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
import pin_suite

MUTANTS = {
    "phi_drops_plus_one": ("return x > 0.0 ? x + 1.0 : exp(x); }", "return x > 0.0 ? x : exp(x); }"),
    "phi_wrong_branch": ("return x > 0.0 ? x + 1.0 : exp(x); }", "return x >= 1.0 ? x + 1.0 : exp(x); }"),
    "dphi_constant": ("static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }",
                      "static double dphi(double x) { return 1.0; }"),
    "causal_read_before_update": (
        "            for (int e = 0; e < dk; ++e) {\n                double fk = phi(ki[e]);\n"
        "                z[e] += fk;\n                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += fk * vi[c];\n"
        "            }\n            double d = 0.0;\n            for (int e = 0; e < dk; ++e) {\n"
        "                fq[e] = phi(qi[e]);\n                d += fq[e] * z[e];\n            }\n",
        "            double d = 0.0;\n            for (int e = 0; e < dk; ++e) {\n"
        "                fq[e] = phi(qi[e]);\n                d += fq[e] * (z[e] + phi(ki[e]) * 0.0 + (i == 0));\n            }\n"
        "            for (int e = 0; e < dk; ++e) {\n                double fk = phi(ki[e]);\n"
        "                z[e] += fk;\n                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += fk * vi[c];\n"
        "            }\n"),
    "causal_transposed_state_read": ("for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];\n"
                                     "                ob[(long)i * dv + c] = num / d;\n            }\n"
                                     "            if (den)",
                                     "for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)(c % dk) * dv + (e % dv)];\n"
                                     "                ob[(long)i * dv + c] = num / d;\n            }\n"
                                     "            if (den)"),
    "noncausal_drops_normaliser": ("            fq[e] = phi(qb[(long)i * dk + e]);\n                d += fq[e] * z[e];\n"
                                   "            }\n            for (int c = 0; c < dv; ++c) {\n                double num = 0.0;\n"
                                   "                for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];\n"
                                   "                ob[(long)i * dv + c] = num / d;\n            }\n        }\n        free(S);",
                                   "            fq[e] = phi(qb[(long)i * dk + e]);\n                d += fq[e];\n"
                                   "            }\n            for (int c = 0; c < dv; ++c) {\n                double num = 0.0;\n"
                                   "                for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];\n"
                                   "                ob[(long)i * dv + c] = num / d;\n            }\n        }\n        free(S);"),
    "decode_uses_k_for_q": ("for (int e = 0; e < dk; ++e) d += phi(qb[e]) * zb[e];",
                            "for (int e = 0; e < dk; ++e) d += phi(kb[e]) * zb[e];"),
    "bwd_eps_sign": ("Gp[(long)i * dv1 + dv] = -go / den[i];", "Gp[(long)i * dv1 + dv] = go / den[i];"),
    "bwd_drops_ones_column": ("double acc = Sp[(long)e * dv1 + dv]; /* times V'_j[dv] = 1 */",
                              "double acc = 0.0;"),
    "bwd_reverse_exclusive": ("        for (int j = N - 1; j >= 0; --j) {\n            for (int e = 0; e < dk; ++e) {\n"
                              "                double fq = phi(qb[(long)j * dk + e]);\n"
                              "                for (int c = 0; c < dv1; ++c) Sp[(long)e * dv1 + c] += fq * Gp[(long)j * dv1 + c];\n"
                              "            }\n",
                              "        for (int j = N - 1; j >= 0; --j) {\n            if (j < N - 1) for (int e = 0; e < dk; ++e) {\n"
                              "                double fq = phi(qb[(long)(j + 1) * dk + e]);\n"
                              "                for (int c = 0; c < dv1; ++c) Sp[(long)e * dv1 + c] += fq * Gp[(long)(j + 1) * dv1 + c];\n"
                              "            }\n"),
    "bwd_dv_uses_q": ("for (int e = 0; e < dk; ++e) acc += Sp[(long)e * dv1 + c] * phi(kb[(long)j * dk + e]);",
                      "for (int e = 0; e < dk; ++e) acc += Sp[(long)e * dv1 + c] * phi(qb[(long)j * dk + e]);"),
    "bwd_dq_missing_chain_rule": ("dqb[(long)i * dk + e] = acc * dphi(qb[(long)i * dk + e]);",
                                  "dqb[(long)i * dk + e] = acc;"),
    "decay_misses_z": ("z[e] = g * z[e] + fk;", "z[e] = z[e] + fk;"),
    "decay_after_update": ("S[(long)e * dv + c] = g * S[(long)e * dv + c] + fk * vi[c];",
                           "S[(long)e * dv + c] = g * (S[(long)e * dv + c] + fk * vi[c]);"),
    "decay_gamma_by_batch": ("const double g = gamma[bh % H];\n        const double *qb = q + bh * (long)N * dk;",
                             "const double g = gamma[(bh / H) % H];\n        const double *qb = q + bh * (long)N * dk;"),
    "decode_decay_misses_S": ("Sb[(long)e * dv + c] = g * Sb[(long)e * dv + c] + fk * vb[c];",
                              "Sb[(long)e * dv + c] = Sb[(long)e * dv + c] + fk * vb[c];"),
    "dbwd_reverse_undecayed": ("Sp[(long)e * dv1 + c] = gm * Sp[(long)e * dv1 + c] + fq * Gp[(long)j * dv1 + c];",
                               "Sp[(long)e * dv1 + c] = Sp[(long)e * dv1 + c] + fq * Gp[(long)j * dv1 + c];"),
    "dbwd_z_undecayed": ("Sp[(long)e * dv1 + dv] = gm * Sp[(long)e * dv1 + dv] + fk;",
                         "Sp[(long)e * dv1 + dv] = Sp[(long)e * dv1 + dv] + fk;"),
    "fm_drops_half_norm": ("out[r] = exp(a - 0.5 * nx) / sqrt((double)m);", "out[r] = exp(a) / sqrt((double)m);"),
    "fm_normalised_by_m": ("out[r] = exp(a - 0.5 * nx) / sqrt((double)m);", "out[r] = exp(a - 0.5 * nx) / (double)m;"),
    "fm_direction_sign": ("a += Wh[(long)r * dk + e] * x[e];", "a -= Wh[(long)r * dk + e] * x[e];"),
    "fm_directions_transposed": ("a += Wh[(long)r * dk + e] * x[e];", "a += Wh[(long)(e % m) * dk + (r % dk)] * x[e];"),
    "fm_vjp_drops_x": ("dx[e] += u * (Wh[(long)r * dk + e] - x[e]);", "dx[e] += u * Wh[(long)r * dk + e];"),
    "fm_vjp_drops_phi": ("double u = dphi_in[r] * f[r];", "double u = dphi_in[r];"),
    "fm_identity_vjp_elu": ("for (int e = 0; e < dk; ++e) dx[e] = dphi_in[e];",
                            "for (int e = 0; e < dk; ++e) dx[e] = dphi_in[e] * dphi(x[e]);"),
    "fm_causal_drops_z": ("for (int e = 0; e < mf; ++e) d += fq[e] * z[e];", "for (int e = 0; e < mf; ++e) d += fq[e];"),
    "fm_bwd_dv_uses_q": ("for (int e = 0; e < mf; ++e) acc += Sp[(long)e * dv1 + c] * fk[e];",
                         "for (int e = 0; e < mf; ++e) acc += Sp[(long)e * dv1 + c] * fq[e];"),
    "nbwd_eps_sign": ("Gi[dv] = -go / d;", "Gi[dv] = go / d;"),
    "nbwd_drops_ones_column": ("double acc = Rp[(long)e * dv1 + dv]; /* times V'_j[dv] = 1 */",
                               "double acc = 0.0;"),
    "nbwd_R_from_k": ("double fq = phi(qb[(long)i * dk + e]);\n                for (int c = 0; c < dv1; ++c) Rp",
                      "double fq = phi(kb[(long)i * dk + e]);\n                for (int c = 0; c < dv1; ++c) Rp"),
    "nbwd_dv_transposed": ("acc += Rp[(long)e * dv1 + c] * phi(kb[(long)j * dk + e]);",
                           "acc += Rp[(long)(c % dk) * dv1 + (e % dv)] * phi(kb[(long)j * dk + e]);"),
    "nbwd_dq_drops_normaliser_term": ("for (int c = 0; c < dv1; ++c) acc += Sp[(long)e * dv1 + c] * Gi[c];",
                                      "for (int c = 0; c < dv; ++c) acc += Sp[(long)e * dv1 + c] * Gi[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, oracle_lib, name):
    old, new = MUTANTS[name]
    src = open(oracle.source_path()).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    cfile = os.path.join(tmp_path, "mutant.c")
    sofile = os.path.join(tmp_path, "libmutant.so")
    with open(cfile, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-shared", "-fPIC", "-std=c99", "-o", sofile, cfile, "-lm"], check=True)
    lib = oracle.load_variant(sofile)
    failed = pin_suite.failing_checks(lib)
    assert failed, f"planted mistake {name} passed every pin"
