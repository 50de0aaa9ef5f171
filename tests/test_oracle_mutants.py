"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Each mutant is the oracle's C source with one snippet replaced (a dropped term,
a flipped sign, a transposed operand, a wrong order or index).  The mutant is
compiled into a temporary library and the oracle pin suite is run against it
in a subprocess; the suite must fail.  The real oracle is untouched.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hypic_ref.c")

MUTANTS = {
    "delta_decay_dropped_on_erase": (
        "a * (s - x->beta * x->k[i] * work[j])",
        "a * s - x->beta * x->k[i] * work[j]"),
    "delta_erase_sign": (
        "a * (s - x->beta * x->k[i] * work[j])",
        "a * (s + x->beta * x->k[i] * work[j])"),
    "delta_write_weight_dropped": (
        "+ x->beta * x->k[i] * x->v[j];",
        "+ x->k[i] * x->v[j];"),
    "delta_U_beta_dropped": (
        "U[(size_t)i * dk + j] -= x->beta * x->k[i] * dot;",
        "U[(size_t)i * dk + j] -= x->k[i] * dot;"),
    "scalar_gate_not_accumulated": (
        "          S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + x->k[i] * x->v[j];\n"
        "      if (g) g[0] += x->lg;",
        "          S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + x->k[i] * x->v[j];\n"
        "      if (g) g[0] += 0.0;"),
    "diag_gate_on_value_axis": (
        "          S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + x->k[i] * x->v[j];\n"
        "        if (g) g[i] += x->lgv[i];",
        "          S[(size_t)i * dv + j] = exp(x->lgv[j % dk]) * S[(size_t)i * dv + j] + x->k[i] * x->v[j];\n"
        "        if (g) g[i] += x->lgv[i];"),
    "compose_transition_transposed": (
        "acc += U[(size_t)i * dk + l] * S[(size_t)l * dv + j];",
        "acc += U[(size_t)l * dk + i] * S[(size_t)l * dv + j];"),
    "compose_add_before_transition": (
        "      apply_T(fam, dk, dv, g + pu * gl, REF_DENSE(fam) ? U + pu * dk * dk : NULL, cur, tmp);\n"
        "      const double* Si = S + pu * sz;\n"
        "      for (size_t e = 0; e < sz; ++e) cur[e] += Si[e];",
        "      const double* Si = S + pu * sz;\n"
        "      for (size_t e = 0; e < sz; ++e) cur[e] += Si[e];\n"
        "      apply_T(fam, dk, dv, g + pu * gl, REF_DENSE(fam) ? U + pu * dk * dk : NULL, cur, tmp);"),
    "compose_total_order_reversed": (
        "acc += Us[(size_t)i * dk + l] * ut[(size_t)l * dk + j];",
        "acc += ut[(size_t)i * dk + l] * Us[(size_t)l * dk + j];"),
    "compose_total_gate_not_summed": (
        "gacc[i] += g[pu * gl + i];",
        "gacc[i] = g[pu * gl + i];"),
    "compose_prefix_after_update": (
        "      if (prefix) memcpy(prefix + pu * sz, cur, sizeof(double) * sz);\n"
        "      apply_T(fam, dk, dv, g + pu * gl, REF_DENSE(fam) ? U + pu * dk * dk : NULL, cur, tmp);\n"
        "      const double* Si = S + pu * sz;\n"
        "      for (size_t e = 0; e < sz; ++e) cur[e] += Si[e];",
        "      apply_T(fam, dk, dv, g + pu * gl, REF_DENSE(fam) ? U + pu * dk * dk : NULL, cur, tmp);\n"
        "      const double* Si = S + pu * sz;\n"
        "      for (size_t e = 0; e < sz; ++e) cur[e] += Si[e];\n"
        "      if (prefix) memcpy(prefix + pu * sz, cur, sizeof(double) * sz);"),
    "build_first_token_skipped": (
        "for (int t = offsets[s]; t < offsets[s + 1]; ++t)",
        "for (int t = offsets[s] + 1; t < offsets[s + 1]; ++t)"),
    "seam_output_before_update": (
        "        token_step(fam, dk, dv, &x, S, NULL, NULL, work);\n"
        "        if (wS || wU || wg) token_step(fam, dk, dv, &x, pS, pg, REF_DENSE(fam) ? pU : NULL, work);\n"
        "        const double* qt = q + ((size_t)t * n_chain + h) * dk;\n"
        "        double* ot = o_out + ((size_t)t * n_chain + h) * dv;\n"
        "        for (int c = 0; c < dv; ++c) {\n"
        "          double acc = 0.0;\n"
        "          for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + c] * qt[i];\n"
        "          ot[c] = acc;\n"
        "        }\n",
        "        if (wS || wU || wg) token_step(fam, dk, dv, &x, pS, pg, REF_DENSE(fam) ? pU : NULL, work);\n"
        "        const double* qt = q + ((size_t)t * n_chain + h) * dk;\n"
        "        double* ot = o_out + ((size_t)t * n_chain + h) * dv;\n"
        "        for (int c = 0; c < dv; ++c) {\n"
        "          double acc = 0.0;\n"
        "          for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + c] * qt[i];\n"
        "          ot[c] = acc;\n"
        "        }\n"
        "        token_step(fam, dk, dv, &x, S, NULL, NULL, work);\n"),
    "seam_body_skipped_for_last_segment": (
        "      if (body_S) {\n        apply_T(",
        "      if (body_S && s + 1 < n_seg) {\n        apply_T("),
    "kda_erase_before_decay": (
        "      for (i = 0; i < dk; ++i) {\n"
        "        const double a = exp(x->lgv[i]);\n"
        "        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;\n"
        "      }\n"
        "      for (j = 0; j < dv; ++j) work[j] = 0.0;\n"
        "      for (i = 0; i < dk; ++i)\n"
        "        for (j = 0; j < dv; ++j) work[j] += x->k[i] * S[(size_t)i * dv + j];\n"
        "      for (i = 0; i < dk; ++i)\n"
        "        for (j = 0; j < dv; ++j)\n"
        "          S[(size_t)i * dv + j] += x->beta * x->k[i] * (x->v[j] - work[j]);\n",
        "      for (j = 0; j < dv; ++j) work[j] = 0.0;\n"
        "      for (i = 0; i < dk; ++i)\n"
        "        for (j = 0; j < dv; ++j) work[j] += x->k[i] * S[(size_t)i * dv + j];\n"
        "      for (i = 0; i < dk; ++i)\n"
        "        for (j = 0; j < dv; ++j)\n"
        "          S[(size_t)i * dv + j] -= x->beta * x->k[i] * work[j];\n"
        "      for (i = 0; i < dk; ++i) {\n"
        "        const double a = exp(x->lgv[i]);\n"
        "        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;\n"
        "      }\n"
        "      for (i = 0; i < dk; ++i)\n"
        "        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += x->beta * x->k[i] * x->v[j];\n"),
    "kda_scale_not_moved_into_g": (
        "        if (g) g[0] += m;",
        "        if (g) g[0] += 0.0;"),
    "kda_gate_of_wrong_channel": (
        "          const double a = exp(x->lgv[i] - m);",
        "          const double a = exp(x->lgv[dk - 1 - i] - m);"),
    "rope_sin_sign": (
        "R[(2 * i) * dk + 2 * i + 1] = -sn;",
        "R[(2 * i) * dk + 2 * i + 1] = sn;"),
    "rope_frequency_exponent": (
        "pow(base, -2.0 * i / dk)",
        "pow(base, -1.0 * i / dk)"),
    "rope_transition_rotated_on_one_side": (
        "acc += tmp[(size_t)i * dk + j] * R[c * dk + j];",
        "acc += tmp[(size_t)i * dk + j] * (j == c);"),
    "rope_offset_of_wrong_segment": (
        "rope_matrix(R, dk, delta[u / n_chain], base);",
        "rope_matrix(R, dk, delta[u % n_seg], base);"),
}


def _run_mutant(name, tmpdir):
    orig, mutated = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == 1, "snippet for %s not found exactly once" % name
    msrc = os.path.join(tmpdir, name + ".c")
    mlib = os.path.join(tmpdir, name + ".so")
    with open(msrc, "w") as f:
        f.write(src.replace(orig, mutated))
    oracle.compile_to(msrc, mlib)
    env = dict(os.environ, HYPIC_REF_LIB=mlib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda n: _run_mutant(n, tmp), sorted(MUTANTS)))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by the oracle pins: %s" % survivors
    # every run must have failed on a test, not on a crash of the harness
    for n, rc, out in results:
        assert rc == 1, (n, rc, out)
