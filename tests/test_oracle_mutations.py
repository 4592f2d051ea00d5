"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of ``oracle/sv_oracle.c``,
builds that copy with the oracle's own compile line, and runs the named pins
of ``tests/test_oracle_pins.py`` and ``tests/test_oracle_tree.py`` against it
in a child process: the pins must fail.  The unmutated oracle passing the same pins is the ordinary pin run.
Nothing here touches the GPU library; the planted mistakes live only in a
temporary directory.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sv_oracle.c")

# (id, text in sv_oracle.c, replacement, pins expected to catch it (pytest -k))
MUTATIONS = [
    # decision margins (they decide which GPU/oracle disagreements are excused)
    ("accept-margin-zero", "margin = fabs(u - fmin(1.0, rho));", "margin = 0.0;", "accept_margin"),
    ("accept-margin-no-min", "margin = fabs(u - fmin(1.0, rho));", "margin = fabs(u - rho);", "accept_margin"),
    ("draw-margin-zero", "*margin = fmin(t - prev, run - t) / W;", "*margin = 0.0;", "draw_margin"),
    ("draw-margin-no-div-W", "*margin = fmin(t - prev, run - t) / W;", "*margin = fmin(t - prev, run - t);",
     "draw_margin"),
    ("topp-margin-zero", "out->margin = fmin(fabs(c_gt - top_p), fabs(c_ge - top_p));", "out->margin = 0.0;",
     "topp_margin"),
    ("topp-margin-ge-only", "out->margin = fmin(fabs(c_gt - top_p), fabs(c_ge - top_p));",
     "out->margin = fabs(c_ge - top_p);", "topp_margin"),
    ("topp-margin-gt-only", "out->margin = fmin(fabs(c_gt - top_p), fabs(c_ge - top_p));",
     "out->margin = fabs(c_gt - top_p);", "topp_margin"),
    # the method itself
    ("residual-from-p", "wbuf[v] = p - q > 0.0 ? p - q : 0.0;", "wbuf[v] = p;", "chi2_residual or draw_margin"),
    ("no-posterior-update",
     "if (i < Lr)\n            for (int32_t z = 0; z < K; ++z) logpost[z] += orc_branch_logq(&mx, z, i, x[i]);",
     "if (i < Lr) {}", "posterior_brute_force"),
    ("topp-cut-shifted", "cut = it[k].v;", "cut = it[k + 1 < V ? k + 1 : k].v;", "row_stats_vs_library or two_level"),
    ("accept-u-below-p", "accept = u < rho;", "accept = u < p;", "chi2_dense or expected_accepted"),
    ("dvl-ties-reversed", "if (x->r != y->r) return x->r < y->r ? -1 : 1;",
     "if (x->r != y->r) return x->r > y->r ? -1 : 1;", "dvl_special_cases"),
    ("lse-without-temperature", "S += exp(orc_val(row, dtype, v) / T - M);\n  double lse = M + log(S);",
     "S += exp(orc_val(row, dtype, v) - m);\n  double lse = m + log(S);", "row_stats_vs_library"),
    ("draw-from-next-slot", "const int32_t j = n_acc;", "const int32_t j = n_acc < Lr ? n_acc + 1 : n_acc;",
     "chi2_residual or greedy_is_longest"),
    # tree verification
    ("tree-no-residual-between-siblings",
     "const double px = have_res ? pcur[x] : orc_p_of(trow, in->dtype, x, T, &st);",
     "const double px = orc_p_of(trow, in->dtype, x, T, &st);", "tree"),
    ("tree-final-draw-from-p", "        if (!(W > 0.0))\n          for (int32_t v = 0; v < V; ++v) wbuf[v] = orc_p_of",
     "        if (1)\n          for (int32_t v = 0; v < V; ++v) wbuf[v] = orc_p_of", "tree"),
    ("tree-draft-row-of-the-child", "in->draft_row0[r] + depth[u], in->draft_ld);",
     "in->draft_row0[r] + depth[u] + 1, in->draft_ld);", "tree"),
    ("tree-uniform-counter-shifted", "orc_words_at(in->seed, r, j - 1, w4);", "orc_words_at(in->seed, r, j, w4);",
     "tree"),
]


@pytest.mark.parametrize("name,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_its_pins(name, old, new, pins, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    mutated = tmp_path / "sv_oracle.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    hdr = os.path.join(ROOT, "oracle")
    cmd = oracle.compile_command(str(mutated), str(lib))
    cmd.insert(1, f"-I{hdr}")
    subprocess.check_call(cmd)
    env = dict(os.environ, SV_ORACLE_LIB=str(lib))
    run = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          os.path.join(ROOT, "tests", "test_oracle_tree.py"), "-k", pins],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = run.stdout[-1500:]
    assert "passed" in tail or "failed" in tail, tail
    assert run.returncode == 1, f"planted mistake {name} passed the pins '{pins}':\n{tail}"
