"""Plant plausible mistakes in copies of the oracle: every copy must fail a pin.

Each mutant is oracle.c with one textual change (a dropped term, a sign, an
index, the tie-break, the row numbering), built with gcc into a temporary
directory and run through every pin in a subprocess.  Only the oracle is
mutated, only on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "drop_max_in_lse": ("const double lse = zmax + log(s);", "const double lse = log(s);"),
    "drop_cumulative": ("const double score = cum[k] + logp;", "const double score = logp;"),
    "ascending_scores": ("if (x->score > y->score) return -1;\n  if (x->score < y->score) return 1;",
                         "if (x->score > y->score) return 1;\n  if (x->score < y->score) return -1;"),
    "tie_break_beam_desc": ("return (x->beam < y->beam) ? -1 : 1;", "return (x->beam < y->beam) ? 1 : -1;"),
    "tie_break_token_desc": ("return (x->token < y->token) ? -1 : (x->token > y->token);",
                             "return (x->token > y->token) ? -1 : (x->token < y->token);"),
    "slot_instead_of_token": ("const float* w = W + (int64_t)legal[j] * d;",
                              "const float* w = W + (int64_t)j * d;"),
    "reversed_hidden": ("acc += (double)w[i] * (double)hk[i];",
                        "acc += (double)w[i] * (double)hk[d - 1 - i];"),
    "row_off_by_one": ("c->depth_keys[len][i] == k) ? i : -1;", "c->depth_keys[len][i] == k) ? i + 1 : -1;"),
    "drop_last_child": ("const int64_t hi = lower_bound_u64(a, n, (p + 1) << c->bits);",
                        "const int64_t hi = lower_bound_u64(a, n, (p + 1) << c->bits) - 1;"),
    "denominator_sum_wrong": ("for (int64_t j = 0; j < n; ++j) s += exp(z[j] - zmax);",
                              "for (int64_t j = 1; j < n; ++j) s += exp(z[j] - zmax);"),
    "all_v_max_dropped": ("const double lse_all = zmax_all + log(s_all);",
                          "const double lse_all = log(s_all);"),
    "all_v_sum_skips_first": ("for (int32_t v = 0; v < c->V; ++v) s_all += exp(z[v] - zmax_all);",
                              "for (int32_t v = 1; v < c->V; ++v) s_all += exp(z[v] - zmax_all);"),
    "score_first_keeps_illegal": ("if (mode == 1) {", "if (mode == 3) {"),
    "unconstrained_drops_last_token": ("n = c->V;\n", "n = c->V - 1;\n"),
    "score_first_uses_slot": ("lp[j] = z[legal[j]] - lse_all;", "lp[j] = z[j] - lse_all;"),
    "keep_one_more": ("const int32_t keep = (m_all < K) ? (int32_t)m_all : K;",
                      "const int32_t keep = (m_all < K) ? (int32_t)m_all : K - 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", str(mut), "-lm", "-o", str(so)])
    env = dict(os.environ, ORACLE_LIB=str(so))
    p = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py")], env=env,
                       capture_output=True, text=True, timeout=600)
    last = p.stdout.strip().splitlines()[-1] if p.stdout.strip() else ""
    assert p.returncode != 0, f"mutant {name} passed every pin"
    assert last.startswith("FAILED:") and last != "FAILED: none", p.stdout[-2000:] + p.stderr[-2000:]
