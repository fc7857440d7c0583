"""Mutation sweep of the CPU oracle (CPU only, no GPU).

Each mutant plants one plausible mistake in a copy of oracle/oracle.c - a
dropped term, a wrong sign, index or comparison, a transposed operand, a
missing max subtraction, a misread threshold - builds it with gcc into a
temporary library, and runs the oracle pins (tests/test_oracle_pins.py)
against that library in a child process (ORACLE_LIB names it).  The sweep
passes when every mutant makes at least one pin fail, i.e. no such mistake can
hide behind the pins.  The original source must pass the same pins (the
control run).
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement): each text occurs exactly once.
MUTANTS = [
    ("score_min_not_max", "s += (a > b) ? a : b;", "s += (a < b) ? a : b;"),
    ("score_max_read_as_min", "double b = qc * widen(mx[i * d + c]);",
     "double b = qc * widen(mn[i * d + c]);"),
    ("group_score_head0_only", "if (s > best) best = s;", "if (h == 0) best = s;"),
    ("summary_min_compare_flipped", "if (widen(x) < widen(lo)) lo = x;",
     "if (widen(x) > widen(lo)) lo = x;"),
    ("window_off_by_one", "if (j >= N - (int64_t)W) return 1;",
     "if (j > N - (int64_t)W) return 1;"),
    ("sinks_dropped", "if (j < (int64_t)n_s) return 1;", "if (j < 0) return 1;"),
    ("candidate_test_negated", "if (!oracle_in_dense(j, N, n_s, W)) any = 1;",
     "if (oracle_in_dense(j, N, n_s, W)) any = 1;"),
    ("budget_floor_not_ceil", "int64_t k = (budget_ppm * N + den - 1) / den;",
     "int64_t k = (budget_ppm * N) / den;"),
    ("flag_without_block_size", "return maw * (double)n_dense > beta * (double)S;",
     "return maw * (double)n_dense > beta;"),
    ("flag_without_dense_count", "return maw * (double)n_dense > beta * (double)S;",
     "return maw > beta * (double)S;"),
    ("tie_break_index_desc", "return a < b ? -1 : (a > b ? 1 : 0);\n}\n\nstatic int cmp_int32",
     "return a > b ? -1 : (a < b ? 1 : 0);\n}\n\nstatic int cmp_int32"),
    ("flag_ranked_last", "return g_order.flag[a] > g_order.flag[b] ? -1 : 1;",
     "return g_order.flag[a] > g_order.flag[b] ? 1 : -1;"),
    ("softmax_scale_dropped", "s[t] = scale * acc;", "s[t] = acc;"),
    ("lse_without_max", "lse[h] = mx + log(z);", "lse[h] = log(z);"),
    ("output_reads_keys", "const uint16_t *vr = V + tok[t] * ldv;",
     "const uint16_t *vr = K + tok[t] * ldk;"),
    ("fusion_weight_from_max", "double w = exp(lse_parts[i] - *lse);",
     "double w = exp(lse_parts[i] - m);"),
    ("decay_swapped", "maw[i] = r * maw[i] + (1.0 - r) * a[i];\n}\n\n/* One MAW step",
     "maw[i] = (1.0 - r) * maw[i] + r * a[i];\n}\n\n/* One MAW step"),
    ("maw_step_updates_every_block", "if (inside) maw[i] = r * maw[i] + (1.0 - r) * a[i];",
     "maw[i] = r * maw[i] + (1.0 - r) * a[i];"),
    ("maw_step_decays_outside_dense",
     "if (inside) maw[i] = r * maw[i] + (1.0 - r) * a[i];",
     "maw[i] = inside ? r * maw[i] + (1.0 - r) * a[i] : r * maw[i];"),
    ("maw_step_updates_blocks_touching_dense",
     "if (!oracle_in_dense(j, N, n_s, W)) inside = 0;",
     "if (oracle_in_dense(j, N, n_s, W)) inside = 2;\n    inside = inside == 2;"),
    ("dense_mass_head0_only", "a_blk[tok[tt] / S] += p[(int64_t)h * nD + tt] / (double)G;",
     "a_blk[tok[tt] / S] += p[tt] / (double)G;"),
    ("dense_mass_not_averaged", "a_blk[tok[tt] / S] += p[(int64_t)h * nD + tt] / (double)G;",
     "a_blk[tok[tt] / S] += p[(int64_t)h * nD + tt];"),
    ("dense_mass_block_index", "a_blk[tok[tt] / S] += p[(int64_t)h * nD + tt] / (double)G;",
     "a_blk[tt / S] += p[(int64_t)h * nD + tt] / (double)G;"),
    ("select_heads_group_of_all", "k = oracle_select(q + (int64_t)h * d, 1, d,",
     "k = oracle_select(q, G, d,"),
    ("select_heads_first_head_only", "k = oracle_select(q + (int64_t)h * d, 1, d,",
     "k = oracle_select(q, 1, d,"),
    ("attend_heads_first_selection", "sel + (int64_t)h * ld_sel, k[h], scale,",
     "sel, k[0], scale,"),
    ("lfps_growth_offsets_mirrored", "int64_t c = i - e;", "int64_t c = i + e;"),
    ("lfps_mean_filter_dropped", "inC[i] = (int8_t)(grown && above && cand[i]);",
     "inC[i] = (int8_t)(grown && cand[i]);"),
    ("lfps_slash_offset_from_start",
     "for (int64_t i = 0; i <= b; ++i) c0[i] = (int8_t)(phi_v[i] > tau_v || phi_s[b - i] > tau_s);",
     "for (int64_t i = 0; i <= b; ++i) c0[i] = (int8_t)(phi_v[i] > tau_v || phi_s[i] > tau_s);"),
    ("lfps_threshold_at_max", "double tau_v = mu_v + a * (mx_v - mu_v), tau_s = mu_s + a * (mx_s - mu_s);",
     "double tau_v = mx_v, tau_s = mx_s;"),
    ("lfps_slash_update_unmirrored",
     "for (int64_t o = 0; o <= b; ++o) phi_s[o] = r * phi_s[o] + (1.0 - r) * a_blk[b - o];",
     "for (int64_t o = 0; o <= b; ++o) phi_s[o] = r * phi_s[o] + (1.0 - r) * a_blk[o];"),
    ("lfps_init_not_causal", "for (int64_t j = 0; j <= pos; ++j) tok[j] = j;\n    oracle_attend_tokens(q + (int64_t)u * G * d, G, d, K, ldk, K, ldk, tok, pos + 1,",
     "for (int64_t j = 0; j <= pos; ++j) tok[j] = j;\n    oracle_attend_tokens(q + (int64_t)u * G * d, G, d, K, ldk, K, ldk, tok, pos,"),
    ("attend_mass_first_head_only", "for (int64_t tt = 0; tt < nT; ++tt) a_blk[tok[tt] / S] += p[(int64_t)h * nT + tt] / (double)G;",
     "for (int64_t tt = 0; tt < nT; ++tt) a_blk[tok[tt] / S] += p[tt] / (double)G;"),
    ("selected_block_last_token_dropped",
     "for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S && j < N; ++j)\n      inT[j] = 1;\n  int64_t n_tok = 0;",
     "for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S - 1 && j < N; ++j)\n      inT[j] = 1;\n  int64_t n_tok = 0;"),
    ("attend_mass_selected_block_last_token_dropped",
     "for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S && j < N; ++j)\n      inT[j] = 1;\n  int64_t nT = 0;",
     "for (int64_t j = (int64_t)sel[t] * S; j < ((int64_t)sel[t] + 1) * S - 1 && j < N; ++j)\n      inT[j] = 1;\n  int64_t nT = 0;"),
]


def _build(src_text, out_dir, name):
    c_path = os.path.join(out_dir, name + ".c")
    so_path = os.path.join(out_dir, "lib" + name + ".so")
    with open(c_path, "w") as fh:
        fh.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-w",
                           "-I", os.path.join(ROOT, "oracle"), "-o", so_path, c_path, "-lm"])
    return so_path


def _run_pins(so_path):
    env = dict(os.environ, ORACLE_LIB=so_path)
    p = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    return p.returncode, p.stdout[-2000:]


def test_every_mutant_fails_a_pin():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, "mutant %s: its text occurs %d times" % (name, src.count(old))
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [("control", src)] + [(n, src.replace(old, new)) for n, old, new in MUTANTS]
        libs = {n: _build(t, tmp, n) for n, t in jobs}
        workers = max(1, min(6, (os.cpu_count() or 2) - 1))
        with cf.ThreadPoolExecutor(workers) as ex:
            res = dict(zip(libs, ex.map(_run_pins, libs.values())))
    rc, out = res.pop("control")
    assert rc == 0, "the unmutated oracle must pass the pins:\n" + out
    survivors = [n for n, (rc, _) in res.items() if rc == 0]
    assert not survivors, "mutants that pass every pin: %s" % survivors
