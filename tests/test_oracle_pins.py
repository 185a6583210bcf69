"""The CPU oracle against its pins (no GPU).  See oracle_pins.py."""
import os
import re
import tempfile

import pytest

import oracle
import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_QUICK, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_accept_example_full_grid():
    pins.check_accept_example_grid()


def test_grid_one_decision_full():
    pins.check_grid_one_decision_full()


def test_config0_chi_square_2e20():
    pins.check_config0_chi_square()


def test_oracle_under_sanitizers():
    """The oracle built with gcc's address and undefined-behaviour
    sanitizers (host code only) passes every quick pin: no out-of-bounds
    access, use after free or undefined arithmetic in the oracle's C."""
    import subprocess
    import sys
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's address sanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        so = oracle.build(out=os.path.join(d, "san.so"),
                          flags=("-O1", "-g", "-fno-omit-frame-pointer",
                                 "-fsanitize=address,undefined",
                                 "-fno-sanitize-recover=all"))
        here = os.path.dirname(os.path.abspath(__file__))
        code = ("import sys; sys.path[:0] = [%r, %r]\n"
                "import oracle, oracle_pins as p\n"
                "oracle.use_library(oracle.open_library(%r))\n"
                "for c in p.ALL_QUICK: c()\n"
                "p.check_accept_example_grid(chunk=1 << 18)\n"
                "print('sanitized pins ok')\n" % (here, os.path.dirname(here), so))
        env = dict(os.environ, LD_PRELOAD=asan,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, timeout=900)
        assert r.returncode == 0 and "sanitized pins ok" in r.stdout, r.stderr[-4000:]


# Planted mistakes: each is a plausible slip in the oracle's source.  A copy
# of the source with the slip is compiled and the pins must reject it.
MUTANTS = {
    "residual_q_minus_p": ("double d = p[i] - q[i];", "double d = q[i] - p[i];"),
    "ratio_inverted": ("if (qx > 0.0) return px / qx;", "if (qx > 0.0) return qx / px;"),
    "draw_not_strict": ("if (C > theta) {", "if (C >= theta) {"),
    "uniform_words_swapped": ("*u_acc = (double)(w[0] >> 40)", "*u_acc = (double)(w[1] >> 40)"),
    "philox_constant": ("0xD2E7470EE14C6C93ULL", "0xD2E7470EE14C6C95ULL"),
    "greedy_last_tie": ("if (v[i] > v[best]) best = i;", "if (v[i] >= v[best]) best = i;"),
    "temperature_ignored": ("p[i] = exp((logits[i] - m) / T);", "p[i] = exp((logits[i] - m));"),
    "no_stop_at_rejection": ("rejected = 1;\n        break;", "rejected = 1;"),
    "onehot_x_not_zeroed": ("if (x >= 0 && x < V) r[x] = 0.0;", "(void)x;"),
    "bonus_from_draft": ("memcpy(r, p, sizeof(double) * (size_t)V);\n      }\n      double u = u_rec",
                         "memcpy(r, p, sizeof(double) * (size_t)V);\n        if (mode == SVO_MODE_PROB && n > 0) { load_row(draft, draft_dtype, drow0 + n - 1, V, dl); svo_softmax(dl, V, (double)T, r); }\n      }\n      double u = u_rec"),
    "draft_counter_word": ("uint64_t ctr[4] = {offset, b, j, 1};", "uint64_t ctr[4] = {offset, b, j, 0};"),
    "draft_temperature_ignored": ("svo_softmax(l, V, (double)T, q);", "svo_softmax(l, V, 1.0, q);"),
    "draft_rows_past_n": ("      if (j < n) {", "      if (j <= n && j < K) {"),
    "draft_same_uniform_all_rows": ("(uint64_t)b, (uint64_t)j),\n", "(uint64_t)b, 0),\n"),
    "ngram_earliest_occurrence": ("for (int e = N - 2; e >= n - 1; --e) {", "for (int e = n - 1; e <= N - 2; ++e) {"),
    "ngram_shortest_first": ("for (int n = max_n; n >= min_n && start < 0; --n) {",
                             "for (int n = min_n; n <= max_n && start < 0; ++n) {"),
    "ngram_self_match": ("for (int e = N - 2; e >= n - 1; --e) {", "for (int e = N - 1; e >= n - 1; --e) {"),
    "ngram_no_length_limit": ("if (count > max_model_len - N) count = max_model_len - N;", ""),
    "typical_rank_off_by_one": ("if (valid && above < top_k) {", "if (valid && above <= top_k) {"),
    "typical_threshold_on_logit": ("const double px = valid ? p[x] : 0.0;", "const double px = valid ? l[x] : 0.0;"),
    "typical_no_stop": ("      if (!accept) break;\n      n_acc++;", "      if (accept) n_acc++;"),
    "typical_draw_from_bonus_row": ("load_row(target, target_dtype, row0 + n_acc, V, l);",
                                    "load_row(target, target_dtype, row0 + n, V, l);"),
    "tree_no_residual_update": ("          ck += Zk;\n", "          (void)ck;\n"),
    "tree_onehot_no_renormalize": ("ratio = removed[x] ? 0.0 : p[x] / Zk;", "ratio = removed[x] ? 0.0 : p[x];"),
    "tree_children_reversed": ("for (int c = v + 1; c < n && next < 0; ++c) {",
                               "for (int c = n - 1; c > v && next < 0; --c) {"),
    "tree_uniform_of_node": ("(uint64_t)(c - 1), &ua, &ur);", "(uint64_t)c, &ua, &ur);"),
    # the margins that decide which requests the parity rule lets differ
    "draw_margin_zero": ("*margin = (lo < hi ? lo : hi) / S;", "*margin = 0.0;"),
    "draw_margin_not_over_total": ("*margin = (lo < hi ? lo : hi) / S;",
                                   "*margin = (lo < hi ? lo : hi);"),
    "accept_margin_zero": ("out_margin_acc[(size_t)b * K + j] = fabs(u - ratio);",
                           "out_margin_acc[(size_t)b * K + j] = 0.0;"),
    "accept_margin_wrong_uniform": ("out_margin_acc[(size_t)b * K + j] = fabs(u - ratio);",
                                    "out_margin_acc[(size_t)b * K + j] = fabs(u_rec[(size_t)b * (K + 1) + j] - ratio);"),
    "tree_probs_softmaxed": ("if (!draft_is_probs) svo_softmax(q, V, (double)T, q);",
                             "svo_softmax(q, V, (double)T, q);"),
    # evaluation along a given path (the checks of flagged requests)
    "interval_through_token": ("for (int i = 0; i < y; ++i) C += r[i];",
                               "for (int i = 0; i <= y; ++i) C += r[i];"),
    "path_stop_not_decided": ("for (int j = 0; j <= n_path && j < n; ++j) {",
                              "for (int j = 0; j < n_path && j < n; ++j) {"),
    "path_draw_uniform_of_row0": ("path_emit(r, V, u_rec[n_path], y, out_tok, out_margin_rec, out_y);",
                                  "path_emit(r, V, u_rec[0], y, out_tok, out_margin_rec, out_y);"),
    "path_bonus_drops_token0": ("svo_residual(p, q, mode, draft_ids[n_path], V, r);\n    } else {\n      memcpy(r, p,",
                                 "svo_residual(p, q, mode, draft_ids[n_path], V, r);\n    } else {\n      memset(r, 0, sizeof(double)); memcpy(r + 1, p + 1, sizeof(double) * (size_t)(V - 1)); (void)("),
    "tree_path_outcome": ("out_tests[4 * nt + 1] = c == next;", "out_tests[4 * nt + 1] = 0;"),
    "tree_path_no_residual_update": ("        ck += Zk;\n        for (int i = 0; i < V; ++i) {\n          const double d",
                                     "        for (int i = 0; i < V; ++i) {\n          const double d"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    # a site that occurs in a walk and in its path copy is changed in both
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = oracle.open_library(oracle.build(src=path, out=os.path.join(d, "m.so"),
                                               flags=("-Wno-error",)))
        oracle.use_library(lib)
        caught = []
        try:
            for check in pins.ALL_QUICK:
                try:
                    check()
                except AssertionError:
                    caught.append(check.__name__)
        finally:
            oracle.use_library(None)
    assert caught, f"no pin caught the planted mistake {name}"
