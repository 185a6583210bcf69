"""Pins for the CPU oracle: checks against facts the pages and the mathematics
fix, written so that they can also be run against a deliberately broken copy
of the oracle (see test_oracle_pins.py::test_planted_mistakes_are_caught).

Every check raises AssertionError on failure.  None of them re-types the
oracle's own formulas: they compare with the pages' worked examples, with
numpy / scipy routines the oracle does not use, with exact enumeration of the
output law, with brute force on tiny inputs and with statistical tests.
"""
from __future__ import annotations

import json
import os

import numpy as np
import scipy.special
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Philox4x64-10 against numpy's independent implementation
# --------------------------------------------------------------------------
def _numpy_block(counter, key):
    """numpy's Philox advances its 256-bit counter before producing a block,
    so the block of counter c is the first output of a generator started at
    c - 1."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)]
    g = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                         key=np.array([int(k) for k in key], dtype=np.uint64))
    return g.random_raw(4)


def check_philox_known_answers(n=4000, seed=1234):
    rng = np.random.default_rng(seed)
    counters = [[0, 0, 0, 0], [(1 << 64) - 1, 0, 0, 0],
                [(1 << 64) - 1, (1 << 64) - 1, 7, 0], [5, 6, 7, 8]]
    for _ in range(n):
        counters.append([int(x) for x in rng.integers(0, 1 << 63, 4, dtype=np.uint64)])
    for i, c in enumerate(counters):
        key = [int(rng.integers(0, 1 << 63)), 0] if i % 2 else [i, i * 3]
        ours = oracle.philox4x64_10(c, key)
        ref = _numpy_block(c, key)
        assert np.array_equal(ours, ref), (c, key, ours, ref)


def check_uniform_mapping(n=2000, seed=99):
    """u_acc / u_rec are words 0 / 1 of the block at counter (offset, b, j, 0)
    with key (seed, 0), mapped as (w >> 40) * 2^-24."""
    rng = np.random.default_rng(seed)
    for _ in range(n):
        s, o = (int(x) for x in rng.integers(0, 1 << 62, 2, dtype=np.uint64))
        b, j = int(rng.integers(0, 4096)), int(rng.integers(0, 8))
        w = _numpy_block([o, b, j, 0], [s, 0])
        ua, ur = oracle.uniforms(s, o, b, j)
        assert ua == (int(w[0]) >> 40) / 2.0 ** 24
        assert ur == (int(w[1]) >> 40) / 2.0 ** 24


# --------------------------------------------------------------------------
# The pages' acceptance example: q(x) = 0.4, p(x) = 0.2 -> accept half the time
# --------------------------------------------------------------------------
def _accept_example_inputs(B):
    ex = _golden("accept_worked_example.json")
    p, q = ex["p_x"], ex["q_x"]
    target = np.empty((B, 2, 2), np.float32)
    target[:, 0] = [np.log(p), np.log(1 - p)]   # p_0 = (0.2, 0.8)
    target[:, 1] = [np.log(0.3), np.log(0.7)]   # bonus row p_1 = (0.3, 0.7)
    draft = np.empty((B, 1, 2), np.float32)
    draft[:, 0] = [q, 1 - q]                    # normalized q_0 = (0.4, 0.6)
    return ex, target, draft


def check_accept_example_grid(chunk=1 << 21):
    """Over every u on the 2^24 grid, exactly half (up to the rounding of
    ln / exp, i.e. +-1 grid point) of the decisions accept."""
    ex, target, draft = _accept_example_inputs(chunk)
    accepted = 0
    for start in range(0, 1 << 24, chunk):
        ua = np.zeros((chunk, 2))
        ua[:, 0] = (start + np.arange(chunk)) / 2.0 ** 24
        r = oracle.verify(target, draft, np.zeros((chunk, 1)), np.ones(chunk),
                          np.ones(chunk), draft_is_probs=True, u_acc=ua,
                          u_rec=np.full((chunk, 2), 0.5))
        accepted += int(r["num_accepted"].sum())
        # a rejected x = 0 is replaced by a draw from max(0, p - q) = (0, 0.4)
        rej = r["num_accepted"] == 0
        assert np.all(r["tokens"][rej, 0] == 1)
    expect = ex["accept_probability"] * 2 ** 24
    assert abs(accepted - expect) <= 1, (accepted, expect)


def check_accept_example_philox(B=1 << 20):
    """With Philox uniforms (seed 0, request index b) the acceptance rate is
    0.5 within 3 sigma; rejections always emit token 1; after an acceptance
    the bonus token follows p_1 = (0.3, 0.7)."""
    ex, target, draft = _accept_example_inputs(B)
    r = oracle.verify(target, draft, np.zeros((B, 1)), np.ones(B), np.ones(B),
                      draft_is_probs=True, seed=0, offset=0)
    acc = r["num_accepted"] == 1
    rate = acc.mean()
    sigma = np.sqrt(0.25 / B)
    assert abs(rate - ex["accept_probability"]) < 3 * sigma, rate
    assert np.all(r["tokens"][~acc, 0] == 1)
    bonus0 = (r["tokens"][acc, 1] == 0).mean()
    s2 = np.sqrt(0.21 / acc.sum())
    assert abs(bonus0 - 0.3) < 4 * s2, bonus0


# --------------------------------------------------------------------------
# Greedy (temperature 0): exact match against the target's top-1
# --------------------------------------------------------------------------
def check_bpd_greedy_example():
    ex = _golden("bpd_greedy_example.json")
    vocab = ex["vocab"]
    V, K = len(vocab), len(ex["drafts"])
    rng = np.random.default_rng(7)
    target = rng.normal(0, 1, (1, K + 1, V)).astype(np.float32)
    for j, w in enumerate(ex["target_top1"]):
        target[0, j, vocab.index(w)] = 10.0
    ids = [[vocab.index(w) for w in ex["drafts"]]]
    r = oracle.verify(target, None, ids, [K], [0.0])
    n = int(r["num_accepted"][0])
    toks = [vocab[t] for t in r["tokens"][0, : n + 1]]
    assert toks[:n] == ex["expected_accepted"], toks
    assert toks[n] == ex["expected_emitted"], toks
    assert list(r["tokens"][0, n + 1:]) == [-1] * (K - n)


def check_greedy_bruteforce(cases=300, seed=3):
    """Integer-valued logits (many ties): n_acc is the longest prefix whose
    draft attains the row maximum; the emitted token is numpy's argmax (lowest
    index among ties) of the row after that prefix."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        V = int(rng.choice([1, 2, 3, 5, 8]))
        K = int(rng.integers(0, 5))
        B = 4
        target = rng.integers(-2, 3, (B, K + 1, V)).astype(np.float32)
        ids = rng.integers(0, V, (B, K)).astype(np.int32)
        nd = rng.integers(0, K + 1, B).astype(np.int32)
        T = rng.choice([0.0, -1.0, np.nan], B).astype(np.float32)
        r = oracle.verify(target, None, ids, nd, T)
        for b in range(B):
            n = 0
            while n < nd[b] and target[b, n, ids[b, n]] == target[b, n].max():
                n += 1
            assert r["num_accepted"][b] == n
            assert r["tokens"][b, n] == int(np.argmax(target[b, n]))
            assert np.array_equal(r["tokens"][b, :n], ids[b, :n])
            assert np.all(r["tokens"][b, n + 1:] == -1)


# --------------------------------------------------------------------------
# Exact output law (V = 4, K = 2): every emitted position follows p_j
# --------------------------------------------------------------------------
def _position_law(p, q, mode, x_fixed=None):
    """Law of the token emitted at a position, by enumeration over the draft
    x ~ q (or the fixed one-hot draft), the acceptance probability
    min(1, ratio) and the oracle's residual law r / sum(r)."""
    V = len(p)
    law = np.zeros(V)
    drafts = [(x, q[x]) for x in range(V)] if mode == oracle.MODE_PROB else [(x_fixed, 1.0)]
    for x, wx in drafts:
        if wx == 0:
            continue
        ratio = oracle.accept_ratio(p[x], q[x] if mode == oracle.MODE_PROB else 1.0)
        a = min(1.0, ratio)
        law[x] += wx * a
        if a < 1:
            r = oracle.residual(p, q if mode == oracle.MODE_PROB else None, mode, x)
            law += wx * (1 - a) * r / r.sum()
    return law


def check_enumeration_law(cases=60, seed=11):
    rng = np.random.default_rng(seed)
    for c in range(cases):
        V = 4
        T = float(rng.choice([0.4, 1.0, 1.7]))
        for j in range(2):
            lt = rng.normal(0, 2, V)
            ld = lt + rng.normal(0, 1.5, V)
            p = oracle.softmax(lt, T)
            # the oracle's softmax itself against scipy's
            assert np.allclose(p, scipy.special.softmax(lt / T), rtol=1e-13, atol=0)
            q = oracle.softmax(ld, T)
            law = _position_law(p, q, oracle.MODE_PROB)
            assert np.max(np.abs(law - p)) < 1e-12, (law, p)
            x = int(rng.integers(0, V))
            law1 = _position_law(p, None, oracle.MODE_ONEHOT, x_fixed=x)
            assert np.max(np.abs(law1 - p)) < 1e-12, (law1, p)


def check_grid_law_through_verify(G=1 << 14, seed=5):
    """The same law, but through the full verify entry on a grid of uniforms:
    per draft x0 of a V=4 row, the acceptance count over a u_acc grid and the
    emitted-token histogram over a u_rec grid (forced rejection) rebuild p_0
    within 3/G."""
    rng = np.random.default_rng(seed)
    V, K = 4, 2
    lt = rng.normal(0, 2, (K + 1, V)).astype(np.float32)
    ld = (lt[:K] + rng.normal(0, 1.5, (K, V))).astype(np.float32)
    p0 = scipy.special.softmax(lt[0].astype(np.float64))
    q0 = scipy.special.softmax(ld[0].astype(np.float64))
    grid = np.arange(G) / G
    law = np.zeros(V)
    for x0 in range(V):
        target = np.broadcast_to(lt, (G, K + 1, V)).copy()
        draft = np.broadcast_to(ld, (G, K, V)).copy()
        ids = np.tile([[x0, 0]], (G, 1))
        ua = np.zeros((G, K + 1)); ua[:, 0] = grid; ua[:, 1] = 0.0
        ur = np.full((G, K + 1), 0.25)
        r = oracle.verify(target, draft, ids, np.full(G, 2), np.ones(G),
                          u_acc=ua, u_rec=ur)
        acc = (r["num_accepted"] >= 1).mean()
        ua2 = np.full((G, K + 1), 1.0 - 2.0 ** -24)
        ur2 = np.zeros((G, K + 1)); ur2[:, 0] = grid
        r2 = oracle.verify(target, draft, ids, np.full(G, 2), np.ones(G),
                           u_acc=ua2, u_rec=ur2)
        if (r2["num_accepted"] == 0).all():
            hist = np.bincount(r2["tokens"][:, 0], minlength=V) / G
        else:
            hist = np.zeros(V)  # ratio >= 1: never rejected
        law[x0] += q0[x0] * acc
        law += q0[x0] * (1 - acc) * hist
    assert np.max(np.abs(law - p0)) < 3.0 / G, (law, p0)


# --------------------------------------------------------------------------
# Monte Carlo: first and second emitted tokens, acceptance rate closed form
# --------------------------------------------------------------------------
def _chisq_ok(counts, probs, alpha=1e-3):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return scipy.stats.chisquare(obs, ex).pvalue > alpha


def check_monte_carlo(B=1 << 20, V=8, T=0.7, seed=21):
    rng = np.random.default_rng(seed)
    K = 2
    lt = rng.normal(0, 2, (K + 1, V)).astype(np.float32)
    ld = (lt[:K] + rng.normal(0, 1.0, (K, V))).astype(np.float32)
    p = [scipy.special.softmax(lt[j].astype(np.float64) / T) for j in range(K + 1)]
    q = [scipy.special.softmax(ld[j].astype(np.float64) / T) for j in range(K)]
    # drafts drawn from q_j with a generator of the test's own
    ids = np.stack([rng.choice(V, B, p=q[j]) for j in range(K)], 1).astype(np.int32)
    target = np.broadcast_to(lt, (B, K + 1, V)).copy()
    draft = np.broadcast_to(ld, (B, K, V)).copy()
    r = oracle.verify(target, draft, ids, np.full(B, K), np.full(B, T),
                      seed=seed, offset=3)
    first = r["tokens"][:, 0]
    assert _chisq_ok(np.bincount(first, minlength=V), p[0])
    reached = r["num_accepted"] >= 1
    second = r["tokens"][reached, 1]
    assert _chisq_ok(np.bincount(second, minlength=V), p[1])
    # P(accept at 0) = sum_x min(p(x), q(x)) = 1 - TV(p, q)
    pa = np.minimum(p[0], q[0]).sum()
    rate = reached.mean()
    assert abs(rate - pa) < 4 * np.sqrt(pa * (1 - pa) / B), (rate, pa)


def check_monte_carlo_onehot(B=1 << 18, V=6, T=1.3, seed=8):
    rng = np.random.default_rng(seed)
    K = 1
    lt = rng.normal(0, 1.5, (K + 1, V)).astype(np.float32)
    p0 = scipy.special.softmax(lt[0].astype(np.float64) / T)
    x = int(np.argsort(p0)[-2])
    target = np.broadcast_to(lt, (B, K + 1, V)).copy()
    r = oracle.verify(target, None, np.full((B, K), x), np.full(B, K),
                      np.full(B, T), seed=seed, offset=0)
    assert _chisq_ok(np.bincount(r["tokens"][:, 0], minlength=V), p0)
    rate = (r["num_accepted"] == 1).mean()
    assert abs(rate - p0[x]) < 4 * np.sqrt(p0[x] * (1 - p0[x]) / B)


# --------------------------------------------------------------------------
# Special cases that reduce to library routines, and invariants
# --------------------------------------------------------------------------
def check_no_draft_is_plain_sampling(cases=200, seed=31):
    """n_b = 0: the step is one inverse-CDF draw from softmax(l/T), i.e.
    searchsorted(cumsum(p), u * sum(p), 'right') with scipy's softmax."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        V = int(rng.integers(1, 300))
        T = float(rng.uniform(0.2, 2.0))
        l = rng.normal(0, 3, (1, 1, V)).astype(np.float32)
        r = oracle.verify(l, None, np.zeros((1, 0)), [0], [T], seed=c, offset=c)
        p = scipy.special.softmax(l[0, 0].astype(np.float64) / T)
        _, u = oracle.uniforms(c, c, 0, 0)
        cdf = np.cumsum(p)
        y = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        if r["margin_rec"][0] > 1e-9:
            assert r["tokens"][0, 0] == y, (r["tokens"], y)
        assert r["num_accepted"][0] == 0


def check_identical_draft_always_accepted(seed=41):
    """q = p (draft logits equal to target logits): ratio is exactly 1, so
    every draft is accepted and the bonus row is sampled."""
    rng = np.random.default_rng(seed)
    B, K, V = 64, 5, 50
    lt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    ids = rng.integers(0, V, (B, K)).astype(np.int32)
    r = oracle.verify(lt, lt[:, :K].copy(), ids, np.full(B, K),
                      rng.uniform(0.3, 2, B), seed=1, offset=2)
    assert np.all(r["num_accepted"] == K)


def check_certain_onehot_always_accepted(seed=43):
    rng = np.random.default_rng(seed)
    B, K, V = 32, 3, 40
    lt = np.full((B, K + 1, V), -100.0, np.float32)
    ids = rng.integers(0, V, (B, K)).astype(np.int32)
    for b in range(B):
        for j in range(K):
            lt[b, j, ids[b, j]] = 100.0
    lt[:, K, 0] = 0.0
    r = oracle.verify(lt, None, ids, np.full(B, K), np.ones(B), seed=2)
    assert np.all(r["num_accepted"] == K)


def check_zero_mass_never_drawn():
    """The inverse CDF skips tokens of zero mass even at u = 0."""
    y, _ = oracle.draw(np.array([0.0, 0.0, 0.5, 0.5]), 0.0)
    assert y == 2
    y, _ = oracle.draw(np.array([0.3, 0.0, 0.7, 0.0]), 1.0 - 2.0 ** -24)
    assert y == 2


def check_invariants(seed=51):
    """0 <= n_acc <= n_b, accepted prefix = drafts, one emitted token then -1
    padding, a rejected sampling draft is never re-emitted, and NaN padding
    rows are never read."""
    import torch
    import synth
    for i, kw in enumerate([dict(temps=(1.0, 0.0, 0.6), n_mode="ragged"),
                            dict(temps=(0.8,), onehot_frac=0.5, n_mode="ragged"),
                            dict(temps=(1.2, 0.0), dtype=torch.bfloat16),
                            dict(temps=(0.9,), draft_is_probs=True)]):
        w = synth.make_random(48, 6, 300, seed=seed + i, **kw)
        h = w.host_arrays()
        r = oracle.verify(h["target"], h["draft"], h["draft_ids"],
                          h["num_drafts"], h["temperatures"],
                          draft_mode=h["draft_mode"],
                          draft_is_probs=h["draft_is_probs"], seed=i, offset=7)
        assert r["flags"] == 0
        for b in range(w.B):
            n = int(r["num_accepted"][b]); nb = int(h["num_drafts"][b])
            assert 0 <= n <= nb
            assert np.array_equal(r["tokens"][b, :n], h["draft_ids"][b, :n])
            y = int(r["tokens"][b, n])
            assert 0 <= y < w.V
            assert np.all(r["tokens"][b, n + 1:] == -1)
            if n < nb and oracle.is_sampling(h["temperatures"][b]):
                assert y != h["draft_ids"][b, n]


# --------------------------------------------------------------------------
# Draft-token sampler
# --------------------------------------------------------------------------
def check_draft_uniform_mapping(n=2000, seed=7):
    """The sampler's uniform is word 0 of the block at counter
    (offset, b, j, 1) with key (seed, 0), mapped as (w >> 40) * 2^-24."""
    rng = np.random.default_rng(seed)
    for _ in range(n):
        s, o = (int(x) for x in rng.integers(0, 1 << 62, 2, dtype=np.uint64))
        b, j = int(rng.integers(0, 4096)), int(rng.integers(0, 32))
        w = _numpy_block([o, b, j, 1], [s, 0])
        assert oracle.draft_uniform(s, o, b, j) == (int(w[0]) >> 40) / 2.0 ** 24


def _greedy_temperature(T):
    T = np.float32(T)
    return not (np.isfinite(T) and T >= np.finfo(np.float32).tiny)


def check_draft_sample_vs_library(cases=120, seed=61):
    """Every sampled row equals an independent computation: scipy's softmax
    of l/T, numpy's Philox for the uniform, searchsorted over the cumulative
    sum.  Greedy rows equal np.argmax (lowest index on ties) with q = 1; rows
    past n_b are -1; an out-of-range count is clamped and flagged."""
    rng = np.random.default_rng(seed)
    temps_pool = [1.0, 0.7, 1.6, 0.05, 0.0, -1.0, float("nan"), 1e-40]
    for c in range(cases):
        B, K, V = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 300))
        l = rng.normal(0, 3, (B, K, V)).astype(np.float32)
        if c % 3 == 0:
            l = np.round(l)  # integer logits: ties for the greedy rows
        temps = np.array([temps_pool[i] for i in rng.integers(0, len(temps_pool), B)],
                         dtype=np.float32)
        nd = rng.integers(0, K + 1, B).astype(np.int32)
        bad = c % 10 == 5
        if bad:
            nd[0] = K + 2
        r = oracle.draft_sample(l, nd, temps, seed=c, offset=3 * c)
        assert r["flags"] == (2 if bad else 0)
        for b in range(B):
            n = min(int(nd[b]), K)
            for j in range(K):
                x, qx = int(r["ids"][b, j]), r["q"][b, j]
                if j >= n:
                    assert x == -1 and np.isnan(qx)
                    continue
                row = l[b, j].astype(np.float64)
                if _greedy_temperature(temps[b]):
                    assert x == int(np.argmax(row)) and qx == 1.0
                    continue
                p = scipy.special.softmax(row / float(temps[b]))
                w = _numpy_block([3 * c, b, j, 1], [c, 0])
                u = (int(w[0]) >> 40) / 2.0 ** 24
                cdf = np.cumsum(p)
                y = min(int(np.searchsorted(cdf, u * cdf[-1], side="right")), V - 1)
                if r["margin"][b, j] > 1e-9:
                    assert x == y, (c, b, j, x, y)
                assert abs(qx - p[x]) <= 1e-12 * p[x] + 1e-300


def check_draft_sample_monte_carlo(B=1 << 17, V=8, T=0.8, seed=71):
    """One draft row repeated over B requests (each has its own Philox
    counter): the histogram of the sampled tokens follows softmax(l/T), at
    both positions of a two-position draft."""
    rng = np.random.default_rng(seed)
    l1 = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    l = np.broadcast_to(l1, (B, 2, V)).copy()
    r = oracle.draft_sample(l, None, np.full(B, T, np.float32), seed=seed,
                            offset=1, diagnostics=False)
    for j in range(2):
        q = scipy.special.softmax(l1[j].astype(np.float64) / T)
        assert _chisq_ok(np.bincount(r["ids"][:, j], minlength=V), q), j


# --------------------------------------------------------------------------
# n-gram prompt-lookup proposer
# --------------------------------------------------------------------------
def _rfind_propose(tokens, N, min_n, max_n, k, max_model_len):
    """The same rule through CPython's string search: tokens become code
    points, and str.rfind over s[0:N-1] gives the latest occurrence of each
    suffix that ends before the last token."""
    s = "".join(chr(0x100 + int(t)) for t in tokens[:N])
    for n in range(min(max_n, N - 1), min_n - 1, -1):
        pos = s.rfind(s[N - n:], 0, N - 1)
        if pos >= 0:
            start = pos + n
            count = max(0, min(k, N - start, max_model_len - N))
            return [int(t) for t in tokens[start:start + count]]
    return []


def check_ngram_golden():
    ex = _golden("ngram_lookup_example.json")
    d, n = oracle.ngram_propose(np.array([ex["context"]]), [len(ex["context"])],
                                min_n=ex["min_n"], max_n=ex["max_n"], k=ex["k"],
                                max_model_len=ex["max_model_len"])
    assert int(n[0]) == ex["num_drafts"] and d[0, :n[0]].tolist() == ex["drafts"], (d, n)


def check_ngram_vs_rfind(cases=400, seed=81):
    rng = np.random.default_rng(seed)
    for c in range(cases):
        B, stride = int(rng.integers(1, 5)), int(rng.integers(1, 120))
        alphabet = int(rng.integers(2, 9))
        ctx = rng.integers(0, alphabet, (B, stride)).astype(np.int32)
        lens = rng.integers(0, stride + 1, B).astype(np.int32)
        min_n = int(rng.integers(1, 4))
        max_n = min_n + int(rng.integers(0, 5))
        k = int(rng.integers(1, 8))
        mml = int(rng.integers(1, 2 * stride + 2))
        d, n = oracle.ngram_propose(ctx, lens, min_n=min_n, max_n=max_n, k=k, max_model_len=mml)
        for b in range(B):
            ref = _rfind_propose(ctx[b], int(lens[b]), min_n, max_n, k, mml)
            assert int(n[b]) == len(ref) and d[b, :n[b]].tolist() == ref, (c, b, ref, d[b], n[b])
            assert np.all(d[b, n[b]:] == -1)


def check_ngram_edge_cases():
    prop = lambda ctx, N, **kw: oracle.ngram_propose(np.array([ctx]), [N], **kw)
    kw = dict(min_n=1, max_n=4, k=3, max_model_len=100)
    for N in (0, 1):  # nothing to match against
        assert prop([4, 4, 4], N, **kw)[1][0] == 0
    assert prop([1, 2, 3, 4, 5], 5, **kw)[1][0] == 0            # no repeated token
    d, n = prop([7, 7, 7, 7], 4, **kw)                          # overlapping occurrence
    assert n[0] == 1 and d[0, 0] == 7
    d, n = prop([1, 2, 9, 1, 2], 5, **kw)                       # only 3 tokens follow
    assert n[0] == 3 and d[0].tolist() == [9, 1, 2]
    d, n = prop([1, 2, 9, 1, 2], 5, min_n=1, max_n=4, k=3, max_model_len=6)
    assert n[0] == 1 and d[0].tolist() == [9, -1, -1]           # stops at max_model_len
    assert prop([1, 2, 9, 1, 2], 5, min_n=1, max_n=4, k=3, max_model_len=5)[1][0] == 0
    assert prop([1, 2, 9, 1, 2], 5, min_n=3, max_n=4, k=3, max_model_len=100)[1][0] == 0
    d, n = prop([3, 1, 5, 3, 1, 6, 3, 1], 8, **kw)              # latest of equal matches
    assert n[0] == 3 and d[0].tolist() == [6, 3, 1]


# --------------------------------------------------------------------------
# Typical acceptance
# --------------------------------------------------------------------------
def check_typical_golden():
    ex = _golden("typical_acceptance_example.json")
    t = np.log(np.array(ex["probs"], dtype=np.float64)).astype(np.float32)[None]
    for case in ex["cases"]:
        r = oracle.verify_typical(t, np.array([ex["draft_ids"]]), [2], [1.0],
                                  eps=ex["eps"], top_k=case["top_k"])
        assert r["num_accepted"][0] == case["num_accepted"], (case, r["num_accepted"])


def _typical_case(rng, B, K, V):
    t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    ids = rng.integers(0, V, (B, K)).astype(np.int32)
    top = np.argsort(-t[:, :K], axis=-1)[..., :3]  # some drafts among the top tokens
    pick = rng.random((B, K)) < 0.6
    ids = np.where(pick, np.take_along_axis(top, rng.integers(0, 3, (B, K, 1)), -1)[..., 0], ids)
    nd = rng.integers(0, K + 1, B).astype(np.int32)
    return t, ids.astype(np.int32), nd


def check_typical_vs_library(cases=60, seed=91):
    """Acceptances, the accepted prefix and the emitted token against numpy /
    scipy: accept iff softmax(l/T)[x] > eps or #{l_i > l_x} < top_k; the
    emitted token is searchsorted over p's cumulative sum (skipping draws
    within 1e-9 of a boundary and decisions within 1e-12 of eps)."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        B, K, V = int(rng.integers(1, 6)), int(rng.integers(1, 6)), int(rng.integers(2, 200))
        t, ids, nd = _typical_case(rng, B, K, V)
        temps = rng.choice([1.0, 0.6, 1.5, 0.0], B).astype(np.float32)
        eps, top_k = float(rng.choice([0.0, 0.01, 0.05, 0.2, 1.0])), int(rng.integers(0, 4))
        r = oracle.verify_typical(t, ids, nd, temps, eps=eps, top_k=top_k, seed=c, offset=c)
        for b in range(B):
            T = float(temps[b])
            n_acc, ambiguous = 0, False
            for j in range(int(nd[b])):
                row, x = t[b, j].astype(np.float64), int(ids[b, j])
                if T == 0.0:
                    ok = row[x] == row.max()
                else:
                    p = scipy.special.softmax(row / T)
                    ok = p[x] > eps or int(np.sum(row > row[x])) < top_k
                    if abs(p[x] - eps) < 1e-12 and int(np.sum(row > row[x])) >= top_k:
                        ambiguous = True
                        break
                if not ok:
                    break
                n_acc += 1
            if ambiguous:
                continue
            assert r["num_accepted"][b] == n_acc, (c, b, r["num_accepted"][b], n_acc)
            assert np.array_equal(r["tokens"][b, :n_acc], ids[b, :n_acc])
            row = t[b, n_acc].astype(np.float64)
            if T == 0.0:
                y = int(np.argmax(row))
            else:
                p = scipy.special.softmax(row / T)
                _, u = oracle.uniforms(c, c, b, n_acc)
                cdf = np.cumsum(p)
                y = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
                if r["margin_rec"][b] <= 1e-9:
                    continue
            assert r["tokens"][b, n_acc] == y, (c, b, r["tokens"][b], y)


def check_typical_special_cases(seed=93):
    """eps = 1 with top_k = 1 accepts exactly the drafts the greedy rule
    accepts (x a row max); eps = 0 accepts every valid draft; eps = 1 with
    top_k = 0 rejects at once and emits the plain temperature sample of row 0,
    the token of the verify step with n_b = 0."""
    rng = np.random.default_rng(seed)
    B, K, V = 64, 4, 40
    t, ids, nd = _typical_case(rng, B, K, V)
    t = np.round(t)  # ties at the max
    g = oracle.verify(t, None, ids, nd, np.zeros(B, np.float32))
    r = oracle.verify_typical(t, ids, nd, np.ones(B, np.float32), eps=1.0, top_k=1)
    assert np.array_equal(r["num_accepted"], g["num_accepted"])
    r = oracle.verify_typical(t, ids, nd, np.full(B, 0.8, np.float32), eps=0.0)
    assert np.array_equal(r["num_accepted"], nd)
    r = oracle.verify_typical(t, ids, nd, np.full(B, 0.8, np.float32), eps=1.0, top_k=0,
                              seed=4, offset=6)
    assert np.all(r["num_accepted"] == 0)
    plain = oracle.verify(t, None, ids, np.zeros(B, np.int32), np.full(B, 0.8, np.float32),
                          seed=4, offset=6)
    assert np.array_equal(r["tokens"][:, 0], plain["tokens"][:, 0])


def check_typical_correction_law(B=1 << 17, V=6, T=0.9, seed=95):
    """A draft that is always rejected: the emitted token follows p_0."""
    rng = np.random.default_rng(seed)
    row = rng.normal(0, 1, V).astype(np.float32)
    t = np.broadcast_to(np.stack([row, row]), (B, 2, V)).copy()
    x = int(np.argmin(row))
    r = oracle.verify_typical(t, np.full((B, 1), x, np.int32), np.ones(B, np.int32),
                              np.full(B, T, np.float32), eps=0.99, top_k=0, seed=seed,
                              diagnostics=False)
    assert np.all(r["num_accepted"] == 0)
    p = scipy.special.softmax(row.astype(np.float64) / T)
    assert _chisq_ok(np.bincount(r["tokens"][:, 0], minlength=V), p)


# --------------------------------------------------------------------------
# Token-tree verification
# --------------------------------------------------------------------------
def _chain_tree(t, d, ids, nd):
    """The chain verify inputs laid out as a tree: node i = position i."""
    B, K1, V = t.shape
    N = K1
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = ids
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    dt = None
    if d is not None:
        dt = np.zeros((B, N, V), d.dtype)
        dt[:, :N - 1] = d
    return tokens, parents, dt, np.asarray(nd, np.int32) + 1


def check_tree_chain_equals_verify(seed=101):
    """A chain-shaped tree reproduces the verify step bit for bit: tokens,
    counts and the smallest decision margin, for probabilistic, one-hot and
    greedy requests."""
    rng = np.random.default_rng(seed)
    for c in range(12):
        B, K, V = 24, int(rng.integers(1, 6)), int(rng.integers(2, 300))
        t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
        d = (t[:, :K] + rng.normal(0, 0.7, (B, K, V))).astype(np.float32)
        ids = rng.integers(0, V, (B, K)).astype(np.int32)
        am = np.argmax(d, -1)
        ids = np.where(rng.random((B, K)) < 0.5, am, ids).astype(np.int32)
        nd = rng.integers(0, K + 1, B).astype(np.int32)
        temps = rng.choice([1.0, 0.7, 0.0, 1.4], B).astype(np.float32)
        onehot = c % 3 == 2
        dd = None if onehot else d
        ref = oracle.verify(t, dd, ids, nd, temps, seed=c, offset=7 * c)
        tok, par, dt, nn = _chain_tree(t, dd, ids, nd)
        r = oracle.verify_tree(t, dt, tok, par, nn, temps, seed=c, offset=7 * c)
        assert np.array_equal(r["num_accepted"], ref["num_accepted"]), c
        assert np.array_equal(r["tokens"], ref["tokens"]), c
        assert np.array_equal(r["last_node"], ref["num_accepted"]), c
        for b in range(B):
            m = ref["margin_acc"][b, :min(nd[b], ref["num_accepted"][b] + 1)]
            m = m[np.isfinite(m)] if np.any(np.isfinite(m)) else np.array([np.inf])
            assert r["margin_acc"][b] == m.min(), (c, b)
            assert r["margin_rec"][b] == ref["margin_rec"][b], (c, b)


def check_tree_lossless_monte_carlo(B=1 << 17, V=6, T=0.8, seed=103):
    """Multi-step speculative sampling keeps the target law: three children
    of the root drawn i.i.d. from q (duplicates allowed), and three fixed
    distinct one-hot children; the first emitted token follows p_root."""
    rng = np.random.default_rng(seed)
    lp = rng.normal(0, 1, V).astype(np.float32)
    lq = (lp + rng.normal(0, 1.2, V)).astype(np.float32)
    p = scipy.special.softmax(lp.astype(np.float64) / T)
    q = scipy.special.softmax(lq.astype(np.float64) / T)
    N = 4
    t = np.broadcast_to(lp, (B, N, V)).copy()
    d = np.broadcast_to(lq, (B, N, V)).copy()
    par = np.tile(np.array([-1, 0, 0, 0], np.int32), (B, 1))
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = rng.choice(V, size=(B, 3), p=q)
    temps = np.full(B, T, np.float32)
    r = oracle.verify_tree(t, d, tok, par, np.full(B, N, np.int32), temps, seed=seed)
    assert _chisq_ok(np.bincount(r["tokens"][:, 0], minlength=V), p)
    tok[:, 1:] = [1, 4, 2]
    r = oracle.verify_tree(t, None, tok, par, np.full(B, N, np.int32), temps, seed=seed + 1)
    assert _chisq_ok(np.bincount(r["tokens"][:, 0], minlength=V), p)


def check_tree_greedy_walk(cases=200, seed=105):
    """Greedy trees against a walk written with numpy: follow the first
    child (in index order) whose token attains its parent's row max; emit
    the lowest argmax where none does."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        N, V = int(rng.integers(1, 12)), int(rng.integers(2, 12))
        t = np.round(rng.normal(0, 1.5, (1, N, V))).astype(np.float32)
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)], np.int32)
        tok = rng.integers(0, V, N).astype(np.int32)
        r = oracle.verify_tree(t, None, tok[None], par[None], [N], [0.0])
        v, path = 0, []
        while True:
            kids = [i for i in range(v + 1, N) if par[i] == v and t[0, v, tok[i]] == t[0, v].max()]
            if not kids:
                break
            v = kids[0]
            path.append(int(tok[v]))
        want = path + [int(np.argmax(t[0, v]))] + [-1] * (N - len(path) - 1)
        assert r["tokens"][0].tolist() == want and r["last_node"][0] == v, (c, r, want)


def check_tree_flags():
    t = np.zeros((2, 3, 4), np.float32)
    r = oracle.verify_tree(t, None, np.array([[0, 9, 1], [0, 1, 2]]),
                           np.array([[-1, 0, 0], [-1, 2, 0]]), [3, 3], [1.0, 1.0])
    assert r["flags"] & oracle.FLAG_BAD_DRAFT_ID and r["flags"] & oracle.FLAG_BAD_TREE
    assert r["last_node"][1] in (0, 2)  # node 1 (parent 2 > 1) is never visited
    r = oracle.verify_tree(t, None, np.zeros((2, 3)), np.full((2, 3), -1), [0, 7], [1.0, 1.0])
    assert r["flags"] & oracle.FLAG_BAD_NUM_DRAFTS


# --------------------------------------------------------------------------
# Margins: the distance of each decision's uniform to its threshold and of
# each draw's u * S to the chosen token's CDF boundaries, recomputed with
# numpy / scipy.  They decide which requests the parity rule lets differ,
# so they are pinned against an independent computation, not only used.
# --------------------------------------------------------------------------
def _np_draw(r, u):
    """numpy's inverse CDF of the unnormalized law r: the token
    searchsorted(cumsum(r), u * S, 'right') picks, the distance of u * S to
    its nearer boundary over S, and its boundaries (C_{y-1}, C_y) over S.
    Past the end (rounding): the last token with mass, margin 0."""
    C = np.cumsum(r)
    S = C[-1]
    theta = u * S
    y = int(np.searchsorted(C, theta, side="right"))
    if y >= len(r):
        y = int(np.flatnonzero(r > 0)[-1])
        return y, 0.0, (C[y - 1] if y else 0.0) / S, C[y] / S
    lo = C[y - 1] if y else 0.0
    return y, min(theta - lo, C[y] - theta) / S, lo / S, C[y] / S


def check_draw_margin_vs_library(cases=400, seed=111):
    """svo_draw's token and margin, and svo_draw_interval's (lo, hi, mass),
    against numpy's cumulative sum and searchsorted on random laws with
    zeros and totals far from 1."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        V = int(rng.integers(1, 60))
        r = rng.random(V) * (rng.random(V) < 0.7) * float(rng.choice([1e-3, 0.3, 1.0, 40.0]))
        if not r.sum() > 0:
            r[int(rng.integers(V))] = 0.25
        u = float(rng.integers(0, 1 << 24)) / 2.0 ** 24
        y, m = oracle.draw(r, u)
        yn, mn, lo, hi = _np_draw(r, u)
        if mn > 1e-12:
            assert y == yn, (c, y, yn)
        assert abs(m - mn) <= 1e-12, (c, m, mn)
        lo_o, hi_o, mass = oracle.draw_interval(r, yn)
        assert abs(lo_o - lo) <= 1e-12 and abs(hi_o - hi) <= 1e-12, (c, lo_o, lo, hi_o, hi)
        assert abs(mass - r[yn] / r.sum()) <= 1e-12, (c, mass)
        z = int(rng.integers(V))
        lo_z, hi_z, mass_z = oracle.draw_interval(r, z)
        C = np.cumsum(r)
        assert abs(lo_z - (C[z - 1] if z else 0.0) / C[-1]) <= 1e-12
        assert abs(hi_z - C[z] / C[-1]) <= 1e-12 and abs(mass_z - r[z] / C[-1]) <= 1e-12
    lo, hi, m = oracle.draw_interval(np.array([0.5, 0.5]), 2)
    assert m == 0.0 and np.isnan(lo) and np.isnan(hi)


def _np_uniforms(seed, offset, b, j):
    w = _numpy_block([offset, b, j, 0], [seed, 0])
    return (int(w[0]) >> 40) / 2.0 ** 24, (int(w[1]) >> 40) / 2.0 ** 24


def _np_laws(h, b, j, T, need_q=True):
    """scipy's p_j and q_j of request b (q None for one-hot, or when not
    needed), from the raw input rows."""
    p = scipy.special.softmax(oracle.row_f64(h["target"], (b, j)) / T)
    onehot = h["draft"] is None or (h["draft_mode"] is not None and h["draft_mode"][b] != 0)
    if onehot or not need_q:
        return p, None
    d = oracle.row_f64(h["draft"], (b, j))
    return p, (d if h["draft_is_probs"] else scipy.special.softmax(d / T))


def _np_request(h, b, seed, offset, n_path=None):
    """The verify step of one sampling request with numpy / scipy: the
    decisions [(accept, |u - ratio|)] of the walk (to the first rejection, or
    along the path with n_path accepts) and the emitted draw (token, margin,
    lo, hi, law) at its end; None where a value lies within 1e-12 of a
    threshold (rounding could take either side)."""
    K = h["target"].shape[1] - 1
    T = float(np.float32(h["temperatures"][b]))
    n = int(np.clip(h["num_drafts"][b], 0, K))
    dec, j = [], 0
    while j < n:
        p, q = _np_laws(h, b, j, T)
        x = int(h["draft_ids"][b, j])
        ua, _ = _np_uniforms(seed, offset, b, j)
        if not 0 <= x < p.size:
            ratio = 0.0
        elif q is None:
            ratio = p[x]
        else:
            ratio = p[x] / q[x] if q[x] > 0 else (np.inf if p[x] > 0 else 0.0)
        m = abs(ua - ratio)
        if m < 1e-12:
            return None
        dec.append((ua < ratio, m))
        stop = (not ua < ratio) if n_path is None else j == n_path
        if stop:
            break
        j += 1
    if n_path is not None:
        j = n_path
    p, q = _np_laws(h, b, j, T, need_q=j < n)
    if j < n:
        x = int(h["draft_ids"][b, j])
        if q is None:
            r = p.copy()
            if 0 <= x < p.size:
                r[x] = 0.0
        else:
            r = np.maximum(p - q, 0.0)
    else:
        r = p
    if not r.sum() > 0:
        return None
    _, ur = _np_uniforms(seed, offset, b, j)
    y, m, lo, hi = _np_draw(r, ur)
    if m < 1e-11:
        return None
    return dec, (y, m, lo, hi, r)


def _margin_batches(seed):
    import torch
    import synth
    kws = [dict(temps=(1.0, 0.6, 1.5), n_mode="ragged", corr=0.8),
           dict(temps=(0.8,), onehot_frac=0.5, n_mode="ragged"),
           dict(temps=(1.2, 0.9), dtype=torch.bfloat16, corr=0.95),
           dict(temps=(0.9, 1.1), draft_is_probs=True, n_mode="ragged", corr=0.7)]
    for i, kw in enumerate(kws):
        yield i, synth.make_random(24, 4, 120, seed=seed + i, **kw).host_arrays()


def check_margins_vs_library(seed=121):
    """Every decision margin |u - p(x)/q(x)| the oracle reports and its
    draw margin, against scipy's softmax, numpy's Philox and numpy's
    inverse CDF (probabilistic, one-hot, probability and bf16 drafts)."""
    checked = 0
    for i, h in _margin_batches(seed):
        r = oracle.verify(h["target"], h["draft"], h["draft_ids"], h["num_drafts"],
                          h["temperatures"], draft_mode=h["draft_mode"],
                          draft_is_probs=h["draft_is_probs"], seed=i, offset=5 + i)
        for b in range(h["target"].shape[0]):
            got = _np_request(h, b, i, 5 + i)
            if got is None:
                continue
            dec, (y, m, lo, hi, _) = got
            for j, (acc, mj) in enumerate(dec):
                mo = r["margin_acc"][b, j]
                assert abs(mo - mj) <= 1e-12 * max(1.0, mj), (i, b, j, mo, mj)
            assert np.all(np.isnan(r["margin_acc"][b, len(dec):])), (i, b)
            assert int(r["num_accepted"][b]) == sum(a for a, _ in dec), (i, b)
            a = int(r["num_accepted"][b])
            assert int(r["tokens"][b, a]) == y, (i, b, r["tokens"][b], y)
            assert abs(r["margin_rec"][b] - m) <= 1e-11, (i, b, r["margin_rec"][b], m)
            checked += 1
    assert checked > 60, checked


def check_forced_path_vs_library(seed=131):
    """oracle.verify_path along paths the walk did not take (any count of
    accepts up to n_b): the decisions and margins on the path, the emitted
    draw there, and where another token sits in that draw's law, against
    scipy / numpy."""
    rng = np.random.default_rng(seed)
    checked = 0
    for i, h in _margin_batches(seed):
        K = h["target"].shape[1] - 1
        r = oracle.verify(h["target"], h["draft"], h["draft_ids"], h["num_drafts"],
                          h["temperatures"], draft_mode=h["draft_mode"],
                          draft_is_probs=h["draft_is_probs"], seed=i, offset=9)
        for b in range(h["target"].shape[0]):
            n = int(np.clip(h["num_drafts"][b], 0, K))
            n_path = int(rng.integers(0, n + 1))
            z = int(rng.integers(0, h["target"].shape[2]))
            ev = oracle.verify_path(r, b, n_path, z)
            got = _np_request(h, b, i, 9, n_path=n_path)
            if got is None:
                continue
            dec, (y, m, lo, hi, law) = got
            assert len(dec) == min(n_path + 1, n), (i, b)
            for j, (acc, mj) in enumerate(dec):
                assert ev["accept"][j] == acc, (i, b, j)
                assert abs(ev["margin"][j] - mj) <= 1e-12 * max(1.0, mj), (i, b, j)
            assert np.all(np.isnan(ev["accept"][len(dec):]))
            assert ev["token"] == y and abs(ev["margin_rec"] - m) <= 1e-11, (i, b, ev, y, m)
            C = np.cumsum(law)
            assert abs(ev["lo"] - (C[z - 1] if z else 0.0) / C[-1]) <= 1e-12, (i, b)
            assert abs(ev["hi"] - C[z] / C[-1]) <= 1e-12, (i, b)
            assert abs(ev["mass"] - law[z] / C[-1]) <= 1e-12, (i, b)
            checked += 1
    assert checked > 60, checked


def check_typical_path_vs_library(cases=40, seed=141):
    """oracle.verify_typical_path along any path: decisions by scipy's
    softmax and numpy's ranks, the draw from p at the stop by numpy."""
    rng = np.random.default_rng(seed)
    for c in range(cases):
        B, K, V = 3, int(rng.integers(1, 5)), int(rng.integers(2, 150))
        t, ids, nd = _typical_case(rng, B, K, V)
        temps = rng.choice([1.0, 0.6, 0.0], B).astype(np.float32)
        eps, top_k = float(rng.choice([0.01, 0.05, 0.2])), int(rng.integers(0, 3))
        r = oracle.verify_typical(t, ids, nd, temps, eps=eps, top_k=top_k, seed=c, offset=1)
        for b in range(B):
            n = int(nd[b])
            n_path = int(rng.integers(0, n + 1))
            z = int(rng.integers(0, V))
            ev = oracle.verify_path(r, b, n_path, z)
            T = float(temps[b])
            for j in range(min(n_path + 1, n)):
                row, x = t[b, j].astype(np.float64), int(ids[b, j])
                if T == 0.0:
                    assert ev["accept"][j] == (row[x] == row.max()) and np.isinf(ev["margin"][j])
                    continue
                p = scipy.special.softmax(row / T)
                rank_ok = int(np.sum(row > row[x])) < top_k
                assert ev["accept"][j] == (rank_ok or p[x] > eps), (c, b, j)
                if not rank_ok:
                    assert abs(ev["margin"][j] - abs(p[x] - eps)) <= 1e-12, (c, b, j)
            row = t[b, n_path].astype(np.float64)
            if T == 0.0:
                assert ev["token"] == int(np.argmax(row))
                continue
            p = scipy.special.softmax(row / T)
            _, u = _np_uniforms(c, 1, b, n_path)
            y, m, lo, hi = _np_draw(p, u)
            if m > 1e-11:
                assert ev["token"] == y and abs(ev["margin_rec"] - m) <= 1e-11, (c, b)
            C = np.cumsum(p)
            assert abs(ev["lo"] - (C[z - 1] if z else 0.0) / C[-1]) <= 1e-12
            assert abs(ev["hi"] - C[z] / C[-1]) <= 1e-12


def check_tree_chain_probs_equals_verify(seed=151):
    """The tree's probability-draft branch: a chain-shaped tree whose draft
    rows are normalized q (draft_is_probs) reproduces the verify step with
    draft_is_probs bit for bit, tokens, counts and margins."""
    rng = np.random.default_rng(seed)
    for c in range(6):
        B, K, V = 16, int(rng.integers(1, 5)), int(rng.integers(2, 200))
        t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
        dl = t[:, :K] + rng.normal(0, 0.8, (B, K, V))
        d = scipy.special.softmax(dl / 0.9, axis=-1).astype(np.float32)
        ids = np.array([[rng.choice(V, p=d[b, j] / d[b, j].sum()) for j in range(K)]
                        for b in range(B)], np.int32)
        nd = rng.integers(0, K + 1, B).astype(np.int32)
        temps = rng.choice([1.0, 0.7, 1.3], B).astype(np.float32)
        ref = oracle.verify(t, d, ids, nd, temps, draft_is_probs=True, seed=c, offset=3)
        tok, par, dt, nn = _chain_tree(t, d, ids, nd)
        r = oracle.verify_tree(t, dt, tok, par, nn, temps, seed=c, offset=3, draft_is_probs=True)
        assert np.array_equal(r["tokens"], ref["tokens"]), c
        assert np.array_equal(r["num_accepted"], ref["num_accepted"]), c
        for b in range(B):
            m = ref["margin_acc"][b, :min(nd[b], ref["num_accepted"][b] + 1)]
            assert r["margin_acc"][b] == (m.min() if m.size else np.inf), (c, b)
            assert r["margin_rec"][b] == ref["margin_rec"][b], (c, b)


def check_tree_path_chain_equals_verify_path(seed=161):
    """oracle.verify_tree_path on a chain-shaped tree equals
    oracle.verify_path (pinned above against scipy / numpy) for every
    forced count of accepts: the same decisions, margins and draw."""
    rng = np.random.default_rng(seed)
    for c in range(4):
        B, K, V = 8, int(rng.integers(1, 5)), int(rng.integers(2, 120))
        t = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
        d = (t[:, :K] + rng.normal(0, 0.7, (B, K, V))).astype(np.float32)
        ids = rng.integers(0, V, (B, K)).astype(np.int32)
        nd = rng.integers(0, K + 1, B).astype(np.int32)
        temps = rng.choice([1.0, 0.7, 0.0], B).astype(np.float32)
        dd = None if c == 3 else d
        ref = oracle.verify(t, dd, ids, nd, temps, seed=c, offset=2)
        tok, par, dt, nn = _chain_tree(t, dd, ids, nd)
        rt = oracle.verify_tree(t, dt, tok, par, nn, temps, seed=c, offset=2)
        for b in range(B):
            for n_path in range(int(nd[b]) + 1):
                z = int(rng.integers(0, V))
                ev = oracle.verify_path(ref, b, n_path, z)
                et = oracle.verify_tree_path(rt, b, list(range(n_path + 1)), z)
                tests = et["tests"]
                assert tests is not None and len(tests) == min(n_path + 1, int(nd[b])), (c, b)
                for j, (child, walk, orc, m) in enumerate(tests):
                    assert child == j + 1 and walk == (j < n_path), (c, b, j)
                    assert orc == ev["accept"][j] and (m == ev["margin"][j]), (c, b, j)
                for key in ("token", "margin_rec", "lo", "hi", "mass", "u"):
                    a1, a2 = et[key], ev[key]
                    assert a1 == a2 or (np.isnan(a1) and np.isnan(a2)), (c, b, key, a1, a2)


# --------------------------------------------------------------------------
# Long statistical pins (run once, not for every planted mistake)
# --------------------------------------------------------------------------
def check_config0_chi_square(total=1 << 20, batch=4096, seed=171, threads=8):
    """The distribution claim at the size the task states, on the B=1, K=4,
    V=1000 workload's own rows: 2^20 verify steps, each with fresh drafts
    x_j ~ q_j drawn by numpy, over distinct Philox counters (one offset per
    batch of requests).  The first emitted token follows p_0 and, given an
    acceptance at position 0, the second follows p_1 (chi-square, p > 1e-3);
    the acceptance rate at position 0 equals sum_x min(p_0, q_0) within 4
    sigma."""
    from concurrent.futures import ThreadPoolExecutor
    import synth
    w = synth.make_config(0)
    h = w.host_arrays()
    K, V = w.K, w.V
    T = float(h["temperatures"][0])
    p = [scipy.special.softmax(h["target"][0, j].astype(np.float64) / T) for j in range(K + 1)]
    q = [scipy.special.softmax(h["draft"][0, j].astype(np.float64) / T) for j in range(K)]
    tgt = np.broadcast_to(h["target"][0], (batch, K + 1, V)).copy()
    dft = np.broadcast_to(h["draft"][0], (batch, K, V)).copy()

    def run(i):
        rng = np.random.default_rng([seed, i])
        ids = np.stack([rng.choice(V, batch, p=q[j]) for j in range(K)], 1).astype(np.int32)
        r = oracle.verify(tgt, dft, ids, np.full(batch, K), np.full(batch, T, np.float32),
                          seed=seed, offset=i, diagnostics=False)
        acc0 = r["num_accepted"] >= 1
        return (np.bincount(r["tokens"][:, 0], minlength=V),
                np.bincount(r["tokens"][acc0, 1], minlength=V), int(acc0.sum()))

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(run, range(total // batch)))
    first = sum(x[0] for x in parts)
    second = sum(x[1] for x in parts)
    n_acc0 = sum(x[2] for x in parts)
    assert first.sum() == total
    assert _chisq_ok(first, p[0]), "first emitted token vs p_0"
    assert _chisq_ok(second, p[1]), "second emitted token vs p_1"
    pa = np.minimum(p[0], q[0]).sum()
    assert abs(n_acc0 / total - pa) < 4 * np.sqrt(pa * (1 - pa) / total), (n_acc0 / total, pa)


def check_grid_one_decision_full(seed=181, chunk=1 << 21):
    """One decision and its recovery draw over the whole 2^24 grid of
    uniforms, through the full verify entry (V = 4, T = 0.8, a draft x with
    p(x) < q(x)).  Acceptances: #{k : k / 2^24 < p(x)/q(x)}, within 1 of
    ratio * 2^24 with the ratio from scipy.  Recovery (the decision forced to
    reject): the count of grid points drawing token i is r_i / S * 2^24
    within 1, r = max(0, p - q) from scipy."""
    rng = np.random.default_rng(seed)
    V, T, G = 4, 0.8, 1 << 24
    while True:
        lt = rng.normal(0, 1.5, (2, V)).astype(np.float32)
        ld = (lt[:1] + rng.normal(0, 1.2, (1, V))).astype(np.float32)
        p = scipy.special.softmax(lt[0].astype(np.float64) / T)
        q = scipy.special.softmax(ld[0].astype(np.float64) / T)
        x = int(np.argmin(p / q))
        if p[x] / q[x] < 0.9 and np.count_nonzero(p > q) >= 2:
            break
    ratio = p[x] / q[x]
    r = np.maximum(p - q, 0.0)
    tgt = np.broadcast_to(lt, (chunk, 2, V)).copy()
    dft = np.broadcast_to(ld, (chunk, 1, V)).copy()
    ids = np.full((chunk, 1), x, np.int32)
    accepted, hist = 0, np.zeros(V, np.int64)
    for start in range(0, G, chunk):
        grid = (start + np.arange(chunk)) / G
        ua = np.zeros((chunk, 2))
        ua[:, 0] = grid
        res = oracle.verify(tgt, dft, ids, np.ones(chunk), np.full(chunk, T), u_acc=ua,
                            u_rec=np.full((chunk, 2), 0.5), diagnostics=False)
        accepted += int(res["num_accepted"].sum())
        ua[:, 0] = 1.0 - 2.0 ** -24
        ur = np.zeros((chunk, 2))
        ur[:, 0] = grid
        res = oracle.verify(tgt, dft, ids, np.ones(chunk), np.full(chunk, T), u_acc=ua,
                            u_rec=ur, diagnostics=False)
        assert np.all(res["num_accepted"] == 0)
        hist += np.bincount(res["tokens"][:, 0], minlength=V)
    assert abs(accepted - ratio * G) <= 1.0, (accepted, ratio * G)
    assert hist[x] == 0 and np.all(hist[r == 0] == 0), hist
    assert np.all(np.abs(hist - r / r.sum() * G) <= 1.0), (hist, r / r.sum() * G)


ALL_QUICK = [check_philox_known_answers, check_uniform_mapping,
             check_accept_example_philox, check_bpd_greedy_example,
             check_greedy_bruteforce, check_enumeration_law,
             check_grid_law_through_verify, check_monte_carlo,
             check_monte_carlo_onehot, check_no_draft_is_plain_sampling,
             check_identical_draft_always_accepted,
             check_certain_onehot_always_accepted, check_zero_mass_never_drawn,
             check_invariants, check_draft_uniform_mapping,
             check_draft_sample_vs_library, check_draft_sample_monte_carlo,
             check_ngram_golden, check_ngram_vs_rfind, check_ngram_edge_cases,
             check_typical_golden, check_typical_vs_library, check_typical_special_cases,
             check_typical_correction_law, check_tree_chain_equals_verify,
             check_tree_lossless_monte_carlo, check_tree_greedy_walk, check_tree_flags,
             check_draw_margin_vs_library, check_margins_vs_library,
             check_forced_path_vs_library, check_typical_path_vs_library,
             check_tree_chain_probs_equals_verify, check_tree_path_chain_equals_verify_path]
