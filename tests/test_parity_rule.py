"""The parity rule itself (no GPU): it must accept the oracle's own outputs
and reject planted differences."""
import numpy as np
import torch

import oracle
import synth
from oracle.parity import compare


def _case():
    w = synth.make_random(40, 5, 400, temps=(1.0, 0.0, 0.7), n_mode="ragged",
                          onehot_frac=0.3, seed=17)
    h = w.host_arrays()
    ref = oracle.verify(h["target"], h["draft"], h["draft_ids"], h["num_drafts"],
                        h["temperatures"], draft_mode=h["draft_mode"], seed=2,
                        offset=9)
    dbg = np.stack([ref["p"], ref["q"]], -1).astype(np.float32)
    return h, ref, dbg


def test_oracle_outputs_pass():
    h, ref, dbg = _case()
    rep = compare(h, ref, ref["tokens"], ref["num_accepted"], dbg)
    assert rep.ok(), rep.mismatches
    assert rep.prob_checked > 0


def test_planted_differences_are_reported():
    h, ref, dbg = _case()
    n = np.clip(h["num_drafts"], 0, 5)
    b = int(np.argmax(n > 0))
    # a different emitted token
    t = ref["tokens"].copy()
    t[b, ref["num_accepted"][b]] = (t[b, ref["num_accepted"][b]] + 1) % 400
    assert not compare(h, ref, t, ref["num_accepted"], dbg).ok()
    # a different accepted count (with a consistent token layout)
    a = ref["num_accepted"].copy()
    t = ref["tokens"].copy()
    k = int(np.argmax((a < n) & (a >= 0)))
    a[k] += 1
    t[k, : a[k]] = h["draft_ids"][k, : a[k]]
    t[k, a[k]] = 0
    t[k, a[k] + 1:] = -1
    assert not compare(h, ref, t, a, dbg).ok()
    # garbage after the emitted token
    t = ref["tokens"].copy()
    r = int(np.argmax(ref["num_accepted"] < 5))
    if ref["num_accepted"][r] < 5:
        t[r, -1] = 3
        assert not compare(h, ref, t, ref["num_accepted"], dbg).ok()
    # a probability off by 1e-4 relative
    d2 = dbg.copy()
    live = np.argwhere(np.isfinite(d2[..., 0]))
    i, j = live[0]
    d2[i, j, 0] *= 1.0001
    assert not compare(h, ref, ref["tokens"], ref["num_accepted"], d2).ok()
    # a debug slot that should be NaN
    d3 = dbg.copy()
    dead = np.argwhere(~np.isfinite(d3[..., 0]))
    i, j = dead[0]
    d3[i, j] = 0.5
    assert not compare(h, ref, ref["tokens"], ref["num_accepted"], d3).ok()


def test_draft_rule_accepts_oracle_and_rejects_differences():
    from oracle.parity import compare_draft
    rng = np.random.default_rng(3)
    l = rng.normal(0, 2, (6, 4, 300)).astype(np.float32)
    ref = oracle.draft_sample(l, np.array([4, 3, 0, 2, 4, 1]),
                              np.array([1.0, 0.5, 1.0, 0.0, 2.0, 1.0]), seed=5, offset=1)
    assert compare_draft(ref, ref["ids"], ref["q"]).ok()
    ids = ref["ids"].copy()
    ids[0, 1] = (ids[0, 1] + 1) % 300
    assert not compare_draft(ref, ids, ref["q"]).ok()
    ids = ref["ids"].copy()
    ids[2, 0] = 7  # a row past n_b must stay -1
    assert not compare_draft(ref, ids, ref["q"]).ok()
    q = ref["q"].copy()
    q[1, 0] *= 1.001
    assert not compare_draft(ref, ref["ids"], q).ok()
