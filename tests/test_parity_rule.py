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


# ---------------------------------------------------------------------------
# Flagged requests: an output along the other branch of a decision or draw
# within the band passes; one that strays further is reported.
# ---------------------------------------------------------------------------
def _uniform_case(seed=23):
    """A probabilistic batch with explicit uniforms (Philox values of the
    request's own counter), so single uniforms can be moved."""
    w = synth.make_random(12, 4, 200, temps=(1.0, 0.8), seed=seed, n_mode="full",
                          corr=0.9)
    h = w.host_arrays()
    B, K = w.B, w.K
    ua, ur = np.empty((B, K + 1)), np.empty((B, K + 1))
    for b in range(B):
        for j in range(K + 1):
            ua[b, j], ur[b, j] = oracle.uniforms(1, 2, b, j)
    return h, ua, ur


def _run(h, ua, ur):
    return oracle.verify(h["target"], h["draft"], h["draft_ids"], h["num_drafts"],
                         h["temperatures"], u_acc=ua, u_rec=ur)


def test_flagged_decision_other_branch_passes():
    h, ua, ur = _uniform_case()
    ref0 = _run(h, ua, ur)
    b = 0
    ratio = ref0["p"][b, 0] / ref0["q"][b, 0]
    assert 0.01 < ratio < 0.99
    ua_a, ua_r = ua.copy(), ua.copy()
    ua_a[b, 0] = ratio - 4e-7  # accepted, within the band
    ua_r[b, 0] = ratio + 4e-7  # rejected, within the band
    ref = _run(h, ua_r, ur)    # the oracle's walk rejects at 0: flagged
    other = _run(h, ua_a, ur)  # an output that accepted there
    assert ref["num_accepted"][b] == 0 and other["num_accepted"][b] >= 1
    rep = compare(h, ref, other["tokens"], other["num_accepted"])
    assert rep.ok(), rep.mismatches
    assert rep.flagged_decision >= 1 and rep.flagged_mismatch >= 1
    # the other branch, but a wrong token emitted after it
    t = other["tokens"].copy()
    a = other["num_accepted"][b]
    ev = oracle.verify_path(ref, b, a, int(t[b, a]))
    t[b, a] = (t[b, a] + 1) % 200
    if ev["margin_rec"] >= 1e-6:
        assert not compare(h, ref, t, other["num_accepted"]).ok()
    # an accepted count past a clear rejection is reported
    ua_far = ua_r.copy()
    ua_far[b, 0] = min(0.999, ratio + 0.2)
    ref_far = _run(h, ua_far, ur)
    assert not compare(h, ref_far, other["tokens"], other["num_accepted"]).ok()


def test_flagged_draw_neighbour_passes():
    h, ua, ur = _uniform_case(seed=29)
    ref0 = _run(h, ua, ur)
    b = 1
    a = int(ref0["num_accepted"][b])
    y = int(ref0["tokens"][b, a])
    ev = oracle.verify_path(ref0, b, a, y)
    ur2 = ur.copy()
    ur2[b, a] = ev["hi"] - 3e-7  # just below y's upper boundary: flagged draw
    ref = _run(h, ua, ur2)
    assert ref["margin_rec"][b] < 1e-6 and int(ref["tokens"][b, a]) == y
    # the next token with mass, as a draw that rounded the other way
    law_ev = [oracle.verify_path(ref, b, a, z) for z in range(y + 1, 200)]
    z = next(y + 1 + i for i, e in enumerate(law_ev) if e["mass"] > 0)
    t = ref["tokens"].copy()
    t[b, a] = z
    rep = compare(h, ref, t, ref["num_accepted"])
    assert rep.ok(), rep.mismatches
    assert rep.flagged_draw >= 1 and rep.flagged_mismatch == 1
    # a token with mass further away is reported
    far = [y + 1 + i for i, e in enumerate(law_ev) if e["mass"] > 0 and y + 1 + i != z]
    t[b, a] = far[-1]
    assert not compare(h, ref, t, ref["num_accepted"]).ok()


def test_rejected_draft_reemitted_is_reported():
    h, ref, dbg = _case()
    n = np.clip(h["num_drafts"], 0, 5)
    samp = np.isfinite(h["temperatures"]) & (h["temperatures"] > 0)
    rej = np.flatnonzero((ref["num_accepted"] < n) & samp)
    b = int(rej[0])
    a = int(ref["num_accepted"][b])
    t = ref["tokens"].copy()
    t[b, a] = h["draft_ids"][b, a]
    assert not compare(h, ref, t, ref["num_accepted"]).ok()


def test_tree_rule_flagged_walks():
    from oracle.parity import compare_tree
    w = synth.make_tree(16, 6, 50, seed=4, temps=(1.0, 0.7), corr=0.9)
    h = w.host_arrays()
    ref = oracle.verify_tree(h["target"], h["draft"], h["tokens"], h["parents"],
                             h["num_nodes"], h["temperatures"], seed=3, offset=1)
    rep = compare_tree(h["tokens"], h["parents"], h["num_nodes"], w.V, ref, ref["tokens"],
                       ref["num_accepted"], ref["last_node"])
    assert rep.ok(), rep.mismatches
    # the oracle's own walk evaluated as a path agrees with it everywhere
    for b in range(w.B):
        a, v = int(ref["num_accepted"][b]), int(ref["last_node"][b])
        path, node = [], v
        while node != 0:
            path.append(node)
            node = int(h["parents"][b, node])
        ev = oracle.verify_tree_path(ref, b, [0] + path[::-1], int(ref["tokens"][b, a]))
        assert ev["tests"] is not None
        assert np.all(ev["tests"][:, 1] == ev["tests"][:, 2])
        assert ev["token"] == int(ref["tokens"][b, a])
    # a wrong emitted token on an unflagged request is reported
    t = ref["tokens"].copy()
    b = int(np.argmax((ref["margin_rec"] > 1e-3) & (ref["margin_acc"] > 1e-3)))
    a = int(ref["num_accepted"][b])
    t[b, a] = (t[b, a] + 1) % w.V
    assert not compare_tree(h["tokens"], h["parents"], h["num_nodes"], w.V, ref, t,
                            ref["num_accepted"], ref["last_node"]).ok()
