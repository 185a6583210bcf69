"""Parity rule between an implementation's verify outputs and the oracle's.

TEST INFRASTRUCTURE (see the package docstring).  Works on numpy arrays and
the oracle's own functions.

Rule.  A request is flagged when one of the decisions the oracle's walk
evaluated lies within ``band`` of its threshold (|u - p(x)/q(x)| < band) or
its draw uniform lies within ``band`` of a CDF boundary (relative to the
law's total): there rounding may send an implementation the other way.

  * An unflagged request must match the oracle bit for bit: accepted count
    and every token.
  * A flagged request that matches is fine.  One that differs is checked
    along the path it took (oracle.verify_path evaluates the method there
    with the oracle's arithmetic): every position it accepted must be an
    oracle accept or lie within ``band``; the position where it stopped must
    be an oracle reject or lie within ``band``; its emitted token must be the
    oracle's token for that path, or, when that draw lies within ``band`` of
    a boundary, a token with positive mass whose CDF interval [lo, hi) lies
    within ``band`` of the draw uniform.
  * Every output must be valid whatever the flags: n_acc in [0, n_b], the
    accepted prefix equal to the drafts, one token in [0, V), then -1; a
    sampling rejection never re-emits its draft.
  * Acceptance probabilities p_j(x_j), q_j(x_j) must agree to ``prob_rtol``
    relative (an absolute floor of 1e-35 below 1e-30).
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle


@dataclasses.dataclass
class ParityReport:
    requests: int = 0
    flagged: int = 0
    flagged_decision: int = 0   # flagged at a decision of the oracle's walk
    flagged_draw: int = 0       # flagged at the oracle's draw only
    flagged_mismatch: int = 0   # flagged requests whose outputs differ (each path-checked)
    mismatches: list = dataclasses.field(default_factory=list)
    prob_checked: int = 0
    prob_max_rel: float = 0.0
    accepted: int = 0
    proposed: int = 0

    def ok(self):
        return not self.mismatches


def _is_sampling(T):
    T = np.asarray(T, dtype=np.float32)
    return (T >= np.finfo(np.float32).tiny) & (T <= np.finfo(np.float32).max)


def _draw_ok(ev, y, band):
    """The emitted token of a path: the oracle's, or, for a draw within band
    of a boundary, one with mass whose interval lies within band of u."""
    if not ev["margin_rec"] < band:
        return y == ev["token"]
    return ev["mass"] > 0 and ev["lo"] - band <= ev["u"] < ev["hi"] + band


def _path_errors(ev, n, ga, band):
    """Why the path "ga accepted, then stop" is not the oracle's within band
    (an empty list if it is)."""
    errs = []
    for j in range(min(ga, n)):
        if ev["accept"][j] != 1 and not ev["margin"][j] < band:
            errs.append(f"accepted position {j} that the oracle rejects "
                        f"(margin {ev['margin'][j]:.3g})")
    if ga < n and ev["accept"][ga] != 0 and not ev["margin"][ga] < band:
        errs.append(f"rejected position {ga} that the oracle accepts "
                    f"(margin {ev['margin'][ga]:.3g})")
    return errs


def compare(host, ref, tokens, nacc, dbg=None, *, band=1e-6, prob_rtol=1e-5,
            max_report=20) -> ParityReport:
    """host: the input arrays (synth.Workload.host_arrays()); ref: the
    oracle's result dict (oracle.verify or oracle.verify_typical, on those
    inputs); tokens [B, K+1], nacc [B], dbg [B, K, 2] or None: the
    implementation's outputs."""
    tokens = np.asarray(tokens)
    nacc = np.asarray(nacc)
    B, K1 = tokens.shape
    K = K1 - 1
    V = host["target"].shape[2]
    nd = np.clip(np.asarray(host["num_drafts"]), 0, K)
    ids = np.asarray(host["draft_ids"]).reshape(B, K)
    samp = _is_sampling(host["temperatures"])
    typical = ref["call"]["kind"] == "typical"
    rep = ParityReport(requests=B)

    def bad(b, why):
        rep.mismatches.append((b, why) if len(rep.mismatches) < max_report else (b, "..."))

    for b in range(B):
        n = int(nd[b])
        ga, oa = int(nacc[b]), int(ref["num_accepted"][b])
        rep.accepted += ga
        rep.proposed += n
        # validity, whatever the flags
        if not (0 <= ga <= n):
            bad(b, f"n_acc {ga} outside [0, {n}]")
            continue
        if not np.array_equal(tokens[b, :ga], ids[b, :ga]):
            bad(b, "accepted prefix differs from the drafts")
        y = int(tokens[b, ga])
        if not (0 <= y < V):
            bad(b, f"emitted token {y} outside [0, {V})")
            continue
        if np.any(tokens[b, ga + 1:] != -1):
            bad(b, "padding after the emitted token is not -1")
        if samp[b] and not typical and ga < n and y == int(ids[b, ga]):
            bad(b, f"rejected draft {y} at position {ga} re-emitted")
        # flagged by the oracle's own walk?
        flag_at = None
        for j in range(oa + 1 if oa < n else n):
            m = ref["margin_acc"][b, j]
            if np.isfinite(m) and m < band:
                flag_at = j
                break
        rec_flag = flag_at is None and ref["margin_rec"][b] < band
        same = ga == oa and np.array_equal(tokens[b], ref["tokens"][b])
        if flag_at is None and not rec_flag:
            if ga != oa:
                bad(b, f"n_acc {ga} != oracle {oa}")
            elif not same:
                bad(b, f"tokens {tokens[b].tolist()} != oracle {ref['tokens'][b].tolist()}")
            continue
        rep.flagged += 1
        rep.flagged_decision += flag_at is not None
        rep.flagged_draw += rec_flag
        if same:
            continue
        rep.flagged_mismatch += 1
        ev = oracle.verify_path(ref, b, ga, y)
        for why in _path_errors(ev, n, ga, band):
            bad(b, why)
        if not _draw_ok(ev, y, band):
            bad(b, f"emitted {y} at position {ga}: oracle draws {ev['token']} (draw margin "
                   f"{ev['margin_rec']:.3g}; u {ev['u']:.9f} vs [{ev['lo']:.9f}, "
                   f"{ev['hi']:.9f}), mass {ev['mass']:.3g})")

    if dbg is not None:
        dbg = np.asarray(dbg, dtype=np.float64)
        for b in range(B):
            for j in range(K):
                op, oq = ref["p"][b, j], ref["q"][b, j]
                gp, gq = dbg[b, j, 0], dbg[b, j, 1]
                live = samp[b] and j < nd[b] and 0 <= ids[b, j] < V
                if not live:
                    if not (np.isnan(gp) and np.isnan(gq)):
                        bad(b, f"debug probs at j={j} should be NaN")
                    continue
                for o, g in ((op, gp), (oq, gq)):
                    rep.prob_checked += 1
                    if abs(o) < 1e-30:
                        if abs(g - o) > 1e-35:
                            bad(b, f"prob at j={j}: {g} vs {o} (abs floor)")
                        continue
                    rel = abs(g - o) / abs(o)
                    rep.prob_max_rel = max(rep.prob_max_rel, rel)
                    if not rel <= prob_rtol:
                        bad(b, f"prob at j={j}: {g} vs {o} rel {rel:.3g}")
    return rep


def compare_draft(ref, ids, qx=None, *, band=1e-6, prob_rtol=1e-5,
                  max_report=20) -> ParityReport:
    """Parity of the draft sampler's outputs.  ref: oracle.draft_sample's
    result; ids [B, K] and qx [B, K] (or None): the implementation's.

    A row is flagged when its draw uniform lies within ``band`` of a CDF
    boundary (relative to the total).  Unflagged rows must match the oracle's
    token exactly; a flagged row that differs must hold a token with mass
    whose CDF interval lies within ``band`` of the row's uniform.  Rows past
    n_b must be -1.  q_j(x_j) must agree to ``prob_rtol`` relative wherever
    the token matches (an absolute floor of 1e-35 below 1e-30)."""
    ids = np.asarray(ids)
    B, K = ids.shape
    rep = ParityReport(requests=B * K)

    def bad(where, why):
        rep.mismatches.append((where, why) if len(rep.mismatches) < max_report else (where, "..."))

    for b in range(B):
        for j in range(K):
            o, g = int(ref["ids"][b, j]), int(ids[b, j])
            if o < 0:
                if g != -1:
                    bad((b, j), f"row past n_b holds {g}, not -1")
                continue
            rep.proposed += 1
            if g < 0:
                bad((b, j), f"no token ({g}) where the oracle drew {o}")
                continue
            if ref["margin"][b, j] < band:
                rep.flagged += 1
                rep.flagged_draw += 1
                if g != o:
                    rep.flagged_mismatch += 1
                    lo, hi, mass, u = oracle.draft_sample_interval(ref, b, j, g)
                    if not (mass > 0 and lo - band <= u < hi + band):
                        bad((b, j), f"token {g} (mass {mass:.3g}, [{lo:.9f}, {hi:.9f})) is "
                                    f"not within the band of u {u:.9f}")
            elif g != o:
                bad((b, j), f"token {g} != oracle {o}")
            if qx is None or g != o:
                continue
            oq, gq = float(ref["q"][b, j]), float(qx[b, j])
            rep.prob_checked += 1
            if abs(oq) < 1e-30:
                if abs(gq - oq) > 1e-35:
                    bad((b, j), f"q(x) {gq} vs {oq} (abs floor)")
                continue
            rel = abs(gq - oq) / abs(oq)
            rep.prob_max_rel = max(rep.prob_max_rel, rel)
            if not rel <= prob_rtol:
                bad((b, j), f"q(x) {gq} vs {oq} rel {rel:.3g}")
    return rep


def compare_tree(tokens_in, parents, num_nodes, V, ref, tokens, nacc, last, *, band=1e-6,
                 max_report=20) -> ParityReport:
    """Parity of token-tree verification.  tokens_in / parents [B, N] and
    num_nodes [B]: the tree; ref: oracle.verify_tree's result; tokens [B, N],
    nacc [B], last [B]: the implementation's.

    A request is flagged when one of its sampling tests lay within ``band``
    of its threshold or its draw within ``band`` of a CDF boundary.
    Unflagged requests must match exactly (tokens, count, last node).  A
    flagged request that differs is checked along the walk it took
    (oracle.verify_tree_path): every child test on it agrees with the oracle
    or lies within ``band``, and the emitted token is the oracle's for that
    walk or, for a draw within ``band`` of a boundary, one with mass whose
    interval lies within ``band`` of the uniform.  Every output must be
    valid: the accepted path climbs from the last node to the root through
    parents, its tokens are those nodes' tokens, then one token in [0, V),
    then -1."""
    tokens, nacc, last = np.asarray(tokens), np.asarray(nacc), np.asarray(last)
    B, N = tokens.shape
    rep = ParityReport(requests=B)

    def bad(b, why):
        rep.mismatches.append((b, why) if len(rep.mismatches) < max_report else (b, "..."))

    for b in range(B):
        n = int(np.clip(num_nodes[b], 1, N))
        a, v = int(nacc[b]), int(last[b])
        rep.accepted += a
        path = []
        node, ok = v, 0 <= v < n
        while ok and node != 0:
            path.append(node)
            pn = int(parents[b, node])
            ok = 0 <= pn < node
            node = pn
        path = path[::-1]
        if not ok or len(path) != a:
            bad(b, f"last node {v} is not {a} accepted steps below the root")
            continue
        if [int(tokens_in[b, i]) for i in path] != tokens[b, :a].tolist():
            bad(b, "accepted tokens differ from the path's node tokens")
        y = int(tokens[b, a])
        if not 0 <= y < V:
            bad(b, f"emitted token {y} outside [0, {V})")
            continue
        if np.any(tokens[b, a + 1:] != -1):
            bad(b, "padding after the emitted token is not -1")
        same = (a == int(ref["num_accepted"][b]) and v == int(ref["last_node"][b])
                and np.array_equal(tokens[b], ref["tokens"][b]))
        if not (ref["margin_acc"][b] < band or ref["margin_rec"][b] < band):
            if a != int(ref["num_accepted"][b]) or v != int(ref["last_node"][b]):
                bad(b, f"accepted {a} / last {v} != oracle {int(ref['num_accepted'][b])} / "
                       f"{int(ref['last_node'][b])}")
            elif not same:
                bad(b, f"tokens {tokens[b].tolist()} != oracle {ref['tokens'][b].tolist()}")
            continue
        rep.flagged += 1
        if same:
            continue
        rep.flagged_mismatch += 1
        ev = oracle.verify_tree_path(ref, b, [0] + path, y)
        if ev["tests"] is None:
            bad(b, "the accepted path is not a walk of the tree")
            continue
        for child, walk, orc, m in ev["tests"]:
            if walk != orc and not m < band:
                bad(b, f"child {int(child)} {'accepted' if walk else 'rejected'} where the "
                       f"oracle {'accepts' if orc else 'rejects'} (margin {m:.3g})")
        if not _draw_ok(ev, y, band):
            bad(b, f"emitted {y} at node {v}: oracle draws {ev['token']} (draw margin "
                   f"{ev['margin_rec']:.3g}; u {ev['u']:.9f} vs [{ev['lo']:.9f}, "
                   f"{ev['hi']:.9f}), mass {ev['mass']:.3g})")
    return rep
