"""Parity rule between an implementation's verify outputs and the oracle's.

TEST INFRASTRUCTURE (see the package docstring).  Works on numpy arrays only.

Rule: a request is flagged when one of the decisions the oracle evaluated
lies within ``band`` of its threshold (|u - p(x)/q(x)| < band) or the draw
uniform lies within ``band`` of a CDF boundary (relative to the law's total).
Unflagged requests must match bit for bit in the accepted count and in every
token.  A request flagged at decision j must still agree on tokens 0..j-1; a
request flagged only at the draw must agree on the accepted count and the
accepted tokens.  Every output must be valid whatever the flags.  Acceptance
probabilities p_j(x_j), q_j(x_j) must agree to ``prob_rtol`` relative (an
absolute floor of 1e-35 below 1e-30).
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class ParityReport:
    requests: int = 0
    flagged: int = 0
    flagged_mismatch: int = 0   # flagged requests whose outputs differ
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


def compare(host, ref, tokens, nacc, dbg=None, *, band=1e-6, prob_rtol=1e-5,
            max_report=20) -> ParityReport:
    """host: the input arrays (synth.Workload.host_arrays()); ref: the
    oracle's result dict; tokens [B, K+1], nacc [B], dbg [B, K, 2] or None:
    the implementation's outputs."""
    tokens = np.asarray(tokens)
    nacc = np.asarray(nacc)
    B, K1 = tokens.shape
    K = K1 - 1
    V = host["target"].shape[2]
    nd = np.clip(np.asarray(host["num_drafts"]), 0, K)
    ids = np.asarray(host["draft_ids"]).reshape(B, K)
    samp = _is_sampling(host["temperatures"])
    rep = ParityReport(requests=B)

    def bad(b, why):
        if len(rep.mismatches) < max_report:
            rep.mismatches.append((b, why))
        else:
            rep.mismatches.append((b, "..."))

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
        if np.any(tokens[b, ga + 1:] != -1):
            bad(b, "padding after the emitted token is not -1")
        # flag position
        flag_at = None
        for j in range(oa + 1 if oa < n else n):
            m = ref["margin_acc"][b, j]
            if np.isfinite(m) and m < band:
                flag_at = j
                break
        rec_flag = flag_at is None and ref["margin_rec"][b] < band
        if flag_at is not None or rec_flag:
            rep.flagged += 1
            if ga != oa or not np.array_equal(tokens[b], ref["tokens"][b]):
                rep.flagged_mismatch += 1
            if flag_at is not None:
                if ga < flag_at:
                    bad(b, f"flagged at decision {flag_at} but n_acc {ga} < {flag_at}")
            elif ga != oa:
                bad(b, f"flagged at the draw only but n_acc {ga} != oracle {oa}")
            continue
        if ga != oa:
            bad(b, f"n_acc {ga} != oracle {oa}")
        elif not np.array_equal(tokens[b], ref["tokens"][b]):
            bad(b, f"tokens {tokens[b].tolist()} != oracle {ref['tokens'][b].tolist()}")

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
    token exactly; a flagged row must still be a valid token.  Rows past n_b
    must be -1.  q_j(x_j) must agree to ``prob_rtol`` relative wherever the
    token matches (an absolute floor of 1e-35 below 1e-30)."""
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
                rep.flagged_mismatch += int(g != o)
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
    Unflagged requests must match exactly (tokens, count, last node).  Every
    output must be valid: the accepted path climbs from the last node to the
    root through parents, its tokens are those nodes' tokens, then one token
    in [0, V), then -1."""
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
        if not 0 <= int(tokens[b, a]) < V:
            bad(b, f"emitted token {int(tokens[b, a])} outside [0, {V})")
        if np.any(tokens[b, a + 1:] != -1):
            bad(b, "padding after the emitted token is not -1")
        if ref["margin_acc"][b] < band or ref["margin_rec"][b] < band:
            rep.flagged += 1
            rep.flagged_mismatch += int(not np.array_equal(tokens[b], ref["tokens"][b]))
            continue
        if a != int(ref["num_accepted"][b]) or v != int(ref["last_node"][b]):
            bad(b, f"accepted {a} / last {v} != oracle {int(ref['num_accepted'][b])} / "
                   f"{int(ref['last_node'][b])}")
        elif not np.array_equal(tokens[b], ref["tokens"][b]):
            bad(b, f"tokens {tokens[b].tolist()} != oracle {ref['tokens'][b].tolist()}")
    return rep
