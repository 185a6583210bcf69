"""GPU parity of token-tree verification (spec_verify_run_tree) against the
CPU oracle (oracle.verify_tree), with oracle.parity.compare_tree: accepted
paths, counts, last nodes and emitted tokens bit-exact outside the 1e-6
decision and draw bands, every output a valid walk of its tree."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.parity import compare_tree

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def svlib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import rejection_sampling_verify_temp_amd as m
    m.load_library()
    return m


def check(svlib, w, seed=0, offset=0, draft_is_probs=False, expect_flags=0, members=0):
    say(f"[gpu] tree {w.name} seed={seed} offset={offset} members={members or 'picked'}")
    w = w.to("cuda")
    h = svlib.SpecVerify(w.B, 1, w.V, w.target.dtype,
                         draft_dtype=w.draft.dtype if w.draft is not None else None,
                         draft_is_probs=draft_is_probs)
    if members:
        h.set_tree_team_size(members)
        assert h.tree_team_size(w.B, w.draft is not None) == members
    tokens, nacc, last = h.run_tree(w.target, w.draft, w.tokens, w.parents, w.num_nodes,
                                    w.temperatures, seed=seed, offset=offset)
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    h.close()
    hs = w.host_arrays()
    ref = oracle.verify_tree(hs["target"], hs["draft"], hs["tokens"], hs["parents"],
                             hs["num_nodes"], hs["temperatures"], seed=seed, offset=offset,
                             draft_is_probs=draft_is_probs)
    rep = compare_tree(hs["tokens"], hs["parents"], hs["num_nodes"], w.V, ref,
                       tokens.cpu().numpy(), nacc.cpu().numpy(), last.cpu().numpy())
    say(f"      requests={rep.requests} flagged={rep.flagged} (differing "
        f"{rep.flagged_mismatch}) accepted={rep.accepted} flags={flags}")
    assert rep.ok(), rep.mismatches
    assert flags & ~8 == expect_flags, (flags, expect_flags)
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    assert ref["flags"] == expect_flags
    return rep, ref


CASES = {
    "f32_V1001_random": dict(B=32, N=12, V=1001, temps=(1.0, 0.0, 0.6)),
    "bf16_V4099_random": dict(B=32, N=16, V=4099, dtype=torch.bfloat16, temps=(0.8, 1.3)),
    "bf16_wide": dict(B=24, N=9, V=3000, dtype=torch.bfloat16, temps=(1.0,), shape="wide"),
    "chain": dict(B=24, N=8, V=2051, temps=(1.0, 0.0, 0.7), shape="chain"),
    "onehot_random": dict(B=32, N=12, V=777, temps=(1.0, 0.5, 0.0), onehot=True),
    "onehot_wide": dict(B=24, N=7, V=500, temps=(0.9,), onehot=True, shape="wide"),
    "mixed_dtypes": dict(B=16, N=10, V=2000, dtype=torch.bfloat16, draft_dtype=torch.float32,
                         temps=(1.1,)),
    "V2": dict(B=64, N=6, V=2, temps=(1.0, 0.5, 0.0)),
    "V1": dict(B=8, N=4, V=1, temps=(1.0, 0.0)),
    "N1_root_only": dict(B=16, N=1, V=300, temps=(1.0, 0.0)),
    "low_corr": dict(B=32, N=14, V=1500, temps=(1.0,), corr=0.2),
    "tiny_T": dict(B=16, N=8, V=300, temps=(1e-3, 0.05)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_random_trees(svlib, name):
    for seed in (0, 1):
        w = synth.make_tree(seed=seed, **CASES[name])
        check(svlib, w, seed=seed, offset=5 * seed)


def test_chain_tree_equals_verify(svlib):
    """A chain-shaped tree on the GPU gives the verify step's outputs."""
    w = synth.make_random(32, 5, 3000, dtype=torch.bfloat16, temps=(1.0, 0.7, 0.0),
                          n_mode="ragged", seed=6, nan_padding=False)
    B, K, V = w.B, w.K, w.V
    N = K + 1
    tokens = torch.zeros((B, N), dtype=torch.int32)
    tokens[:, 1:] = w.draft_ids
    parents = torch.arange(-1, N - 1, dtype=torch.int32).repeat(B, 1)
    draft = torch.zeros((B, N, V), dtype=w.draft.dtype)
    draft[:, :K] = w.draft
    t = synth.TreeWorkload("chain of a verify batch", w.target, draft, tokens, parents,
                           w.num_drafts + 1, w.temperatures)
    rep, ref = check(svlib, t, seed=2, offset=3)
    hs = w.host_arrays()
    chain = oracle.verify(hs["target"], hs["draft"], hs["draft_ids"], hs["num_drafts"],
                          hs["temperatures"], seed=2, offset=3)
    assert np.array_equal(ref["tokens"], chain["tokens"])


def test_probability_drafts(svlib):
    w = synth.make_tree(24, 10, 1200, temps=(1.0, 0.8), seed=3)
    w.draft = torch.softmax(w.draft.float(), -1)
    check(svlib, w, seed=1, draft_is_probs=True)


def test_malformed_trees_are_flagged(svlib):
    w = synth.make_tree(8, 6, 300, temps=(1.0, 0.0), seed=4, ragged=False)
    w.parents[0, 3] = 5      # parent after the node: never visited
    w.tokens[1, 1] = -4      # bad id: never accepted
    w.tokens[2, 2] = 300
    w.num_nodes[3] = 0       # clamped into [1, N]
    w.num_nodes[4] = 9
    check(svlib, w, expect_flags=16 | 1 | 2)


def test_malformed_large_trees_are_flagged(svlib):
    """Trees of 200 nodes, where the parent check runs over several groups
    of 64 nodes: a parent after its node at index 70, one at index 150, and
    a negative parent at index 2, each in a request of its own, against two
    well-formed requests."""
    w = synth.make_tree(5, 200, 700, temps=(1.0, 0.0, 0.7), seed=41, ragged=False)
    w.parents[0, 70] = 120
    w.parents[1, 150] = 150
    w.parents[2, 2] = -1
    check(svlib, w, seed=5, offset=2, expect_flags=16)


def test_realistic_size(svlib):
    """64 requests, trees of 16 nodes over a 32000-token vocabulary."""
    w = synth.make_tree(64, 16, 32000, dtype=torch.bfloat16, temps=(1.0, 0.6, 0.0), seed=8,
                        corr=0.95, device="cuda")
    rep, _ = check(svlib, w, seed=9, offset=1)
    assert rep.accepted > 0


@pytest.mark.parametrize("members", [0, 1])
def test_max_nodes(svlib, members):
    """Trees of 256 nodes, the most the entry point takes, in teams (the
    pick) and in one 1024-thread workgroup per request."""
    w = synth.make_tree(8, 256, 600, temps=(1.0, 0.0, 0.7), seed=12, corr=0.97)
    check(svlib, w, seed=3, offset=2, members=members)
    w = synth.make_tree(8, 256, 600, temps=(1.0, 0.8), seed=13, onehot=True, shape="wide")
    check(svlib, w, seed=4, offset=1, members=members)


@pytest.mark.parametrize("members", [0, 1])
def test_max_vocab(svlib, members):
    """V = 983040.  In one 1024-thread workgroup per request, fp32 rows fill
    the draw's slot table (3840 slots of 64 vectors plus head and tail) and
    bf16 rows take two rounds per pass; teams (the pick) split both."""
    for dtype, seed in ((torch.float32, 14), (torch.bfloat16, 15)):
        w = synth.make_tree(4, 6, 983040, dtype=dtype, temps=(1.0, 0.0, 0.6, 1.0), seed=seed,
                            corr=0.97, device="cuda")
        check(svlib, w, seed=seed, offset=3, members=members)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_onehot_dominant_sibling(svlib, dtype):
    """One-hot trees whose first child holds almost all of the root's p
    (about 0.99 at T = 0.3): after its rare rejection the second child and
    the draw see the remaining 1%, so the removed token must leave its draw
    slot exactly, not as a difference of rounded sums."""
    g = torch.Generator().manual_seed(43)
    B, N, V, T = 2048, 3, 20000, 0.3
    t = torch.randn((B, N, V), generator=g) * 0.5
    tok = torch.randint(0, V, (B, N), generator=g, dtype=torch.int32)
    tok[:, 0] = 0
    for b in range(B):
        t[b, 0, tok[b, 1]] = 4.6 + 0.3 * float(np.log(V / 50000))
    w = synth.TreeWorkload("one-hot trees, dominant first child", t.to(dtype), None, tok,
                           torch.tensor([[-1, 0, 0]] * B, dtype=torch.int32),
                           torch.full((B,), N, dtype=torch.int32), torch.full((B,), T))
    rep, ref = check(svlib, w, seed=6, offset=2)
    assert int((ref["last_node"] == 0).sum()) >= 10  # enough walks past the first child


def test_benchmark_shape(svlib):
    """The tree benchmark's own shape and law: 256 random recursive trees of
    16 nodes over V = 152064, bf16 target and draft logits, T in
    {0.6, 1.0, 0.0, 0.8}, correlation 0.95, every node in use."""
    w = synth.make_tree(256, 16, 152064, dtype=torch.bfloat16, seed=31,
                        temps=(0.6, 1.0, 0.0, 0.8), corr=0.95, ragged=False, device="cuda")
    rep, _ = check(svlib, w, seed=0, offset=0)
    assert rep.accepted > 0


# Batches and team settings whose walks differ on MI355X (256 compute
# units).  Picked: eight workgroups per request up to B = 256 (at B = 200 each
# of the 128 teams of eight walks one or two requests), four beyond, where at
# B = 300 each team of four walks one or two requests.  Set: teams of four at
# B = 100, teams of eight that walk two or three requests each, and one
# 1024-thread workgroup per request, at B = 300.
TEAM_CASES = {
    (40, 0): dict(dtype=torch.bfloat16, temps=(1.0, 0.6, 0.0)),
    (100, 0): dict(temps=(0.9, 0.0)),
    (100, 4): dict(dtype=torch.bfloat16, temps=(1.0, 0.0, 0.7)),
    (200, 0): dict(dtype=torch.bfloat16, temps=(0.8, 0.0, 1.2)),
    (300, 0): dict(temps=(1.0, 0.7)),
    (300, 1): dict(temps=(1.0, 0.7)),
    (300, 8): dict(dtype=torch.bfloat16, temps=(1.0, 0.0, 0.6)),
}


@pytest.mark.parametrize("B,members", sorted(TEAM_CASES))
def test_team_sizes(svlib, B, members):
    """Logit, one-hot and probability-draft trees at batches and team
    settings that run teams of 8 and 4 workgroups (one request per team, or
    several in turn) and single workgroups, against the oracle."""
    V = 20011  # an odd vocabulary: unaligned rows, a head and a tail in every row
    h = svlib.SpecVerify(B, 1, V, torch.float32)
    say(f"[gpu] tree team size picked at B={B}: {h.tree_team_size(B)} "
        f"(one-hot {h.tree_team_size(B, False)}); set: {members or 'none'}")
    h.close()
    w = synth.make_tree(B, 12, V, seed=50 + B + members, corr=0.9, device="cuda",
                        **TEAM_CASES[(B, members)])
    check(svlib, w, seed=B, offset=1, members=members)
    w = synth.make_tree(B, 10, V, seed=51 + B + members, onehot=True, temps=(1.0, 0.5),
                        device="cuda")
    check(svlib, w, seed=B, offset=2, members=members)
    w = synth.make_tree(B, 8, V, seed=52 + B + members, temps=(1.0,), device="cuda")
    w.draft = torch.softmax(w.draft.float(), -1)
    check(svlib, w, seed=B, offset=3, draft_is_probs=True, members=members)


def test_many_requests_per_team(svlib):
    """B = 1000 requests on 256 teams of four: each team takes about four
    requests from the launch's counter, in an order that depends on timing.
    The outputs match the oracle, and five launches in a row on one handle
    repeat the first bit for bit (the counter is back at 0 after every
    launch)."""
    B, V = 1000, 2053
    w = synth.make_tree(B, 10, V, dtype=torch.bfloat16, seed=80, corr=0.9,
                        temps=(1.0, 0.0, 0.7), device="cuda")
    check(svlib, w, seed=9, offset=1)
    h = svlib.SpecVerify(B, 1, V, torch.bfloat16, draft_dtype=torch.bfloat16)
    assert h.tree_team_size(B) == 4
    outs = [[x.cpu() for x in h.run_tree(w.target, w.draft, w.tokens, w.parents, w.num_nodes,
                                         w.temperatures, seed=9, offset=off)]
            for off in (1, 2, 3, 4, 1)]
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    h.close()
    assert flags & ~8 == 0, flags
    for a, b in zip(outs[0], outs[-1]):
        assert torch.equal(a, b)


def test_team_size_setting(svlib):
    """The setting's contract on the host: 0, 1, 4 and 8 are taken and
    reported, anything else is refused, and 0 restores the pick."""
    h = svlib.SpecVerify(64, 1, 1000, torch.float32)
    picked = h.tree_team_size(300)
    for m in (1, 4, 8):
        h.set_tree_team_size(m)
        assert h.tree_team_size(300) == m and h.tree_team_size(8, False) == m
    for bad in (2, 3, 16, -1):
        with pytest.raises(svlib.SpecVerifyError):
            h.set_tree_team_size(bad)
    h.set_tree_team_size(0)
    assert h.tree_team_size(300) == picked == 4
    h.close()


@pytest.mark.parametrize("B", [40, 100, 200, 300])
def test_team_launches_in_a_row(svlib, B):
    """One handle, the same trees launched five times with a different
    offset each and then again with the first: a team walk returns its
    exchange words to 0 at its end, so every launch starts clean and the
    repeat matches the first launch bit for bit."""
    V = 8192
    w = synth.make_tree(B, 16, V, dtype=torch.bfloat16, seed=60 + B, corr=0.95,
                        temps=(1.0, 0.8, 0.0), ragged=False, device="cuda")
    h = svlib.SpecVerify(B, 1, V, torch.bfloat16, draft_dtype=torch.bfloat16)
    assert h.tree_team_size(B) in (4, 8)
    outs = []
    for off in (0, 1, 2, 3, 4, 0):
        outs.append([x.cpu() for x in h.run_tree(w.target, w.draft, w.tokens, w.parents,
                                                   w.num_nodes, w.temperatures, seed=5,
                                                   offset=off)])
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    h.close()
    assert flags & ~8 == 0, flags
    for a, b in zip(outs[0], outs[-1]):
        assert torch.equal(a, b)
    hs = w.host_arrays()
    ref = oracle.verify_tree(hs["target"], hs["draft"], hs["tokens"], hs["parents"],
                             hs["num_nodes"], hs["temperatures"], seed=5, offset=4)
    rep = compare_tree(hs["tokens"], hs["parents"], hs["num_nodes"], V, ref,
                       outs[4][0].numpy(), outs[4][1].numpy(), outs[4][2].numpy())
    assert rep.ok(), rep.mismatches


@pytest.mark.parametrize("B", [40, 100, 200, 300])
def test_team_members_finishing_alone(svlib, B):
    """With the team wait bound at 0 the members give up on their partners at
    once, in a mix of team and solo walks that differs run to run; each then
    computes every member's share itself, so the outputs match a normal run's
    bit for bit, and the condition is flagged."""
    V = 20011
    w = synth.make_tree(B, 12, V, dtype=torch.bfloat16, seed=70 + B, corr=0.9,
                        temps=(1.0, 0.6, 0.0), device="cuda")
    outs, flags = [], []
    for wait in (20000, 0, 0):
        h = svlib.SpecVerify(B, 1, V, torch.bfloat16, draft_dtype=torch.bfloat16)
        assert h.tree_team_size(B) in (4, 8)
        h.set_tree_wait_us(wait)
        outs.append([x.cpu() for x in h.run_tree(w.target, w.draft, w.tokens, w.parents,
                                                   w.num_nodes, w.temperatures, seed=3,
                                                   offset=1)])
        torch.cuda.synchronize()
        flags.append(h.device_errors(clear=True))
        h.close()
    say(f"      device flags by wait bound 20000/0/0 us: {flags}")
    assert flags[0] & ~8 == 0
    for f in flags[1:]:
        assert f & ~(8 | 32) == 0
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)
