"""GPU parity of typical acceptance (spec_verify_run_typical) against the CPU
oracle (oracle.verify_typical), with the parity rule of oracle/parity.py:
accepted counts and tokens bit-exact outside the 1e-6 bands (the threshold
band is |p(x) - eps|; top-k ranks are integer counts and never flagged),
p(x) to 1e-5 relative."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.parity import compare

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


def check(svlib, w, eps, top_k, seed=0, offset=0, chunk=0, expect_flags=0):
    say(f"[gpu] typical {w.name} eps={eps} top_k={top_k} seed={seed} offset={offset}")
    w = w.to("cuda")
    h = svlib.SpecVerify(w.B, w.K, w.V, w.target.dtype, chunk_elems=chunk)
    dbg = torch.empty((w.B, w.K, 2), dtype=torch.float32, device="cuda")
    tokens, nacc = h.run_typical(w.target, w.draft_ids, w.num_drafts, w.temperatures,
                                 eps, top_k, seed=seed, offset=offset, out_debug_probs=dbg)
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    h.close()
    hs = w.host_arrays()
    ref = oracle.verify_typical(hs["target"], hs["draft_ids"], hs["num_drafts"],
                                hs["temperatures"], eps=eps, top_k=top_k, seed=seed,
                                offset=offset)
    rep = compare(hs, ref, tokens.cpu().numpy(), nacc.cpu().numpy(), dbg.cpu().numpy())
    say(f"      requests={rep.requests} flagged={rep.flagged} (differing "
        f"{rep.flagged_mismatch}) accept={rep.accepted}/{rep.proposed} "
        f"prob_max_rel={rep.prob_max_rel:.2e} flags={flags}")
    assert rep.ok(), rep.mismatches
    assert flags & ~8 == expect_flags, (flags, expect_flags)
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    assert ref["flags"] == expect_flags
    return rep


@pytest.mark.parametrize("cfg,eps,top_k", [(3, 0.05, 0), (3, 0.05, 2), (1, 0.1, 1),
                                           (2, 0.02, 3)])
def test_config_typical(svlib, cfg, eps, top_k):
    w = synth.make_config(cfg, device="cpu" if cfg <= 1 else "cuda")
    check(svlib, w, eps, top_k, seed=3, offset=cfg)


@pytest.mark.parametrize("eps,top_k", [(0.0, 0), (0.01, 0), (0.1, 1), (0.3, 4), (1.0, 0),
                                       (1.0, 2)])
def test_random_cases(svlib, eps, top_k):
    for seed, kw in enumerate([dict(B=24, K=5, V=1001, temps=(1.0, 0.0, 0.5, 1.7)),
                               dict(B=32, K=4, V=4099, dtype=torch.bfloat16, temps=(0.8, 1.2)),
                               dict(B=16, K=3, V=33333, dtype=torch.bfloat16, temps=(0.7,))]):
        w = synth.make_random(n_mode="ragged", seed=seed, corr=0.95, **kw)
        check(svlib, w, eps, top_k, seed=seed, offset=2 * seed)


def test_ranks_with_ties(svlib):
    """Integer logits: many tokens share a value, so the top-k clause is
    decided by exact counts of strictly larger logits."""
    g = torch.Generator().manual_seed(7)
    B, K, V = 64, 4, 700
    t = torch.randint(-3, 3, (B, K + 1, V), generator=g).float()
    ids = torch.randint(0, V, (B, K), generator=g).int()
    w = synth.Workload("integer logits", t, None, None, ids,
                       torch.randint(0, K + 1, (B,), generator=g).int(),
                       torch.full((B,), 0.5))
    for top_k in (1, 50, 200, 400):
        check(svlib, w, 0.9, top_k, offset=top_k)
    w.target = t.to(torch.bfloat16)
    check(svlib, w, 0.9, 120, offset=1)


def test_extremes(svlib):
    w = synth.make_random(16, 5, 3000, dtype=torch.bfloat16, temps=(1.0, 0.6), seed=4)
    rep = check(svlib, w, 0.0, 0)          # every valid draft accepted
    assert rep.accepted == rep.proposed
    rep = check(svlib, w, 1.0, 0, offset=1)  # none accepted
    assert rep.accepted == 0


def test_bad_data_and_k0(svlib):
    w = synth.make_random(16, 4, 300, temps=(1.0, 0.0), seed=4, nan_padding=False)
    w.draft_ids[0, 0] = -1
    w.draft_ids[1, 1] = 300
    w.num_drafts[2] = -3
    w.num_drafts[3] = 9
    check(svlib, w, 0.01, 2, expect_flags=1 | 2)
    w = synth.make_random(40, 0, 513, temps=(1.0, 0.3, 0.0), seed=2)
    check(svlib, w, 0.1, 1)


def test_chunk_sizes(svlib):
    w = synth.make_random(20, 4, 20000, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.6),
                          n_mode="ragged", seed=9)
    for chunk in (256, 1024, 15360):
        check(svlib, w, 0.002, 3, chunk=chunk)


def test_max_vocab(svlib):
    """V = 983040 (64 chunks): rank counts summed over every chunk."""
    w = synth.make_random(6, 3, 983040, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.6),
                          n_mode="ragged", corr=0.97, seed=3, device="cuda")
    check(svlib, w, 1e-6, 3, seed=2, offset=1)


def test_draw_sizes(svlib):
    """Batches whose draw count selects each draw workgroup size."""
    for B in (700, 800, 900):
        w = synth.make_random(B, 2, 1500, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.8),
                              n_mode="ragged", corr=0.97, seed=B, device="cuda")
        check(svlib, w, 0.02, 2, seed=2, offset=B)
