"""GPU parity of the n-gram prompt-lookup proposer (spec_ngram_propose)
against the CPU oracle (oracle.ngram_propose): integer work, so drafts and
counts must match bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

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


def check(svlib, name, ctx, lens, **kw):
    say(f"[gpu] ngram {name} B={ctx.shape[0]} stride={ctx.shape[1]} {kw}")
    c = ctx.to(torch.int32).contiguous().cuda()
    l = lens.to(torch.int32).contiguous().cuda()
    d, n = svlib.ngram_propose(c, l, **kw)
    torch.cuda.synchronize()
    rd, rn = oracle.ngram_propose(c.cpu().numpy(), l.cpu().numpy(), **kw)
    assert np.array_equal(n.cpu().numpy(), rn), (n.cpu().numpy(), rn)
    if kw["k"] > 0:
        assert np.array_equal(d.cpu().numpy(), rd)
    say(f"      proposals={int((rn > 0).sum())}/{len(rn)} drafts={int(rn.sum())}")
    return d, n, rd, rn


PARAMS = [dict(min_n=1, max_n=1, k=1, max_model_len=10 ** 6),
          dict(min_n=1, max_n=4, k=3, max_model_len=10 ** 6),
          dict(min_n=2, max_n=5, k=7, max_model_len=10 ** 6),
          dict(min_n=3, max_n=32, k=16, max_model_len=10 ** 6),
          dict(min_n=1, max_n=6, k=5, max_model_len=150)]


@pytest.mark.parametrize("pi", range(len(PARAMS)))
@pytest.mark.parametrize("alphabet", [2, 5, 50])
def test_random_small_alphabets(svlib, pi, alphabet):
    g = torch.Generator().manual_seed(17 * pi + alphabet)
    B, stride = 96, 300
    ctx = torch.randint(0, alphabet, (B, stride), generator=g)
    lens = torch.randint(0, stride + 1, (B,), generator=g)
    check(svlib, f"alphabet {alphabet}", ctx, lens, **PARAMS[pi])


def test_zipf_contexts_at_benchmark_size(svlib):
    ctx, lens = synth.make_contexts(512, 2048, 129280, seed=7, copy_spans=4,
                                    tail_copy_frac=0.5, device="cuda")
    _, _, _, rn = check(svlib, "zipf 512x2048", ctx, lens, min_n=2, max_n=5, k=3,
                        max_model_len=8192)
    assert (rn > 0).sum() > 100


def test_long_contexts(svlib):
    ctx, lens = synth.make_contexts(8, 32768, 129280, seed=3, copy_spans=8,
                                    tail_copy_frac=1.0, ragged=True, device="cuda")
    check(svlib, "32k", ctx, lens, min_n=1, max_n=8, k=5, max_model_len=10 ** 6)


def test_longest_n_and_runs(svlib):
    B, stride = 6, 200
    ctx = torch.full((B, stride), 4)  # runs: matches as long as max_n allows
    ctx[1, ::7] = 9
    ctx[2, 100:] = torch.arange(100) % 13
    ctx[3] = torch.arange(stride) % 40
    lens = torch.tensor([200, 200, 200, 200, 33, 2])
    for max_n in (1, 2, 31, 32):
        check(svlib, f"runs max_n={max_n}", ctx, lens, min_n=1, max_n=max_n, k=9,
              max_model_len=10 ** 6)


def test_lengths_clamped_and_degenerate(svlib):
    g = torch.Generator().manual_seed(2)
    ctx = torch.randint(0, 3, (8, 64), generator=g)
    lens = torch.tensor([-5, 0, 1, 2, 64, 65, 1000, 40])
    check(svlib, "clamped lengths", ctx, lens, min_n=1, max_n=3, k=4, max_model_len=100)
    check(svlib, "at max_model_len", ctx, lens, min_n=1, max_n=3, k=4, max_model_len=40)
    c = ctx.to(torch.int32).cuda()
    l = lens.to(torch.int32).cuda()
    _, n = svlib.ngram_propose(c, l, min_n=1, max_n=3, k=0, max_model_len=100)
    torch.cuda.synchronize()
    assert (n.cpu() == 0).all()


def test_proposals_feed_the_verify_step(svlib):
    """n-gram drafts on the GPU, then verified as one-hot drafts on the GPU:
    both match the oracle."""
    from oracle.parity import compare
    B, K, V = 64, 3, 4096
    ctx, lens = synth.make_contexts(B, 512, V, seed=11, copy_spans=3,
                                    tail_copy_frac=0.7, device="cuda")
    d, n, rd, rn = check(svlib, "drafts for verify", ctx, lens, min_n=2, max_n=4, k=K,
                         max_model_len=4096)
    w = synth.make_random(B, K, V, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.8),
                          with_draft=False, seed=5, device="cuda")
    w.draft_ids = torch.where(d < 0, torch.zeros_like(d), d).contiguous()
    w.num_drafts = n.clone()
    # the padding rows of the target are NaN past each request's own count
    tf = w.target.float()
    jt = torch.arange(K + 1, device="cuda").view(1, -1)
    tf = torch.where(jt.unsqueeze(-1) > n.view(-1, 1, 1), torch.full_like(tf, float("nan")),
                     torch.nan_to_num(tf, nan=0.0))
    w.target = tf.to(torch.bfloat16).contiguous()
    h = svlib.SpecVerify(B, K, V, torch.bfloat16)
    tokens, nacc = h.run(w.target, None, None, w.draft_ids, w.num_drafts, w.temperatures,
                         seed=9, offset=2)
    torch.cuda.synchronize()
    hs = w.host_arrays()
    ref = oracle.verify(hs["target"], None, hs["draft_ids"], hs["num_drafts"],
                        hs["temperatures"], seed=9, offset=2)
    rep = compare(hs, ref, tokens.cpu().numpy(), nacc.cpu().numpy())
    assert rep.ok(), rep.mismatches
    flags = h.device_errors(clear=True)
    assert flags & ~8 == 0
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    h.close()
