"""GPU parity of the draft-token sampler (spec_draft_sample) against the CPU
oracle (oracle.draft_sample), through the C ABI.

Every case samples on the GPU, copies the exact input bytes back, runs the
oracle with the same Philox seed and offset and applies oracle.parity's
compare_draft: tokens bit-exact outside the 1e-6 draw band, q(x) to 1e-5
relative, -1 past each request's draft count.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.parity import compare_draft

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


def run_gpu(svlib, draft, nd, temps, seed, offset, chunk=0, handle=None):
    B, K, V = draft.shape
    h = handle or svlib.SpecVerify(max(B, 1), max(K, 1), V, draft.dtype,
                                   draft_dtype=draft.dtype, chunk_elems=chunk)
    q = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ids = h.sample(draft, nd, temps, seed=seed, offset=offset, out_q=q)
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    out = ids.cpu().numpy(), q.cpu().numpy(), flags
    if handle is None:
        h.close()
    return out


def host(t):
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check(svlib, name, draft, nd, temps, seed=0, offset=0, chunk=0, expect_flags=0,
          handle=None):
    say(f"[gpu] draft sample {name} shape={tuple(draft.shape)} seed={seed} "
        f"offset={offset} chunk={chunk}")
    draft = draft.to("cuda").contiguous()
    nd_d = None if nd is None else nd.to("cuda").contiguous()
    temps_d = temps.to("cuda").contiguous()
    ids, q, flags = run_gpu(svlib, draft, nd_d, temps_d, seed, offset, chunk, handle)
    ref = oracle.draft_sample(host(draft), host(nd_d), host(temps_d), seed=seed,
                              offset=offset)
    rep = compare_draft(ref, ids, q)
    say(f"      rows={rep.proposed} flagged={rep.flagged} (differing "
        f"{rep.flagged_mismatch}) q_max_rel={rep.prob_max_rel:.2e} flags={flags}")
    assert rep.ok(), rep.mismatches
    assert flags & ~8 == expect_flags, (flags, expect_flags)
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    assert ref["flags"] == expect_flags
    return ids, ref


# ---------------------------------------------------------------------------
# Draft rows of the full-size workloads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_config_draft_rows(svlib, cfg):
    w = synth.make_config(cfg, device="cpu" if cfg <= 1 else "cuda")
    check(svlib, w.name, w.draft, w.num_drafts, w.temperatures, seed=7, offset=cfg)


# ---------------------------------------------------------------------------
# Small and edge cases
# ---------------------------------------------------------------------------
def _rows(B, K, V, dtype, seed, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, K, V), generator=g) * scale).to(dtype)


CASES = {
    "f32_V1001_mixT": dict(B=24, K=5, V=1001, temps=(1.0, 0.0, 0.5, 1.7)),
    "bf16_V4099": dict(B=32, K=4, V=4099, dtype=torch.bfloat16, temps=(0.8, 1.2, -1.0)),
    "bf16_V33333_nan_inf_T": dict(B=12, K=7, V=33333, dtype=torch.bfloat16,
                                  temps=(0.7, float("nan"), float("inf"), 1e-40)),
    "V1": dict(B=8, K=3, V=1, temps=(1.0, 0.0)),
    "V2": dict(B=64, K=2, V=2, temps=(1.0, 0.5, 0.0)),
    "V5": dict(B=64, K=6, V=5, temps=(1.0, 2.0, 0.0)),
    "tiny_T": dict(B=16, K=3, V=300, temps=(1e-3, 0.05)),
    "huge_logits": dict(B=16, K=3, V=1500, temps=(1.0,), scale=40.0),
    "K1_one_position": dict(B=200, K=1, V=2048, temps=(0.9,)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_random_case(svlib, name):
    kw = dict(CASES[name])
    B, K, V = kw["B"], kw["K"], kw["V"]
    dtype = kw.get("dtype", torch.float32)
    for seed in (0, 1):
        l = _rows(B, K, V, dtype, seed, kw.get("scale", 2.0))
        temps = torch.tensor([kw["temps"][b % len(kw["temps"])] for b in range(B)],
                             dtype=torch.float32)
        g = torch.Generator().manual_seed(100 + seed)
        nd = torch.randint(0, K + 1, (B,), generator=g).to(torch.int32)
        check(svlib, name, l, nd, temps, seed=seed, offset=3 * seed)


def test_all_rows_when_counts_are_null(svlib):
    l = _rows(20, 4, 3000, torch.bfloat16, 5)
    temps = torch.tensor([1.0, 0.0, 0.6, 1.3] * 5)
    ids, _ = check(svlib, "null counts", l, None, temps, seed=2, offset=4)
    assert (ids >= 0).all()


@pytest.mark.parametrize("chunk", [256, 1024, 15360])
def test_chunk_sizes(svlib, chunk):
    l = _rows(16, 4, 20000, torch.bfloat16, 9)
    temps = torch.tensor([1.0, 0.0, 0.6, 2.0] * 4)
    nd = torch.tensor([4, 3, 0, 1] * 4, dtype=torch.int32)
    check(svlib, "chunks", l, nd, temps, seed=1, offset=2, chunk=chunk)


def test_bad_counts_are_flagged(svlib):
    l = _rows(8, 3, 500, torch.float32, 4)
    nd = torch.tensor([3, -2, 9, 1, 0, 3, 2, 3], dtype=torch.int32)
    check(svlib, "bad counts", l, nd, torch.ones(8), expect_flags=2)


def test_greedy_ties_take_lowest_index(svlib):
    g = torch.Generator().manual_seed(5)
    l = torch.randint(-3, 2, (64, 4, 700), generator=g).float()
    ids, _ = check(svlib, "greedy ties", l, None, torch.zeros(64))
    am = torch.argmax(l, -1).numpy()  # lowest index of the max
    assert np.array_equal(ids, am)


def test_monte_carlo_law_on_gpu(svlib):
    """One row repeated over 2^17 requests: the sampled tokens follow
    softmax(l / T) (chi-square), and match the oracle token for token."""
    import scipy.stats
    B, V, T = 1 << 17, 8, 0.8
    row = torch.tensor([0.3, -1.2, 2.0, 0.0, 1.1, -0.4, 0.9, -2.5])
    l = row.view(1, 1, V).expand(B, 1, V).contiguous()
    ids, ref = check(svlib, "monte carlo", l, None, torch.full((B,), T), seed=11, offset=0)
    qv = torch.softmax(row.double() / T, 0).numpy()
    counts = np.bincount(ids[:, 0], minlength=V)
    assert scipy.stats.chisquare(counts, qv * B).pvalue > 1e-3


def test_sampler_and_verify_share_a_handle(svlib):
    """Sample the drafts on the GPU, then verify them with the same handle:
    both steps match the oracle."""
    from oracle.parity import compare
    w = synth.make_random(32, 4, 5000, dtype=torch.bfloat16, temps=(1.0, 0.7, 0.0),
                          n_mode="ragged", seed=3, device="cuda")
    h = svlib.SpecVerify(32, 4, 5000, torch.bfloat16, draft_dtype=torch.bfloat16)
    ids, _ = check(svlib, "shared handle", w.draft, w.num_drafts, w.temperatures,
                   seed=4, offset=1, handle=h)
    w.draft_ids = torch.from_numpy(np.where(ids < 0, 0, ids)).to("cuda").int()
    tokens, nacc = h.run(w.target, w.draft, w.draft_mode, w.draft_ids, w.num_drafts,
                         w.temperatures, seed=4, offset=1)
    torch.cuda.synchronize()
    hs = w.host_arrays()
    ref = oracle.verify(hs["target"], hs["draft"], hs["draft_ids"], hs["num_drafts"],
                        hs["temperatures"], seed=4, offset=1)
    rep = compare(hs, ref, tokens.cpu().numpy(), nacc.cpu().numpy())
    assert rep.ok(), rep.mismatches
    flags = h.device_errors(clear=True)
    assert flags & ~8 == 0
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    h.close()


def test_empty_and_unsupported(svlib):
    h = svlib.SpecVerify(4, 2, 100, torch.float32)
    assert svlib.spec_draft_sample(h.handle, 0, 2, 0, 0, 0, 0, 0, 0, 0, None) == 0
    assert svlib.spec_draft_sample(h.handle, 4, 0, 0, 0, 0, 0, 0, 0, 0, None) == 0
    assert svlib.spec_draft_sample(h.handle, 5, 2, 1, 0, 1, 0, 0, 1, 0, None) == -3
    h.close()
    hp = svlib.SpecVerify(4, 2, 100, torch.float32, draft_is_probs=True)
    assert svlib.spec_draft_sample(hp.handle, 4, 2, 1, 0, 1, 0, 0, 1, 0, None) == -2
    hp.close()


def test_max_vocab_and_drafts(svlib):
    """The largest sizes a handle takes: V = 983040 (64 chunks) and K = 31."""
    l = _rows(3, 2, 983040, torch.bfloat16, 11)
    temps = torch.tensor([1.0, 0.0, 0.7])
    nd = torch.tensor([2, 2, 1], dtype=torch.int32)
    check(svlib, "max vocab", l, nd, temps, seed=1, offset=5)
    l = _rows(6, 31, 2000, torch.float32, 12)
    temps = torch.tensor([1.0, 0.0, 0.7, 1.5, 0.3, 1.0])
    nd = torch.tensor([31, 30, 0, 17, 31, 1], dtype=torch.int32)
    check(svlib, "max drafts", l, nd, temps, seed=2, offset=6)


def test_draw_sizes(svlib):
    """Row counts on each side of the draw workgroup sizes (1024 threads up to
    768 rows, 512 up to 896, 256 above)."""
    for B, K in ((192, 4), (160, 5), (180, 5)):
        l = _rows(B, K, 3000, torch.bfloat16, 20 + B)
        temps = torch.tensor([(1.0, 0.0, 0.6)[b % 3] for b in range(B)])
        check(svlib, f"{B * K} rows", l, None, temps, seed=3, offset=B)
