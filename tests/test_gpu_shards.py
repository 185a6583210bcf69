"""A batch split into shards, each run with spec_verify_set_request_base set
to its first request's index, gives bit for bit the outputs of one call over
the whole batch: the property a batch-sharded (data-parallel) deployment
relies on, since every shard draws its Philox counters at the requests'
global indices.  Covers the verify step, typical acceptance, the draft
sampler and token trees."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

SHARDS = ((0, 16), (16, 21), (21, 48))


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


def shard(t, a, b):
    return None if t is None else t[a:b].contiguous()


def check_equal(name, full, parts):
    for k, (f, p) in enumerate(zip(full, parts)):
        got = torch.cat(p).cpu().numpy()
        ref = f.cpu().numpy()
        assert np.array_equal(got, ref, equal_nan=True), (name, k)


def test_verify_shards(svlib):
    w = synth.make_random(48, 4, 3000, dtype=torch.bfloat16, temps=(1.0, 0.7, 0.0),
                          n_mode="ragged", onehot_frac=0.3, seed=21, device="cuda")
    say("[gpu] shards verify B=48 K=4 V=3000")
    h = svlib.SpecVerify(w.B, w.K, w.V, torch.bfloat16, draft_dtype=torch.bfloat16)

    def run(a, b):
        dbg = torch.empty((b - a, w.K, 2), dtype=torch.float32, device="cuda")
        t, n = h.run(shard(w.target, a, b), shard(w.draft, a, b), shard(w.draft_mode, a, b),
                     shard(w.draft_ids, a, b), shard(w.num_drafts, a, b),
                     shard(w.temperatures, a, b), seed=7, offset=3, out_debug_probs=dbg)
        return t, n, dbg

    full = run(0, w.B)
    parts = [[], [], []]
    for a, b in SHARDS:
        h.set_request_base(a)
        for k, x in enumerate(run(a, b)):
            parts[k].append(x)
    h.set_request_base(0)
    torch.cuda.synchronize()
    check_equal("verify", full, parts)
    # without the base the later shards draw other uniforms
    t, _, _ = run(16, 48)
    torch.cuda.synchronize()
    assert not torch.equal(t, full[0][16:])
    assert h.device_errors(clear=True) & ~8 == 0
    h.close()


def test_typical_shards(svlib):
    w = synth.make_random(48, 3, 2500, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.8),
                          n_mode="ragged", corr=0.97, seed=22, device="cuda")
    say("[gpu] shards typical B=48 K=3 V=2500")
    h = svlib.SpecVerify(w.B, w.K, w.V, torch.bfloat16)

    def run(a, b):
        return h.run_typical(shard(w.target, a, b), shard(w.draft_ids, a, b),
                             shard(w.num_drafts, a, b), shard(w.temperatures, a, b),
                             0.02, 2, seed=5, offset=1)

    full = run(0, w.B)
    parts = [[], []]
    for a, b in SHARDS:
        h.set_request_base(a)
        for k, x in enumerate(run(a, b)):
            parts[k].append(x)
    torch.cuda.synchronize()
    check_equal("typical", full, parts)
    h.close()


def test_sampler_shards(svlib):
    g = torch.Generator(device="cuda").manual_seed(23)
    B, K, V = 48, 5, 2000
    draft = (torch.randn((B, K, V), generator=g, device="cuda") * 2).to(torch.bfloat16)
    nd = torch.randint(0, K + 1, (B,), generator=g, device="cuda").to(torch.int32)
    temps = torch.tensor([(1.0, 0.0, 0.6)[b % 3] for b in range(B)], device="cuda")
    say("[gpu] shards sampler B=48 K=5 V=2000")
    h = svlib.SpecVerify(B, K, V, torch.bfloat16, draft_dtype=torch.bfloat16)

    def run(a, b):
        q = torch.empty((b - a, K), dtype=torch.float32, device="cuda")
        ids = h.sample(shard(draft, a, b), shard(nd, a, b), shard(temps, a, b), seed=9,
                       offset=4, out_q=q)
        return ids, q

    full = run(0, B)
    parts = [[], []]
    for a, b in SHARDS:
        h.set_request_base(a)
        for k, x in enumerate(run(a, b)):
            parts[k].append(x)
    torch.cuda.synchronize()
    check_equal("sampler", full, parts)
    h.close()


def test_tree_shards(svlib):
    w = synth.make_tree(48, 10, 1500, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.7), seed=24,
                        corr=0.97, device="cuda")
    say("[gpu] shards tree B=48 N=10 V=1500")
    h = svlib.SpecVerify(w.B, 1, w.V, torch.bfloat16, draft_dtype=torch.bfloat16)

    def run(a, b):
        return h.run_tree(shard(w.target, a, b), shard(w.draft, a, b), shard(w.tokens, a, b),
                          shard(w.parents, a, b), shard(w.num_nodes, a, b),
                          shard(w.temperatures, a, b), seed=11, offset=2)

    full = run(0, w.B)
    parts = [[], [], []]
    for a, b in SHARDS:
        h.set_request_base(a)
        for k, x in enumerate(run(a, b)):
            parts[k].append(x)
    torch.cuda.synchronize()
    check_equal("tree", full, parts)
    h.close()
