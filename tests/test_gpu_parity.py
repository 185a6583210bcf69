"""GPU parity: the HIP verify step through the C ABI against the CPU oracle.

Every case runs the library on the GPU, copies the exact input bytes back to
the host, runs the oracle on them with the same Philox seed and offset and
applies the parity rule of oracle/parity.py: bit-exact accepted counts and
tokens outside the 1e-6 decision / draw bands, acceptance probabilities to
1e-5 relative.
"""
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


def run_gpu(svlib, w, seed=0, offset=0, chunk=0, dbg=True, handle=None):
    w = w.to("cuda")
    h = handle or svlib.SpecVerify(
        w.B, w.K, w.V, w.target.dtype,
        draft_dtype=w.draft.dtype if w.draft is not None else None,
        draft_is_probs=w.draft_is_probs, chunk_elems=chunk)
    out_dbg = torch.empty((w.B, w.K, 2), dtype=torch.float32, device="cuda") if dbg else None
    tokens, nacc = h.run(w.target, w.draft, w.draft_mode, w.draft_ids,
                         w.num_drafts, w.temperatures, seed=seed,
                         offset=offset, out_debug_probs=out_dbg)
    torch.cuda.synchronize()
    flags = h.device_errors(clear=True)
    res = (tokens.cpu().numpy(), nacc.cpu().numpy(),
           out_dbg.cpu().numpy() if dbg else None, flags)
    if handle is None:
        h.close()
    return res


def run_oracle(w, seed, offset):
    hs = w.host_arrays()
    ref = oracle.verify(hs["target"], hs["draft"], hs["draft_ids"],
                        hs["num_drafts"], hs["temperatures"],
                        draft_mode=hs["draft_mode"],
                        draft_is_probs=hs["draft_is_probs"], seed=seed,
                        offset=offset)
    return hs, ref


def check(svlib, w, seed=0, offset=0, chunk=0, expect_flags=0):
    say(f"[gpu] {w.name} seed={seed} offset={offset} chunk={chunk}")
    tokens, nacc, dbg, flags = run_gpu(svlib, w, seed, offset, chunk)
    hs, ref = run_oracle(w, seed, offset)
    rep = compare(hs, ref, tokens, nacc, dbg)
    say(f"      requests={rep.requests} flagged={rep.flagged} "
        f"(differing {rep.flagged_mismatch}) accept={rep.accepted}/{rep.proposed} "
        f"prob_max_rel={rep.prob_max_rel:.2e} flags={flags}")
    assert rep.ok(), rep.mismatches
    assert flags & ~8 == expect_flags, (flags, expect_flags)
    # a draw on a rounding tie at a chunk boundary (device flag 8) is a draw
    # within the band of a CDF boundary: only a batch the oracle flags has one
    assert not flags & 8 or rep.flagged > 0, (flags, rep.flagged)
    assert ref["flags"] == expect_flags
    return rep


# ---------------------------------------------------------------------------
# The five workloads, full size, default launch configuration
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_config_parity(svlib, cfg):
    dev = "cpu" if cfg <= 1 else "cuda"  # large ones are generated on the GPU
    w = synth.make_config(cfg, device=dev)
    check(svlib, w, seed=0, offset=0)
    if cfg <= 2:
        check(svlib, w, seed=12345, offset=7)


@pytest.mark.parametrize("cfg", [3, 4])
def test_config_second_stream(svlib, cfg):
    """The two largest workloads again at another (seed, offset): other
    uniforms, so other rejection positions and draws."""
    w = synth.make_config(cfg, device="cuda")
    check(svlib, w, seed=777, offset=11)


@pytest.mark.parametrize("offset", range(12))
def test_config0_many_offsets(svlib, offset):
    w = synth.make_config(0)
    check(svlib, w, seed=3, offset=offset)


# ---------------------------------------------------------------------------
# Small and edge cases (several chunks, ragged tails, odd V)
# ---------------------------------------------------------------------------
CASES = {
    "f32_V1001_ragged_mixT": dict(B=24, K=5, V=1001, temps=(1.0, 0.0, 0.5, 1.7), n_mode="ragged"),
    "bf16_V4099_onehot_mix": dict(B=32, K=4, V=4099, dtype=torch.bfloat16, temps=(0.8, 1.2), onehot_frac=0.5, n_mode="ragged"),
    "bf16_tgt_f32_draft": dict(B=16, K=3, V=3000, dtype=torch.bfloat16, draft_dtype=torch.float32, temps=(0.9,)),
    "f32_tgt_bf16_draft": dict(B=16, K=3, V=2051, dtype=torch.float32, draft_dtype=torch.bfloat16, temps=(1.1,)),
    "probs_f32": dict(B=32, K=4, V=777, temps=(1.0, 0.6), draft_is_probs=True, n_mode="ragged"),
    "probs_bf16": dict(B=16, K=4, V=5000, dtype=torch.bfloat16, temps=(1.0,), draft_is_probs=True),
    "K0_plain_sampling": dict(B=40, K=0, V=513, temps=(1.0, 0.3, 0.0)),
    "V1": dict(B=8, K=3, V=1, temps=(1.0, 0.0)),
    "V2": dict(B=64, K=2, V=2, temps=(1.0, 0.5, 0.0)),
    "V5_tiny": dict(B=64, K=6, V=5, temps=(1.0, 2.0, 0.0), n_mode="ragged"),
    "V33333_bf16": dict(B=12, K=7, V=33333, dtype=torch.bfloat16, temps=(0.7, 0.0, 1.0), n_mode="ragged"),
    "no_draft_all_onehot": dict(B=24, K=3, V=900, temps=(1.0, 0.0), with_draft=False),
    "high_corr": dict(B=32, K=5, V=2000, temps=(1.0,), corr=0.999),
    "low_corr": dict(B=32, K=5, V=2000, temps=(1.0,), corr=0.0),
    "tiny_T": dict(B=16, K=3, V=300, temps=(1e-3, 0.05)),
    "huge_logits": dict(B=16, K=3, V=1500, temps=(1.0,), scale=40.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_random_case(svlib, name):
    kw = dict(CASES[name])
    for seed in (0, 1):
        w = synth.make_random(seed=seed, **kw)
        check(svlib, w, seed=seed, offset=seed * 3)


@pytest.mark.parametrize("chunk", [256, 320, 1024, 4096, 15360])
def test_chunk_sizes(svlib, chunk):
    w = synth.make_random(20, 4, 20000, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.6),
                          n_mode="ragged", onehot_frac=0.3, seed=9)
    check(svlib, w, seed=1, offset=2, chunk=chunk)
    w = synth.make_config(1)
    check(svlib, w, seed=0, offset=1, chunk=chunk)


def test_greedy_ties(svlib):
    """Integer logits: many ties in the max; accept on equality, lowest
    index emitted."""
    g = torch.Generator().manual_seed(5)
    B, K, V = 64, 4, 700
    t = torch.randint(-3, 2, (B, K + 1, V), generator=g).float()
    ids = torch.randint(0, V, (B, K), generator=g).int()
    am = torch.argmax(t[:, :K], -1).int()
    ids = torch.where(torch.rand(B, K, generator=g) < 0.7, am, ids)
    w = synth.Workload("greedy ties", t, None, None, ids,
                       torch.randint(0, K + 1, (B,), generator=g).int(),
                       torch.zeros(B))
    check(svlib, w)
    w.target = t.to(torch.bfloat16)
    check(svlib, w, offset=1)


def test_bad_device_data_is_flagged(svlib):
    w = synth.make_random(16, 4, 300, temps=(1.0, 0.0), seed=4, nan_padding=False)
    w.draft_ids[0, 0] = -1
    w.draft_ids[1, 1] = 300
    w.num_drafts[2] = -3
    w.num_drafts[3] = 9
    check(svlib, w, expect_flags=1 | 2)


def test_accept_example_on_gpu(svlib):
    """The pages' worked example (q = 0.4, p = 0.2) over 2^20 Philox draws:
    exactly the oracle's decisions, and a rate of 0.5 within 3 sigma."""
    B = 1 << 20
    t = torch.empty((B, 2, 2))
    t[:, 0] = torch.tensor([np.log(0.2), np.log(0.8)])
    t[:, 1] = torch.tensor([np.log(0.3), np.log(0.7)])
    d = torch.empty((B, 1, 2))
    d[:, 0] = torch.tensor([0.4, 0.6])
    w = synth.Workload("accept example", t, d, None, torch.zeros((B, 1), dtype=torch.int32),
                       torch.ones(B, dtype=torch.int32), torch.ones(B), draft_is_probs=True)
    say("[gpu] accept example B=2^20")
    tokens, nacc, _, _ = run_gpu(svlib, w, dbg=False)
    hs, ref = run_oracle(w, 0, 0)
    assert np.array_equal(nacc, ref["num_accepted"])
    assert np.array_equal(tokens, ref["tokens"])
    assert abs(nacc.mean() - 0.5) < 3 * np.sqrt(0.25 / B)


def test_deterministic_and_offsets_differ(svlib):
    w = synth.make_config(1)
    a = run_gpu(svlib, w, seed=0, offset=5)
    b = run_gpu(svlib, w, seed=0, offset=5)
    c = run_gpu(svlib, w, seed=0, offset=6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2], b[2], equal_nan=True)
    assert not np.array_equal(a[0], c[0])


@pytest.mark.parametrize("cfg", [3, 4])
def test_deterministic_many_runs(svlib, cfg):
    """100 steps of a full-size workload on one handle, with other runs in
    between: every output (tokens, counts, debug probabilities) is
    bit-identical to the first step's."""
    w = synth.make_config(cfg, device="cuda")
    say(f"[gpu] determinism {w.name} x100")
    h = svlib.SpecVerify(w.B, w.K, w.V, w.target.dtype,
                         draft_dtype=w.draft.dtype if w.draft is not None else None)
    first = run_gpu(svlib, w, seed=3, offset=4, handle=h)
    for i in range(99):
        if i % 10 == 5:  # another stream of uniforms on the same workspace
            run_gpu(svlib, w, seed=3, offset=100 + i, handle=h)
        again = run_gpu(svlib, w, seed=3, offset=4, handle=h)
        assert np.array_equal(again[0], first[0]) and np.array_equal(again[1], first[1]), i
        assert np.array_equal(again[2], first[2], equal_nan=True), i
        assert again[3] == first[3], i
    h.close()


def test_empty_batch_is_noop(svlib):
    h = svlib.SpecVerify(4, 2, 100, torch.float32)
    rc = svlib.spec_verify_run(h.handle, 0, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, None)
    assert rc == 0
    tgt = torch.zeros((5, 3, 100), device="cuda")
    with pytest.raises(svlib.SpecVerifyError):
        h.run(tgt, None, None, torch.zeros((5, 2), dtype=torch.int32, device="cuda"),
              torch.zeros(5, dtype=torch.int32, device="cuda"),
              torch.ones(5, device="cuda"))
    h.close()


# ---------------------------------------------------------------------------
# The largest sizes a handle takes
# ---------------------------------------------------------------------------
def test_max_vocab(svlib):
    """V = 983040: 64 chunks of 15360, one decide lane per chunk.  bf16 and
    fp32 rows; sampling, greedy and one-hot requests, ragged counts."""
    for dtype, seed in ((torch.bfloat16, 0), (torch.float32, 1)):
        w = synth.make_random(6, 2, 983040, dtype=dtype, temps=(1.0, 0.0, 0.7),
                              n_mode="ragged", onehot_frac=0.3, seed=seed, device="cuda")
        check(svlib, w, seed=seed, offset=4)


def test_max_drafts(svlib):
    """K = 31: 2K + 1 = 63 row slots, one wavefront lane each in the decision."""
    w = synth.make_random(16, 31, 3000, dtype=torch.bfloat16, temps=(1.0, 0.0, 0.8),
                          n_mode="ragged", onehot_frac=0.25, corr=0.97, seed=5, device="cuda")
    rep = check(svlib, w, seed=2, offset=7)
    assert rep.accepted > 0


def test_draw_sizes(svlib):
    """Batches whose size selects each draw workgroup size: up to 768
    requests take 1024 threads, up to 896 take 512, more take 256."""
    for B in (768, 800, 900):
        w = synth.make_random(B, 3, 2000, dtype=torch.bfloat16, temps=(1.0, 0.7, 0.0),
                              n_mode="ragged", onehot_frac=0.2, seed=B, device="cuda")
        check(svlib, w, seed=1, offset=B)


@pytest.mark.parametrize("B", [800, 900])
@pytest.mark.parametrize("dtypes", ["f32_f32", "bf16_f32", "f32_bf16", "f32_probs"])
def test_draw_sizes_pair_dtypes(svlib, B, dtypes):
    """The 512- and 256-thread draws (B = 800 and 900) on the residual pairs
    with an fp32 row (4 parts per chunk, the heaviest draws' registers) and
    with probability drafts; ragged counts, moderate correlation so most
    requests reject."""
    f32, bf16 = torch.float32, torch.bfloat16
    dt, ddt, probs = {"f32_f32": (f32, f32, False), "bf16_f32": (bf16, f32, False),
                      "f32_bf16": (f32, bf16, False), "f32_probs": (f32, f32, True)}[dtypes]
    w = synth.make_random(B, 3, 3000, dtype=dt, draft_dtype=ddt, temps=(1.0, 0.7),
                          n_mode="ragged", corr=0.6, draft_is_probs=probs, seed=B + 7,
                          device="cuda")
    check(svlib, w, seed=2, offset=B)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_onehot_dominant_draft(svlib, dtype):
    """One-hot drafts that hold almost all of p (p(x) about 0.99 at T = 0.3):
    the rare rejections draw from the remaining 1% of the mass, so x's share
    must leave its chunk exactly, not as a difference of rounded sums.  Every
    request has its own Philox counter; about 1% reject."""
    g = torch.Generator().manual_seed(41)
    B, K, V, T = 4096, 1, 20000, 0.3
    t = torch.randn((B, K + 1, V), generator=g) * 0.5
    ids = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    for b in range(B):  # x about 0.99 of p_0 (1 - 1e-2 of the mass)
        t[b, 0, ids[b, 0]] = 4.6 + 0.3 * float(np.log(V / 50000))
    w = synth.Workload("one-hot dominant drafts", t.to(dtype), None,
                       torch.ones(B, dtype=torch.uint8), ids,
                       torch.full((B,), K, dtype=torch.int32), torch.full((B,), T))
    rep = check(svlib, w, seed=5, offset=3)
    assert rep.proposed - rep.accepted >= 10  # enough rejections drawn from the rest


def test_mode_bytes_at_the_end_of_an_allocation(svlib):
    """draft_mode is read through the aligned 4-byte word that holds each
    byte.  With the array alone in its own hipMalloc allocation of B = 37
    bytes, the last word reaches past the array's end: the run must give the
    same outputs as with the array inside a larger tensor."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipFree.argtypes = [ctypes.c_void_p]
    w = synth.make_random(37, 3, 4099, dtype=torch.bfloat16, temps=(1.0, 0.7, 0.0),
                          onehot_frac=0.5, n_mode="ragged", seed=37).to("cuda")
    assert w.draft_mode is not None and w.B % 4 == 1
    ref = run_gpu(svlib, w, seed=8, offset=2)
    ptr = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(ptr), w.B) == 0
    try:
        assert hip.hipMemcpy(ptr, w.draft_mode.data_ptr(), w.B, 3) == 0  # device to device
        h = svlib.SpecVerify(w.B, w.K, w.V, w.target.dtype, draft_dtype=w.draft.dtype)
        tok = torch.empty((w.B, w.K + 1), dtype=torch.int32, device="cuda")
        nacc = torch.empty((w.B,), dtype=torch.int32, device="cuda")
        rc = svlib.spec_verify_run(h.handle, w.B, w.K, w.target.data_ptr(), w.draft.data_ptr(),
                                   ptr.value, w.draft_ids.data_ptr(), w.num_drafts.data_ptr(),
                                   w.temperatures.data_ptr(), 8, 2, tok.data_ptr(),
                                   nacc.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), ref[0]) and np.array_equal(nacc.cpu().numpy(), ref[1])
        h.close()
    finally:
        hip.hipFree(ptr)
