"""The C ABI on the host (no GPU): the library loads, exports every function
include/spec_verify.h declares, and rejects bad arguments before touching
the device."""
import ctypes

import rejection_sampling_verify_temp_amd as sv
from rejection_sampling_verify_temp_amd import binding


def test_library_exports_header_functions():
    lib = sv.load_library()
    names = sv.header_functions()
    assert "spec_verify_run" in names and "spec_verify_create" in names
    assert "spec_draft_sample" in names and "spec_ngram_propose" in names
    assert "spec_verify_run_typical" in names and "spec_verify_run_tree" in names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert sv.spec_verify_status_string(code)
    assert sv.spec_verify_status_string(99) == "unknown status"


def test_kernel_names():
    names = [sv.spec_verify_kernel_name(i) for i in range(4)]
    assert names == ["stats", "decide", "resid", "locate"]
    assert sv.spec_verify_kernel_name(4) is None


def test_create_rejects_bad_config_without_device():
    lib = sv.load_library()
    h = ctypes.c_void_p(1)
    assert lib.spec_verify_create(None, ctypes.byref(h)) == binding.SV_ERR_INVALID_ARG
    assert h.value is None
    bad = [dict(max_batch=0), dict(max_drafts=-1), dict(max_drafts=32),
           dict(vocab=0), dict(vocab=983041), dict(chunk_elems=100),
           dict(chunk_elems=15424), dict(device=-1)]
    for b in bad:
        f = dict(max_batch=4, max_drafts=4, vocab=1000, target_dtype=0,
                 draft_dtype=0, draft_is_probs=0, device=0, chunk_elems=0)
        f.update(b)
        cfg = binding.sv_config(**f)
        assert lib.spec_verify_create(ctypes.byref(cfg), ctypes.byref(h)) == \
            binding.SV_ERR_INVALID_ARG, b
    for b in [dict(target_dtype=2), dict(draft_dtype=-1), dict(draft_is_probs=2)]:
        f = dict(max_batch=4, max_drafts=4, vocab=1000, target_dtype=0,
                 draft_dtype=0, draft_is_probs=0, device=0, chunk_elems=0)
        f.update(b)
        cfg = binding.sv_config(**f)
        assert lib.spec_verify_create(ctypes.byref(cfg), ctypes.byref(h)) == \
            binding.SV_ERR_UNSUPPORTED, b


def test_run_and_queries_reject_null_handle():
    assert sv.spec_verify_run(None, 1, 1, 1, 0, 0, 1, 1, 1, 0, 0, 1, 1, 0, None) == \
        binding.SV_ERR_INVALID_ARG
    assert sv.spec_draft_sample(None, 1, 1, 1, 0, 1, 0, 0, 1, 0, None) == \
        binding.SV_ERR_INVALID_ARG
    assert sv.spec_verify_run_typical(None, 1, 1, 1, 1, 1, 1, 0.1, 0, 0, 0, 1, 1, 0,
                                      None) == binding.SV_ERR_INVALID_ARG
    assert sv.spec_verify_run_tree(None, 1, 4, 1, 0, 1, 1, 1, 1, 0, 0, 1, 1, 1, None) == \
        binding.SV_ERR_INVALID_ARG


def test_ngram_rejects_bad_arguments_without_device():
    bad = [dict(B=-1), dict(min_n=0), dict(max_n=0), dict(min_n=3, max_n=2),
           dict(max_n=33), dict(k=-1), dict(max_model_len=-1), dict(stride=0),
           dict(context=None), dict(context=2)]
    for b in bad:
        a = dict(B=1, context=4, stride=8, context_lens=4, min_n=1, max_n=4, k=3,
                 max_model_len=100, out_drafts=4, out_num_drafts=4, stream=None)
        a.update(b)
        assert sv.spec_ngram_propose(**a) == binding.SV_ERR_INVALID_ARG, b
    assert sv.spec_ngram_propose(0, None, 0, None, 1, 4, 3, 100, None, None, None) == 0
    lib = sv.load_library()
    f = ctypes.c_uint32()
    assert lib.spec_verify_get_device_errors(None, ctypes.byref(f), 0) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_timing_enable(None, 1) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_timing_read(None, None, 0, None) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_chunk_elems(None) == 0
    assert lib.spec_verify_tree_team_size(None, 8, 1) == 0
    assert lib.spec_verify_set_tree_wait_us(None, 10) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_set_tree_team_size(None, 4) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_set_request_base(None, 0) == binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_destroy(None) == 0


def test_noalloc_rejects_before_touching_the_device():
    """The no-alloc entry point checks its configuration, arguments and the
    size of its fixed workspace on the host: a null configuration, a bad
    field and a step too large for the array are rejected with no device
    call (this machine has no GPU)."""
    assert "spec_verify_run_noalloc" in sv.header_functions()
    lib = sv.load_library()
    P = 256  # an aligned stand-in address: nothing is dereferenced on these paths
    args = lambda B, K: [B, K, P, P, None, P, P, P, 0, 0, P, P, None, None, None]
    assert lib.spec_verify_run_noalloc(None, *args(1, 1)) == binding.SV_ERR_INVALID_ARG
    f = dict(max_batch=512, max_drafts=31, vocab=983040, target_dtype=1, draft_dtype=1,
             draft_is_probs=0, device=0, chunk_elems=0)
    cfg = binding.sv_config(**f)
    # 512 requests x 63 row slots x 64 chunks of partials alone are 33 MB
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), *args(512, 31)) == \
        binding.SV_ERR_CAPACITY
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), *args(513, 1)) == \
        binding.SV_ERR_CAPACITY  # above cfg.max_batch
    bad = binding.sv_config(**dict(f, vocab=0))
    assert lib.spec_verify_run_noalloc(ctypes.byref(bad), *args(1, 1)) == \
        binding.SV_ERR_INVALID_ARG
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), *args(0, 1)) == binding.SV_OK
