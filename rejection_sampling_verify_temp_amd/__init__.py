"""Speculative-sampling verify step, and the draft-token sampler and n-gram
proposer that feed it, on MI355X (gfx950).

The compute lives in the HIP library ``lib/libspecverify.so`` (kernels and
C ABI under ``csrc/``, declared in ``include/spec_verify.h``); ``binding``
holds the ctypes binding with the C entry-point names and a small
torch-tensor wrapper.
"""
from .binding import (SpecVerify, SpecVerifyError, load_library, sv_config,  # noqa: F401
                      spec_verify_create, spec_verify_destroy,
                      spec_verify_get_device_errors, spec_verify_kernel_name,
                      spec_verify_run, spec_verify_status_string,
                      spec_verify_timing_enable, spec_verify_timing_read,
                      spec_verify_chunk_elems, spec_draft_sample,
                      spec_ngram_propose, ngram_propose, spec_verify_run_typical,
                      spec_verify_run_tree, spec_verify_set_request_base,
                      spec_verify_run_noalloc, spec_verify_tree_team_size,
                      spec_verify_set_tree_wait_us, spec_verify_set_tree_team_size,
                      header_functions)
