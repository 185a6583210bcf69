"""ctypes binding of the C ABI in include/spec_verify.h (the verify step, the
draft-token sampler and the n-gram proposer).

The functions here carry the C names and only marshal arguments: every step
of the verify path runs in the HIP kernels of libspecverify.so.  There is no
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libspecverify.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "spec_verify.h")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_CAPACITY, SV_ERR_HIP = (
    0, -1, -2, -3, -4)
SV_F32, SV_BF16 = 0, 1
SV_DEVERR_BAD_DRAFT_ID = 1
SV_DEVERR_BAD_NUM_DRAFTS = 2
SV_DEVERR_ZERO_RESIDUAL = 4
SV_DEVERR_DRAW_ROUNDING = 8
SV_DEVERR_BAD_TREE = 16
SV_DEVERR_TREE_SYNC = 32


class sv_config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_drafts", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("target_dtype", ctypes.c_int32),
                ("draft_dtype", ctypes.c_int32),
                ("draft_is_probs", ctypes.c_int32),
                ("device", ctypes.c_int32), ("chunk_elems", ctypes.c_int32)]


class SpecVerifyError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({spec_verify_status_string(status)})")


_lib = None


def load_library(path: str = None) -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built).  The
    SPEC_VERIFY_LIB environment variable names another build of the same
    library (for comparing compile-time variants)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SPEC_VERIFY_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    P, i32, u64, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64,
                        ctypes.c_uint32)
    lib.spec_verify_create.argtypes = [ctypes.POINTER(sv_config), ctypes.POINTER(P)]
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_run.argtypes = [P, i32, i32, P, P, P, P, P, P, u64, u64,
                                    P, P, P, P]
    lib.spec_verify_run.restype = ctypes.c_int
    lib.spec_verify_run_noalloc.argtypes = [ctypes.POINTER(sv_config), i32, i32, P, P, P, P,
                                            P, P, u64, u64, P, P, P, P, P]
    lib.spec_verify_run_noalloc.restype = ctypes.c_int
    lib.spec_verify_run_typical.argtypes = [P, i32, i32, P, P, P, P, ctypes.c_float, i32,
                                            u64, u64, P, P, P, P]
    lib.spec_verify_run_typical.restype = ctypes.c_int
    lib.spec_verify_run_tree.argtypes = [P, i32, i32, P, P, P, P, P, P, u64, u64, P, P, P, P]
    lib.spec_verify_run_tree.restype = ctypes.c_int
    lib.spec_draft_sample.argtypes = [P, i32, i32, P, P, P, u64, u64, P, P, P]
    lib.spec_draft_sample.restype = ctypes.c_int
    lib.spec_ngram_propose.argtypes = [i32, P, i32, P, i32, i32, i32, i32, P, P, P]
    lib.spec_ngram_propose.restype = ctypes.c_int
    lib.spec_verify_get_device_errors.argtypes = [P, ctypes.POINTER(u32), i32]
    lib.spec_verify_get_device_errors.restype = ctypes.c_int
    lib.spec_verify_set_request_base.argtypes = [P, i32]
    lib.spec_verify_set_request_base.restype = ctypes.c_int
    lib.spec_verify_timing_enable.argtypes = [P, i32]
    lib.spec_verify_timing_enable.restype = ctypes.c_int
    lib.spec_verify_timing_read.argtypes = [P, ctypes.POINTER(ctypes.c_float),
                                            i32, ctypes.POINTER(i32)]
    lib.spec_verify_timing_read.restype = ctypes.c_int
    lib.spec_verify_kernel_name.argtypes = [i32]
    lib.spec_verify_kernel_name.restype = ctypes.c_char_p
    lib.spec_verify_chunk_elems.argtypes = [P]
    lib.spec_verify_chunk_elems.restype = i32
    lib.spec_verify_tree_team_size.argtypes = [P, i32, i32]
    lib.spec_verify_tree_team_size.restype = i32
    lib.spec_verify_set_tree_wait_us.argtypes = [P, i32]
    lib.spec_verify_set_tree_wait_us.restype = ctypes.c_int
    lib.spec_verify_set_tree_team_size.argtypes = [P, i32]
    lib.spec_verify_set_tree_team_size.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [P]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/spec_verify.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


# --- the C entry points, same names ---------------------------------------
def spec_verify_status_string(status: int) -> str:
    return load_library().spec_verify_status_string(int(status)).decode()


def spec_verify_kernel_name(i: int):
    s = load_library().spec_verify_kernel_name(int(i))
    return None if s is None else s.decode()


def spec_verify_create(cfg: sv_config) -> int:
    h = ctypes.c_void_p()
    rc = load_library().spec_verify_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_create", rc)
    return h.value


def spec_verify_run(h, B, K, target_logits, draft_probs, draft_mode, draft_ids,
                    num_drafts_per_req, temperatures, philox_seed, philox_offset,
                    out_tokens, out_num_accepted, out_debug_probs, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_verify_run(
        h, int(B), int(K), target_logits, draft_probs, draft_mode, draft_ids,
        num_drafts_per_req, temperatures, int(philox_seed) & (2 ** 64 - 1),
        int(philox_offset) & (2 ** 64 - 1), out_tokens, out_num_accepted,
        out_debug_probs, stream)


def spec_verify_run_noalloc(cfg: sv_config, B, K, target_logits, draft_probs, draft_mode,
                            draft_ids, num_drafts_per_req, temperatures, philox_seed,
                            philox_offset, out_tokens, out_num_accepted, out_debug_probs,
                            out_device_flags, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_verify_run_noalloc(
        ctypes.byref(cfg), int(B), int(K), target_logits, draft_probs, draft_mode, draft_ids,
        num_drafts_per_req, temperatures, int(philox_seed) & (2 ** 64 - 1),
        int(philox_offset) & (2 ** 64 - 1), out_tokens, out_num_accepted, out_debug_probs,
        out_device_flags, stream)


def spec_verify_run_typical(h, B, K, target_logits, draft_ids, num_drafts_per_req,
                            temperatures, threshold, top_k, philox_seed, philox_offset,
                            out_tokens, out_num_accepted, out_debug_probs, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_verify_run_typical(
        h, int(B), int(K), target_logits, draft_ids, num_drafts_per_req, temperatures,
        float(threshold), int(top_k), int(philox_seed) & (2 ** 64 - 1),
        int(philox_offset) & (2 ** 64 - 1), out_tokens, out_num_accepted,
        out_debug_probs, stream)


def spec_verify_run_tree(h, B, N, target_logits, draft_logits, tokens, parents, num_nodes,
                         temperatures, philox_seed, philox_offset, out_tokens,
                         out_num_accepted, out_last_node, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_verify_run_tree(
        h, int(B), int(N), target_logits, draft_logits, tokens, parents, num_nodes,
        temperatures, int(philox_seed) & (2 ** 64 - 1), int(philox_offset) & (2 ** 64 - 1),
        out_tokens, out_num_accepted, out_last_node, stream)


def spec_draft_sample(h, B, K, draft_logits, num_drafts_per_req, temperatures,
                      philox_seed, philox_offset, out_ids, out_q, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_draft_sample(
        h, int(B), int(K), draft_logits, num_drafts_per_req, temperatures,
        int(philox_seed) & (2 ** 64 - 1), int(philox_offset) & (2 ** 64 - 1),
        out_ids, out_q, stream)


def spec_ngram_propose(B, context, stride, context_lens, min_n, max_n, k,
                       max_model_len, out_drafts, out_num_drafts, stream) -> int:
    """Pointers are integers (device addresses); returns the status code."""
    return load_library().spec_ngram_propose(
        int(B), context, int(stride), context_lens, int(min_n), int(max_n),
        int(k), int(max_model_len), out_drafts, out_num_drafts, stream)


def ngram_propose(context, context_lens, *, min_n, max_n, k, max_model_len,
                  out_drafts=None, out_num=None, stream=None):
    """torch wrapper: context [B, stride] int32 and context_lens [B] int32
    device tensors -> (drafts [B, k] with -1 padding, num [B])."""
    import torch
    if context.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("context and context_lens must be int32")
    if not (context.is_cuda and context.is_contiguous() and context_lens.is_cuda
            and context_lens.is_contiguous()):
        raise ValueError("inputs must be contiguous device tensors")
    B, stride = context.shape
    if tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be [B]")
    dev = context.device
    if out_drafts is None:
        out_drafts = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out_num is None:
        out_num = torch.empty((B,), dtype=torch.int32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = spec_ngram_propose(B, context.data_ptr(), stride, context_lens.data_ptr(),
                            min_n, max_n, k, max_model_len,
                            out_drafts.data_ptr() if k > 0 else None,
                            out_num.data_ptr(), stream.cuda_stream)
    if rc != SV_OK:
        raise SpecVerifyError("spec_ngram_propose", rc)
    return out_drafts, out_num


def spec_verify_set_request_base(h, base: int) -> None:
    rc = load_library().spec_verify_set_request_base(h, int(base))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_set_request_base", rc)


def spec_verify_tree_team_size(h, B: int, has_draft: bool) -> int:
    return load_library().spec_verify_tree_team_size(h, int(B), int(bool(has_draft)))


def spec_verify_set_tree_wait_us(h, microseconds: int) -> None:
    rc = load_library().spec_verify_set_tree_wait_us(h, int(microseconds))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_set_tree_wait_us", rc)


def spec_verify_set_tree_team_size(h, members: int) -> None:
    rc = load_library().spec_verify_set_tree_team_size(h, int(members))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_set_tree_team_size", rc)


def spec_verify_get_device_errors(h, clear: bool = False) -> int:
    f = ctypes.c_uint32()
    rc = load_library().spec_verify_get_device_errors(h, ctypes.byref(f), int(clear))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_get_device_errors", rc)
    return f.value


def spec_verify_timing_enable(h, enable: bool = True) -> None:
    rc = load_library().spec_verify_timing_enable(h, int(enable))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_timing_enable", rc)


def spec_verify_timing_read(h, n: int = 4):
    buf = (ctypes.c_float * n)()
    runs = ctypes.c_int32()
    rc = load_library().spec_verify_timing_read(h, buf, n, ctypes.byref(runs))
    if rc != SV_OK:
        raise SpecVerifyError("spec_verify_timing_read", rc)
    return list(buf), runs.value


def spec_verify_chunk_elems(h) -> int:
    return int(load_library().spec_verify_chunk_elems(h))


def spec_verify_destroy(h) -> int:
    return load_library().spec_verify_destroy(h)


# --- torch-tensor convenience wrapper (marshalling only) --------------------
def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def chk(t, shape, dtype=None):
    """The device address of a contiguous device tensor of the given shape
    (and dtype), None for None; raises otherwise."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("inputs must be contiguous device tensors")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"shape {tuple(t.shape)} != {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"dtype {t.dtype} != {dtype}")
    return t.data_ptr()


class SpecVerify:
    """A handle bound to one device; run() takes torch device tensors."""

    def __init__(self, max_batch, max_drafts, vocab, target_dtype,
                 draft_dtype=None, draft_is_probs=False, device=0,
                 chunk_elems=0):
        import torch
        code = lambda d: SV_BF16 if d == torch.bfloat16 else SV_F32
        self.cfg = sv_config(int(max_batch), int(max_drafts), int(vocab),
                             code(target_dtype),
                             code(draft_dtype or target_dtype),
                             int(bool(draft_is_probs)), int(device),
                             int(chunk_elems))
        self.device = int(device)
        self.handle = spec_verify_create(self.cfg)

    def close(self):
        if self.handle:
            spec_verify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def chunk_elems(self):
        return spec_verify_chunk_elems(self.handle)

    def run(self, target, draft, draft_mode, draft_ids, num_drafts,
            temperatures, seed=0, offset=0, out_tokens=None,
            out_num_accepted=None, out_debug_probs=None, stream=None):
        import torch
        B, K1, V = target.shape
        K = K1 - 1
        if V != self.cfg.vocab:
            raise ValueError(f"vocab {V} != handle vocab {self.cfg.vocab}")

        if _dtype_code(target) != self.cfg.target_dtype:
            raise TypeError("target dtype differs from the handle's")
        if draft is not None and _dtype_code(draft) != self.cfg.draft_dtype:
            raise TypeError("draft dtype differs from the handle's")
        dev = target.device
        if out_tokens is None:
            out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
        ptrs = [chk(target, (B, K + 1, V)), chk(draft, (B, K, V)),
                chk(draft_mode, (B,), torch.uint8),
                chk(draft_ids, (B, K), torch.int32),
                chk(num_drafts, (B,), torch.int32),
                chk(temperatures, (B,), torch.float32)]
        outs = [chk(out_tokens, (B, K + 1), torch.int32),
                chk(out_num_accepted, (B,), torch.int32),
                chk(out_debug_probs, (B, K, 2), torch.float32)]
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = spec_verify_run(self.handle, B, K, *ptrs, seed, offset, *outs,
                             stream.cuda_stream)
        if rc != SV_OK:
            raise SpecVerifyError("spec_verify_run", rc)
        return out_tokens, out_num_accepted

    def run_typical(self, target, draft_ids, num_drafts, temperatures, threshold,
                    top_k=0, seed=0, offset=0, out_tokens=None, out_num_accepted=None,
                    out_debug_probs=None, stream=None):
        """Typical acceptance: target [B, K+1, V] logits, draft ids [B, K]."""
        import torch
        B, K1, V = target.shape
        K = K1 - 1
        if V != self.cfg.vocab:
            raise ValueError(f"vocab {V} != handle vocab {self.cfg.vocab}")
        if _dtype_code(target) != self.cfg.target_dtype:
            raise TypeError("target dtype differs from the handle's")

        dev = target.device
        if out_tokens is None:
            out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        if out_num_accepted is None:
            out_num_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
        ptrs = [chk(target, (B, K + 1, V)), chk(draft_ids, (B, K), torch.int32),
                chk(num_drafts, (B,), torch.int32), chk(temperatures, (B,), torch.float32)]
        outs = [chk(out_tokens, (B, K + 1), torch.int32),
                chk(out_num_accepted, (B,), torch.int32),
                chk(out_debug_probs, (B, K, 2), torch.float32)]
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = spec_verify_run_typical(self.handle, B, K, *ptrs, threshold, top_k, seed,
                                     offset, *outs, stream.cuda_stream)
        if rc != SV_OK:
            raise SpecVerifyError("spec_verify_run_typical", rc)
        return out_tokens, out_num_accepted

    def run_tree(self, target, draft, tokens, parents, num_nodes, temperatures, seed=0,
                 offset=0, stream=None):
        """Token-tree verification: target [B, N, V] (and draft [B, N, V] or
        None) logits, tokens / parents [B, N] int32, num_nodes [B] int32 ->
        (tokens [B, N], num_accepted [B], last_node [B])."""
        import torch
        B, N, V = target.shape
        if V != self.cfg.vocab:
            raise ValueError(f"vocab {V} != handle vocab {self.cfg.vocab}")
        if _dtype_code(target) != self.cfg.target_dtype:
            raise TypeError("target dtype differs from the handle's")
        if draft is not None and _dtype_code(draft) != self.cfg.draft_dtype:
            raise TypeError("draft dtype differs from the handle's")

        dev = target.device
        out = torch.empty((B, N), dtype=torch.int32, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        last = torch.empty((B,), dtype=torch.int32, device=dev)
        ptrs = [chk(target, (B, N, V)), chk(draft, (B, N, V)),
                chk(tokens, (B, N), torch.int32), chk(parents, (B, N), torch.int32),
                chk(num_nodes, (B,), torch.int32), chk(temperatures, (B,), torch.float32)]
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = spec_verify_run_tree(self.handle, B, N, *ptrs, seed, offset, out.data_ptr(),
                                  nacc.data_ptr(), last.data_ptr(), stream.cuda_stream)
        if rc != SV_OK:
            raise SpecVerifyError("spec_verify_run_tree", rc)
        return out, nacc, last

    def sample(self, draft, num_drafts, temperatures, seed=0, offset=0,
               out_ids=None, out_q=None, stream=None):
        """Draft-token sampler: draft [B, K, V] logits (the handle's draft
        dtype) -> ids [B, K] (-1 past n_b); q(x) into out_q if given."""
        import torch
        B, K, V = draft.shape
        if V != self.cfg.vocab:
            raise ValueError(f"vocab {V} != handle vocab {self.cfg.vocab}")
        if _dtype_code(draft) != self.cfg.draft_dtype:
            raise TypeError("draft dtype differs from the handle's")
        dev = draft.device
        if out_ids is None:
            out_ids = torch.empty((B, K), dtype=torch.int32, device=dev)

        ptrs = [chk(draft, (B, K, V)), chk(num_drafts, (B,), torch.int32),
                chk(temperatures, (B,), torch.float32)]
        outs = [chk(out_ids, (B, K), torch.int32), chk(out_q, (B, K), torch.float32)]
        if stream is None:
            stream = torch.cuda.current_stream(dev)
        rc = spec_draft_sample(self.handle, B, K, *ptrs, seed, offset, *outs,
                               stream.cuda_stream)
        if rc != SV_OK:
            raise SpecVerifyError("spec_draft_sample", rc)
        return out_ids

    def device_errors(self, clear=False):
        return spec_verify_get_device_errors(self.handle, clear)

    def set_tree_wait_us(self, microseconds):
        """Bound on a tree team member's wait at an exchange."""
        spec_verify_set_tree_wait_us(self.handle, microseconds)

    def tree_team_size(self, B, has_draft=True):
        """Workgroups per request that run_tree uses for a batch of B."""
        return spec_verify_tree_team_size(self.handle, B, has_draft)

    def set_tree_team_size(self, members):
        """Workgroups per request for later run_tree calls (0: the handle's pick)."""
        spec_verify_set_tree_team_size(self.handle, members)

    def set_request_base(self, base):
        """Global index of request 0 for later runs (a shard of a batch)."""
        spec_verify_set_request_base(self.handle, base)
