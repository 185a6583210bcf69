"""CPU oracle for the speculative-sampling verify step (rejection sampling,
typical acceptance, token trees), the draft-token sampler and the n-gram
prompt-lookup proposer that feed it.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The product path
(the HIP library and its binding) never imports, links or calls it, and it
imports nothing from the product path.

The arithmetic lives in ``sv_oracle.c`` (plain C, double precision,
sequential); this module only builds it with gcc and marshals numpy arrays
through ctypes.  See ``sv_oracle.c`` for the method and its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "libsvoracle.so")

F32, BF16 = 0, 1
MODE_PROB, MODE_ONEHOT = 0, 1
FLAG_BAD_DRAFT_ID, FLAG_BAD_NUM_DRAFTS, FLAG_ZERO_RESIDUAL = 1, 2, 4
FLAG_BAD_TREE = 16


def build(force: bool = True, src: str = _SRC, out: str = _LIB, flags=()) -> str:
    """Compile the oracle's C source into a shared library with gcc
    (-O2, no fast-math); `flags` are extra gcc options (the tests build
    sanitizer and planted-mistake copies this way)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-Wall",
             "-Werror", *flags, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def open_library(path: str):
    """Load a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, u64, u32, dbl, flt = (ctypes.c_int, ctypes.c_uint64,
                               ctypes.c_uint32, ctypes.c_double,
                               ctypes.c_float)
    lib.svo_philox4x64_10.argtypes = [P, P, P]
    lib.svo_philox4x64_10.restype = None
    lib.svo_uniforms.argtypes = [u64, u64, u64, u64, P, P]
    lib.svo_uniforms.restype = None
    lib.svo_is_sampling.argtypes = [flt]
    lib.svo_is_sampling.restype = i32
    lib.svo_softmax.argtypes = [P, i32, dbl, P]
    lib.svo_softmax.restype = None
    lib.svo_argmax.argtypes = [P, i32]
    lib.svo_argmax.restype = i32
    lib.svo_accept_ratio.argtypes = [dbl, dbl]
    lib.svo_accept_ratio.restype = dbl
    lib.svo_residual.argtypes = [P, P, i32, i32, i32, P]
    lib.svo_residual.restype = None
    lib.svo_draw.argtypes = [P, i32, dbl, P]
    lib.svo_draw.restype = i32
    lib.svo_draw_interval.argtypes = [P, i32, i32, P, P]
    lib.svo_draw_interval.restype = dbl
    lib.svo_verify_path.argtypes = [i32, i32, i32, P, i32, P, i32, i32, P, i32, flt, P, P,
                                    i32, i32, P, P, P, P, P]
    lib.svo_verify_path.restype = u32
    lib.svo_verify_typical_path.argtypes = [i32, i32, i32, P, P, i32, flt, dbl, i32, P, i32,
                                            i32, P, P, P, P, P]
    lib.svo_verify_typical_path.restype = u32
    lib.svo_verify_tree_path.argtypes = [i32, i32, i32, P, i32, P, i32, P, P, i32, flt, P, P,
                                         i32, P, i32, P, P, P, P, P]
    lib.svo_verify_tree_path.restype = u32
    common = [i32, i32, i32, i32, P, i32, P, i32, P, P, P, P]
    lib.svo_verify_with_uniforms.argtypes = common + [P, P] + [P] * 6
    lib.svo_verify_with_uniforms.restype = u32
    lib.svo_verify.argtypes = common + [u64, u64] + [P] * 6
    lib.svo_verify.restype = u32
    lib.svo_draft_uniform.argtypes = [u64, u64, u64, u64]
    lib.svo_draft_uniform.restype = dbl
    lib.svo_draft_sample.argtypes = [i32, i32, i32, i32, P, P, P, u64, u64,
                                     P, P, P]
    lib.svo_draft_sample.restype = u32
    lib.svo_ngram_propose.argtypes = [i32, P, i32, P, i32, i32, i32, i32, P, P]
    lib.svo_ngram_propose.restype = None
    lib.svo_verify_typical.argtypes = [i32, i32, i32, i32, P, P, P, P, dbl, i32,
                                       u64, u64, P, P, P, P, P]
    lib.svo_verify_typical.restype = u32
    lib.svo_verify_tree.argtypes = [i32, i32, i32, i32, P, i32, P, i32, P, P, P, P, u64, u64,
                                    P, P, P, P, P]
    lib.svo_verify_tree.restype = u32
    return lib


_lib = None
_override = None  # a library handle installed by use_library()


def use_library(lib):
    """Route this module's functions through another compiled oracle (the
    pin tests use this to check that planted mistakes are caught).  Pass
    None to restore the default."""
    global _override
    _override = lib


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        _lib = open_library(_LIB)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def philox4x64_10(counter, key):
    """Philox4x64-10 block for a 4-word counter and a 2-word key."""
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    _load().svo_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniforms(seed, offset, b, j):
    """(u_acc, u_rec) of request b at position j."""
    ua, ur = ctypes.c_double(), ctypes.c_double()
    _load().svo_uniforms(seed, offset, b, j, ctypes.byref(ua), ctypes.byref(ur))
    return ua.value, ur.value


def is_sampling(T: float) -> bool:
    return bool(_load().svo_is_sampling(float(T)))


def softmax(logits, T):
    l = np.ascontiguousarray(logits, dtype=np.float64)
    p = np.empty_like(l)
    _load().svo_softmax(_ptr(l), l.size, float(T), _ptr(p))
    return p


def argmax(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    return int(_load().svo_argmax(_ptr(v), v.size))


def accept_ratio(px, qx):
    return float(_load().svo_accept_ratio(float(px), float(qx)))


def residual(p, q, mode, x):
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q if q is not None else p, dtype=np.float64)
    r = np.empty_like(p)
    _load().svo_residual(_ptr(p), _ptr(q), int(mode), int(x), p.size, _ptr(r))
    return r


def draw(r, u):
    """(token, margin) of the inverse-CDF draw from unnormalized law r."""
    r = np.ascontiguousarray(r, dtype=np.float64)
    m = ctypes.c_double()
    y = _load().svo_draw(_ptr(r), r.size, float(u), ctypes.byref(m))
    return int(y), m.value


def draw_interval(r, y):
    """(lo, hi, mass) of token y in the inverse CDF of the unnormalized law
    r: u selects y iff lo <= u < hi; mass = r_y / sum(r)."""
    r = np.ascontiguousarray(r, dtype=np.float64)
    lo, hi = ctypes.c_double(), ctypes.c_double()
    m = _load().svo_draw_interval(_ptr(r), r.size, int(y), ctypes.byref(lo),
                                  ctypes.byref(hi))
    return lo.value, hi.value, float(m)


def row_f64(a, idx):
    """Row idx (a tuple of leading indices) of a float32 or bf16-bits array
    as float64: the input conversion the oracle makes."""
    row = np.asarray(a[idx])
    if row.dtype == np.uint16:
        row = (row.astype(np.uint32) << 16).view(np.float32)
    return row.astype(np.float64)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bf16 bits
        return BF16
    raise TypeError("oracle inputs are float32 or raw bf16 bits (uint16)")


def verify(target, draft, draft_ids, num_drafts, temperatures, *,
           draft_mode=None, draft_is_probs=False, seed=0, offset=0,
           u_acc=None, u_rec=None, diagnostics=True):
    """Run the oracle on host arrays.

    target: [B, K+1, V] float32, or uint16 holding bf16 bits.
    draft:  [B, K, V] (same convention) or None for all one-hot.
    Uniforms come from Philox(seed, offset) unless u_acc/u_rec ([B, K+1])
    are given.  Returns a dict with tokens, num_accepted, p, q, margin_acc,
    margin_rec and flags; with diagnostics=False only tokens, num_accepted
    and flags are computed.
    """
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    if draft is not None:
        draft = np.ascontiguousarray(draft)
        assert draft.shape == (B, K, V)
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32).reshape(B, K)
    nd = np.ascontiguousarray(num_drafts, dtype=np.int32).reshape(B)
    temps = np.ascontiguousarray(temperatures, dtype=np.float32).reshape(B)
    mode = None if draft_mode is None else np.ascontiguousarray(
        draft_mode, dtype=np.uint8).reshape(B)
    tokens = np.empty((B, K + 1), dtype=np.int32)
    nacc = np.empty(B, dtype=np.int32)
    p = np.empty((B, K), dtype=np.float64)
    q = np.empty((B, K), dtype=np.float64)
    macc = np.empty((B, K), dtype=np.float64)
    mrec = np.empty(B, dtype=np.float64)
    lib = _load()
    head = [B, K, V, _dtype_code(target), _ptr(target),
            _dtype_code(draft) if draft is not None else F32, _ptr(draft),
            int(bool(draft_is_probs)), _ptr(mode), _ptr(ids), _ptr(nd),
            _ptr(temps)]
    if diagnostics:
        tail = [_ptr(tokens), _ptr(nacc), _ptr(p), _ptr(q), _ptr(macc),
                _ptr(mrec)]
    else:
        tail = [_ptr(tokens), _ptr(nacc), None, None, None, None]
    if u_acc is not None or u_rec is not None:
        ua = np.ascontiguousarray(u_acc, dtype=np.float64).reshape(B, K + 1)
        ur = np.ascontiguousarray(u_rec, dtype=np.float64).reshape(B, K + 1)
        flags = lib.svo_verify_with_uniforms(*head, _ptr(ua), _ptr(ur), *tail)
    else:
        ua = ur = None
        flags = lib.svo_verify(*head, int(seed), int(offset), *tail)
    call = dict(kind="verify", target=target, draft=draft, draft_ids=ids,
                num_drafts=nd, temperatures=temps, draft_mode=mode,
                draft_is_probs=bool(draft_is_probs), seed=int(seed),
                offset=int(offset), u_acc=ua, u_rec=ur)
    return dict(tokens=tokens, num_accepted=nacc, p=p, q=q, margin_acc=macc,
                margin_rec=mrec, flags=int(flags), call=call)


def draft_uniform(seed, offset, b, j):
    """The draft sampler's uniform for request b, position j."""
    return float(_load().svo_draft_uniform(int(seed), int(offset), int(b), int(j)))


def draft_sample(draft, num_drafts, temperatures, *, seed=0, offset=0,
                 diagnostics=True):
    """Sample draft tokens x_j ~ softmax(l_j / T_b) for rows j < n_b.

    draft: [B, K, V] float32, or uint16 holding bf16 bits.  num_drafts [B]
    or None (all K rows).  Returns a dict with ids [B, K] (-1 past n_b),
    q [B, K] = q_j(x_j), margin [B, K] (draw margins) and flags.
    """
    draft = np.ascontiguousarray(draft)
    B, K, V = draft.shape
    nd = None if num_drafts is None else np.ascontiguousarray(
        num_drafts, dtype=np.int32).reshape(B)
    temps = np.ascontiguousarray(temperatures, dtype=np.float32).reshape(B)
    ids = np.empty((B, K), dtype=np.int32)
    q = np.empty((B, K), dtype=np.float64)
    margin = np.empty((B, K), dtype=np.float64)
    flags = _load().svo_draft_sample(
        B, K, V, _dtype_code(draft), _ptr(draft), _ptr(nd), _ptr(temps),
        int(seed), int(offset), _ptr(ids),
        _ptr(q) if diagnostics else None, _ptr(margin) if diagnostics else None)
    call = dict(kind="draft_sample", draft=draft, num_drafts=nd,
                temperatures=temps, seed=int(seed), offset=int(offset))
    return dict(ids=ids, q=q, margin=margin, flags=int(flags), call=call)


def ngram_propose(context, lens, *, min_n, max_n, k, max_model_len):
    """n-gram prompt lookup: context [B, stride] int32, lens [B] ->
    (drafts [B, k] with -1 padding, num [B])."""
    ctx = np.ascontiguousarray(context, dtype=np.int32)
    B, stride = ctx.shape
    ln = np.ascontiguousarray(lens, dtype=np.int32).reshape(B)
    drafts = np.empty((B, k), dtype=np.int32)
    num = np.empty(B, dtype=np.int32)
    _load().svo_ngram_propose(B, _ptr(ctx), stride, _ptr(ln), int(min_n),
                              int(max_n), int(k), int(max_model_len),
                              _ptr(drafts), _ptr(num))
    return drafts, num


def verify_typical(target, draft_ids, num_drafts, temperatures, *, eps, top_k=0,
                   seed=0, offset=0, diagnostics=True):
    """Typical acceptance on host arrays (target [B, K+1, V] float32 or bf16
    bits).  Returns a dict with tokens, num_accepted, p (= p_j(x_j)),
    margin_acc, margin_rec and flags, in the layout of verify()."""
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32).reshape(B, K)
    nd = np.ascontiguousarray(num_drafts, dtype=np.int32).reshape(B)
    temps = np.ascontiguousarray(temperatures, dtype=np.float32).reshape(B)
    tokens = np.empty((B, K + 1), dtype=np.int32)
    nacc = np.empty(B, dtype=np.int32)
    p = np.empty((B, K), dtype=np.float64)
    macc = np.empty((B, K), dtype=np.float64)
    mrec = np.empty(B, dtype=np.float64)
    d = diagnostics
    flags = _load().svo_verify_typical(
        B, K, V, _dtype_code(target), _ptr(target), _ptr(ids), _ptr(nd), _ptr(temps),
        float(eps), int(top_k), int(seed), int(offset), _ptr(tokens), _ptr(nacc),
        _ptr(p) if d else None, _ptr(macc) if d else None, _ptr(mrec) if d else None)
    call = dict(kind="typical", target=target, draft_ids=ids, num_drafts=nd,
                temperatures=temps, eps=float(eps), top_k=int(top_k),
                seed=int(seed), offset=int(offset))
    return dict(tokens=tokens, num_accepted=nacc, p=p, q=np.ones_like(p),
                margin_acc=macc, margin_rec=mrec, flags=int(flags), call=call)


def verify_tree(target, draft, tokens, parents, num_nodes, temperatures, *, seed=0,
                offset=0, draft_is_probs=False):
    """Token-tree verification.  target [B, N, V] (float32 or bf16 bits),
    draft [B, N, V] logits (normalized q with draft_is_probs) or None
    (one-hot tree), tokens / parents [B, N] int32,
    num_nodes [B].  Returns a dict with tokens [B, N], num_accepted,
    last_node, margin_acc, margin_rec and flags."""
    target = np.ascontiguousarray(target)
    B, N, V = target.shape
    if draft is not None:
        draft = np.ascontiguousarray(draft)
        assert draft.shape == (B, N, V)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, N)
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, N)
    nn = np.ascontiguousarray(num_nodes, dtype=np.int32).reshape(B)
    temps = np.ascontiguousarray(temperatures, dtype=np.float32).reshape(B)
    out = np.empty((B, N), dtype=np.int32)
    nacc = np.empty(B, dtype=np.int32)
    last = np.empty(B, dtype=np.int32)
    macc = np.empty(B, dtype=np.float64)
    mrec = np.empty(B, dtype=np.float64)
    flags = _load().svo_verify_tree(
        B, N, V, _dtype_code(target), _ptr(target),
        _dtype_code(draft) if draft is not None else F32, _ptr(draft),
        int(bool(draft_is_probs)), _ptr(tok), _ptr(par),
        _ptr(nn), _ptr(temps), int(seed), int(offset), _ptr(out), _ptr(nacc), _ptr(last),
        _ptr(macc), _ptr(mrec))
    call = dict(kind="tree", target=target, draft=draft, tokens=tok, parents=par,
                num_nodes=nn, temperatures=temps, draft_is_probs=bool(draft_is_probs),
                seed=int(seed), offset=int(offset))
    return dict(tokens=out, num_accepted=nacc, last_node=last, margin_acc=macc,
                margin_rec=mrec, flags=int(flags), call=call)


# --------------------------------------------------------------------------
# Evaluation along a given path (checks of flagged requests)
# --------------------------------------------------------------------------
def _request_uniforms(call, b, n):
    """u_acc, u_rec [n] of request b of a recorded call."""
    if call.get("u_acc") is not None:
        return (np.ascontiguousarray(call["u_acc"][b], dtype=np.float64),
                np.ascontiguousarray(call["u_rec"][b], dtype=np.float64))
    ua, ur = np.empty(n), np.empty(n)
    for j in range(n):
        ua[j], ur[j] = uniforms(call["seed"], call["offset"], b, j)
    return ua, ur


def _path_result(acc, margin, tok, mrec, out_y, flags):
    return dict(accept=acc, margin=margin, token=int(tok.value),
                margin_rec=float(mrec.value), lo=float(out_y[0]), hi=float(out_y[1]),
                mass=float(out_y[2]), u=float(out_y[3]), flags=int(flags))


def verify_path(ref, b, n_path, y):
    """Request b of an oracle.verify() (or verify_typical()) result
    evaluated along the path "n_path drafts accepted, then token y emitted
    at position n_path".  Returns a dict: accept / margin [K] (the oracle's
    decision and |u - threshold| at every position the path decides, NaN
    elsewhere), token / margin_rec (the oracle's own emitted token at n_path
    and its draw margin), lo / hi / mass / u (where y sits in that draw's
    law: u selects y iff lo <= u < hi) and flags."""
    c = ref["call"]
    if c["kind"] == "typical":
        return verify_typical_path(ref, b, n_path, y)
    t = np.ascontiguousarray(c["target"][b])
    K = t.shape[0] - 1
    V = t.shape[1]
    d = None if c["draft"] is None else np.ascontiguousarray(c["draft"][b])
    onehot = c["draft_mode"] is not None and int(c["draft_mode"][b]) != 0
    ua, ur = _request_uniforms(c, b, K + 1)
    ids = np.ascontiguousarray(c["draft_ids"][b], dtype=np.int32)
    acc, margin = np.empty(K), np.empty(K)
    tok, mrec, out_y = ctypes.c_int32(), ctypes.c_double(), np.empty(4)
    flags = _load().svo_verify_path(
        K, V, _dtype_code(t), _ptr(t), _dtype_code(d) if d is not None else F32, _ptr(d),
        int(c["draft_is_probs"]), int(onehot), _ptr(ids), int(c["num_drafts"][b]),
        float(c["temperatures"][b]), _ptr(ua), _ptr(ur), int(n_path), int(y), _ptr(acc),
        _ptr(margin), ctypes.byref(tok), ctypes.byref(mrec), _ptr(out_y))
    return _path_result(acc, margin, tok, mrec, out_y, flags)


def verify_typical_path(ref, b, n_path, y):
    """verify_path for a verify_typical() result (margin = |p(x) - eps|, or
    +inf where the rank decides)."""
    c = ref["call"]
    t = np.ascontiguousarray(c["target"][b])
    K = t.shape[0] - 1
    V = t.shape[1]
    _, ur = _request_uniforms(c, b, K + 1)
    ids = np.ascontiguousarray(c["draft_ids"][b], dtype=np.int32)
    acc, margin = np.empty(K), np.empty(K)
    tok, mrec, out_y = ctypes.c_int32(), ctypes.c_double(), np.empty(4)
    flags = _load().svo_verify_typical_path(
        K, V, _dtype_code(t), _ptr(t), _ptr(ids), int(c["num_drafts"][b]),
        float(c["temperatures"][b]), c["eps"], c["top_k"], _ptr(ur), int(n_path), int(y),
        _ptr(acc), _ptr(margin), ctypes.byref(tok), ctypes.byref(mrec), _ptr(out_y))
    return _path_result(acc, margin, tok, mrec, out_y, flags)


def verify_tree_path(ref, b, path, y):
    """Request b of an oracle.verify_tree() result evaluated along the walk
    `path` (node 0 first, then the accepted nodes in order) with token y
    emitted at its last node.  Returns a dict: tests [k, 4] (child tested,
    the walk's outcome 1/0, the oracle's decision 1/0, |u - ratio|; None if
    the path is not a walk of the tree), token / margin_rec / lo / hi / mass
    / u as in verify_path, and flags."""
    c = ref["call"]
    t = np.ascontiguousarray(c["target"][b])
    N, V = t.shape
    d = None if c["draft"] is None else np.ascontiguousarray(c["draft"][b])
    ua, ur = _request_uniforms(c, b, N)
    path = np.ascontiguousarray(path, dtype=np.int32)
    tests = np.empty((N, 4))
    nt = ctypes.c_int()
    tok, mrec, out_y = ctypes.c_int32(), ctypes.c_double(), np.empty(4)
    flags = _load().svo_verify_tree_path(
        N, V, _dtype_code(t), _ptr(t), _dtype_code(d) if d is not None else F32, _ptr(d),
        int(c["draft_is_probs"]), _ptr(c["tokens"][b]), _ptr(c["parents"][b]),
        int(c["num_nodes"][b]), float(c["temperatures"][b]), _ptr(ua), _ptr(ur),
        len(path) - 1, _ptr(path), int(y), _ptr(tests), ctypes.byref(nt), ctypes.byref(tok),
        ctypes.byref(mrec), _ptr(out_y))
    res = _path_result(None, None, tok, mrec, out_y, flags)
    del res["accept"], res["margin"]
    res["tests"] = None if nt.value < 0 else tests[:nt.value].copy()
    return res


def draft_sample_interval(ref, b, j, y):
    """Where token y sits in the law of row (b, j) of an oracle.draft_sample()
    result: (lo, hi, mass, u), u selecting y iff lo <= u < hi."""
    c = ref["call"]
    q = softmax(row_f64(c["draft"], (b, j)), float(c["temperatures"][b]))
    lo, hi, mass = draw_interval(q, y)
    return lo, hi, mass, draft_uniform(c["seed"], c["offset"], b, j)
