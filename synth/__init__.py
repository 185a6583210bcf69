"""Seeded synthetic inputs for the speculative-sampling verify step.

This module only draws random inputs (logits, draft ids, draft counts,
temperatures).  It holds none of the verify step's arithmetic and is shared,
as plain data, by the oracle tests, the GPU parity tests and the benchmark.

Draft ids are drawn the way a drafter would: from the draft distribution the
verifier sees (the logits after bf16 rounding), with the Gumbel-max trick for
sampling requests and plain argmax for greedy ones.

Tensors are generated with ``torch`` on the requested device; the CPU and GPU
generators give different (equally seeded) streams, so a test always hands the
oracle the very bytes the kernel saw.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

CONFIG_NAMES = {
    0: "tiny verify B=1 K=4 V=1000 fp32",
    1: "B=8 K=5 V=32000 bf16, half greedy / half T=0.7",
    2: "B=64 K=4 V=128256 fp32 Zipf, T=1",
    3: "B=256 K=7 V=152064 bf16 ragged n_b, per-request T and correlation",
    4: "B=512 K=3 V=129280 bf16, half probabilistic / half one-hot n-gram",
}

CONFIG_SHAPES = {  # (B, K, V, dtype)
    0: (1, 4, 1000, torch.float32),
    1: (8, 5, 32000, torch.bfloat16),
    2: (64, 4, 128256, torch.float32),
    3: (256, 7, 152064, torch.bfloat16),
    4: (512, 3, 129280, torch.bfloat16),
}


@dataclasses.dataclass
class Workload:
    name: str
    target: torch.Tensor            # [B, K+1, V] float32 / bfloat16 logits
    draft: torch.Tensor | None      # [B, K, V] logits or probabilities
    draft_mode: torch.Tensor | None  # [B] uint8: 0 probabilistic, 1 one-hot
    draft_ids: torch.Tensor         # [B, K] int32
    num_drafts: torch.Tensor        # [B] int32
    temperatures: torch.Tensor      # [B] float32
    draft_is_probs: bool = False

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def K(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    def to(self, device) -> "Workload":
        mv = lambda t: None if t is None else t.to(device)
        return Workload(self.name, mv(self.target), mv(self.draft),
                        mv(self.draft_mode), mv(self.draft_ids),
                        mv(self.num_drafts), mv(self.temperatures),
                        self.draft_is_probs)

    def clone(self) -> "Workload":
        cl = lambda t: None if t is None else t.clone()
        return Workload(self.name, cl(self.target), cl(self.draft),
                        cl(self.draft_mode), cl(self.draft_ids),
                        cl(self.num_drafts), cl(self.temperatures),
                        self.draft_is_probs)

    def host_arrays(self, requests=None):
        """numpy views for the oracle (bf16 as raw uint16 bits).

        ``requests`` selects a subset of requests (a list or slice)."""
        def np_of(t):
            if t is None:
                return None
            t = t.detach()
            if requests is not None:
                t = t[requests]
            t = t.cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return dict(target=np_of(self.target), draft=np_of(self.draft),
                    draft_mode=np_of(self.draft_mode),
                    draft_ids=np_of(self.draft_ids),
                    num_drafts=np_of(self.num_drafts),
                    temperatures=np_of(self.temperatures),
                    draft_is_probs=self.draft_is_probs)

    def elt(self):
        return self.target.element_size()

    def verified_elems(self):
        """sum_b (n_b + 1) * V: the rows the step verifies or samples."""
        n = self.num_drafts.clamp(0, self.K).to(torch.int64)
        return int((n + 1).sum().item()) * self.V

    def algorithmic_bytes(self):
        """Each needed input element read once: target rows 0..n_b, plus draft
        rows 0..n_b-1 for probabilistic sampling requests (greedy and one-hot
        requests read no draft row)."""
        n = self.num_drafts.clamp(0, self.K).to(torch.int64).cpu()
        T = self.temperatures.float().cpu()
        sampling = (T > 0) & torch.isfinite(T) & (T >= torch.finfo(torch.float32).tiny)
        prob = torch.ones_like(n, dtype=torch.bool)
        if self.draft is None:
            prob[:] = False
        elif self.draft_mode is not None:
            prob = self.draft_mode.cpu() == 0
        rows_t = int((n + 1).sum())
        rows_d = int((n * (prob & sampling)).sum())
        delt = self.draft.element_size() if self.draft is not None else 0
        return rows_t * self.V * self.elt() + rows_d * self.V * delt

    def nominal_bytes(self):
        delt = self.draft.element_size() if self.draft is not None else self.elt()
        return self.B * self.V * ((self.K + 1) * self.elt() + self.K * delt)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(g, shape, std, device):
    return torch.randn(shape, generator=g, device=device,
                       dtype=torch.float32) * std


def _gumbel_argmax(logits_over_T, g):
    u = torch.rand(logits_over_T.shape, generator=g, device=logits_over_T.device,
                   dtype=torch.float32)
    gumbel = -torch.log(-torch.log(u))
    return torch.argmax(logits_over_T + gumbel, dim=-1)


def _zipf_base(g, B, R, V, device):
    """Per-request permutation: logit_i = -1.1 ln(rank_i) + N(0, 0.3^2),
    rank_i = pi_b(i) + 1, the same permutation for every row of a request."""
    out = torch.empty((B, R, V), device=device, dtype=torch.float32)
    ranks = torch.empty((B, V), device=device, dtype=torch.float32)
    for b in range(B):
        perm = torch.randperm(V, generator=g, device=device)
        ranks[b] = (perm + 1).to(torch.float32)
        out[b] = -1.1 * torch.log(ranks[b]).unsqueeze(0)
    out += _normal(g, (B, R, V), 0.3, device)
    return out, ranks


def make_contexts(B, N, V, *, seed=0, device="cpu", alpha=1.1, ragged=False,
                  copy_spans=0, span=(8, 33), tail_copy_frac=0.0):
    """Token contexts for the n-gram proposer: row b holds N ids drawn i.i.d.
    from request b's Zipf unigram law (weight rank^-alpha under a per-request
    permutation of the V ids), as the n-gram requests of the B=512 workload.
    With copy_spans > 0, that many spans (lengths in [span[0], span[1])) are
    copied from earlier in the row to later positions, the repeats that make
    prompt lookup pay off; with tail_copy_frac, that fraction of rows also
    ends in a copy of an earlier span (a suffix that occurred before).
    ragged: lengths uniform in [1, N], else all N.
    Returns (context [B, N] int32, lens [B] int32)."""
    device = torch.device(device)
    g = _gen(device, seed)
    ctx = torch.empty((B, N), dtype=torch.int64, device=device)
    for b0 in range(0, B, 64):
        b1 = min(B, b0 + 64)
        w = torch.empty((b1 - b0, V), device=device, dtype=torch.float32)
        for b in range(b0, b1):
            perm = torch.randperm(V, generator=g, device=device)
            w[b - b0] = (perm + 1).to(torch.float32).pow(-alpha)
        ctx[b0:b1] = torch.multinomial(w, N, replacement=True, generator=g)
    if copy_spans > 0 and N > 2 * span[0]:
        for b in range(B):
            for _ in range(copy_spans):
                L = int(torch.randint(span[0], span[1], (1,), generator=g, device=device))
                L = min(L, N // 2)
                src = int(torch.randint(0, N - 2 * L + 1, (1,), generator=g, device=device))
                dst = int(torch.randint(src + L, N - L + 1, (1,), generator=g, device=device))
                ctx[b, dst:dst + L] = ctx[b, src:src + L].clone()
    if ragged:
        lens = torch.randint(1, N + 1, (B,), generator=g, device=device)
    else:
        lens = torch.full((B,), N, device=device)
    if tail_copy_frac > 0 and N > 2 * span[0]:
        pick = torch.rand(B, generator=g, device=device) < tail_copy_frac
        for b in range(B):
            n_b = int(lens[b])
            if not bool(pick[b]) or n_b <= 2 * span[0]:
                continue
            L = min(int(torch.randint(span[0], span[1], (1,), generator=g, device=device)),
                    n_b // 2)
            src = int(torch.randint(0, n_b - 2 * L + 1, (1,), generator=g, device=device))
            ctx[b, n_b - L:n_b] = ctx[b, src:src + L].clone()
    return ctx.to(torch.int32).contiguous(), lens.to(torch.int32)


@dataclasses.dataclass
class TreeWorkload:
    """Inputs of token-tree verification (layout of spec_verify_run_tree)."""
    name: str
    target: torch.Tensor        # [B, N, V] logits after each node
    draft: torch.Tensor | None  # [B, N, V] draft logits at each node, or None
    tokens: torch.Tensor        # [B, N] int32, node 0 unused
    parents: torch.Tensor       # [B, N] int32, node 0: -1
    num_nodes: torch.Tensor     # [B] int32
    temperatures: torch.Tensor  # [B] float32

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def N(self):
        return self.target.shape[1]

    @property
    def V(self):
        return self.target.shape[2]

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return TreeWorkload(self.name, f(self.target), f(self.draft), f(self.tokens),
                            f(self.parents), f(self.num_nodes), f(self.temperatures))

    def host_arrays(self):
        def np_of(t):
            if t is None:
                return None
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return {k: np_of(getattr(self, k)) for k in
                ("target", "draft", "tokens", "parents", "num_nodes", "temperatures")}


def make_tree(B, N, V, *, dtype=torch.float32, draft_dtype=None, seed=0, device="cpu",
              temps=(1.0,), onehot=False, corr=0.9, scale=2.0, ragged=True,
              shape="random"):
    """Seeded token trees.  Shape "random": node i's parent is uniform over the
    earlier nodes (a random recursive tree); "chain": parent of i is i - 1;
    "wide": the root has every other node as a child.  Draft logits at each
    node are N(0, scale^2); target logits are corr * draft + noise.  Child
    tokens are drawn from the parent's tempered draft law by Gumbel-max,
    independently (siblings may repeat), or, for one-hot trees, half from the
    parent's target top tokens and half uniformly; greedy requests take the
    parent's draft argmax with random perturbations."""
    device = torch.device(device)
    g = _gen(device, seed)
    draft_dtype = draft_dtype or dtype
    D = _normal(g, (B, N, V), scale, device)
    tgt = corr * D + math.sqrt(max(0.0, 1 - corr * corr)) * _normal(g, (B, N, V), scale, device)
    target = tgt.to(dtype)
    T = torch.tensor([temps[b % len(temps)] for b in range(B)], dtype=torch.float32,
                     device=device)
    par = torch.full((B, N), -1, dtype=torch.int64, device=device)
    for i in range(1, N):
        if shape == "chain":
            par[:, i] = i - 1
        elif shape == "wide":
            par[:, i] = 0
        else:
            par[:, i] = torch.randint(0, i, (B,), generator=g, device=device)
    tok = torch.zeros((B, N), dtype=torch.int64, device=device)
    base = D.to(draft_dtype).float()
    tq = torch.where(T > 0, T, torch.ones_like(T)).view(-1, 1, 1)
    pg = torch.gather(base, 1, par.clamp_min(0).unsqueeze(-1).expand(B, N, V))
    if onehot:
        pt = torch.gather(target.float(), 1, par.clamp_min(0).unsqueeze(-1).expand(B, N, V))
        top = torch.topk(pt, 3, dim=-1).indices
        pick = torch.randint(0, 3, (B, N, 1), generator=g, device=device)
        tok_top = torch.gather(top, 2, pick)[..., 0]
        tok_rnd = torch.randint(0, V, (B, N), generator=g, device=device)
        tok = torch.where(torch.rand((B, N), generator=g, device=device) < 0.5, tok_top, tok_rnd)
    else:
        tok = _gumbel_argmax(pg / tq, g)
        am = torch.argmax(pg, -1)
        greedy = (T <= 0).view(-1, 1)
        tok = torch.where(greedy & (torch.rand((B, N), generator=g, device=device) < 0.7), am, tok)
    tok[:, 0] = 0
    if ragged:
        nn = torch.randint(1, N + 1, (B,), generator=g, device=device)
    else:
        nn = torch.full((B,), N, device=device)
    return TreeWorkload(f"tree B={B} N={N} V={V} {shape}{' one-hot' if onehot else ''}",
                        target.contiguous(),
                        None if onehot else D.to(draft_dtype).contiguous(),
                        tok.to(torch.int32).contiguous(), par.to(torch.int32).contiguous(),
                        nn.to(torch.int32), T)


def make_config(idx: int, device="cpu", seed: int | None = None) -> Workload:
    """The five verify workloads (shapes, value laws and draft structure)."""
    device = torch.device(device)
    seed = 1000 + idx if seed is None else seed
    g = _gen(device, seed)
    B, K, V, dt = CONFIG_SHAPES[idx]
    name = CONFIG_NAMES[idx]
    i32 = dict(device=device, dtype=torch.int32)

    if idx == 0:
        D = _normal(g, (B, K + 1, V), 2.0, device)
        target = D + _normal(g, (B, K + 1, V), 0.5, device)
        draft = D[:, :K].to(dt)
        ids = _gumbel_argmax(draft.float(), g)
        return Workload(name, target.to(dt), draft.contiguous(), None,
                        ids.to(torch.int32), torch.full((B,), K, **i32),
                        torch.ones(B, device=device))

    if idx == 1:
        D = _normal(g, (B, K + 1, V), 2.0, device)
        target = (D + _normal(g, (B, K + 1, V), 1.0, device)).to(dt)
        draft = D[:, :K].to(dt).contiguous()
        temps = torch.tensor([0.0] * (B // 2) + [0.7] * (B - B // 2),
                             device=device)
        ids = torch.empty((B, K), **i32)
        ids[: B // 2] = torch.argmax(draft[: B // 2].float(), -1).to(torch.int32)
        ids[B // 2:] = _gumbel_argmax(draft[B // 2:].float() / 0.7, g).to(torch.int32)
        return Workload(name, target, draft, None, ids,
                        torch.full((B,), K, **i32), temps)

    if idx == 2:
        D, _ = _zipf_base(g, B, K + 1, V, device)
        target = (D + _normal(g, (B, K + 1, V), 0.7, device)).to(dt)
        draft = D[:, :K].to(dt).contiguous()
        ids = _gumbel_argmax(draft.float(), g).to(torch.int32)
        return Workload(name, target, draft, None, ids,
                        torch.full((B,), K, **i32), torch.ones(B, device=device))

    if idx == 3:
        n = torch.randint(0, K + 1, (B,), generator=g, device=device)
        temps = 0.3 + 0.9 * torch.rand(B, generator=g, device=device)
        rho = 0.5 + 0.45 * torch.rand(B, generator=g, device=device)
        target = torch.empty((B, K + 1, V), device=device, dtype=dt)
        draft = torch.empty((B, K, V), device=device, dtype=dt)
        ids = torch.empty((B, K), **i32)
        for b0 in range(0, B, 32):  # bounded temporaries
            b1 = min(B, b0 + 32)
            D = _normal(g, (b1 - b0, K + 1, V), 2.0, device)
            r = rho[b0:b1].view(-1, 1, 1)
            tgt = r * D + torch.sqrt(1 - r * r) * _normal(
                g, (b1 - b0, K + 1, V), 2.0, device)
            dq = D[:, :K].to(dt)
            x = _gumbel_argmax(dq.float() / temps[b0:b1].view(-1, 1, 1), g)
            target[b0:b1] = tgt.to(dt)
            draft[b0:b1] = dq
            ids[b0:b1] = x.to(torch.int32)
        # Padding rows are never read by the step: fill them with NaN.
        jt = torch.arange(K + 1, device=device).view(1, -1)
        target[jt > n.view(-1, 1)] = float("nan")
        jd = torch.arange(K, device=device).view(1, -1)
        draft[jd >= n.view(-1, 1)] = float("nan")
        return Workload(name, target, draft, None, ids, n.to(torch.int32),
                        temps.float())

    if idx == 4:
        target = torch.empty((B, K + 1, V), device=device, dtype=dt)
        draft = torch.full((B, K, V), float("nan"), device=device, dtype=dt)
        ids = torch.empty((B, K), **i32)
        mode = (torch.arange(B, device=device) % 2).to(torch.uint8)
        for b0 in range(0, B, 32):
            b1 = min(B, b0 + 32)
            D, ranks = _zipf_base(g, b1 - b0, K + 1, V, device)
            target[b0:b1] = (D + _normal(g, (b1 - b0, K + 1, V), 0.7,
                                         device)).to(dt)
            dq = D[:, :K].to(dt)
            x_prob = _gumbel_argmax(dq.float(), g)
            # n-gram drafts: a random span of a 2048-token context drawn from
            # the request's Zipf unigram law (weight rank^-1.1).
            ctx = torch.multinomial(ranks.pow(-1.1), 2048, replacement=True,
                                    generator=g)
            s = torch.randint(0, 2048 - K + 1, (b1 - b0, 1), generator=g,
                              device=device)
            x_gram = torch.gather(ctx, 1, s + torch.arange(K, device=device))
            for bb in range(b0, b1):
                if mode[bb] == 0:
                    draft[bb] = dq[bb - b0]
                    ids[bb] = x_prob[bb - b0].to(torch.int32)
                else:
                    ids[bb] = x_gram[bb - b0].to(torch.int32)
        return Workload(name, target, draft, mode, ids,
                        torch.full((B,), K, **i32), torch.ones(B, device=device))

    raise ValueError(f"unknown config {idx}")


def make_random(B, K, V, *, dtype=torch.float32, draft_dtype=None, seed=0,
                device="cpu", temps=(1.0,), n_mode="full", onehot_frac=0.0,
                draft_is_probs=False, corr=0.9, scale=2.0, with_draft=True,
                nan_padding=True) -> Workload:
    """Small seeded cases for parity tests: Gaussian draft logits, target
    correlated with them, drafts sampled from q (or argmax for greedy),
    temperatures cycled from ``temps``, n_b all K ("full") or uniform in
    {0..K} ("ragged")."""
    device = torch.device(device)
    g = _gen(device, seed)
    draft_dtype = draft_dtype or dtype
    D = _normal(g, (B, K + 1, V), scale, device)
    tgt = corr * D + math.sqrt(max(0.0, 1 - corr * corr)) * _normal(
        g, (B, K + 1, V), scale, device)
    target = tgt.to(dtype)
    T = torch.tensor([temps[b % len(temps)] for b in range(B)],
                     dtype=torch.float32, device=device)
    if n_mode == "full":
        n = torch.full((B,), K, dtype=torch.int32, device=device)
    else:
        n = torch.randint(0, K + 1, (B,), generator=g, device=device).to(torch.int32)
    mode = None
    if onehot_frac > 0:
        mode = (torch.rand(B, generator=g, device=device) < onehot_frac).to(torch.uint8)
    draft = None
    ids = torch.empty((B, K), dtype=torch.int32, device=device)
    if with_draft and K > 0:
        dq = D[:, :K]
        if draft_is_probs:
            Tq = torch.where(T > 0, T, torch.ones_like(T)).view(-1, 1, 1)
            draft = torch.softmax(dq / Tq, dim=-1).to(draft_dtype)
            base = torch.log(draft.float().clamp_min(1e-38))
        else:
            draft = dq.to(draft_dtype)
            base = draft.float()
        for b in range(B):
            if T[b] > 0:
                tb = 1.0 if draft_is_probs else float(T[b])
                ids[b] = _gumbel_argmax(base[b] / tb, g).to(torch.int32)
            else:
                ids[b] = torch.argmax(base[b], -1).to(torch.int32)
        draft = draft.contiguous()
    elif K > 0:
        ids[:] = torch.randint(0, V, (B, K), generator=g,
                               device=device).to(torch.int32)
    if mode is not None and K > 0:
        # one-hot requests: copy some ids from the target's own argmax so that
        # acceptances happen, the rest random
        am = torch.argmax(target.float()[:, :K], -1).to(torch.int32)
        rnd = torch.randint(0, V, (B, K), generator=g, device=device).to(torch.int32)
        pick = torch.rand((B, K), generator=g, device=device) < 0.5
        oh = torch.where(pick, am, rnd)
        ids = torch.where(mode.view(-1, 1).bool(), oh, ids)
    if nan_padding and K > 0:
        jt = torch.arange(K + 1, device=device).view(1, -1)
        tf = target.float()
        tf[jt > n.view(-1, 1)] = float("nan")
        target = tf.to(dtype)
        if draft is not None:
            jd = torch.arange(K, device=device).view(1, -1)
            df = draft.float()
            df[jd >= n.view(-1, 1)] = float("nan")
            if mode is not None:
                df[mode.bool()] = float("nan")
            draft = df.to(draft_dtype).contiguous()
    return Workload(f"random B={B} K={K} V={V}", target.contiguous(), draft,
                    mode, ids.contiguous(), n, T, draft_is_probs)
