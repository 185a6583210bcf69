"""Benchmark of the speculative-sampling verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
    python bench.py --op draft_sample     # the draft-token sampler instead
    python bench.py --op ngram            # the n-gram prompt-lookup proposer
    python bench.py --op typical          # verify with typical acceptance
    python bench.py --op tree             # token-tree verification

One step = one spec_verify_run over a whole batch: row statistics, decisions,
residual sums of rejected probabilistic drafts, and the draws.  Inputs are
generated on the GPU and stay resident; steps rotate through --rotate copies
of them so each step's rows were last
touched more than the 256 MB Infinity Cache earlier.  The timed region is
bracketed by torch.cuda.synchronize() and timed with events on the stream
the library launches on.  A second loop of the same length times each kernel
with the library's own HIP events (spec_verify_timing_*), which gives the
dominant kernel's duration for the roofline.

Before the warm-up, untimed steps run for --ramp-ms of GPU time so that the
clocks have ramped up (reported as clock_ramp); the warm-up and timed steps
are then exactly --warmup and --steps.

Prints ONE JSON line.  value = verified (request x position x vocabulary)
elements per second = sum_b (n_b + 1) * V / step time.  With --op
draft_sample a step is one spec_draft_sample over the workload's draft rows
(j < n_b) and value = sampled elements per second = sum_b n_b * V / step time.
roofline.frac is the dominant (row statistics) kernel's algorithmic GB/s over
the 8 TB/s peak; roofline.step_frac is the same bytes over the whole step.
With --op verify the other large workloads (--also, default B=64 and B=512)
are measured the same way afterwards and reported under "workloads".

The CPU leg (skipped with --no-cpu-baseline) runs the fp64 oracle twice: once,
untimed, on the exact inputs of the last timed step of each workload, whose
outputs it checks by the parity rule ("parity"), and once timed on a bounded
sample ("cpu_baseline").
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified (req×pos×vocab) elems/s + achieved HBM GB/s vs peak, spec-verify step"
METRIC_SAMPLE = "sampled (row×vocab) elems/s + achieved HBM GB/s vs peak, draft-token sampler"
METRIC_TYPICAL = "verified (req×pos×vocab) elems/s + achieved HBM GB/s vs peak, typical acceptance"
HBM_PEAK_GBPS = 8000.0
DOMINANT = "stats"  # the kernel that streams every needed logits row
# the sources the verify kernels are built from (the traffic summary is valid
# only for the sources it was measured on)
KERNEL_SRC = [os.path.join(ROOT, "rejection_sampling_verify_temp_amd", "csrc", f)
              for f in ("sv_kernels.hip", "sv_device.h", "sv_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stats_traffic_B256_K7_V152064_bf16.txt")
TREE_SRC = [os.path.join(ROOT, "rejection_sampling_verify_temp_amd", "csrc", f)
            for f in ("sv_tree.hip", "sv_tree.h", "sv_device.h", "sv_internal.h")]
TREE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tree_traffic_B256_N16_V152064_bf16.txt")


def _code_only(text):
    """The source with comments removed and whitespace collapsed, so that an
    edit to a comment keeps a measurement that the compiled kernel still
    matches.  (Comment markers inside string literals do not occur in these
    sources.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(paths=None):
    h = hashlib.sha256()
    for path in paths or KERNEL_SRC:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload_idx, path=TRAFFIC_FILE, src=None):
    """HBM bytes per launch of the dominant kernel measured with rocprofv3
    --pmc (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), valid
    only for the workload and the kernel source it was taken on."""
    if workload_idx != 3 or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seconds=12.0):
    """Time the CPU oracle, as it stands, on a bounded sample: slices of 8
    requests of the same batch, cycling through the batch (a new Philox offset
    each pass) until about `seconds` of single-threaded work is done."""
    import oracle
    hs = w.host_arrays()
    V = w.V
    n_req, elems, t, passes = 0, 0, 0.0, 0
    start = 0
    while t < seconds and passes < 64:
        sl = slice(start, min(w.B, start + 8))
        sub = {k: (v[sl] if hasattr(v, "shape") and v.shape[:1] == (w.B,) else v)
               for k, v in hs.items()}
        t0 = time.perf_counter()
        oracle.verify(sub["target"], sub["draft"], sub["draft_ids"],
                      sub["num_drafts"], sub["temperatures"],
                      draft_mode=sub["draft_mode"],
                      draft_is_probs=sub["draft_is_probs"], seed=0,
                      offset=passes, diagnostics=False)
        t += time.perf_counter() - t0
        n = sub["num_drafts"].clip(0, w.K)
        elems += int((n + 1).sum()) * V
        n_req += sl.stop - sl.start
        start = sl.stop
        if start >= w.B:
            start, passes = 0, passes + 1
    return dict(value=elems / t, unit="elems/s", cores=1, kind="oracle",
                sample=f"{n_req} requests of the same batch (the batch cycled "
                       f"with a new Philox offset per pass), {elems} verified "
                       f"elems, {t:.1f} s of the single-threaded fp64 C oracle")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads():
    """Worker threads for the all-cores leg: the CPUs this process may run on,
    at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_threads(w, seconds=6.0):
    """The same oracle on all the host cores this process may use: each
    worker thread runs slices of 8 requests (the C oracle releases the
    interpreter lock), cycling through the batch with a new Philox offset per
    pass, until about `seconds` of wall time; requests are independent, so
    this is the oracle as it stands, only run side by side."""
    import threading
    import oracle
    hs = w.host_arrays()
    V, B, K = w.V, w.B, w.K
    nthreads = cpu_threads()
    lock = threading.Lock()
    state = {"next": 0, "elems": 0, "req": 0}
    stop = time.perf_counter() + seconds

    def worker():
        while time.perf_counter() < stop:
            with lock:
                k = state["next"]
                state["next"] += 1
            start = (k * 8) % B
            sl = slice(start, min(B, start + 8))
            sub = {kk: (v[sl] if hasattr(v, "shape") and v.shape[:1] == (B,) else v)
                   for kk, v in hs.items()}
            oracle.verify(sub["target"], sub["draft"], sub["draft_ids"], sub["num_drafts"],
                          sub["temperatures"], draft_mode=sub["draft_mode"],
                          draft_is_probs=sub["draft_is_probs"], seed=0,
                          offset=(k * 8) // B, diagnostics=False)
            n = sub["num_drafts"].clip(0, K)
            with lock:
                state["elems"] += int((n + 1).sum()) * V
                state["req"] += sl.stop - sl.start

    t0 = time.perf_counter()
    threads = [threading.Thread(target=worker) for _ in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    dt = time.perf_counter() - t0
    return dict(value=state["elems"] / dt, unit="elems/s", cores=nthreads, kind="oracle",
                cpu=cpu_model(),
                sample=f"{state['req']} requests of the same batch on {nthreads} threads "
                       f"(slices of 8, a new Philox offset per pass over the batch), "
                       f"{state['elems']} verified elems, {dt:.1f} s wall time")


def cpu_baseline_typical(w, eps, top_k, seconds=12.0):
    """The CPU oracle's typical acceptance, as it stands, on slices of 8
    requests of the same batch until about `seconds` of single-threaded work."""
    import oracle
    hs = w.host_arrays()
    V = w.V
    n_req, elems, t, passes, start = 0, 0, 0.0, 0, 0
    while t < seconds and passes < 64:
        sl = slice(start, min(w.B, start + 8))
        t0 = time.perf_counter()
        oracle.verify_typical(hs["target"][sl], hs["draft_ids"][sl], hs["num_drafts"][sl],
                              hs["temperatures"][sl], eps=eps, top_k=top_k, seed=0,
                              offset=passes, diagnostics=False)
        t += time.perf_counter() - t0
        elems += int((hs["num_drafts"][sl].clip(0, w.K) + 1).sum()) * V
        n_req += sl.stop - sl.start
        start = sl.stop
        if start >= w.B:
            start, passes = 0, passes + 1
    return dict(value=elems / t, unit="elems/s", cores=1, kind="oracle",
                sample=f"{n_req} requests of the same batch (the batch cycled "
                       f"with a new Philox offset per pass), {elems} verified "
                       f"elems, {t:.1f} s of the single-threaded fp64 C oracle")


def cpu_baseline_sample(w, nd, seconds=12.0):
    """The CPU oracle's draft sampler, as it stands, on slices of 8 requests
    of the same batch until about `seconds` of single-threaded work."""
    import oracle
    hs = w.host_arrays()
    hs["num_drafts"] = nd.cpu().numpy()
    V = w.V
    n_req, elems, t, passes, start = 0, 0, 0.0, 0, 0
    while t < seconds and passes < 64:
        sl = slice(start, min(w.B, start + 8))
        t0 = time.perf_counter()
        oracle.draft_sample(hs["draft"][sl], hs["num_drafts"][sl],
                            hs["temperatures"][sl], seed=0, offset=passes,
                            diagnostics=False)
        t += time.perf_counter() - t0
        elems += int(hs["num_drafts"][sl].clip(0, w.K).sum()) * V
        n_req += sl.stop - sl.start
        start = sl.stop
        if start >= w.B:
            start, passes = 0, passes + 1
    return dict(value=elems / t, unit="elems/s", cores=1, kind="oracle",
                sample=f"{n_req} requests of the same batch (the batch cycled "
                       f"with a new Philox offset per pass), {elems} sampled "
                       f"elems, {t:.1f} s of the single-threaded fp64 C oracle")


METRIC_NGRAM = "scanned context tokens/s + achieved HBM GB/s vs peak, n-gram prompt-lookup proposer"
NGRAM = dict(B=512, N=2048, V=129280, min_n=2, max_n=5, k=3, max_model_len=8192)


def bench_ngram(args):
    """n-gram proposer: 512 Zipf-unigram contexts of 2048 tokens (V = 129280,
    four copied spans each, half ending in a copy of an earlier span), n in
    [2, 5], k = 3.  A step is one spec_ngram_propose over the batch."""
    import torch
    import synth
    import rejection_sampling_verify_temp_amd as sv
    c = NGRAM
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = [synth.make_contexts(c["B"], c["N"], c["V"], seed=21 + i, copy_spans=4,
                                  tail_copy_frac=0.5, device=dev) for i in range(args.rotate)]
    drafts = torch.empty((c["B"], c["k"]), dtype=torch.int32, device=dev)
    num = torch.empty((c["B"],), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    kw = {k: c[k] for k in ("min_n", "max_n", "k", "max_model_len")}

    def step(i):
        ctx, lens = copies[i % len(copies)]
        sv.ngram_propose(ctx, lens, out_drafts=drafts, out_num=num, stream=stream, **kw)

    ramp = clock_ramp(step, args.ramp_ms, first=1 << 20)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    tokens = sum(int(l.sum().item()) for _, l in copies) / len(copies)
    alg = tokens * 4 + c["B"] * (c["k"] + 1) * 4  # each context token read once, outputs
    proposals = int((num > 0).sum().item())
    out = {
        "metric": METRIC_NGRAM,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "n-gram proposer, B=512 Zipf(1.1) contexts of 2048 tokens, "
                               "V=129280, n in [2, 5], k=3",
                   **c, "input_copies": len(copies), "requests_with_drafts": proposals,
                   "parallelism": "single GPU"},
        "clock_ramp": {"steps": ramp[0], "ms": round(ramp[1], 1)},
        "roofline": {"bound": "hbm", "kernel": "ngram", "achieved": alg / (ms_step * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        # parity of the last timed step: the oracle's proposals on its
        # contexts, bit for bit (integer work)
        last = args.warmup + args.steps - 1
        lc, ll = (t.cpu().numpy() for t in copies[last % len(copies)])
        rd, rn = oracle.ngram_propose(lc, ll, **kw)
        gd, gn = drafts.cpu().numpy(), num.cpu().numpy()
        bad = int(np.sum((gn != rn) | np.any(gd != rd, axis=1)))
        out["parity"] = {"status": "ok" if bad == 0 else "FAIL", "checked": int(c["B"]),
                         "mismatches": bad,
                         "what": "the last timed step's drafts and counts against the C oracle, "
                                 "bit for bit"}
        ctx, lens = (t.cpu().numpy() for t in copies[0])
        t0, reps = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0:
            oracle.ngram_propose(ctx, lens, **kw)
            reps += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=reps * float(lens.sum()) / dt, unit="tokens/s", cores=1,
                                   kind="oracle",
                                   sample=f"{reps} passes over the same 512 contexts, {dt:.1f} s "
                                          "of the single-threaded C oracle")
    print(json.dumps(out), flush=True)


METRIC_TREE = "tree elems/s (req×node×vocab) + achieved HBM GB/s vs peak, token-tree verification"
TREE = dict(B=256, N=16, V=152064)


def bench_tree(args):
    """Token-tree verification: 256 requests, random recursive trees of 16
    nodes over V = 152064 (bf16 target and draft logits, child tokens drawn
    from the parent's draft law, per-request T in {0.6, 1.0, 0.0, 0.8}).  A
    step is one spec_verify_run_tree over the batch."""
    import torch
    import synth
    import rejection_sampling_verify_temp_amd as sv
    c = TREE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copies = [synth.make_tree(c["B"], c["N"], c["V"], dtype=torch.bfloat16, seed=31 + i,
                              temps=(0.6, 1.0, 0.0, 0.8), corr=0.95, ragged=False, device=dev)
              for i in range(args.rotate)]
    w = copies[0]
    h = sv.SpecVerify(w.B, 1, w.V, torch.bfloat16, draft_dtype=torch.bfloat16)
    stream = torch.cuda.current_stream(dev)
    outs = []

    def step(i):
        t = copies[i % len(copies)]
        outs.append(h.run_tree(t.target, t.draft, t.tokens, t.parents, t.num_nodes,
                               t.temperatures, seed=0, offset=i, stream=stream))
        del outs[:-len(copies)]

    ramp = clock_ramp(step, args.ramp_ms, first=1 << 40)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    assert h.device_errors() & ~8 == 0
    if args.copy_probe_mib:  # a known-size reference for HBM counters
        a = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
    # bytes of the visited nodes' rows (target and draft), from the last
    # steps' walks: the least the walk must read
    row = c["V"] * 2
    visited, accepted = 0, 0
    for k in range(len(copies)):
        _, nacc, _ = outs[k]
        visited += int((nacc + 1).sum().item())
        accepted += int(nacc.sum().item())
    visited /= len(copies)
    alg = visited * 2 * row
    elems = sum(int(t.num_nodes.sum().item()) for t in copies) / len(copies) * c["V"]
    out = {
        "metric": METRIC_TREE,
        "value": elems / (ms_step * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "token-tree verification, B=256 random trees of 16 nodes, "
                               "V=152064 bf16",
                   **c, "input_copies": len(copies), "visited_rows_per_step": visited,
                   "accepted_per_request": accepted / len(copies) / c["B"],
                   "parallelism": "single GPU"},
        "clock_ramp": {"steps": ramp[0], "ms": round(ramp[1], 1)},
        "roofline": {"bound": "hbm", "kernel": "tree", "achieved": alg / (ms_step * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "traffic": read_traffic(3, TREE_TRAFFIC_FILE, TREE_SRC)},
        "team_size": h.tree_team_size(c["B"]),
    }
    if not args.no_cpu_baseline:
        import oracle
        from oracle.parity import compare_tree
        # parity of the last timed step (whole batch, its inputs, seed and
        # offset) against the oracle, untimed
        last = args.warmup + args.steps - 1
        t0 = time.perf_counter()
        hl = copies[last % len(copies)].host_arrays()
        ref = oracle.verify_tree(hl["target"], hl["draft"], hl["tokens"], hl["parents"],
                                 hl["num_nodes"], hl["temperatures"], seed=0, offset=last)
        tok, nacc, lastn = (x.cpu().numpy() for x in outs[-1])
        rep = compare_tree(hl["tokens"], hl["parents"], hl["num_nodes"], c["V"], ref, tok, nacc,
                           lastn)
        out["parity"] = {"status": "ok" if rep.ok() else "FAIL", "checked": rep.requests,
                         "flagged": rep.flagged, "flagged_differing": rep.flagged_mismatch,
                         "mismatches": len(rep.mismatches),
                         "first_mismatches": [str(m) for m in rep.mismatches[:3]],
                         "what": f"the whole batch of the last timed step (Philox offset {last}) "
                                 f"against the fp64 C oracle, {time.perf_counter() - t0:.1f} s"}
        hs = w.host_arrays()
        t0, n_req = time.perf_counter(), 0
        while time.perf_counter() - t0 < 12.0 and n_req < c["B"]:
            sl = slice(n_req, n_req + 4)
            oracle.verify_tree(hs["target"][sl], hs["draft"][sl], hs["tokens"][sl],
                               hs["parents"][sl], hs["num_nodes"][sl], hs["temperatures"][sl])
            n_req += 4
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=n_req * c["N"] * c["V"] / dt, unit="elems/s", cores=1,
                                   kind="oracle",
                                   sample=f"{n_req} requests of the same batch, {dt:.1f} s of "
                                          "the single-threaded fp64 C oracle")
    h.close()
    del copies, outs, w
    if args.tree_batches:
        out["batches"] = {str(b): tree_batch(b, args) for b in args.tree_batches.split(",")
                          if b.strip()}
    print(json.dumps(out), flush=True)


def tree_batch(B, args):
    """The tree workload's recipe at another batch size: step time, tree
    elements per second and the workgroups per request the library picks."""
    import torch
    import synth
    import rejection_sampling_verify_temp_amd as sv
    B = int(B)
    c = TREE
    dev = torch.device("cuda:0")
    copies = [synth.make_tree(B, c["N"], c["V"], dtype=torch.bfloat16, seed=31 + i,
                              temps=(0.6, 1.0, 0.0, 0.8), corr=0.95, ragged=False, device=dev)
              for i in range(args.rotate)]
    h = sv.SpecVerify(B, 1, c["V"], torch.bfloat16, draft_dtype=torch.bfloat16)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = copies[i % len(copies)]
        return h.run_tree(t.target, t.draft, t.tokens, t.parents, t.num_nodes, t.temperatures,
                          seed=0, offset=i, stream=stream)

    clock_ramp(step, args.ramp_ms, first=1 << 40)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert h.device_errors() & ~8 == 0
    team = h.tree_team_size(B)
    h.close()
    return {"ms_per_step": ms, "value": B * c["N"] * c["V"] / (ms * 1e-3), "unit": "elems/s",
            "team_size": team}


def clock_ramp(step, ms, first):
    """Untimed steps until about `ms` of GPU time has passed, so the clocks
    have ramped up before the warm-up and the timed steps (offsets start at
    `first`, away from the timed ones).  Returns (steps, wall ms)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(first + n)
            n += 1
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def measure(args, widx, op):
    """Ramp, warm-up and timed steps of one workload.  Returns the numbers
    and the context the parity check of the CPU leg needs."""
    import torch
    import synth
    import rejection_sampling_verify_temp_amd as sv

    dev = torch.device("cuda:0")
    base = synth.make_config(widx, device=dev)
    copies = [base] + [base.clone() for _ in range(max(0, args.rotate - 1))]
    torch.cuda.synchronize()
    w = base
    h = sv.SpecVerify(w.B, w.K, w.V, w.target.dtype,
                      draft_dtype=w.draft.dtype if w.draft is not None else None,
                      draft_is_probs=w.draft_is_probs, device=0,
                      chunk_elems=args.chunk)
    tok = torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((w.B,), dtype=torch.int32, device=dev)
    ids = torch.empty((w.B, w.K), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sample, typical = op == "draft_sample", op == "typical"
    # the sampler draws the draft rows that hold logits: rows j < n_b of the
    # probabilistic requests (one-hot requests have no draft distribution)
    nd_sample = w.num_drafts if w.draft_mode is None else torch.where(
        w.draft_mode == 0, w.num_drafts, torch.zeros_like(w.num_drafts))

    def step(i):
        c = copies[i % len(copies)]
        if sample:
            h.sample(c.draft, nd_sample, c.temperatures, seed=0, offset=i,
                     out_ids=ids, stream=stream)
        elif typical:
            h.run_typical(c.target, c.draft_ids, c.num_drafts, c.temperatures,
                          args.threshold, args.top_k, seed=0, offset=i, out_tokens=tok,
                          out_num_accepted=nacc, stream=stream)
        else:
            h.run(c.target, c.draft, c.draft_mode, c.draft_ids, c.num_drafts,
                  c.temperatures, seed=0, offset=i, out_tokens=tok,
                  out_num_accepted=nacc, stream=stream)

    ramp_steps, ramp_ms = clock_ramp(step, args.ramp_ms, first=1 << 40)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # whole-step timing
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-kernel timing (library events on the same stream), separate loop
    # over the same steps: its last step leaves the outputs of the last timed
    # step (same inputs, same offset)
    sv.spec_verify_timing_enable(h.handle, True)
    for i in range(args.steps):
        step(args.warmup + i)
    nk = 0
    while sv.spec_verify_kernel_name(nk) is not None:
        nk += 1
    tot, runs = sv.spec_verify_timing_read(h.handle, nk)
    sv.spec_verify_timing_enable(h.handle, False)
    torch.cuda.synchronize()
    kern_ms = {sv.spec_verify_kernel_name(k): tot[k] / runs for k in range(nk) if tot[k] > 0}
    # bit 8: a draw met a rounding tie at a chunk boundary (a valid token is
    # taken); any other bit would be bad input data
    dev_flags = h.device_errors()
    assert dev_flags & ~8 == 0, dev_flags

    if sample:
        n_rows = int(nd_sample.clamp(0, w.K).sum().item())
        elems = n_rows * w.V
        alg = n_rows * w.V * w.draft.element_size()  # each sampled row read once
    elif typical:  # target rows 0..n_b only: no draft rows are read
        elems = w.verified_elems()
        alg = elems * w.elt()
    else:
        elems = w.verified_elems()
        alg = w.algorithmic_bytes()
    last = args.warmup + args.steps - 1
    ctx = dict(w=w, copy=copies[last % len(copies)], offset=last, tok=tok, nacc=nacc,
               ids=ids, nd_sample=nd_sample)
    res = dict(ms_step=ms_step, kern_ms=kern_ms, elems=elems, alg=alg, h=h,
               ramp=dict(steps=ramp_steps, ms=round(ramp_ms, 1)), dev_flags=dev_flags)
    return res, ctx


def cpu_parity(ctx, op, args):
    """Part of the CPU leg: the oracle on the exact inputs of the last timed
    step (whole batch, same seed and offset), compared with the GPU's outputs
    of that step by the parity rule.  Untimed."""
    import oracle
    from oracle.parity import compare, compare_draft
    t0 = time.perf_counter()
    c = ctx["copy"]
    hs = c.host_arrays()
    if op == "draft_sample":
        ref = oracle.draft_sample(hs["draft"], ctx["nd_sample"].cpu().numpy(),
                                  hs["temperatures"], seed=0, offset=ctx["offset"])
        rep = compare_draft(ref, ctx["ids"].cpu().numpy())
    elif op == "typical":
        ref = oracle.verify_typical(hs["target"], hs["draft_ids"], hs["num_drafts"],
                                    hs["temperatures"], eps=args.threshold, top_k=args.top_k,
                                    seed=0, offset=ctx["offset"])
        rep = compare(hs, ref, ctx["tok"].cpu().numpy(), ctx["nacc"].cpu().numpy())
    else:
        ref = oracle.verify(hs["target"], hs["draft"], hs["draft_ids"], hs["num_drafts"],
                            hs["temperatures"], draft_mode=hs["draft_mode"],
                            draft_is_probs=hs["draft_is_probs"], seed=0,
                            offset=ctx["offset"])
        rep = compare(hs, ref, ctx["tok"].cpu().numpy(), ctx["nacc"].cpu().numpy())
    return {"status": "ok" if rep.ok() else "FAIL", "checked": rep.requests,
            "flagged": rep.flagged, "flagged_differing": rep.flagged_mismatch,
            "mismatches": len(rep.mismatches), "first_mismatches": [str(m) for m in
                                                                   rep.mismatches[:3]],
            "what": f"the whole batch of the last timed step (Philox offset {ctx['offset']}) "
                    f"against the fp64 C oracle, {time.perf_counter() - t0:.1f} s"}


def step_fractions(res):
    """Achieved HBM GB/s of the dominant kernel and of the whole step."""
    k_ms = res["kern_ms"][DOMINANT]
    return (res["alg"] / (k_ms * 1e-3) / 1e9, res["alg"] / (res["ms_step"] * 1e-3) / 1e9)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    # the GPU clocks take ~10 ms of load to ramp up: untimed steps before the
    # warm-up, reported in the output
    ap.add_argument("--ramp-ms", type=float, default=40.0)
    ap.add_argument("--workload", type=int, default=3, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--also", default="2,4",
                    help="--op verify: other workloads measured after the main one "
                         "and reported under 'workloads' (comma list, '' for none)")
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--op", choices=["verify", "draft_sample", "ngram", "typical", "tree"],
                    default="verify")
    ap.add_argument("--threshold", type=float, default=0.05,
                    help="--op typical: the probability threshold")
    ap.add_argument("--top-k", type=int, default=2, help="--op typical: the top-k clause")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tree-batches", default="32,128",
                    help="--op tree: other batch sizes timed with the same recipe")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the steps, run one plain device copy of this "
                         "size (a known-size reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.op == "ngram":
        return bench_ngram(args)
    if args.op == "tree":
        return bench_tree(args)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    op = args.op
    sample, typical = op == "draft_sample", op == "typical"
    res, ctx = measure(args, args.workload, op)
    w = ctx["w"]
    if sample and (w.draft is None or w.draft_is_probs):
        print("--op draft_sample needs a workload with draft logits", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    nacc = ctx["nacc"]
    # bytes the residual pass re-reads: the rejected row pair of every
    # probabilistic sampling request (from the last step's outputs)
    n_b = w.num_drafts.clamp(0, w.K).cpu()
    T = w.temperatures.float().cpu()
    samp = (T >= torch.finfo(torch.float32).tiny) & torch.isfinite(T)
    prob = torch.zeros_like(samp) if w.draft is None else (
        torch.ones_like(samp) if w.draft_mode is None else w.draft_mode.cpu() == 0)
    pairs = int(((nacc.cpu() < n_b) & samp & prob).sum())
    delt = w.draft.element_size() if w.draft is not None else 0
    resid_bytes = pairs * w.V * (w.elt() + delt)
    ms_step, kern_ms, elems, alg = res["ms_step"], res["kern_ms"], res["elems"], res["alg"]
    achieved, step_gbps = step_fractions(res)
    traffic = None if (sample or typical) else read_traffic(args.workload)
    dt = {torch.bfloat16: "bf16", torch.float32: "f32"}[w.target.dtype]
    out = {
        "metric": METRIC_SAMPLE if sample else (METRIC_TYPICAL if typical else METRIC),
        "value": elems / (ms_step * 1e-3),
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": (f"draft-token sampler, draft rows of {w.name}" if sample
                                else f"typical acceptance (threshold {args.threshold}, "
                                     f"top-k {args.top_k}), {w.name}" if typical
                                else f"verify step, {w.name}"),
                   "B": w.B, "K": w.K, "V": w.V, "logits": dt,
                   ("sampled_elems" if sample else "verified_elems"): elems,
                   "algorithmic_bytes": alg,
                   "nominal_bytes": w.nominal_bytes(),
                   "chunk_elems": res["h"].chunk_elems, "input_copies": args.rotate,
                   "parallelism": "single GPU"},
        "clock_ramp": res["ramp"],
        "step_hbm_gbps": step_gbps,
        "resid_pairs": None if (sample or typical) else pairs,
        "resid_bytes": None if (sample or typical) else resid_bytes,
        "resid_gbps": (resid_bytes / (kern_ms["resid"] * 1e-3) / 1e9
                       if "resid" in kern_ms and not (sample or typical) else None),
        "accepted_per_proposed": (int(nacc.sum().item()) / max(1, int(n_b.sum()))
                                  if not sample else None),
        "emitted_per_request": (float((nacc.cpu() + 1).float().mean()) if not sample
                                else None),
        "device_flags": res["dev_flags"],
        "kernels_ms": kern_ms,
        "roofline": {"bound": "hbm", "kernel": DOMINANT,
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "step_achieved": step_gbps,
                     "step_frac": step_gbps / HBM_PEAK_GBPS},
    }
    res["h"].close()
    extra = {}
    also = [int(x) for x in args.also.split(",") if x.strip()] if op == "verify" else []
    for k in also:
        if k == args.workload:
            continue
        r2, c2 = measure(args, k, op)
        a2, s2 = step_fractions(r2)
        extra[str(k)] = {"workload": f"verify step, {c2['w'].name}",
                         "ms_per_step": r2["ms_step"],
                         "value": r2["elems"] / (r2["ms_step"] * 1e-3),
                         "algorithmic_bytes": r2["alg"],
                         "kernels_ms": r2["kern_ms"],
                         "stats_frac": a2 / HBM_PEAK_GBPS,
                         "step_frac": s2 / HBM_PEAK_GBPS,
                         "emitted_per_request": float((c2["nacc"].cpu() + 1).float().mean()),
                         "clock_ramp": r2["ramp"], "device_flags": r2["dev_flags"]}
        if not args.no_cpu_baseline:
            extra[str(k)]["parity"] = cpu_parity(c2, op, args)
        r2["h"].close()
        del c2
        torch.cuda.empty_cache()
    if extra:
        out["workloads"] = extra
    if not args.no_cpu_baseline:
        out["parity"] = cpu_parity(ctx, op, args)
        out["cpu_baseline"] = (cpu_baseline_sample(w, ctx["nd_sample"]) if sample else
                               cpu_baseline_typical(w, args.threshold, args.top_k) if typical
                               else cpu_baseline(w))
        out["cpu_baseline"]["cpu"] = cpu_model()
        if not sample and not typical:
            out["cpu_baseline_threads"] = cpu_baseline_threads(w)
        # the same rates as bytes of input read once (the step's algorithmic
        # bytes per element), for comparison with the GPU's GB/s
        for key in ("cpu_baseline", "cpu_baseline_threads"):
            if key in out:
                out[key]["algorithmic_gbps"] = out[key]["value"] * alg / elems / 1e9
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
