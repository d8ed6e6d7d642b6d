"""Throughput of the DSA forward on one MI355X (prints one JSON line).

A step is one pass of the layer's forward hot path over the whole sequence: for every query
chunk, indexer scores -> top-k -> sparse attention (dsa_forward_chunked).  Inputs are
seeded synthetic tensors, resident on the GPU before timing starts.  `value` is tokens/s of
the whole forward.  A second, instrumented pass calls the three entry points chunk by chunk
with events between launches on the launching stream, which gives each kernel's average
launch duration; from it come per-phase rates and the roofline fraction of the dominant
kernel (algorithmic bytes or flops per launch / measured duration / MI355X peak).  The CPU
oracle is timed on a bounded sample of rows of the same workload (cpu_baseline).

By default the line is the 128k forward (fwd_128k: value, config, roofline, cpu_baseline)
and, after the 128k tensors are freed, the same measurement of one GPU's share of the 1M-token
layer (tp_share_1m) as a nested object of the same line, so that both context lengths of the
metric come from one run.  --workload NAME measures that workload alone; --second NAME (or
"none") changes the nested one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--second NAME]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# The chunked forward selects through the fused indexer -> top-k path (dsa_index_topk) for
# chunks whose first row sees at least this many pools, when k allows it and the indexer has
# more than 16 heads; the same rule is applied here to time the select the way the driver
# runs it.
FUSED_MIN_VISIBLE = 49152
FUSED_MIN_HEADS = 17
FUSED_MAX_K = 2730

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
DEFAULT_WORKLOAD = "fwd_128k"
SECOND_WORKLOAD = "tp_share_1m"
# Timed steps of the nested 1M measurement are capped (one step is about 0.9 s) so that the
# default run stays within a few minutes.
SECOND_MAX_STEPS = 5
SECOND_MAX_WARMUP = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="measure this workload alone (default: %s, then %s nested)"
                         % (DEFAULT_WORKLOAD, SECOND_WORKLOAD))
    ap.add_argument("--second", default=None,
                    help="workload measured after the first and nested in the same line "
                         "(default %s with the default workload; 'none' to skip)"
                         % SECOND_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="first run one plain device copy of this many GiB (a known-size "
                         "kernel that calibrates the HBM byte counters of a profiler run)")
    return ap.parse_args()


# Sources of each kernel whose HBM traffic a committed profile records: the profile is
# used only while these files are unchanged.
KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd.hip", "attn_common.hpp", "common.hpp"],
    "indexer": ["indexer.hip", "common.hpp"],
    "topk": ["topk.hip", "common.hpp"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_context_sparse_index_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload, instance_suffix=None):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter profile
    (profiles/<kernel>_<workload>_traffic.md, a line 'traffic: {json}'), or None when there
    is none, the kernel's sources changed since it was taken, or the recorded kernel instance
    does not end in `instance_suffix` (e.g. the attention's output type parameter)."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
                if rec.get("source_hash") != kernel_source_hash(kernel):
                    return None
                if instance_suffix and not rec.get("kernel", "").endswith(instance_suffix):
                    return None
                return rec["bytes_per_launch"]
    return None


def chunk_ranges(n, chunk):
    return [(t0, min(chunk, n - t0)) for t0 in range(0, n, chunk)]


def visible_pairs(t0, nq, p):
    """sum over t in [t0, t0 + nq) of min(p, floor((t + 1) / 4)), exactly."""
    t = np.arange(t0, t0 + nq, dtype=np.int64)
    return int(np.minimum(p, (t + 1) // 4).sum())


def valid_slots(t0, nq, p, k):
    t = np.arange(t0, t0 + nq, dtype=np.int64)
    return int(np.minimum(k, np.minimum(p, (t + 1) // 4)).sum())


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_sparse_index_amd import binding as B
    from long_context_sparse_index_amd import workloads as W

    first = args.workload or DEFAULT_WORKLOAD
    second = args.second if args.second is not None else (
        SECOND_WORKLOAD if args.workload is None else "none")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load_library()
    if args.copy_probe_gib > 0:
        nb = int(args.copy_probe_gib * (1 << 30))
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads and writes exactly nb bytes
        torch.cuda.synchronize()
        print("bench: copy probe of %d bytes done" % nb, file=sys.stderr, flush=True)
        del src, dst
    line = measure(W.WORKLOADS[first], args.steps, args.warmup, args, dev)
    if second != "none":
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        sub = measure(W.WORKLOADS[second], min(args.steps, SECOND_MAX_STEPS),
                      min(args.warmup, SECOND_MAX_WARMUP), args, dev)
        line[second] = {key: sub[key] for key in (
            "metric", "value", "unit", "steps", "warmup", "ms_per_step", "dtype", "config",
            "roofline", "phases", "cpu_baseline")}
    print(json.dumps(line), flush=True)


def measure(wl, steps, warmup, args, dev):
    """One workload: whole-forward steps timed, then the instrumented passes; returns the
    fields of the JSON line."""
    import torch

    from long_context_sparse_index_amd import binding as B
    from long_context_sparse_index_amd import inputs as I

    n, p, k, chunk = wl.n_tokens, wl.n_pools, wl.topk, wl.chunk
    has_attn = wl.heads > 0
    print("bench: workload %s (N=%d, P=%d, chunk %d)" % (wl.name, n, p, chunk),
          file=sys.stderr, flush=True)

    q_i, k_i, w = I.index_inputs(wl, dev)
    ld = ((p + 3) // 4) * 4
    if has_attn:
        q, kv, _ = I.attn_inputs(wl, dev)
        o_dtype = torch.bfloat16 if wl.attn_out == "bf16" else torch.float32
        o = torch.empty((n, wl.heads, wl.d_v), dtype=o_dtype, device=dev)
        lse = torch.empty((n, wl.heads), dtype=torch.float32, device=dev)
        ws = torch.empty(B.forward_chunked_workspace_bytes(p, chunk, k), dtype=torch.uint8,
                         device=dev)
    scores = torch.empty((chunk, ld), dtype=torch.float32, device=dev)
    idx_chunk = torch.empty((chunk, k), dtype=torch.int32, device=dev)
    sel_ws = (torch.empty(B.index_topk_workspace_bytes(chunk, p, k), dtype=torch.uint8,
                          device=dev) if k <= FUSED_MAX_K else None)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    chunks = chunk_ranges(n, chunk)

    def uses_fused(t0):
        return (sel_ws is not None and wl.h_i >= FUSED_MIN_HEADS and
                min(p, (t0 + 1) // 4) >= FUSED_MIN_VISIBLE)

    def step_select(rec):
        """The select of every chunk as the chunked driver runs it (events per chunk when
        rec is a list)."""
        for t0, nq in chunks:
            if rec is not None:
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(stream)
            if uses_fused(t0):
                B.index_topk(q_i[t0:t0 + nq], k_i, w, idx_chunk[:nq], q_start=t0, n_pools=p,
                             ws=sel_ws)
            else:
                B.index_scores(q_i[t0:t0 + nq], k_i, w, scores[:nq], q_start=t0)
                B.topk(scores[:nq], idx_chunk[:nq], q_start=t0, n_pools=p)
            if rec is not None:
                e[1].record(stream)
                rec.append((uses_fused(t0), e))

    def step_driver():
        B.forward_chunked(q_i, k_i, w, q, kv, o, lse, k=k, chunk=chunk, scale=wl.scale,
                          d_v=wl.d_v, ws=ws)

    def step_phases(events):
        for t0, nq in chunks:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            B.index_scores(q_i[t0:t0 + nq], k_i, w, scores[:nq], q_start=t0)
            e[1].record(stream)
            B.topk(scores[:nq], idx_chunk[:nq], q_start=t0, n_pools=p)
            e[2].record(stream)
            if has_attn:
                B.sparse_attn_fwd(q[t0:t0 + nq], kv, idx_chunk[:nq], o[t0:t0 + nq],
                                  lse[t0:t0 + nq], scale=wl.scale, d_v=wl.d_v)
            e[3].record(stream)
            events.append((t0, nq, e))

    step = step_driver if has_attn else (lambda: step_select(None))

    # ---- timed region: whole forward steps
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / steps
    print("bench: %s %.3f ms/step (wall %.3f s for %d steps)" % (wl.name, ms_per_step, wall,
                                                                 steps),
          file=sys.stderr, flush=True)

    # ---- instrumented pass: per-kernel launch durations on the launching stream
    events = []
    for _ in range(steps):
        step_phases(events)
    torch.cuda.synchronize()
    ph_ms = {"indexer": 0.0, "topk": 0.0, "attn_fwd": 0.0}
    for _, _, e in events:
        ph_ms["indexer"] += e[0].elapsed_time(e[1])
        ph_ms["topk"] += e[1].elapsed_time(e[2])
        ph_ms["attn_fwd"] += e[2].elapsed_time(e[3])
    per_step = {kname: v / steps for kname, v in ph_ms.items()}
    n_launch = len(chunks)
    # ---- the select (indexer + top-k) per chunk as the driver runs it
    sel_rec = []
    for _ in range(steps):
        step_select(sel_rec)
    torch.cuda.synchronize()
    sel_fused = sum(e[0].elapsed_time(e[1]) for f, e in sel_rec if f) / steps
    sel_two = sum(e[0].elapsed_time(e[1]) for f, e in sel_rec if not f) / steps

    # algorithmic work of one step
    pairs = visible_pairs(0, n, p)
    idx_flop = 2.0 * wl.h_i * wl.d_i * pairs
    topk_bytes = 4.0 * pairs + 4.0 * n * k
    slots = valid_slots(0, n, p, k)
    row_bytes = 2 * wl.d_qk if has_attn else 0
    o_bytes = 2 if wl.attn_out == "bf16" else 4
    attn_bytes = (row_bytes * slots + n * wl.heads * wl.d_qk * 2 +
                  n * wl.heads * wl.d_v * o_bytes + n * k * 4) if has_attn else 0.0
    attn_flop = 2.0 * wl.heads * (wl.d_qk + wl.d_v) * slots if has_attn else 0.0
    idx_peak = PEAK_FP8_TFLOPS if wl.index_dtype == "fp8" else PEAK_BF16_TFLOPS

    def tflops(flop, ms):
        return flop / (ms * 1e-3) / 1e12 if ms > 0 else 0.0

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9 if ms > 0 else 0.0

    phases = {
        "indexer": {"ms_per_step": per_step["indexer"], "launches_per_step": n_launch,
                    "avg_launch_ms": per_step["indexer"] / n_launch,
                    "tflops": tflops(idx_flop, per_step["indexer"]),
                    "frac_of_mfma_peak": tflops(idx_flop, per_step["indexer"]) / idx_peak,
                    "visible_pairs_per_s": pairs / (per_step["indexer"] * 1e-3),
                    "tokens_per_s": n / (per_step["indexer"] * 1e-3)},
        "topk": {"ms_per_step": per_step["topk"], "avg_launch_ms": per_step["topk"] / n_launch,
                 "gbs": gbs(topk_bytes, per_step["topk"]),
                 "frac_of_hbm_peak": gbs(topk_bytes, per_step["topk"]) / PEAK_HBM_GBS,
                 "tokens_per_s": n / (per_step["topk"] * 1e-3)},
    }
    n_fused = sum(1 for t0, _ in chunks if uses_fused(t0))
    phases["select"] = {
        "ms_per_step": sel_fused + sel_two, "fused_chunks": n_fused, "chunks": n_launch,
        "fused_ms_per_step": sel_fused, "score_row_ms_per_step": sel_two,
        "tokens_per_s": n / ((sel_fused + sel_two) * 1e-3),
        "note": "indexer + top-k of every chunk as dsa_forward_chunked runs them: the fused "
                "select (dsa_index_topk) on chunks whose rows see >= %d pools when the "
                "indexer has >= %d heads, else dsa_index_scores + dsa_topk (the two phases "
                "above)" % (FUSED_MIN_VISIBLE, FUSED_MIN_HEADS)}
    if has_attn:
        phases["attn_fwd"] = {
            "ms_per_step": per_step["attn_fwd"], "avg_launch_ms": per_step["attn_fwd"] / n_launch,
            "gbs": gbs(attn_bytes, per_step["attn_fwd"]),
            "frac_of_hbm_peak": gbs(attn_bytes, per_step["attn_fwd"]) / PEAK_HBM_GBS,
            "tflops": tflops(attn_flop, per_step["attn_fwd"]),
            "frac_of_mfma_peak": tflops(attn_flop, per_step["attn_fwd"]) / PEAK_BF16_TFLOPS,
            "tokens_per_s": n / (per_step["attn_fwd"] * 1e-3)}

    # roofline of the dominant kernel (largest share of the step)
    dom = max(per_step, key=lambda x: per_step[x])
    if dom == "indexer":
        ach = tflops(idx_flop / n_launch, per_step["indexer"] / n_launch)
        roof = {"kernel": "indexer", "bound": "mfma", "achieved": ach, "peak": idx_peak,
                "unit": "TFLOP/s", "frac": ach / idx_peak,
                "traffic": recorded_traffic("indexer", wl.name)}
    elif dom == "topk":
        ach = gbs(topk_bytes / n_launch, per_step["topk"] / n_launch)
        roof = {"kernel": "topk", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": recorded_traffic("topk", wl.name)}
    else:
        ach = gbs(attn_bytes / n_launch, per_step["attn_fwd"] / n_launch)
        roof = {"kernel": "attn_fwd", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": recorded_traffic(
                    "attn_fwd", wl.name, ", true>" if wl.attn_out == "fp32" else ", false>")}

    if has_attn:
        phases["pool_keys"] = time_pool_keys(wl, dev, stream)

    if has_attn and "attn_bwd" in wl.phases:
        idx_b = idx_for_bwd(wl, q_i, k_i, w, dev)
        phases["attn_bwd"] = time_backward(wl, q, kv, o, lse, idx_b, steps, stream)
        phases["attn_bwd_deterministic"] = time_backward(wl, q, kv, o, lse, idx_b, steps,
                                                         stream, deterministic=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, q_i, k_i, w, q if has_attn else None, kv if has_attn else None,
                           args.cpu_seconds)

    # free this workload's device memory before the next one is generated
    del q_i, k_i, w, scores, idx_chunk, sel_ws
    if has_attn:
        del q, kv, o, lse, ws
    value = n / (ms_per_step * 1e-3)
    line = {
        "metric": ("DSA forward tokens/s (indexer + top-k + sparse attention, chunked)"
                   if has_attn else "DSA select tokens/s (indexer + top-k, chunked)"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # MFMA operand type of the path: bf16 (attention, bf16 indexer) or fp8 e4m3 (indexer
        # of an indexer-only workload); top-k is integer work on the fp32 scores.
        "dtype": "fp8" if (wl.index_dtype == "fp8" and not has_attn) else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_tokens": n, "n_pools": p, "h_i": wl.h_i,
                   "d_i": wl.d_i, "index_dtype": wl.index_dtype, "topk": k,
                   "heads": wl.heads, "d_qk": wl.d_qk, "d_v": wl.d_v, "chunk": chunk,
                   "attn_out": wl.attn_out},
        "roofline": roof,
        "phases": phases,
        "cpu_baseline": cpu,
    }
    return line


def time_pool_keys(wl, dev, stream, reps=20):
    """dsa_pool_keys on token-level latent rows of the workload ([N, d_qk] bf16 and N gate
    scores -> [N / 4, d_qk]), the step upstream of the chunked forward that forms its pooled
    keys (the forward's inputs are pooled already, so this is timed on its own)."""
    import torch

    from long_context_sparse_index_amd import binding as B
    from long_context_sparse_index_amd import inputs as I

    n, d = wl.n_tokens, wl.d_qk
    x = I.normal_bf16((n, d), 0, "kv", dev)
    gate = I.normal_bf16((n,), 0, "d_o", dev).float().contiguous()
    out = torch.empty((n // 4, d), dtype=torch.bfloat16, device=dev)
    B.pool_keys(x, gate, out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        B.pool_keys(x, gate, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = n * d * 2 + n * 4 + (n // 4) * d * 2
    del x, gate, out
    return {"ms_per_call": ms, "bytes_per_call": nbytes,
            "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "note": "dsa_pool_keys of %d token rows of %d bf16 columns (not part of the step: "
                    "the forward's key tables are pooled already), %d calls" % (n, d, reps)}


def idx_for_bwd(wl, q_i, k_i, w, dev):
    """Selections of every query (one chunked forward pass keeping its indices)."""
    import torch

    from long_context_sparse_index_amd import binding as B

    n, p, k, chunk = wl.n_tokens, wl.n_pools, wl.topk, wl.chunk
    ld = ((p + 3) // 4) * 4
    idx = torch.empty((n, k), dtype=torch.int32, device=dev)
    scores = torch.empty((chunk, ld), dtype=torch.float32, device=dev)
    for t0, nq in chunk_ranges(n, chunk):
        B.index_scores(q_i[t0:t0 + nq], k_i, w, scores[:nq], q_start=t0)
        B.topk(scores[:nq], idx[t0:t0 + nq], q_start=t0, n_pools=p)
    torch.cuda.synchronize()
    return idx


def time_backward(wl, q, kv, o, lse, idx, steps, stream, deterministic=False):
    """Times dsa_sparse_attn_bwd over the whole sequence (dQ, and dK / dV by fp32 atomics;
    or dsa_sparse_attn_bwd_deterministic, staged dK / dV rows summed per pool in a fixed
    order) on the forward's outputs;
    flops count the recomputed logits, dP, dV, dQ and dK."""
    import torch

    from long_context_sparse_index_amd import binding as B
    from long_context_sparse_index_amd import inputs as I

    n, p = wl.n_tokens, wl.n_pools
    B.sparse_attn_fwd(q, kv, idx, o, lse, scale=wl.scale, d_v=wl.d_v)
    d_o = I.grad_output(wl, q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dkv = torch.zeros((p, wl.d_qk), dtype=torch.float32, device=q.device)
    if deterministic:
        ws = torch.empty(B.sparse_attn_bwd_deterministic_workspace_bytes(
            n, wl.heads, p, wl.topk, wl.d_qk, wl.d_v, False), dtype=torch.uint8,
            device=q.device)
    else:
        ws = torch.empty(B.sparse_attn_bwd_workspace_bytes(n, wl.heads), dtype=torch.uint8,
                         device=q.device)
    bwd = B.sparse_attn_bwd_deterministic if deterministic else B.sparse_attn_bwd

    def run():
        # V is the first d_v columns of the latent row: its gradient folds into dKV
        dkv.zero_()
        bwd(q, kv, idx, o, lse, d_o, dq, dkv, scale=wl.scale, d_v=wl.d_v, ws=ws)

    run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    slots = valid_slots(0, n, p, wl.topk)
    flop = 2.0 * wl.heads * (3 * wl.d_qk + 2 * wl.d_v) * slots
    return {"ms_per_step": ms, "tflops": flop / (ms * 1e-3) / 1e12,
            "frac_of_mfma_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "tokens_per_s": n / (ms * 1e-3),
            "note": "%s over all rows (dQ, dKV with dV folded in), timed with the zeroing of "
                    "dKV, %d launches" % ("dsa_sparse_attn_bwd_deterministic (no atomics)"
                                          if deterministic else
                                          "dsa_sparse_attn_bwd (fp32 atomics)", steps)}


def cpu_baseline(wl, q_i, k_i, w, q, kv, budget_s):
    """The CPU oracle, as it stands, on uniformly sampled rows of the same workload; its
    tokens/s is rows / seconds (a uniform sample has the workload's mean cost per row)."""
    import torch

    import oracle
    from long_context_sparse_index_amd import inputs as I

    # Every core this process may run on, unless the host assigns a smaller CPU share through
    # OMP_NUM_THREADS (a GPU machine sets it to its per-GPU share): the thread count used is
    # reported as `cores`, next to the host's core count.
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (
        os.cpu_count() or 1)
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(share, usable) if share > 0 else usable
    rng = np.random.default_rng(1234)
    k_bits = I.index_bits(k_i)
    kv_bits = I.bits_u16(kv) if kv is not None else None
    w_h = w.cpu().numpy()

    def run(nrows):
        rows = np.sort(rng.choice(wl.n_tokens, size=nrows, replace=False)).astype(np.int64)
        ridx = torch.from_numpy(rows).to(q_i.device)
        q_rows = I.index_bits(q_i[ridx])
        q_att = I.bits_u16(q[ridx]) if q is not None else None
        t0 = time.perf_counter()
        sc = oracle.index_scores(q_rows, k_bits, w_h, rows, wl.n_pools, threads=threads)
        sel = oracle.topk(sc, rows, wl.n_pools, wl.topk, threads=threads)
        if q is not None:
            oracle.sparse_attn_fwd(q_att, kv_bits, sel, wl.scale, d_v=wl.d_v, threads=threads)
        return time.perf_counter() - t0

    nrows = 2 * threads
    dt = run(nrows)
    target = max(1, min(wl.n_tokens, int(nrows * budget_s / max(dt, 1e-3))))
    if target > nrows:
        nrows = target
        dt = run(nrows)
    # the same oracle on one host thread, on a smaller sample (about a tenth of the budget)
    all_threads = threads
    threads = 1
    n1 = max(1, min(wl.n_tokens, int(0.1 * budget_s * (nrows / max(dt, 1e-3)) / all_threads)))
    dt1 = run(n1)
    return {"value": nrows / dt, "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "host_cores": os.cpu_count(), "usable_cores": usable,
            "threads_from": "OMP_NUM_THREADS" if share > 0 else "affinity",
            "sample": "%d uniformly sampled query rows of %s (seed 1234), all phases of the "
                      "forward, %.1f s; tokens/s = rows / s (a uniform sample has the "
                      "workload's mean cost per row)" % (nrows, wl.name, dt),
            "one_core": {"value": n1 / dt1, "unit": "tokens/s", "cores": 1,
                         "sample": "%d sampled rows, %.1f s" % (n1, dt1)}}


if __name__ == "__main__":
    main()
