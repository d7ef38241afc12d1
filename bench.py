#!/usr/bin/env python3
"""Benchmark of the paged-KV attention forward on one MI355X.

A step is one forward pass of the whole path (main attention kernel plus the
split merge) over one batch of the named synthetic workload, with the plan
already uploaded and every input resident in HBM.  Default workload: the bf16
paged GQA decode batch (32 sequences, one query each, Hq=32, Hkv=8, D=128,
page 16, contexts uniform in [512, 8192], up to 16 splits).

Prints ONE JSON line.  `value` is algorithmic K/V bytes per second (visible
keys only, each K and V row once per (query, KV head)); `roofline` rates the
dominant kernel from HIP timing events that its launch records at the
kernel's own start and end (hipExtLaunchKernel, on the launch stream);
`cpu_baseline` times the fp64 oracle on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "decode KV GB/s (% HBM peak); chunked-prefill TFLOP/s (% bf16 MFMA peak)"


def visible_counts(b):
    """Keys each query sees: t < L, t <= p if causal, t > p - W if windowed."""
    counts = np.zeros(b.num_queries, dtype=np.int64)
    for s in range(b.num_seqs):
        L = int(b.seq_lens[s])
        for i in range(int(b.cu_q[s]), int(b.cu_q[s + 1])):
            p = int(b.q_pos[i])
            hi = p if b.causal else L - 1
            lo = max(0, p - b.window + 1) if b.window > 0 else 0
            counts[i] = hi - lo + 1
    return counts


def algorithmic_work(b, mla=False):
    """(K/V bytes, flops) of the method: bytes count each visible (query, key)
    pair's K and V rows once per KV head (the traffic of decode-style
    queries); flops are 2 (D + Dv) per visible (query row, key) pair."""
    vis = visible_counts(b)
    if mla:
        es = 2
        bytes_ = int(vis.sum()) * (b.r + b.p) * es
        flops = int(vis.sum()) * b.heads * (2 * (b.r + b.p) + 2 * b.r)
        return bytes_, flops
    es = 4 if b.dtype == "f32" else 2
    bytes_ = int(vis.sum()) * b.hkv * (b.d + b.dv) * es
    flops = int(vis.sum()) * b.hq * 2 * (b.d + b.dv)
    return bytes_, flops


def _source_hash():
    """Hash of the sources the forward kernels and their planner are built
    from (the translation units of the backward, the append, the block-sparse
    selection and the no-allocation entry point are left out: no forward
    launch of the benchmark runs their code)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_attention_gqa_amd", "csrc")
    for n in sorted(os.listdir(csrc)):
        if n in ("pa_backward.hip", "pa_append.hip", "pa_sparse.hip", "pa_noalloc.hip"):
            continue
        with open(os.path.join(csrc, n), "rb") as f:
            h.update(n.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """Measured HBM bytes per launch from a committed counter summary, only if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except Exception:
        return None
    rec = data.get(kernel_key)
    if not rec or rec.get("source_hash") != _source_hash():
        return None
    return rec.get("bytes_per_launch")


CPU_BASELINE_SECONDS = 10.0


def cpu_baseline(b, mla, work, hbm):
    """The fp64 oracle on the host cores, over the whole workload (decode)
    or over a bounded sample of query rows (prefill), in the GPU's unit.
    Passes repeat until about `CPU_BASELINE_SECONDS` of work have run (at
    least one pass); the rate is the mean over them."""
    import oracle
    n = oracle.default_threads()
    rows = None
    frac = 1.0
    if not hbm:
        total = b.num_queries * b.hq
        rows = np.random.default_rng(0).choice(total, size=min(total, 8192), replace=False)
        frac = len(rows) / total
    passes, t0 = 0, time.perf_counter()
    while True:
        if mla:
            oracle.mla(b, rows=rows, nthreads=n)
        else:
            oracle.attention(b, rows=rows, nthreads=n)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= CPU_BASELINE_SECONDS:
            break
    scaled = work * frac * passes / dt
    if hbm:
        return {"value": round(scaled / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
                "sample": f"the full workload, {passes} passes ({dt:.2f} s)"}
    return {"value": round(scaled / 1e12, 6), "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": f"{len(rows)} random (query, head) rows of the workload, {passes} passes ({dt:.2f} s), "
                      "flops scaled by the sampled fraction"}


def _is_mla(b):
    return hasattr(b, "latent")


def split_work(b):
    """Algorithmic work split by role: (decode K/V bytes, prefill flops), where
    decode queries are sequences with at most 4 queries."""
    vis = visible_counts(b)
    counts = np.diff(b.cu_q)
    es = 4 if b.dtype == "f32" else 2
    mla = _is_mla(b)
    dec_b, pre_f = 0, 0
    for s in range(b.num_seqs):
        v = int(vis[b.cu_q[s]:b.cu_q[s + 1]].sum())
        if counts[s] <= 4:
            dec_b += v * ((b.r + b.p) * es if mla else b.hkv * (b.d + b.dv) * es)
        else:
            pre_f += v * (b.heads * (2 * (b.r + b.p) + 2 * b.r) if mla else b.hq * 2 * (b.d + b.dv))
    return dec_b, pre_f


def measure(name, steps, warmup, split_tokens=0):
    """Time `steps` forward passes of workload `name` (after `warmup`) with HIP
    events around the main kernel and the wall clock around the whole loop."""
    import torch
    from synth import CONFIGS
    from tests.gpu_harness import GqaRun, MlaRun

    b = CONFIGS[name]()
    mla = _is_mla(b)
    run_ = MlaRun(b, split_tokens=split_tokens, with_lse=False) if mla else \
        GqaRun(b, split_tokens=split_tokens, with_lse=False)

    # Rotate between pool copies so consecutive steps do not re-read a
    # cache-resident pool: the copies together exceed the 256 MB MALL twice over.
    pool_bytes = (run_.latent.numel() + run_.kpos.numel()) * 2 if mla else \
        (run_.k.numel() + run_.v.numel()) * run_.k.element_size()
    copies = max(1, min(4, math.ceil(512e6 / max(pool_bytes, 1)) + 1))
    pools = [(run_.latent, run_.kpos) if mla else (run_.k, run_.v)]
    for _ in range(copies - 1):
        pools.append(tuple(t.clone() for t in pools[0]))

    def step(j, events=None):
        x, y = pools[j % len(pools)]
        if mla:
            run_.latent, run_.kpos = x, y
        else:
            run_.k, run_.v = x, y
        run_(main_events=events)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # The step loop as a caller runs it: back-to-back forward calls, the wall
    # clock (and one event pair) around all of them.
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    t_start.record(stream)
    for j in range(steps):
        step(j)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = t_start.elapsed_time(t_end)

    # The same loop again with timing events handed to the main kernel's
    # launch (hipExtLaunchKernel): each pair holds that kernel's own start and
    # end, as a kernel trace would, with nothing between the kernels.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for e in starts + ends:  # torch creates the HIP event on first record; the launch records it again
        e.record(stream)
    torch.cuda.synchronize()
    for j in range(steps):
        step(j, (starts[j], ends[j]))
    torch.cuda.synchronize()
    mains = [x.elapsed_time(y) for x, y in zip(starts, ends)]

    # Plan creation (validation, host planning and the one upload of tables
    # and work items), timed apart from the steps it serves.
    import paged_kv_attention_gqa_amd as pa
    from tests.gpu_harness import make_plan
    plan_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t = time.perf_counter()
        p = make_plan(b, mla=mla, split_tokens=split_tokens)
        torch.cuda.synchronize()
        plan_ms.append((time.perf_counter() - t) * 1e3)
        pa.pa_plan_destroy(p)
    ms_per_step = max(wall * 1e3, gpu_ms) / steps
    res = {
        "b": b, "mla": mla, "info": run_.info, "copies": len(pools),
        "ms_per_step": ms_per_step,
        "main_ms": min(float(np.mean(mains)), ms_per_step),
        "main_ms_median": float(np.median(mains)),
        "main_ms_min": float(np.min(mains)),
        "plan_ms": float(np.median(plan_ms)),
    }
    del pools, run_
    torch.cuda.empty_cache()
    return res


def summarize(name, r):
    """Per-workload rates against the roofline of what bounds it."""
    b = r["b"]
    kv_bytes, flops = algorithmic_work(b, r["mla"])
    main_s = r["main_ms"] * 1e-3
    step_s = r["ms_per_step"] * 1e-3
    out = {"workload": name, "ms_per_step": round(r["ms_per_step"], 5), "main_kernel_ms": round(r["main_ms"], 5),
           "main_kernel_ms_median": round(r["main_ms_median"], 5), "main_kernel_ms_min": round(r["main_ms_min"], 5),
           "merge_and_gaps_ms": round(r["ms_per_step"] - r["main_ms"], 5), "plan_ms": round(r["plan_ms"], 3),
           "queries_per_s": round(b.num_queries / step_s, 1), "kv_bytes": kv_bytes, "flops": flops}
    traffic = _traffic(f"{name}:main")
    if r["info"]["prefill_items"] == 0:
        out.update(bound="hbm", step_gbs=round(kv_bytes / step_s / 1e9, 2), step_frac=round(
            kv_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4), step_tflops=round(flops / step_s / 1e12, 3))
        out["roofline"] = {"bound": "hbm", "achieved": round(kv_bytes / main_s / 1e9, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(kv_bytes / main_s / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": traffic}
    elif r["info"]["decode_items"] == 0:
        out.update(bound="mfma", step_tflops=round(flops / step_s / 1e12, 2),
                   step_frac=round(flops / step_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4))
        out["roofline"] = {"bound": "mfma", "achieved": round(flops / main_s / 1e12, 2),
                           "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(flops / main_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        # one launch, two bounds: the kernel time against the larger of the
        # decode part's HBM time and the prefill part's MFMA time
        dec_b, pre_f = split_work(b)
        t_bw, t_mf = dec_b / (HBM_PEAK_GBS * 1e9), pre_f / (BF16_MFMA_PEAK_TFLOPS * 1e12)
        out.update(bound="hbm+mfma", decode_kv_bytes=dec_b, prefill_flops=pre_f,
                   decode_gbs_in_kernel=round(dec_b / main_s / 1e9, 2),
                   prefill_tflops_in_kernel=round(pre_f / main_s / 1e12, 2),
                   frac_sum=round((t_bw + t_mf) / main_s, 4))
        out["roofline"] = {"bound": "hbm+mfma", "achieved_ms": round(r["main_ms"], 5),
                           "bound_ms": round(max(t_bw, t_mf) * 1e3, 5), "peak": [HBM_PEAK_GBS, BF16_MFMA_PEAK_TFLOPS],
                           "unit": ["GB/s", "TFLOP/s"], "frac": round(max(t_bw, t_mf) / main_s, 4),
                           "traffic": traffic}
    return out


def measure_append(name, steps, warmup):
    """Paged K/V append of one new K and V row per (query, KV head) of
    workload `name` into its pools (the cache write before attention), timed
    with HIP events around `steps` back-to-back calls.  Bytes: each new row
    read once and written once."""
    import torch
    import paged_kv_attention_gqa_amd as pa
    from synth import CONFIGS
    from tests.gpu_harness import GqaRun

    b = CONFIGS[name]()
    run_ = GqaRun(b, with_lse=False)
    rng = np.random.default_rng(0)
    k_new = torch.from_numpy(rng.standard_normal((b.num_queries, b.hkv, b.d), dtype=np.float32)).to(
        "cuda", dtype=torch.bfloat16)
    v_new = torch.from_numpy(rng.standard_normal((b.num_queries, b.hkv, b.dv), dtype=np.float32)).to(
        "cuda", dtype=torch.bfloat16)
    for _ in range(warmup):
        pa.pa_append_kv(run_.plan, k_new, v_new, run_.k, run_.v)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # one call as a caller makes it (the host's ~10 us per call included) ...
    t0 = time.perf_counter()
    for _ in range(steps):
        pa.pa_append_kv(run_.plan, k_new, v_new, run_.k, run_.v)
    torch.cuda.synchronize()
    call_ms = (time.perf_counter() - t0) * 1e3 / steps
    # ... and the kernels back to back: the GPU first sleeps while the host
    # queues every call, so the events bracket device time only
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6 + steps * 5e4))
    e0.record(stream)
    for _ in range(steps):
        pa.pa_append_kv(run_.plan, k_new, v_new, run_.k, run_.v)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 2 * (k_new.numel() + v_new.numel()) * 2
    del run_
    torch.cuda.empty_cache()
    return {"workload": f"append:{name}", "ms_per_call": round(call_ms, 5), "kernel_ms": round(ms, 5),
            "bytes": nbytes, "bound": "hbm", "kernel_gbs": round(nbytes / (ms * 1e-3) / 1e9, 2),
            "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def measure_backward(name, steps, warmup):
    """Paged GQA backward of workload `name` (pa_attention_bwd: zero the
    gradient pools, D = dO . O, dQ, dK/dV) after one forward call, timed with
    HIP events around `steps` back-to-back calls.  Algorithmic flops per
    visible (query row, key) pair: 2 (3 D + 2 Dv) (scores, dP, dQ, dK, dV)."""
    import torch
    import paged_kv_attention_gqa_amd as pa
    from synth import CONFIGS
    from tests.gpu_harness import GqaRun

    b = CONFIGS[name]()
    f = GqaRun(b)
    f()
    rng = np.random.default_rng(1)
    dout = torch.from_numpy(rng.standard_normal((b.num_queries, b.hq, b.dv), dtype=np.float32)).to(
        "cuda", dtype=torch.bfloat16)
    dq = torch.empty_like(f.q)
    dk, dv = torch.empty_like(f.k), torch.empty_like(f.v)
    n = pa.pa_plan_bwd_workspace_bytes(f.plan, b.dtype, b.d, b.dv)
    ws = torch.empty(n // 4 + 64, dtype=torch.float32, device="cuda")

    def call():
        pa.pa_attention_bwd(f.plan, f.q, f.k, f.v, f.out, f.lse, dout, dq, dk, dv, scale=b.scale, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6 + steps * 5e4))
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = int(visible_counts(b).sum()) * b.hq
    flops = pairs * 2 * (3 * b.d + 2 * b.dv)
    info = pa.pa_plan_get_info(f.plan)
    del f, dq, dk, dv, ws
    torch.cuda.empty_cache()
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"backward:{name}", "kernel_ms": round(ms, 5), "flops": flops, "bound": "mfma",
            "tflops": round(tf, 2), "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "items": {"dq": info["bwd_dq_items"], "dkv": info["bwd_kv_items"]}}


def measure_mla_backward(name, steps, warmup):
    """Absorbed-MLA backward of workload `name` (pa_mla_bwd) after one
    forward call, timed with HIP events around `steps` back-to-back calls.
    Algorithmic flops per visible (query row, key) pair: 2 (R + P) scores,
    2 R dP, 2 (R + P) dq, 2 R + 2 R for the latent's key and value terms and
    2 P for the rotary cache: 10 R + 6 P."""
    import torch
    import paged_kv_attention_gqa_amd as pa
    from synth import CONFIGS
    from tests.gpu_harness import MlaRun

    m = CONFIGS[name]()
    f = MlaRun(m)
    f()
    rng = np.random.default_rng(1)
    dout = torch.from_numpy(rng.standard_normal((m.num_queries, m.heads, m.r), dtype=np.float32)).to(
        "cuda", dtype=torch.bfloat16)
    dqa, dqr = torch.empty_like(f.q_abs), torch.empty_like(f.q_rope)
    dlat, dkp = torch.empty_like(f.latent), torch.empty_like(f.kpos)
    n = pa.pa_plan_bwd_workspace_bytes(f.plan, m.dtype, m.r, m.p)
    ws = torch.empty(n // 4 + 64, dtype=torch.float32, device="cuda")

    def call():
        pa.pa_mla_bwd(f.plan, f.q_abs, f.q_rope, f.latent, f.kpos, f.out, f.lse, dout, dqa, dqr, dlat, dkp,
                      scale=m.scale, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6 + steps * 5e4))
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = int(visible_counts(m).sum()) * m.heads
    flops = pairs * (10 * m.r + 6 * m.p)
    del f, dqa, dqr, dlat, dkp, ws
    torch.cuda.empty_cache()
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"mla_backward:{name}", "kernel_ms": round(ms, 5), "flops": flops, "bound": "mfma",
            "tflops": round(tf, 2), "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}


def measure_sparse(name, steps, warmup, block_size=64, topk=16):
    """Block-sparse top-k attention of workload `name` (pa_sparse_attention_fwd:
    selection, block attention, merge), timed with HIP events around `steps`
    back-to-back calls.  Bytes: the proxy pass reads every visible K row once
    per (query, KV head), the attention reads the K and V rows of the kept
    blocks."""
    import torch
    import paged_kv_attention_gqa_amd as pa
    from synth import CONFIGS
    from tests.gpu_harness import GqaRun

    b = CONFIGS[name]()
    f = GqaRun(b, with_lse=False)
    nbytes, width = pa.pa_sparse_workspace_bytes(f.plan, b.dv, block_size, topk)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device="cuda")
    sel = torch.empty((b.num_queries, b.hkv, width), dtype=torch.int32, device="cuda")

    def call():
        pa.pa_sparse_attention_fwd(f.plan, f.q, f.k, f.v, f.out, None, scale=b.scale, block_size=block_size,
                                   topk=topk, selection=sel, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e6 + steps * 5e4))
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    es = 2 if b.dtype != "f32" else 4
    vis = visible_counts(b)
    proxy_bytes = int(vis.sum()) * b.hkv * b.d * es
    s = sel.cpu().numpy()
    kept_keys = 0
    for si in range(b.num_seqs):
        for i in range(int(b.cu_q[si]), int(b.cu_q[si + 1])):
            hi = int(b.q_pos[i]) if b.causal else int(b.seq_lens[si]) - 1
            lo = max(0, int(b.q_pos[i]) - b.window + 1) if b.window > 0 else 0
            for h in range(b.hkv):
                for r in s[i, h]:
                    if r >= 0:
                        kept_keys += min(hi + 1, (int(r) + 1) * block_size) - max(lo, int(r) * block_size)
    attn_bytes = kept_keys * (b.d + b.dv) * es
    total = proxy_bytes + attn_bytes
    del f, ws, sel
    torch.cuda.empty_cache()
    gbs = total / (ms * 1e-3) / 1e9
    return {"workload": f"sparse_top{topk}_of_{block_size}:{name}", "ms_per_call": round(ms, 5),
            "bytes": total, "proxy_bytes": proxy_bytes, "kept_kv_bytes": attn_bytes, "bound": "hbm",
            "gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4)}


PRIMARY = "bf16_decode_batch"
SECONDARY = ("bf16_chunked_prefill", "bf16_mixed_batch", "bf16_mla_decode", "bf16_mla_decode_h128",
             "bf16_mla_chunked_prefill", "bf16_chunked_prefill_d192", "bf16_chunked_prefill_d256")
APPEND = ("bf16_decode_batch", "bf16_chunked_prefill")  # cache writes of one decode step and of one chunk
BACKWARD = ("bf16_chunked_prefill",)  # gradients of one chunk step
MLA_BACKWARD = ("bf16_mla_chunked_prefill",)
SPARSE = ("bf16_decode_batch",)  # top-16 of 64-key blocks per decode row


def run(args):
    import torch
    import paged_kv_attention_gqa_amd as pa

    pa.load_library()  # fails loudly if the HIP library is missing
    torch.cuda.set_device(0)
    name = args.workload
    r = measure(name, args.steps, args.warmup, args.split_tokens)
    b = r["b"]
    mla = r["mla"]
    bytes_alg, flops_alg = algorithmic_work(b, mla)
    summ = summarize(name, r)
    hbm = summ["bound"] != "mfma"
    if hbm:
        value, vunit = bytes_alg / (r["ms_per_step"] * 1e-3) / 1e9, "GB/s"
    else:
        value, vunit = flops_alg / (r["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": vunit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": name, "seed": b.seed, "sequences": b.num_seqs,
                   "queries": b.num_queries, "page_size": b.page_size, "max_splits": b.max_splits,
                   **({"heads": b.heads, "rank": b.r, "rope_dim": b.p} if mla else
                      {"hq": b.hq, "hkv": b.hkv, "head_dim": b.d}),
                   "causal": b.causal, "window": b.window, "kv_bytes": bytes_alg, "flops": flops_alg,
                   "pool_copies_rotated": r["copies"]},
        "roofline": summ["roofline"],
        "kernels": {"main_ms": round(r["main_ms"], 5), "main_ms_median": round(r["main_ms_median"], 5),
                    "main_ms_min": round(r["main_ms_min"], 5),
                    "merge_and_gaps_ms": round(r["ms_per_step"] - r["main_ms"], 5),
                    "plan_create_ms": round(r["plan_ms"], 3),
                    "queries_per_s": round(r["b"].num_queries / (r["ms_per_step"] * 1e-3), 1), "plan": r["info"]},
    }
    if not args.no_secondary and name == PRIMARY:
        result["secondary"] = []
        for n in SECONDARY:
            try:
                result["secondary"].append(summarize(n, measure(n, args.steps, args.warmup)))
            except pa.PaError as e:  # a workload this build cannot run is reported, not hidden
                result["secondary"].append({"workload": n, "error": str(e)})
        for n in APPEND:
            result["secondary"].append(measure_append(n, args.steps, args.warmup))
        for n in BACKWARD:
            result["secondary"].append(measure_backward(n, args.steps, args.warmup))
        for n in MLA_BACKWARD:
            result["secondary"].append(measure_mla_backward(n, args.steps, args.warmup))
        for n in SPARSE:
            result["secondary"].append(measure_sparse(n, args.steps, args.warmup))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(b, mla, bytes_alg if hbm else flops_alg, hbm)
    return result


def copy_calibration(nbytes, reps):
    """A plain device-to-device copy of `nbytes` (torch's copy kernel), for
    scaling the HBM traffic counters: each launch must read and write exactly
    nbytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "ms": round(dt * 1e3, 4),
                      "gbs_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_decode_batch")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the backward of --workload (one JSON line; as --part backward)")
    ap.add_argument("--part", choices=("backward", "mla-backward", "sparse", "append"),
                    help="only run one of the secondary measurements on --workload (one JSON line)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return
    if args.backward_only:
        args.part = "backward"
    if args.part:
        import torch
        import paged_kv_attention_gqa_amd as pa
        pa.load_library()
        torch.cuda.set_device(0)
        fn = {"backward": measure_backward, "mla-backward": measure_mla_backward, "sparse": measure_sparse,
              "append": measure_append}[args.part]
        print(json.dumps(fn(args.workload, args.steps, args.warmup)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(run(args)), flush=True)


if __name__ == "__main__":
    main()
