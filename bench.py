"""Throughput of the DSA hot path (lightning indexer -> top-2048 -> sparse MLA) on one MI355X.

Default: one step = one pass of the whole path over the L = 32768 causal prefill batch (the
headline workload): dsa_indexer_logits, dsa_topk and dsa_sparse_mla_fwd back to back on one
stream, with HIP events between the stages so every kernel's duration comes from the timed steps
themselves.  The fused entry point (dsa_prefill_paged, the same kernels behind one call) is timed
beside it.  Inputs are generated on the host from the seeded recipe, copied to HBM before timing,
and stay resident; nothing is generated, quantized or copied inside the timed region.  Prints
one JSON line.

``--workload`` selects another configuration (tiny, prefill_4k, chunked_131k, decode_64; decode
times the fused paged decode call against its HBM roofline; quantize_append_32k times the FP8
quantization of the L = 32K queries and the paged append of its tokens; indexer_ue8m0_32k the
indexer with power-of-two scales inside the MFMA; indexer_train_4k / indexer_train_32k one
training step of the indexer: scores, KL loss toward the main attention, backward;
indexer_train_sparse_4k / _32k the sparse-stage step: scores, top-k, sparse attention, the loss over
the selected entries, backward), and
``--all-configs`` prints one line per configuration.  ``--gpus`` above 1 is rejected: the library runs on one GPU (no multi-GPU path).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense bf16 / fp16 MFMA, MI355X published
PEAK_FP8 = 5.0e15       # dense fp8 MFMA
PEAK_HBM = 8.0e12       # HBM3E bytes/s
PMC_FILE = os.path.join(ROOT, "profiles", "sparse_mla_prefill_32k_pmc.json")
MLA_SOURCE = os.path.join(ROOT, "dsa_lightning_indexer_02_amd", "csrc", "sparse_mla.hip")
HEADLINE = "prefill_32k"
METRIC = "query tokens/s (indexer+top-2048+sparse MLA) at L=32K"


def copy_calibration(dev):
    """One 1 GiB device-to-device copy: the reference a counter run scales FETCH_SIZE/WRITE_SIZE by."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def work_model(wl, n=None):
    """Algorithmic work of one pass (masked pairs and skipped dense work excluded).  ``n``: the
    visible key count of every query row (default: the prefill causal counts)."""
    if n is None:
        t = np.arange(wl.T, dtype=np.int64)
        n = np.minimum(wl.S, wl.q_start + t + 1)
    n = np.asarray(n, dtype=np.int64)
    sel = np.minimum(n, wl.topk)
    T = len(n)
    return {
        "indexer_flop": float(2 * wl.H_I * wl.D_I * n.sum()),
        "indexer_bytes": float(n.sum() * (wl.D_I + 4) + T * wl.H_I * (wl.D_I + 8) + 4 * n.sum()),
        "topk_bytes": float(4 * n.sum() + 4 * T * wl.topk),
        "mla_flop": float(2 * wl.H * (wl.D_qk + wl.D_v) * sel.sum()),
        "mla_bytes": float(sel.sum() * wl.D_qk * 2 + T * wl.H * (wl.D_qk + wl.D_v) * 2 + T * wl.topk * 4),
        "visible_pairs": int(n.sum()),
        "selected_rows": int(sel.sum()),
    }


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per sparse-MLA launch at L = 32K from the committed rocprofv3 counter runs, if
    they were taken on the current kernel source; None otherwise."""
    if not os.path.exists(PMC_FILE):
        return None
    with open(PMC_FILE) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != source_hash(MLA_SOURCE):
        return None
    return d.get("hbm_bytes_per_launch")


def percentiles(ms):
    ms = np.asarray(ms, dtype=np.float64)
    return {"p10": float(np.percentile(ms, 10)), "p50": float(np.percentile(ms, 50)),
            "p90": float(np.percentile(ms, 90))}


def host_cpu():
    """The host cores the oracle may use (this process's CPU affinity), nproc and the CPU model."""
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"threads": max(1, threads), "nproc": os.cpu_count(), "model": model}


def cpu_baseline(wl, n_rows: int, threads: int):
    """The oracle (as it stands) on a uniform sample of query rows, scaled to the whole workload by the
    exact per-stage work model (all rows when n_rows >= T)."""
    import oracle
    from dsa_inputs import prefill_inputs
    rows = np.unique(np.linspace(0, wl.T - 1, min(n_rows, wl.T)).round().astype(np.int64))
    inp = prefill_inputs(wl, rows=rows)
    pos = inp.pos
    n = np.minimum(wl.S, pos + 1)
    t0 = time.perf_counter()
    lg = oracle.indexer(inp.q8, inp.qs, inp.w, pos, inp.k8, inp.ks, nthreads=threads)
    t1 = time.perf_counter()
    ix = oracle.topk(lg, pos, wl.topk, nthreads=threads)
    t2 = time.perf_counter()
    oracle.sparse_mla(inp.q, ix, pos, inp.kv, wl.D_v, wl.sm_scale, nthreads=threads)
    t3 = time.perf_counter()
    tn = np.arange(wl.T, dtype=np.int64)
    n_all = np.minimum(wl.S, wl.q_start + tn + 1)
    est = ((t1 - t0) * n_all.sum() / n.sum() + (t2 - t1) * n_all.sum() / n.sum()
           + (t3 - t2) * np.minimum(n_all, wl.topk).sum() / np.minimum(n, wl.topk).sum())
    sample = ("all %d query rows" % wl.T if len(rows) == wl.T else
              "%d query rows evenly spaced over the %d-token batch (full indexer, top-k and MLA per row), "
              "scaled per stage by visible / selected key counts" % (len(rows), wl.T))
    cpu = host_cpu()
    return {
        "value": wl.T / est, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
        "mode": "full" if len(rows) == wl.T else "sampled",
        "sample": sample + "; %.1f s measured" % (t3 - t0), "sample_seconds": t3 - t0,
        "nproc": cpu["nproc"], "cpu_model": cpu["model"],
    }


def cpu_baseline_decode(inp, threads: int):
    """The oracle (as it stands) over every sequence of a decode batch: scores of all visible keys
    read through the block tables, top-k, attention; timed in full."""
    import oracle
    t0 = time.perf_counter()
    oracle.decode(inp, nthreads=threads)
    dt = time.perf_counter() - t0
    cpu = host_cpu()
    B = len(inp.seq_lens)
    return {"value": B / dt, "unit": "query tokens/s", "cores": threads, "kind": "oracle", "mode": "full",
            "sample": "all %d sequences (%d visible keys), one query each; %.1f s measured"
                      % (B, int(inp.seq_lens.astype(np.int64).sum()), dt),
            "sample_seconds": dt, "nproc": cpu["nproc"], "cpu_model": cpu["model"]}


def put(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)


def run_prefill(wl, args, dev):
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import prefill_inputs

    print("generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    inp = prefill_inputs(wl)
    q8, qs, w, k8, ks = (put(x, dev) for x in (inp.q8, inp.qs, inp.w, inp.k8, inp.ks))
    q = put(inp.q, dev).view(torch.bfloat16)
    kv = put(inp.kv, dev).view(torch.bfloat16)
    del inp
    S, T = wl.S, wl.T
    ld = dsa.ld_for(S)
    logits = torch.empty((T, ld), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.topk), dtype=torch.int32, device=dev)
    out = torch.empty((T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
    tk_ws = torch.empty(max(1, dsa.load().dsa_topk_workspace_size(T, S, wl.topk)), dtype=torch.uint8, device=dev)
    mla_ws = torch.empty(max(1, dsa.load().dsa_sparse_mla_workspace_size(T, S, wl.H, wl.D_qk, wl.D_v, wl.topk)),
                         dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        dsa.dsa_indexer_logits(q8, qs, w, k8, ks, wl.q_start, logits)
        if ev:
            ev[1].record(stream)
        dsa.dsa_topk(logits, wl.topk, S, wl.q_start, idx, tk_ws)
        if ev:
            ev[2].record(stream)
        dsa.dsa_sparse_mla_fwd(q, kv, idx, wl.sm_scale, wl.D_v, wl.q_start, out=out, lse=lse, workspace=mla_ws)
        if ev:
            ev[3].record(stream)

    print("warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print("timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    stage_ms = per.mean(axis=0)

    fused_ms = None
    if not args.skip_fused:
        nb = (S + 63) // 64
        pad = nb * 64 - S
        cache = dsa.PagedKV(
            torch.cat([k8, torch.zeros((pad, wl.D_I), dtype=k8.dtype, device=dev)]).view(nb, 64, wl.D_I),
            torch.cat([ks, torch.zeros((pad,), dtype=ks.dtype, device=dev)]).view(nb, 64),
            torch.cat([kv, torch.zeros((pad, wl.D_qk), dtype=kv.dtype, device=dev)]).view(nb, 64, wl.D_qk),
            torch.arange(nb, dtype=torch.int32, device=dev)[None])
        dims = dsa.make_dims(wl.H_I, wl.D_I, wl.H, wl.D_qk, wl.D_v, wl.topk, wl.sm_scale)
        ws = torch.empty(dsa.prefill_workspace_size(dims, T, wl.q_start + T), dtype=torch.uint8, device=dev)
        for _ in range(2):
            dsa.dsa_prefill_paged(cache, 0, dims, wl.q_start, q8, qs, w, q, out=out, workspace=ws)
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for _ in range(args.steps):
            dsa.dsa_prefill_paged(cache, 0, dims, wl.q_start, q8, qs, w, q, out=out, workspace=ws)
        torch.cuda.synchronize()
        fused_ms = (time.perf_counter() - f0) * 1e3 / args.steps

    if args.copy_calibration:
        copy_calibration(dev)

    wm = work_model(wl)
    stages = {
        "indexer": {"ms": float(stage_ms[0]), "bound": "mfma", "achieved_tflops": wm["indexer_flop"] / stage_ms[0] / 1e9,
                    "frac": wm["indexer_flop"] / (stage_ms[0] / 1e3) / PEAK_FP8},
        "topk": {"ms": float(stage_ms[1]), "bound": "hbm", "achieved_gbs": wm["topk_bytes"] / stage_ms[1] / 1e6,
                 "frac": wm["topk_bytes"] / (stage_ms[1] / 1e3) / PEAK_HBM},
        "sparse_mla": {"ms": float(stage_ms[2]), "bound": "mfma", "achieved_tflops": wm["mla_flop"] / stage_ms[2] / 1e9,
                       "frac": wm["mla_flop"] / (stage_ms[2] / 1e3) / PEAK_BF16},
    }
    # dominant kernel: the stage that takes longest
    dom = max(stages, key=lambda k: stages[k]["ms"])
    if dom == "sparse_mla":
        roof = {"kernel": "sparse_mla_kernel<%d,%d>" % (wl.D_qk, wl.D_v), "bound": "mfma",
                "achieved": wm["mla_flop"] / (stage_ms[2] / 1e3) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "traffic": traffic_from_profile() if wl.name == HEADLINE else None,
                "algorithmic_flop_per_launch": wm["mla_flop"]}
    elif dom == "indexer":
        roof = {"kernel": "indexer_prefill_kernel", "bound": "mfma",
                "achieved": wm["indexer_flop"] / (stage_ms[0] / 1e3) / 1e12, "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
                "traffic": None, "algorithmic_flop_per_launch": wm["indexer_flop"]}
    else:
        roof = {"kernel": "topk_row_kernel", "bound": "hbm",
                "achieved": wm["topk_bytes"] / (stage_ms[1] / 1e3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "traffic": None, "algorithmic_bytes_per_launch": wm["topk_bytes"]}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["avg_launch_ms"] = float(stages[dom]["ms"])
    step_ms = per.sum(axis=1)
    return {
        "value": T / (ms_step / 1e3), "ms_per_step": ms_step, "step_ms_events": percentiles(step_ms),
        "roofline": roof, "stages": stages, "fused_ms_per_step": fused_ms,
        "config": {"workload": wl.name, "T": T, "S": S, "q_start": wl.q_start, "H_I": wl.H_I, "D_I": wl.D_I,
                   "topk": wl.topk, "H": wl.H, "D_qk": wl.D_qk, "D_v": wl.D_v, "parallelism": "single GPU"},
    }


def run_decode(wl, args, dev, cpu_threads: int = 0):
    """Fused paged decode (dsa_decode_paged): one new token for each of the 64 sequences.  A second,
    profiled pass brackets each kernel of the call with stage events for its own achieved GB/s."""
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import decode_inputs

    print("generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    inp = decode_inputs(wl)
    cache = dsa.PagedKV(put(inp.k8_pool, dev), put(inp.ks_pool, dev), put(inp.kv_pool, dev).view(torch.bfloat16),
                        put(inp.block_table, dev), put(inp.seq_lens, dev))
    q8, qs, w = put(inp.q8, dev), put(inp.qs, dev), put(inp.w, dev)
    q = put(inp.q, dev).view(torch.bfloat16)
    lens = inp.seq_lens.astype(np.int64)
    max_len = int(lens.max())
    B = len(lens)
    dims = dsa.make_dims(wl.H_I, wl.D_I, wl.H, wl.D_qk, wl.D_v, wl.topk, wl.sm_scale)
    ws = torch.empty(dsa.decode_workspace_size(dims, B, max_len), dtype=torch.uint8, device=dev)
    out = torch.empty((B, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.flush_mall else None
    stream = torch.cuda.current_stream(dev)

    def step():
        dsa.dsa_decode_paged(cache, max_len, dims, q8, qs, w, q, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        if flush is not None:
            flush.zero_()  # evict the previous step's pool lines from the MALL (not timed)
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    # profiled pass: an event before the call and one after each of its kernels.  The events are
    # created (and their HIP events materialised) up front, and two unprofiled calls ahead of each
    # profiled one keep the GPU busy while the host enqueues, so no interval holds host latency.
    nk = 8
    prof = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    for evp in prof:
        for ev in evp:
            ev.record(stream)
    torch.cuda.synchronize()
    names = []
    for evp in prof:
        step()
        step()
        if flush is not None:
            flush.zero_()
        evp[0].record(stream)
        dsa.dsa_profile_begin(evp[1:])
        step()
        names = dsa.dsa_profile_end()
    torch.cuda.synchronize()
    prof = [evp[:len(names) + 1] for evp in prof]
    kms = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(names))] for e in prof]).mean(axis=0)
    if args.copy_calibration:
        copy_calibration(dev)
    n = lens
    sel = np.minimum(n, wl.topk)
    nsplit = max(1, min(-(-256 // B), wl.topk // 64))
    G = -(-max_len // 32768)
    # each kernel's own reads and writes (the logits and split partials included: they are this
    # design's intermediates, so the fused roofline below leaves them out)
    kbytes = {
        "indexer_decode_kernel": float(n.sum() * (wl.D_I + 4) + B * wl.H_I * (wl.D_I + 8)
                                       + ((n + 63) // 64).sum() * 4 + 4 * n.sum()),
        "topk_row_kernel": float(4 * n.sum() + 4 * B * wl.topk),
        # rows over 32768 keys: per-chunk candidates (key + index) written, then merged
        "topk_chunk_kernel": float(4 * n.sum() + B * G * wl.topk * 8),
        "topk_merge_kernel": float(B * G * wl.topk * 8 + 4 * B * wl.topk),
        "sparse_mla_kernel": float(sel.sum() * wl.D_qk * 2 + B * wl.H * wl.D_qk * 2 + B * wl.topk * 4
                                   + B * nsplit * wl.H * (wl.D_v + 1) * 4),
        "mla_combine_kernel": float(B * nsplit * wl.H * (wl.D_v + 1) * 4 + B * wl.H * (wl.D_v * 2 + 4)),
    }
    kernels = []
    for name, t in zip(names, kms):
        rec = {"kernel": name, "ms": float(t)}
        if name in kbytes:
            rec["bytes"] = kbytes[name]
            rec["achieved_gbs"] = rec["bytes"] / (t / 1e3) / 1e9
            rec["frac"] = rec["achieved_gbs"] * 1e9 / PEAK_HBM
        kernels.append(rec)
    # HBM bytes any decode must move: the FP8 keys and scales of every visible position, the latent
    # rows of the selected entries, queries, head weights and outputs (the logits kept between the
    # indexer and the top-k, and the split-K partials, are this design's own and are not counted)
    alg = float(n.sum() * (wl.D_I + 4) + sel.sum() * wl.D_qk * 2 + B * wl.H_I * (wl.D_I + 8)
                + B * wl.H * (wl.D_qk + wl.D_v) * 2 + B * wl.H * 4)
    med = float(np.median(ms))
    roof = {"kernel": "dsa_decode_paged (indexer_decode + top-k + split-K MLA + combine)", "bound": "hbm",
            "achieved": alg / (med / 1e3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s", "traffic": None,
            "algorithmic_bytes_per_launch": alg, "avg_launch_ms": float(ms.mean())}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cpu = cpu_baseline_decode(inp, cpu_threads) if cpu_threads > 0 else None
    del inp
    return {
        "value": B / (med / 1e3), "ms_per_step": med, "step_ms_events": percentiles(ms), "roofline": roof,
        "stages": None, "kernels": kernels, "fused_ms_per_step": med, "mall_flush": bool(args.flush_mall),
        "cpu_baseline": cpu,
        "config": {"workload": wl.name, "B": B, "seq_len_min": int(lens.min()), "seq_len_max": max_len,
                   "seq_len_mean": float(lens.mean()), "topk": wl.topk, "H_I": wl.H_I, "D_I": wl.D_I, "H": wl.H,
                   "D_qk": wl.D_qk, "D_v": wl.D_v, "block_size": wl.block_size, "parallelism": "single GPU"},
    }


def run_quantize_append(args, dev):
    """On-device FP8 quantization of the L = 32K prefill's indexer queries (32768 x 64 rows of 128)
    and the paged append of its 32768 tokens (FP8 key + scale + 576-wide latent row, block 64, a
    seeded permutation of blocks), each timed with HIP events against its algorithmic HBM bytes."""
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get
    wl = get(HEADLINE)
    T, H_I, D_I, D_qk, bs = wl.T, wl.H_I, wl.D_I, wl.D_qk, 64
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    print("generating quantize/append inputs", file=sys.stderr, flush=True)
    q = torch.randn((T, H_I, D_I), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((T, D_I), generator=g, device=dev).to(torch.bfloat16)
    kv = torch.randn((T, D_qk), generator=g, device=dev).to(torch.bfloat16)
    nb = T // bs
    perm = torch.randperm(nb, generator=g, device=dev).to(torch.int32)
    cache = dsa.PagedKV(torch.empty((nb, bs, D_I), dtype=torch.uint8, device=dev),
                        torch.empty((nb, bs), dtype=torch.float32, device=dev),
                        torch.empty((nb, bs, D_qk), dtype=torch.bfloat16, device=dev), perm[None].contiguous())
    seq = torch.zeros(T, dtype=torch.int32, device=dev)
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    codes = torch.empty((T, H_I, D_I), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H_I), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        dsa.dsa_quantize_fp8_rows(q, codes, scales)
        if ev:
            ev[1].record(stream)
        dsa.dsa_append_paged(cache, seq, pos, k, kv)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(2)] for e in evs])
    qms, ams = per.mean(axis=0)
    q_bytes = float(T * H_I * (D_I * 2 + D_I + 4))
    a_bytes = float(T * (D_I * 2 + D_I + 4 + D_qk * 2 * 2 + 8))
    step_ms = per.sum(axis=1)
    stages = {
        "quantize_queries": {"ms": float(qms), "bound": "hbm", "achieved_gbs": q_bytes / qms / 1e6,
                             "frac": q_bytes / (qms / 1e3) / PEAK_HBM, "bytes": q_bytes},
        "append_paged": {"ms": float(ams), "bound": "hbm", "achieved_gbs": a_bytes / ams / 1e6,
                         "frac": a_bytes / (ams / 1e3) / PEAK_HBM, "bytes": a_bytes},
    }
    roof = {"kernel": "quantize_rows_kernel", "bound": "hbm", "achieved": q_bytes / (qms / 1e3) / 1e9,
            "peak": PEAK_HBM / 1e9, "unit": "GB/s", "traffic": None, "algorithmic_bytes_per_launch": q_bytes,
            "avg_launch_ms": float(qms)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    med = float(np.median(step_ms))
    return {
        "value": T / (med / 1e3), "ms_per_step": med, "step_ms_events": percentiles(step_ms), "roofline": roof,
        "stages": stages, "fused_ms_per_step": None,
        "config": {"workload": "quantize_append_32k", "T": T, "H_I": H_I, "D_I": D_I, "D_qk": D_qk,
                   "block_size": bs, "parallelism": "single GPU"},
    }


def run_indexer_ue8m0(args, dev):
    """The L = 32K prefill indexer with power-of-two (UE8M0) scales applied inside the FP8 MFMA
    (dsa_indexer_logits_ue8m0), timed beside the fp32-scale indexer on the same codes (scales
    2^(e - 127)); inputs are seeded bf16 vectors quantized on the device."""
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get
    wl = get(HEADLINE)
    T, S, H_I, D_I = wl.T, wl.S, wl.H_I, wl.D_I
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    print("generating ue8m0 indexer inputs", file=sys.stderr, flush=True)
    q = torch.randn((T, H_I, D_I), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((S, D_I), generator=g, device=dev).to(torch.bfloat16)
    w = (torch.rand((T, H_I), generator=g, device=dev) / H_I).contiguous()
    q8, qe, qs = dsa.dsa_quantize_fp8_rows_ue8m0(q)
    k8, ke, ks = dsa.dsa_quantize_fp8_rows_ue8m0(k)
    del q, k
    logits = torch.empty((T, dsa.ld_for(S)), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        dsa.dsa_indexer_logits_ue8m0(q8, qe, w, k8, ke, 0, logits)
        if ev:
            ev[1].record(stream)
        dsa.dsa_indexer_logits(q8, qs, w, k8, ks, 0, logits)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(2)] for e in evs])
    ums, fms = per.mean(axis=0)
    wm = work_model(wl)
    stages = {
        "indexer_ue8m0": {"ms": float(ums), "bound": "mfma", "achieved_tflops": wm["indexer_flop"] / ums / 1e9,
                          "frac": wm["indexer_flop"] / (ums / 1e3) / PEAK_FP8},
        "indexer_fp32_scales": {"ms": float(fms), "bound": "mfma", "achieved_tflops": wm["indexer_flop"] / fms / 1e9,
                                "frac": wm["indexer_flop"] / (fms / 1e3) / PEAK_FP8},
    }
    roof = {"kernel": "indexer_prefill_kernel (E8M0 operand scales)", "bound": "mfma",
            "achieved": wm["indexer_flop"] / (ums / 1e3) / 1e12, "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
            "traffic": None, "algorithmic_flop_per_launch": wm["indexer_flop"], "avg_launch_ms": float(ums)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    ms = per[:, 0]
    return {
        "value": T / (float(np.median(ms)) / 1e3), "ms_per_step": float(np.median(ms)), "step_ms_events": percentiles(ms),
        "roofline": roof, "stages": stages, "fused_ms_per_step": None,
        "config": {"workload": "indexer_ue8m0_32k", "T": T, "S": S, "q_start": 0, "H_I": H_I, "D_I": D_I,
                   "parallelism": "single GPU"},
    }


def run_indexer_train(name, args, dev):
    """One training step of the indexer at a prefill shape (dense warm-up signal): scores ->
    KL loss toward the head-averaged main attention (dI in place of the scores) -> backward to
    q_I, k_I and w.  The inputs of the prefill configuration; stages timed with events."""
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get, prefill_inputs
    sparse = name.startswith("indexer_train_sparse_")
    wl = get(name.replace("indexer_train_sparse_", "prefill_").replace("indexer_train_", "prefill_"))
    print("generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    inp = prefill_inputs(wl)
    q8, qs, w, k8, ks = (put(x, dev) for x in (inp.q8, inp.qs, inp.w, inp.k8, inp.ks))
    q = put(inp.q, dev).view(torch.bfloat16)
    kv = put(inp.kv, dev).view(torch.bfloat16)
    del inp
    T, S = wl.T, wl.S
    logits = torch.empty((T, dsa.ld_for(S)), dtype=torch.float32, device=dev)
    loss = torch.empty((T,), dtype=torch.float32, device=dev)
    dq = torch.empty((T, wl.H_I, wl.D_I), dtype=torch.float32, device=dev)
    dw = torch.empty((T, wl.H_I), dtype=torch.float32, device=dev)
    dk = torch.empty((S, wl.D_I), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, dsa.indexer_bwd_workspace_size(T, S, wl.D_I)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if sparse:  # sparse stage: top-k lists and the sparse attention's normaliser feed the loss
        idx = torch.empty((T, wl.topk), dtype=torch.int32, device=dev)
        out = torch.empty((T, wl.H, wl.D_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, wl.H), dtype=torch.float32, device=dev)
        tk_ws = torch.empty(max(1, dsa.load().dsa_topk_workspace_size(T, S, wl.topk)), dtype=torch.uint8, device=dev)
        mla_ws = torch.empty(max(1, dsa.load().dsa_sparse_mla_workspace_size(T, S, wl.H, wl.D_qk, wl.D_v, wl.topk)),
                             dtype=torch.uint8, device=dev)
    nstage = 5 if sparse else 3

    def step(ev=None):
        def mark(i):
            if ev:
                ev[i].record(stream)
        mark(0)
        dsa.dsa_indexer_logits(q8, qs, w, k8, ks, wl.q_start, logits)
        mark(1)
        if sparse:
            dsa.dsa_topk(logits, wl.topk, S, wl.q_start, idx, tk_ws)
            mark(2)
            dsa.dsa_sparse_mla_fwd(q, kv, idx, wl.sm_scale, wl.D_v, wl.q_start, out=out, lse=lse, workspace=mla_ws)
            mark(3)
            dsa.dsa_indexer_kl_loss_sparse(q, kv, idx, lse, logits, wl.sm_scale, wl.q_start, dlogits=logits,
                                           loss=loss)
        else:
            dsa.dsa_indexer_kl_loss(q, kv, logits, wl.sm_scale, wl.q_start, dlogits=logits, loss=loss)
        mark(nstage - 1)
        if sparse:  # dI vanishes off the lists: dq / dw over the listed keys only
            dsa.dsa_indexer_bwd_listed(q8, qs, w, k8, ks, idx, logits, wl.q_start, dq, dw, dk, ws)
        else:
            dsa.dsa_indexer_bwd(q8, qs, w, k8, ks, logits, wl.q_start, dq, dw, dk, ws)
        mark(nstage)

    print("warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nstage + 1)] for _ in range(args.steps)]
    print("timing %d steps" % args.steps, file=sys.stderr, flush=True)
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(nstage)] for e in evs])
    step_ms = per.sum(axis=1)
    mean = per.mean(axis=0)
    ims, kms, bms = mean[0], mean[nstage - 2], mean[nstage - 1]
    wm = work_model(wl)
    pairs = wm["visible_pairs"]
    # the loss: one Q K^T over every visible pair (dense) or every selected entry (sparse stage)
    kl_flop = 2.0 * wl.H * wl.D_qk * (wm["selected_rows"] if sparse else pairs)
    # z, dq and dk contractions over the pairs with a nonzero dI (the listed entries in the sparse
    # stage, although its dk kernel still walks every visible pair)
    bwd_flop = 3 * 2.0 * wl.H_I * wl.D_I * (wm["selected_rows"] if sparse else pairs)
    stages = {
        "indexer": {"ms": float(ims), "bound": "mfma", "achieved_tflops": wm["indexer_flop"] / ims / 1e9,
                    "frac": wm["indexer_flop"] / (ims / 1e3) / PEAK_FP8},
        "kl_loss": {"ms": float(kms), "bound": "mfma", "achieved_tflops": kl_flop / kms / 1e9,
                    "frac": kl_flop / (kms / 1e3) / PEAK_BF16},
        "indexer_bwd": {"ms": float(bms), "bound": "mfma", "achieved_tflops": bwd_flop / bms / 1e9,
                        "frac": bwd_flop / (bms / 1e3) / PEAK_BF16},
    }
    if sparse:
        stages["topk"] = {"ms": float(mean[1]), "bound": "hbm", "frac": wm["topk_bytes"] / (mean[1] / 1e3) / PEAK_HBM}
        stages["sparse_mla"] = {"ms": float(mean[2]), "bound": "mfma",
                                "frac": wm["mla_flop"] / (mean[2] / 1e3) / PEAK_BF16}
    kname = "indexer_kl_sparse_kernel<36>" if sparse else "indexer_kl_kernel<36>"
    roof = {"kernel": kname, "bound": "mfma", "achieved": kl_flop / (kms / 1e3) / 1e12,
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "traffic": None, "algorithmic_flop_per_launch": kl_flop,
            "avg_launch_ms": float(kms)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return {
        "value": T / (float(np.median(step_ms)) / 1e3), "ms_per_step": float(np.median(step_ms)),
        "step_ms_events": percentiles(step_ms), "roofline": roof, "stages": stages,
        "config": {"workload": name, "T": T, "S": S, "q_start": wl.q_start, "H": wl.H, "D_qk": wl.D_qk,
                   "H_I": wl.H_I, "D_I": wl.D_I, "parallelism": "single GPU"},
    }


def run_mla_bwd(name, args, dev):
    """Sparse-MLA backward at a prefill shape: indexer -> top-2048 -> forward (for lse) once, then the
    backward (dq, dkv) timed over the steps with a seeded dout; per-kernel times from stage events.
    Algorithmic work per selected (row, head, entry): the score recompute 2 D_qk, dP 2 D_v, dq 2 D_qk,
    dk 2 D_qk, dv 2 D_v flop (the second score pass that forms D and the pass split are this design's
    own)."""
    import torch
    import dsa_lightning_indexer_02_amd as dsa
    from dsa_inputs import get, prefill_inputs
    wl = get(name.replace("sparse_mla_bwd_", "prefill_"))
    print("generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    inp = prefill_inputs(wl)
    q8, qs, w, k8, ks = (put(x, dev) for x in (inp.q8, inp.qs, inp.w, inp.k8, inp.ks))
    q = put(inp.q, dev).view(torch.bfloat16)
    kv = put(inp.kv, dev).view(torch.bfloat16)
    del inp
    T, S = wl.T, wl.S
    lg = dsa.dsa_indexer_logits(q8, qs, w, k8, ks, wl.q_start)
    idx = dsa.dsa_topk(lg, wl.topk, S, wl.q_start)
    del lg
    _, _, lse = dsa.dsa_sparse_mla_fwd(q, kv, idx, wl.sm_scale, wl.D_v, wl.q_start)
    g = torch.Generator(device=dev)
    g.manual_seed(13)
    dout = torch.randn((T, wl.H, wl.D_v), generator=g, device=dev).to(torch.bfloat16)
    dq = torch.empty((T, wl.H, wl.D_qk), dtype=torch.float32, device=dev)
    dkv = torch.empty((S, wl.D_qk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, dsa.load().dsa_sparse_mla_bwd_workspace_size(T, S, wl.H, wl.topk)), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        dsa.dsa_sparse_mla_bwd(q, kv, idx, lse, dout, wl.sm_scale, wl.q_start, dq, dkv, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # stage events after every launch (a zero fill, then five kernels per chunk of 512 rows); an
    # unprofiled call ahead of each keeps the GPU busy while the host enqueues
    nev = 2 + 5 * (-(-T // 512))
    prof = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for ev in prof:
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    names = []
    for ev in prof:
        step()
        ev[0].record(stream)
        dsa.dsa_profile_begin(ev[1:])
        step()
        names = dsa.dsa_profile_end()
    torch.cuda.synchronize()
    prof = [ev[:len(names) + 1] for ev in prof]
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(names))] for e in prof])
    step_ms = per.sum(axis=1)
    # per kernel: its launches summed within a call, averaged over the calls
    order = list(dict.fromkeys(names))
    kms = [float(per[:, [j for j, nm in enumerate(names) if nm == kn]].sum(axis=1).mean()) for kn in order]
    names = order
    wm = work_model(wl)
    sel = wm["selected_rows"]
    flop = 2.0 * wl.H * (3 * wl.D_qk + 2 * wl.D_v) * sel
    kernels = [{"kernel": nm, "ms": float(t)} for nm, t in zip(names, kms)]
    med = float(np.median(step_ms))
    roof = {"kernel": "sparse_mla_bwd (dq, key map, dkv contribution and reduction kernels)", "bound": "mfma", "achieved": flop / (med / 1e3) / 1e12,
            "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "traffic": None, "algorithmic_flop_per_launch": flop,
            "avg_launch_ms": float(step_ms.mean())}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return {"metric": "query tokens/s (sparse MLA backward: dq, dkv, %s)" % name, "value": T / (med / 1e3),
            "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": med,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 scores, bf16 hi/lo dq, fp16 dkv contraction, fp32 accumulation",
            "data": "synthetic (seeded PCG64 recipe; torch-seeded bf16 dout)", "config": {
                "workload": name, "T": T, "S": S, "q_start": wl.q_start, "H": wl.H, "D_qk": wl.D_qk, "D_v": wl.D_v,
                "topk": wl.topk, "parallelism": "single GPU"},
            "roofline": roof, "kernels": kernels, "stages": None, "step_ms_events": percentiles(step_ms),
            "fused_ms_per_step": None, "cpu_baseline": None}


def run_one(name, args, dev, with_cpu: bool):
    from dsa_inputs import get
    if name in ("quantize_append_32k", "indexer_ue8m0_32k"):
        qa = name == "quantize_append_32k"
        res = run_quantize_append(args, dev) if qa else run_indexer_ue8m0(args, dev)
        line = {"metric": ("query tokens/s (FP8 quantize of indexer queries + paged append, L=32K)" if qa else
                           "query tokens/s (indexer with UE8M0 scales in the MFMA, L=32K)"),
                "value": res["value"], "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None,
                "dtype": "bf16 in, fp8-e4m3 out" if qa else "fp8-e4m3 with e8m0 scales",
                "data": "synthetic (seeded torch normal, bf16)", "config": res["config"], "roofline": res["roofline"],
                "stages": res["stages"], "step_ms_events": res["step_ms_events"], "fused_ms_per_step": None,
                "cpu_baseline": None}
        return line
    if name.startswith("sparse_mla_bwd_"):
        return run_mla_bwd(name, args, dev)
    if name.startswith("indexer_train_"):
        res = run_indexer_train(name, args, dev)
        what = ("scores + top-k + sparse attention + sparse-stage KL loss + backward"
                if name.startswith("indexer_train_sparse_") else "scores + KL loss + backward")
        return {"metric": "query tokens/s (indexer training step: %s, %s)" % (what, name),
                "value": res["value"], "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None,
                "dtype": "fp8-e4m3 indexer, bf16 MFMA loss and backward, fp32 gradients",
                "data": "synthetic (seeded PCG64 recipe, FP8 per-row absmax codes, bf16 N(0,1))",
                "config": res["config"], "roofline": res["roofline"], "stages": res["stages"],
                "step_ms_events": res["step_ms_events"], "fused_ms_per_step": None, "cpu_baseline": None}
    wl = get(name)
    threads = host_cpu()["threads"]
    if wl.kind == "decode":
        res = run_decode(wl, args, dev, cpu_threads=threads if with_cpu else 0)
        cpu = res.get("cpu_baseline")
    else:
        res = run_prefill(wl, args, dev)
        cpu = None
        if with_cpu:
            print("cpu baseline (oracle)", file=sys.stderr, flush=True)
            rows = args.cpu_rows if name == HEADLINE else (128 if name == "chunked_131k" else wl.T)
            cpu = cpu_baseline(wl, rows, threads)
    line = {
        "metric": METRIC if name == HEADLINE else "query tokens/s (%s)" % name,
        "value": res["value"],
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer, bf16/fp16 attention",
        "data": "synthetic (seeded PCG64 recipe, FP8 per-row absmax codes, bf16 N(0,1))",
        "config": res["config"],
        "roofline": res["roofline"],
        "stages": res["stages"],
        "step_ms_events": res["step_ms_events"],
        "fused_ms_per_step": res["fused_ms_per_step"],
        "cpu_baseline": cpu,
    }
    if "mall_flush" in res:
        line["mall_flush"] = res["mall_flush"]
    if res.get("kernels"):
        line["kernels"] = res["kernels"]
    return line


def summary(line):
    """The fields of another workload's line that the headline line carries beside its own."""
    keep = ("value", "unit", "ms_per_step", "roofline", "stages", "kernels", "cpu_baseline", "config", "mall_flush")
    return {k: line[k] for k in keep if k in line}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--all-configs", action="store_true", help="one line per configuration (no CPU baseline)")
    ap.add_argument("--cpu-rows", type=int, default=1536)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-fused", action="store_true")
    ap.add_argument("--skip-other-workloads", action="store_true",
                    help="headline run: leave out the decode_64 and chunked_131k summaries")
    ap.add_argument("--flush-mall", action="store_true", help="decode: overwrite 512 MiB between steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy 1 GiB device-to-device (counter scale reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dsa_lightning_indexer_02_amd as dsa
    dev = torch.device("cuda:0")
    dsa.load()
    if args.all_configs:
        for name in ["tiny", "prefill_4k", "prefill_32k", "chunked_131k", "decode_64", "quantize_append_32k",
                     "indexer_ue8m0_32k", "indexer_train_4k", "indexer_train_sparse_4k", "sparse_mla_bwd_4k",
                     "sparse_mla_bwd_32k"]:
            print(json.dumps(run_one(name, args, dev, with_cpu=False)), flush=True)
            torch.cuda.empty_cache()
        return
    line = run_one(args.workload, args, dev, with_cpu=not args.skip_cpu_baseline)
    if args.workload == HEADLINE and not args.skip_other_workloads:
        # the decode and chunked-prefill workloads, each with its own oracle baseline, beside the headline
        other = {}
        for name in ("decode_64", "chunked_131k"):
            torch.cuda.empty_cache()
            other[name] = summary(run_one(name, args, dev, with_cpu=not args.skip_cpu_baseline))
        line["other_workloads"] = other
    print(json.dumps(line))


if __name__ == "__main__":
    main()
