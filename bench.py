"""Benchmark: exact causal GQA attention forward on one MI355X.

One step = one forward over the workload (default: the fp32 causal forward at
L = 30,468, B = 1, Hq = 16, Hkv = 4, D = 256; synthetic N(0,1) inputs already
resident in HBM). Prints ONE JSON line. `value` is TFLOP/s counted as 4*D per
visible (query, key) pair per query head (the causal half of the L x L work).
Secondary workloads (the other lengths, bf16, the shared-prefix branch form and
the packed-segment form) are reported under "secondary".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal GQA attn fwd TFLOP/s + % MFMA peak (fp32 & bf16, L=32k/64k); peak GiB"
HQ, HKV, D = 16, 4, 256
SEG_IDX_NOTE = ", id index built per call"


def dev_inputs(x, torch):
    dev = "cuda:0"
    if x.dtype == "f32":
        return tuple(torch.from_numpy(a).to(dev) for a in (x.q, x.k, x.v))
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float16
    return tuple(torch.from_numpy(b.view(np.int16)).to(dev).view(tdt) for b in (x.q_bits, x.k_bits, x.v_bits))


def time_calls(fn, steps, warmup, torch):
    """Wall time per step (host clock around K synchronized steps) and the mean,
    min and max per-call GPU time from HIP events recorded on the launch stream
    (the median is left in time_calls.last_median)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = [a.elapsed_time(b) for a, b in evs]
    time_calls.last_median = float(np.median(ev_ms))
    return wall_ms, float(np.mean(ev_ms)), float(np.min(ev_ms)), float(np.max(ev_ms))


def run_fwd_workload(name, x, steps, warmup, torch, gqa, work, seg=None, indexed=False):
    """One forward workload. indexed: every timed call first builds the ids'
    range index (gqa_attn_seg_index) and then runs gqa_attn_fwd_indexed."""
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    q, k, v = dev_inputs(x, torch)
    sq = sk = None
    if seg is not None:
        sq = torch.from_numpy(seg[None]).to("cuda:0")
        sk = sq
    o = torch.empty_like(q)
    B, Hq, Lq, Dh = q.shape
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    fn = lambda: gqa.fwd(q, k, v, causal=x.causal, q_offset=x.q_offset, seg_q=sq, seg_k=sk, out=o, lse=lse)
    if indexed and seg is not None:
        ibuf = gqa.seg_index(sk)

        def fn():
            idx = gqa.seg_index(sk, out=ibuf)
            gqa.fwd(q, k, v, causal=x.causal, q_offset=x.q_offset, seg_q=sq, seg_k=sk, out=o, lse=lse,
                    seg_q_index=idx, seg_k_index=idx)
    fn()  # first launch loads the code object; device memory is compared after it
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    wall_ms, ev_ms, ev_min, ev_max = time_calls(fn, steps, warmup, torch)
    free1, _ = torch.cuda.mem_get_info()
    peak = torch.cuda.max_memory_allocated() - base
    Lk, Hkv_ = k.shape[2], k.shape[1]
    fl = work.flops(B, Hq, Lq, Lk, Dh, causal=x.causal, q_offset=x.q_offset,
                    seg_q=None if seg is None else seg[None], seg_k=None if seg is None else seg[None])
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return dict(workload=name, flops=fl, wall_ms=wall_ms, kernel_ms=ev_ms, kernel_ms_min=ev_min,
                kernel_ms_max=ev_max, kernel_ms_median=time_calls.last_median, tflops=fl / (wall_ms * 1e-3) / 1e12,
                kernel_tflops=fl / (ev_ms * 1e-3) / 1e12,
                peak_gib=peak / 2 ** 30, library_alloc_bytes=int(free0 - free1),
                bytes=work.hbm_bytes(B, Hq, Hkv_, Lq, Lk, Dh, 4 if x.dtype == "f32" else 2, seg is not None))


def run_bwd_workload(name, x, steps, warmup, torch, gqa, work, synth, seg=None, indexed=False):
    """The backward (dQ kernel + dK/dV kernel) on the forward's own o and lse;
    dout drawn N(0,1) (seed 1); optional packed segment ids. Times the backward
    call only."""
    torch.cuda.synchronize()
    q, k, v = dev_inputs(x, torch)
    sid = None if seg is None else torch.from_numpy(seg[None]).to("cuda:0")
    g = synth.Grad(x.q.shape, seed=1, dtype=x.dtype)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[x.dtype]
    if x.dtype == "f32":
        do = torch.from_numpy(g.values).to("cuda:0")
    else:
        do = torch.from_numpy(g.bits.view(np.int16)).to("cuda:0").view(tdt)
    del g
    o, lse = gqa.fwd(q, k, v, causal=x.causal, q_offset=x.q_offset, seg_q=sid, seg_k=sid)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    fn = lambda: gqa.bwd(q, k, v, o, lse, do, causal=x.causal, q_offset=x.q_offset, seg_q=sid, seg_k=sid, dq=dq,
                         dk=dk, dv=dv, delta=delta)
    if indexed and seg is not None:
        # the ids' range index built in every timed call, then the indexed backward
        ibuf = gqa.seg_index(sid)

        def fn():
            idx = gqa.seg_index(sid, out=ibuf)
            gqa.bwd(q, k, v, o, lse, do, causal=x.causal, q_offset=x.q_offset, seg_q=sid, seg_k=sid, dq=dq, dk=dk,
                    dv=dv, delta=delta, seg_q_index=idx, seg_k_index=idx)
    fn()
    torch.cuda.synchronize()
    wall_ms, ev_ms, ev_min, ev_max = time_calls(fn, steps, warmup, torch)
    B, Hq, Lq, Dh = q.shape
    Hkv_, Lk = k.shape[1], k.shape[2]
    sk = None if seg is None else seg[None]
    fl = work.bwd_flops(B, Hq, Lq, Lk, Dh, causal=x.causal, q_offset=x.q_offset, seg_q=sk, seg_k=sk)
    ex = work.bwd_exec_flops(B, Hq, Lq, Lk, Dh, causal=x.causal, q_offset=x.q_offset, seg_q=sk, seg_k=sk)
    del q, k, v, do, o, lse, dq, dk, dv, delta, sid
    torch.cuda.empty_cache()
    return dict(workload=name, flops=fl, exec_flops=ex, wall_ms=wall_ms, kernel_ms=ev_ms, kernel_ms_min=ev_min,
                kernel_ms_max=ev_max, kernel_ms_median=time_calls.last_median, tflops=fl / (wall_ms * 1e-3) / 1e12,
                kernel_tflops=fl / (ev_ms * 1e-3) / 1e12,
                exec_tflops=ex / (ev_ms * 1e-3) / 1e12,
                bytes=work.bwd_hbm_bytes(B, Hq, Hkv_, Lq, Lk, Dh, 4 if x.dtype == "f32" else 2, seg is not None))


def run_split_workload(name, x, steps, warmup, torch, gqa, work):
    """Short query block over a long key sequence: gqa_attn_fwd (one launch of
    n_qb * G workgroups) against gqa_attn_fwd_split at the library's split
    count (partials + merge), both timed; the record carries both times, the
    algorithmic flops and the K/V bytes every call must read."""
    q, k, v = dev_inputs(x, torch)
    B, Hq, Lq, Dh = q.shape
    Hkv_, Lk = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    dt = {"f32": gqa.GQA_F32, "bf16": gqa.GQA_BF16, "f16": gqa.GQA_F16}[x.dtype]
    n_split = gqa.split_count(B, Hq, Hkv_, Lq, Lk, dt)
    ws = torch.empty(max(gqa.split_workspace(B, Hq, Lq, Dh, n_split), 16), dtype=torch.uint8, device=q.device)
    plain = lambda: gqa.fwd(q, k, v, causal=x.causal, q_offset=x.q_offset, out=o, lse=lse)
    split = lambda: gqa.fwd_split(q, k, v, causal=x.causal, q_offset=x.q_offset, n_split=n_split, out=o, lse=lse,
                                  workspace=ws)
    plain()
    split()
    torch.cuda.synchronize()
    _, ms_plain, _, _ = time_calls(plain, steps, warmup, torch)
    wall_ms, ms_split, ev_min, ev_max = time_calls(split, steps, warmup, torch)
    med_split = time_calls.last_median
    graph_ms = split_graph_ms(split, o, lse, steps, torch)
    fl = work.flops(B, Hq, Lq, Lk, Dh, causal=x.causal, q_offset=x.q_offset)
    es = 4 if x.dtype == "f32" else 2
    kv_bytes = 2 * B * Hkv_ * Lk * Dh * es
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return dict(workload=name, n_split=n_split, flops=fl, wall_ms=wall_ms, kernel_ms=ms_split,
                kernel_ms_min=ev_min, kernel_ms_max=ev_max, kernel_ms_median=med_split,
                unsplit_ms=ms_plain, speedup=ms_plain / ms_split,
                tflops=fl / (wall_ms * 1e-3) / 1e12, kernel_tflops=fl / (ms_split * 1e-3) / 1e12,
                kv_bytes=kv_bytes, kv_gbs=kv_bytes / (ms_split * 1e-3) / 1e9,
                kv_frac_hbm_peak=kv_bytes / (ms_split * 1e-3) / (work.PEAK_HBM_GBS * 1e9),
                graph_ms=graph_ms, graph_kv_gbs=kv_bytes / (graph_ms * 1e-3) / 1e9 if graph_ms else None,
                graph_kv_frac_hbm_peak=kv_bytes / (graph_ms * 1e-3) / (work.PEAK_HBM_GBS * 1e9) if graph_ms else None)


def split_graph_ms(split, o, lse, steps, torch):
    """GPU time per call of the split-KV pair (partials + merge) replayed from a
    HIP graph: per-call events on a short call also hold the host's launch
    time, which a graph replay leaves out. Every replay's o and lse are checked
    bit for bit against the eager call's; on a mismatch (or a capture error)
    the figure is None."""
    split()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            split()  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            split()
        torch.cuda.synchronize()
    except RuntimeError as e:
        print("graph capture failed: %s" % e, file=sys.stderr)
        return None
    for _ in range(3):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not (torch.equal(o, o_ref) and torch.equal(lse, l_ref)):
            print("graph replay differs from the eager call", file=sys.stderr)
            return None
    # back-to-back replays keep the queue ahead of the GPU, so the time between
    # the events is the GPU's; the best of 3 batches
    reps = max(steps, 20)
    best = None
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / reps
        best = t if best is None else min(best, t)
    return best


def run_branch(steps, warmup, torch, gqa, work, synth):
    """Shared-prefix branch form, fp32: S = 30,468 prefix tokens, 40 branches of
    m = 256 query rows at positions S.. . Prefix part: one non-causal call of all
    n*m rows against the prefix; suffix part: one causal call over the branch keys
    with one segment per branch; then the lse merge."""
    br = synth.Branch(S=30468, n=40, m=256, seed=0, dtype="f32")
    qb, kb, vb, ids = br.branch_layout()
    dev = "cuda:0"
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    q = torch.from_numpy(qb).to(dev)
    kp = torch.from_numpy(br.k_p[None]).to(dev)
    vp = torch.from_numpy(br.v_p[None]).to(dev)
    ks = torch.from_numpy(kb).to(dev)
    vs = torch.from_numpy(vb).to(dev)
    sid = torch.from_numpy(ids[None]).to(dev)
    o1 = torch.empty_like(q)
    o2 = torch.empty_like(q)
    l1 = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    l2 = torch.empty_like(l1)

    def fn():
        gqa.fwd(q, kp, vp, causal=False, out=o1, lse=l1)
        gqa.fwd(q, ks, vs, causal=True, seg_q=sid, seg_k=sid, out=o2, lse=l2)
        gqa.merge(o1, l1, o2, l2, out=o1, out_lse=l1)

    wall_ms, ev_ms, ev_min, ev_max = time_calls(fn, steps, warmup, torch)
    peak = torch.cuda.max_memory_allocated() - base
    n, m, S = br.n, br.m, br.S
    fl = 4 * D * HQ * n * (m * S + m * (m + 1) // 2)
    del q, kp, vp, ks, vs, o1, o2, l1, l2
    torch.cuda.empty_cache()
    return dict(workload="branch f32 S=30468 n=40 m=256 (prefix call + segmented suffix call + merge)",
                flops=fl, wall_ms=wall_ms, kernel_ms=ev_ms, kernel_ms_min=ev_min, kernel_ms_max=ev_max,
                kernel_ms_median=time_calls.last_median, tflops=fl / (wall_ms * 1e-3) / 1e12,
                kernel_tflops=fl / (ev_ms * 1e-3) / 1e12, peak_gib=peak / 2 ** 30)


def zigzag_chunks(L, n_ranks):
    """Rank r's row ranges of a zig-zag context-parallel split: chunks r and
    2N - 1 - r of 2N near-equal chunks (the same rule as tests/test_shard_gpu.py)."""
    edges = [(L * i) // (2 * n_ranks) for i in range(2 * n_ranks + 1)]
    return [[(edges[r], edges[r + 1]), (edges[2 * n_ranks - 1 - r], edges[2 * n_ranks - r])] for r in range(n_ranks)]


def run_shards(x, whole_ms, rank_counts, steps, warmup, torch, gqa):
    """Context-parallel shards of the causal forward, run one after another on
    one GPU: for N ranks (zig-zag rows), rank r's work is two calls (rows
    [a, b), keys [0, b), q_offset = a). Reported per N: each rank's kernel time
    (HIP events), the largest (an N-GPU run's compute time, transfers left out),
    its ratio to the mean (load balance) and to the whole call (speed-up over one
    GPU, transfers left out)."""
    q, k, v = dev_inputs(x, torch)
    L = q.shape[2]
    out = []
    for n in rank_counts:
        ranks = zigzag_chunks(L, n)
        per_rank = []
        for rng in ranks:
            parts = []
            for a, b in rng:
                parts.append((q[:, :, a:b].contiguous(), k[:, :, :b].contiguous(), v[:, :, :b].contiguous(), a))
            fn = lambda parts=parts: [gqa.fwd(qq, kk, vv, q_offset=a) for qq, kk, vv, a in parts]
            fn()
            torch.cuda.synchronize()
            _, ms, _, _ = time_calls(fn, steps, warmup, torch)
            per_rank.append(ms)
            del parts
            torch.cuda.empty_cache()
        mx, mean = max(per_rank), sum(per_rank) / len(per_rank)
        out.append({"ranks": n, "rank_kernel_ms": [round(t, 3) for t in per_rank], "max_rank_ms": round(mx, 3),
                    "max_over_mean": round(mx / mean, 4), "sum_over_whole": round(sum(per_rank) / whole_ms, 4),
                    "speedup_over_one_gpu": round(whole_ms / mx, 3)})
    del q, k, v
    torch.cuda.empty_cache()
    return {"workload": "context-parallel shards, causal GQA fwd fp32 L=%d, zig-zag rows, one GPU in turn" % L,
            "whole_call_ms": round(whole_ms, 3), "splits": out}


def copy_probe(torch):
    """A plain 1 GiB device copy, 3 times: the reference that scales the HBM
    byte counters (FETCH_SIZE, WRITE_SIZE) read under the profiler."""
    n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return {"read": 4 * n, "written": 4 * n}


def cpu_threads():
    """Threads the oracle runs on: the OpenMP thread count the environment sets
    (the host's CPU share for this GPU), else every CPU this process may run on."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() and int(env) > 0 else aff
    return min(n, aff), aff


def oracle_rows(x, rows, threads, seg=None):
    """Seconds for the oracle on query rows `rows` of every head of workload x,
    and the visible (row, key) pairs of one head over those rows."""
    import oracle
    from long_context_causal_amd import work
    sq = None if seg is None else seg[None]
    t0 = time.perf_counter()
    oracle.attn(x.q, x.k, x.v, causal=x.causal, q_offset=x.q_offset, seg_q=sq, seg_k=sq, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    Lk = x.k.shape[2]
    pairs = work.visible_pairs_rows(rows, Lk, causal=x.causal, q_offset=x.q_offset, seg_q=seg, seg_k=seg)
    return dt, pairs


def cpu_entry(name, x, threads, full_pairs, seg=None, target_s=4.0, full=False):
    """The oracle on workload x: the whole workload (full=True), or evenly
    spaced query rows (all heads, all their visible keys) sized to about
    target_s seconds, with the whole workload's time extrapolated by visible
    pairs and labelled so. Rates count 4 D flops per visible pair and head."""
    L = x.q.shape[2]
    Hq, Dh = x.q.shape[1], x.q.shape[3]
    if full:
        rows = np.arange(L, dtype=np.int64)
    else:
        calib = np.linspace(0, L - 1, 16).astype(np.int64)
        dt, pr = oracle_rows(x, calib, threads, seg)
        per_pair = dt / max(pr, 1)
        n = int(max(16, min(L, target_s / max(per_pair * full_pairs / L, 1e-9))))
        rows = np.linspace(0, L - 1, n).astype(np.int64)
    dt, pr = oracle_rows(x, rows, threads, seg)
    fl = 4 * Dh * Hq * pr
    rec = dict(workload=name, threads=threads, rows=int(len(rows)), rows_total=int(L), seconds=round(dt, 3),
               value=fl / dt / 1e12, unit="TFLOP/s")
    if full:
        rec["kind"] = "full"
    else:
        rec["kind"] = "sampled"
        rec["full_seconds_extrapolated"] = round(dt * full_pairs / max(pr, 1), 1)
        rec["note"] = "whole-workload time extrapolated from the sampled rows by visible (row, key) pairs"
    return rec


def cpu_baseline(x, threads, aff, target_s=12.0):
    """The headline line's CPU figure: the oracle (fp64, OpenMP over rows) on a
    bounded sample of evenly spaced query rows of the headline workload, all
    heads, all their visible keys; plus the whole small case (L = 512, inputs
    x 1/16) on one thread and on all threads."""
    import synth
    from long_context_causal_amd import work
    L = x.q.shape[2]
    full_pairs = work.visible_pairs(L, L)
    rec = cpu_entry("causal GQA fwd fp32 L=%d" % L, x, threads, full_pairs, target_s=target_s)
    xs = synth.gqa(1, HQ, HKV, 512, seed=0, scale=1.0 / 16)
    one = cpu_entry("causal GQA fwd fp32 L=512 (inputs x 1/16), one thread", xs, 1, 512 * 513 // 2, full=True)
    allt = cpu_entry("causal GQA fwd fp32 L=512 (inputs x 1/16)", xs, threads, 512 * 513 // 2, full=True)
    return dict(value=rec["value"], unit="TFLOP/s", cores=threads, kind="oracle",
                sample="%d of %d query rows (evenly spaced) x 16 heads of the fp32 causal forward at L=%d, all "
                       "their visible keys; %.1f s on %d threads" % (rec["rows"], L, L, rec["seconds"], threads),
                full_seconds_extrapolated=rec["full_seconds_extrapolated"],
                extrapolated="the whole workload's time, from the sample by visible (row, key) pairs",
                affinity_cpus=aff, cpu_model=cpu_model(), one_thread_L512=one, all_threads_L512=allt)


def cpu_branch(synth, threads, n_sample=2):
    """The oracle on the shared-prefix branch workload (S = 30,468, 40 branches
    of 256 rows): n_sample whole branches, each one call over concat(prefix,
    branch) with q_offset = S; the 40-branch time extrapolated by visible pairs."""
    import oracle
    br = synth.Branch(S=30468, n=40, m=256, seed=0, dtype="f32")
    S, m, n = br.S, br.m, br.n
    t = 0.0
    for b in range(n_sample):
        k_cat = np.concatenate([br.k_p[None], br.k_b[b:b + 1]], axis=2)
        v_cat = np.concatenate([br.v_p[None], br.v_b[b:b + 1]], axis=2)
        t0 = time.perf_counter()
        oracle.attn(br.q_b[b:b + 1], k_cat, v_cat, causal=True, q_offset=S, nthreads=threads)
        t += time.perf_counter() - t0
    pairs_per_branch = m * S + m * (m + 1) // 2
    fl = 4 * D * HQ * pairs_per_branch * n_sample
    return dict(workload="branch f32 S=30468 n=40 m=256", threads=threads, rows=n_sample * m, rows_total=n * m,
                seconds=round(t, 3), value=fl / t / 1e12, unit="TFLOP/s", kind="sampled",
                full_seconds_extrapolated=round(t * n / n_sample, 1),
                note="%d of the 40 branches, whole; the 40-branch time extrapolated by visible pairs" % n_sample)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo, else lscpu), with its family,
    model and stepping numbers where /proc/cpuinfo gives them (a virtual
    machine may list only the brand), or None where neither lists a name."""
    name, ids = None, {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "model name":
                    name = val.strip()
                elif key in ("cpu family", "model", "stepping"):
                    ids[key] = val.strip()
    except OSError:
        pass
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                lname = line.split(":", 1)[1].strip()
                if not name or len(lname) > len(name):
                    name = lname
    except (OSError, subprocess.SubprocessError):
        pass
    if name and len(ids) == 3:
        name += " (family %s, model %s, stepping %s)" % (ids["cpu family"], ids["model"], ids["stepping"])
    return name


# Sources and translation unit of each forward kernel.
KERNEL_SOURCES = {"f32": (["common.hpp", "launch.hpp", "fwd_f32.hpp", "fwd_f32.hip"], "fwd_f32.hip"),
                  "bf16": (["common.hpp", "launch.hpp", "elem16.hpp", "fwd_h16.hpp", "fwd_h16.hip"], "fwd_h16.hip"),
                  "f16": (["common.hpp", "launch.hpp", "elem16.hpp", "fwd_h16.hpp", "fwd_h16.hip"], "fwd_h16.hip")}


def kernel_dtype(name: str) -> str:
    """'bf16', 'f16' or 'f32' from a kernel or workload name; kernel names may be
    mangled (DF16b is __bf16, DF16_ is _Float16)."""
    if "bf16" in name or "DF16b" in name:
        return "bf16"
    if "fp16" in name or "_Float16" in name or "DF16_" in name or name.startswith("f16"):
        return "f16"
    return "f32"


def kernel_source_hash(dtype: str) -> str:
    """Hash of one forward kernel's sources and compile flags, so stored counter
    readings are only used for the kernel build they were taken on."""
    import hashlib
    from long_context_causal_amd import build as gbuild
    files, unit = KERNEL_SOURCES[dtype]
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_causal_amd", "csrc")
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    h.update(repr(gbuild.COMMON_FLAGS + gbuild.UNITS[unit]).encode())
    return h.hexdigest()[:16]


def pmc_dispatches(db_path):
    """Per kernel dispatch of a rocprofv3 database: kernel name, duration (ns)
    and each counter's value (summed over the counter's instances, except
    GRBM_GUI_ACTIVE, one value per XCD, of which the largest is taken)."""
    import sqlite3
    from collections import defaultdict
    con = sqlite3.connect(db_path)
    vals = defaultdict(lambda: defaultdict(list))
    info = {}
    for did, name, dur, cname, val in con.execute(
            "select dispatch_id, name, duration, counter_name, counter_value from pmc_events"):
        vals[did][cname].append(float(val))
        info[did] = (name, float(dur))
    out = []
    for did in sorted(vals):
        c = {k: (max(v) if k == "GRBM_GUI_ACTIVE" else sum(v)) for k, v in vals[did].items()}
        out.append(dict(dispatch=did, name=info[did][0], duration_ns=info[did][1], counters=c))
    return out


def dispatch_groups(disp):
    """Dispatches grouped by kernel name and size: within a name, durations
    more than 4x apart fall in different groups (the branch form launches the
    forward kernel for the long prefix part and the short suffix part). The
    first dispatch of each name (code-object load) is left out when there are
    others."""
    from collections import defaultdict
    byname = defaultdict(list)
    for d in disp:
        byname[d["name"]].append(d)
    groups = []
    for name, ds in byname.items():
        ds = ds[1:] if len(ds) > 1 else ds
        ds = sorted(ds, key=lambda d: d["duration_ns"])
        cur = [ds[0]]
        for d in ds[1:]:
            if d["duration_ns"] > 4 * cur[-1]["duration_ns"]:
                groups.append((name, cur))
                cur = []
            cur.append(d)
        groups.append((name, cur))
    return groups


def group_means(ds):
    keys = set().union(*(d["counters"] for d in ds))
    return (sum(d["duration_ns"] for d in ds) / len(ds),
            {k: sum(d["counters"].get(k, 0.0) for d in ds) / len(ds) for k in keys})


def pmc_summary(dbs):
    """Markdown rows per (kernel, size group) of rocprofv3 --pmc databases:
    mean duration and counters per dispatch, and the derived figures (shader
    clock = GRBM_GUI_ACTIVE / duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE x 1024 SIMDs); busy at 2.4 GHz = SQ_VALU_MFMA_BUSY_CYCLES /
    (1024 x 2.4 GHz x duration); executed MFMA flops = MOPS x 512; L2 hit rate;
    SQ_* cycle counters as fractions of SQ_WAVE_CYCLES)."""
    lines = []
    for db in dbs:
        for name, ds in dispatch_groups(pmc_dispatches(db)):
            dur, c = group_means(ds)
            parts = ["%s x%d" % (name[:60], len(ds)), "%.3f ms" % (dur * 1e-6)]
            if "GRBM_GUI_ACTIVE" in c and dur > 0:
                parts.append("clock %.2f GHz" % (c["GRBM_GUI_ACTIVE"] / dur))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
                b = c["SQ_VALU_MFMA_BUSY_CYCLES"]
                parts.append("MFMA busy %.1f%%" % (100 * b / (c["GRBM_GUI_ACTIVE"] * 1024)))
                parts.append("busy at 2.4 GHz %.1f%%" % (100 * b / (1024 * 2.4 * dur)))
            for m in ("SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16"):
                if c.get(m):
                    parts.append("%s x 512 = %.4g flops" % (m, c[m] * 512))
            if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
                tot = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
                parts.append("L2 hit %.1f%% (%.3g requests)" % (100 * c["TCC_HIT_sum"] / max(tot, 1), tot))
            if c.get("SQ_WAVE_CYCLES"):
                wc = c["SQ_WAVE_CYCLES"]
                parts.append("SQ_WAVE_CYCLES %.4g" % wc)
                for k in sorted(c):
                    if k.startswith("SQ_") and k not in ("SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES") and \
                            not k.startswith("SQ_INSTS_VALU_MFMA"):
                        parts.append("%s %.1f%%" % (k, 100 * c[k] / wc))
            for k in ("FETCH_SIZE", "WRITE_SIZE"):
                if k in c:
                    parts.append("%s %.6g KiB" % (k, c[k]))
            lines.append("| " + " | ".join(parts) + " |")
    return "\n".join(lines)


def pmc_report(fetch_db, write_db, kernel_substr, workload, out_path):
    """HBM traffic per dispatch of the attention kernel from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reports
    for a plain device copy of 1 GiB read + 1 GiB written in the same process.
    Where the kernel name matches dispatches of different sizes, the group of
    the longest ones is taken (the dominant launch)."""
    def pick(db, sub, counter):
        gs = [(n, ds) for n, ds in dispatch_groups(pmc_dispatches(db)) if sub in n]
        assert gs, (sub, counter)
        n, ds = max(gs, key=lambda g: group_means(g[1])[0])
        return group_means(ds)[1][counter], n

    fk, kname = pick(fetch_db, kernel_substr, "FETCH_SIZE")
    wk, _ = pick(write_db, kernel_substr, "WRITE_SIZE")
    fc, _ = pick(fetch_db, "copyBuffer", "FETCH_SIZE")
    wc, _ = pick(write_db, "copyBuffer", "WRITE_SIZE")
    gib = float(1 << 30)
    fetch_scale, write_scale = gib / (fc * 1024.0), gib / (wc * 1024.0)
    rec = {"workload": workload, "kernel": kname, "kernel_src_sha": kernel_source_hash(kernel_dtype(workload)),
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk,
           "copy_fetch_kib": fc, "copy_write_kib": wc, "fetch_scale": fetch_scale, "write_scale": write_scale,
           "traffic_bytes": fk * 1024.0 * fetch_scale + wk * 1024.0 * write_scale}
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def stored_traffic(workload):
    """Counter-derived HBM bytes per launch for `workload`, or None if absent or
    taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    recs = json.load(open(p))
    rec = recs.get(workload)
    if rec is None or rec.get("kernel_src_sha") != kernel_source_hash(kernel_dtype(workload)):
        return None
    return rec["traffic_bytes"]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="primary workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None,
                    help="run one workload: f32-15231, f32-30468, f32-60926, bf16-60926, f16-60926, "
                         "seg-bf16-131072, segidx-bf16-131072, noids-bf16-131072, branch-f32, bwd-f32-30468, bwd-bf16-60926, "
                         "split-decode-bf16, split-decode1-bf16, split-decode-f32, split-decode1-f32, "
                         "split-branch-f32, cp-f32-30468")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle on the whole headline workload (every row, all threads; "
                         "about 90 s on 16 host threads at L=30468)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (3 times) to calibrate HBM byte counters")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DB",
                    help="print per-kernel counter means and derived figures of rocprofv3 --pmc databases")
    ap.add_argument("--pmc-report", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "KERNEL_SUBSTR", "WORKLOAD"),
                    help="turn two rocprofv3 --pmc databases (FETCH_SIZE, WRITE_SIZE) into HBM bytes per "
                         "dispatch and store them in profiles/traffic.json under WORKLOAD")
    args = ap.parse_args()
    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary))
        return
    if args.pmc_report:
        fdb, wdb, sub, wl = args.pmc_report
        tmp = os.path.join(ROOT, "profiles", ".traffic_one.json")
        pmc_report(fdb, wdb, sub, wl, tmp)
        p = os.path.join(ROOT, "profiles", "traffic.json")
        recs = json.load(open(p)) if os.path.exists(p) else {}
        recs[wl] = json.load(open(tmp))
        os.remove(tmp)
        with open(p, "w") as fh:
            json.dump(recs, fh, indent=1, sort_keys=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward is not sharded across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_causal_amd as gqa
    import synth
    from long_context_causal_amd import work

    gqa.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    workloads = {
        "f32-15231": ("causal GQA fwd fp32 B=1 Hq=16 Hkv=4 D=256 L=15231", 15231, "f32"),
        "f32-30468": ("causal GQA fwd fp32 B=1 Hq=16 Hkv=4 D=256 L=30468", 30468, "f32"),
        "f32-60926": ("causal GQA fwd fp32 B=1 Hq=16 Hkv=4 D=256 L=60926", 60926, "f32"),
        "bf16-60926": ("causal GQA fwd bf16 B=1 Hq=16 Hkv=4 D=256 L=60926", 60926, "bf16"),
        "f16-60926": ("causal GQA fwd fp16 B=1 Hq=16 Hkv=4 D=256 L=60926", 60926, "f16"),
    }
    bwd_workloads = {
        "bwd-f32-30468": ("causal GQA bwd fp32 B=1 Hq=16 Hkv=4 D=256 L=30468", 30468, "f32"),
        "bwd-bf16-60926": ("causal GQA bwd bf16 B=1 Hq=16 Hkv=4 D=256 L=60926", 60926, "bf16"),
    }
    split_workloads = {
        "split-decode-bf16": ("split-KV decode bf16 Lq=16 over Lk=60926", 16, 60926, "bf16"),
        "split-decode1-bf16": ("split-KV decode bf16 Lq=1 over Lk=60926", 1, 60926, "bf16"),
        "split-decode-f32": ("split-KV decode fp32 Lq=16 over Lk=60926", 16, 60926, "f32"),
        "split-decode1-f32": ("split-KV decode fp32 Lq=1 over Lk=60926", 1, 60926, "f32"),
        "split-branch-f32": ("split-KV branch fp32 m=256 over S=30468 (Lk=30724)", 256, 30724, "f32"),
    }
    if args.only in split_workloads:
        # a profiling aid: the split-KV workload alone, its record on one line
        nm, Lq_, Lk_, dts = split_workloads[args.only]
        xs = synth.gqa(1, HQ, HKV, Lq_, Lk_, seed=0, dtype=dts, q_offset=Lk_ - Lq_)
        print(json.dumps(run_split_workload(nm, xs, args.steps, args.warmup, torch, gqa, work)), flush=True)
        return
    if args.only == "cp-f32-30468":
        # a profiling aid: the context-parallel shards alone, beside the whole call
        xs = synth.gqa(1, HQ, HKV, 30468, seed=0, dtype="f32")
        whole = run_fwd_workload(workloads["f32-30468"][0], xs, args.steps, args.warmup, torch, gqa, work)
        print(json.dumps(run_shards(xs, whole["kernel_ms"], (2, 4, 8), args.steps, args.warmup, torch, gqa)),
              flush=True)
        return
    if args.only in bwd_workloads:
        # a profiling aid: the backward alone, its record on one line
        nm, Ls, dts = bwd_workloads[args.only]
        r = run_bwd_workload(nm, synth.gqa(1, HQ, HKV, Ls, seed=0, dtype=dts), args.steps, args.warmup, torch, gqa,
                             work, synth)
        r["pct_mfma_peak"] = 100.0 * r["kernel_tflops"] / work.PEAK_TFLOPS[dts]
        r["pct_mfma_peak_exec"] = 100.0 * r["exec_tflops"] / work.PEAK_TFLOPS[dts]
        print(json.dumps(r), flush=True)
        return
    Lseg = 131072
    if args.only in ("seg-bf16-131072", "segidx-bf16-131072", "noids-bf16-131072"):
        # a profiling aid: the packed-segment workload (plain or through the id
        # index) or its id-free comparator alone
        lens = synth.segment_lengths(Lseg, 2048, 32768, seed=1)
        xs = synth.gqa(1, HQ, HKV, Lseg, seed=0, dtype="bf16")
        seg = synth.segment_ids(lens) if args.only.startswith("seg") else None
        indexed = args.only.startswith("segidx")
        nm = ("segmented bf16 L=131072, %d segments (2k-32k)%s" % (len(lens), SEG_IDX_NOTE if indexed else "")
              if seg is not None else "single-segment comparator bf16 L=131072 (no ids)")
        r = run_fwd_workload(nm, xs, args.steps, args.warmup, torch, gqa, work, seg=seg, indexed=indexed)
        r["pct_mfma_peak"] = 100.0 * r["kernel_tflops"] / work.PEAK_TFLOPS["bf16"]
        if args.copy_probe:
            r["copy_probe_bytes"] = copy_probe(torch)
        print(json.dumps(r), flush=True)
        return
    if args.only == "branch-f32":
        # a profiling aid: the shared-prefix branch workload alone
        r = run_branch(args.steps, args.warmup, torch, gqa, work, synth)
        r["pct_mfma_peak"] = 100.0 * r["kernel_tflops"] / work.PEAK_TFLOPS["f32"]
        if args.copy_probe:
            r["copy_probe_bytes"] = copy_probe(torch)
        print(json.dumps(r), flush=True)
        return
    threads, aff = cpu_threads()
    cpu = not args.no_cpu
    cpu_cfg = []
    primary_key = args.only or "f32-30468"
    name, L, dt = workloads[primary_key]
    x = synth.gqa(1, HQ, HKV, L, seed=0, dtype=dt)
    prim = run_fwd_workload(name, x, args.steps, args.warmup, torch, gqa, work)
    peak_t = work.PEAK_TFLOPS[dt]

    secondary = []
    shards = None
    if not args.quick and args.only is None:
        if cpu:
            # the whole small case on all threads and the oracle beside each workload below:
            # whole where it takes seconds (L = 15,231), else sampled rows, extrapolated
            xs = synth.gqa(1, HQ, HKV, 512, seed=0, scale=1.0 / 16)
            cpu_cfg.append(cpu_entry("causal GQA fwd fp32 L=512 (inputs x 1/16)", xs, threads, 512 * 513 // 2,
                                     full=True))
        for key in ("f32-15231", "f32-60926", "bf16-60926", "f16-60926"):
            nm, Ls, dts = workloads[key]
            xs = synth.gqa(1, HQ, HKV, Ls, seed=0, dtype=dts)
            r = run_fwd_workload(nm, xs, max(3, args.steps // 2), 2, torch, gqa, work)
            if cpu and key != "f16-60926":
                cpu_cfg.append(cpu_entry(nm, xs, threads, work.visible_pairs(Ls, Ls), full=(key == "f32-15231")))
            del xs
            secondary.append(r)
        secondary.append(run_branch(max(3, args.steps // 2), 2, torch, gqa, work, synth))
        if cpu:
            cpu_cfg.append(cpu_branch(synth, threads))
        # the backward (training): fp32 at L = 30,468 and bf16 at L = 60,926
        for nm, Ls, dts in bwd_workloads.values():
            xs = synth.gqa(1, HQ, HKV, Ls, seed=0, dtype=dts)
            secondary.append(run_bwd_workload(nm, xs, max(3, args.steps // 2), 2, torch, gqa, work, synth))
            del xs
        # split-KV: 16 and 1 decode positions over the 64k state (bf16 and
        # fp32, the fp32 server's step) and one 256-row branch over the 30k
        # prefix (fp32)
        for nm, Lq_, Lk_, dts in split_workloads.values():
            xs = synth.gqa(1, HQ, HKV, Lq_, Lk_, seed=0, dtype=dts, q_offset=Lk_ - Lq_)
            secondary.append(run_split_workload(nm, xs, max(5, args.steps), 3, torch, gqa, work))
            del xs
        # packed segments, bf16, L = 131,072, lengths uniform in [2k, 32k] (seed 1), and the
        # single-segment comparator at the same L
        Lseg = 131072
        lens = synth.segment_lengths(Lseg, 2048, 32768, seed=1)
        ids = synth.segment_ids(lens)
        xs = synth.gqa(1, HQ, HKV, Lseg, seed=0, dtype="bf16")
        r = run_fwd_workload("segmented bf16 L=131072, %d segments (2k-32k)" % len(lens), xs,
                             max(3, args.steps // 2), 2, torch, gqa, work, seg=ids)
        secondary.append(r)
        if cpu:
            cpu_cfg.append(cpu_entry(r["workload"], xs, threads, r["flops"] // (4 * D * HQ), seg=ids))
        r = run_fwd_workload("segmented bf16 L=131072, %d segments (2k-32k)%s" % (len(lens), SEG_IDX_NOTE), xs,
                             max(3, args.steps // 2), 2, torch, gqa, work, seg=ids, indexed=True)
        secondary.append(r)
        r = run_fwd_workload("single-segment comparator bf16 L=131072 (no ids)", xs, 3, 1, torch, gqa, work)
        secondary.append(r)
        r = run_bwd_workload("segmented bwd bf16 L=131072, %d segments (2k-32k)" % len(lens), xs, 3, 1, torch, gqa,
                             work, synth, seg=ids)
        secondary.append(r)
        r = run_bwd_workload("segmented bwd bf16 L=131072, %d segments (2k-32k)%s" % (len(lens), SEG_IDX_NOTE), xs,
                             3, 1, torch, gqa, work, synth, seg=ids, indexed=True)
        secondary.append(r)
        del xs
        # context-parallel shards of the headline workload, N = 2, 4, 8 ranks
        shards = run_shards(x, prim["kernel_ms"], (2, 4, 8), 3, 1, torch, gqa)
    for r in [prim] + secondary:
        dts = "bf16" if "bf16" in r["workload"] else "f16" if "fp16" in r["workload"] else "f32"
        r["pct_mfma_peak"] = 100.0 * r["kernel_tflops"] / work.PEAK_TFLOPS[dts]
        r["traffic"] = stored_traffic(r["workload"])
        if "exec_tflops" in r:
            r["pct_mfma_peak_exec"] = 100.0 * r["exec_tflops"] / work.PEAK_TFLOPS[dts]

    math_gib = work.score_matrix_bytes(HQ, L, L, 4) / 2 ** 30
    out = {
        "metric": METRIC,
        "value": round(prim["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic: Q/K/V i.i.d. N(0,1), seed 0 (stand-in for post-RoPE activations)",
        "config": {"workload": name, "B": 1, "Hq": HQ, "Hkv": HKV, "D": D, "seq_len": L, "causal": True,
                   "flops_per_step": prim["flops"]},
        "pct_mfma_peak": round(100.0 * prim["kernel_tflops"] / peak_t, 2),
        "peak_gib": round(prim["peak_gib"], 3),
        "math_path_gib": round(math_gib, 2),
        "library_alloc_bytes": prim["library_alloc_bytes"],
        "kernel_ms_stats": {"mean": round(prim["kernel_ms"], 4), "median": round(prim["kernel_ms_median"], 4),
                            "min": round(prim["kernel_ms_min"], 4), "max": round(prim["kernel_ms_max"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(prim["kernel_tflops"], 3), "peak": peak_t,
                     "unit": "TFLOP/s", "frac": round(prim["kernel_tflops"] / peak_t, 4),
                     "traffic": stored_traffic(name), "kernel_ms": round(prim["kernel_ms"], 4),
                     "algorithmic_bytes": prim["bytes"]},
    }
    if secondary:
        out["secondary"] = [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in secondary]
    if shards is not None:
        out["context_parallel_shards"] = shards
    if args.copy_probe:
        out["copy_probe_bytes"] = copy_probe(torch)
    if cpu:
        out["cpu_baseline"] = cpu_baseline(x, threads, aff)
        if args.cpu_full:
            from long_context_causal_amd import work as _work
            Lh = x.q.shape[2]
            print("bench: timing the oracle on the whole fp32 L=%d forward on %d threads" % (Lh, threads),
                  file=sys.stderr, flush=True)
            full = cpu_entry("causal GQA fwd fp32 L=%d, every row" % Lh, x, threads, _work.visible_pairs(Lh, Lh),
                             full=True)
            out["cpu_baseline"]["full"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in full.items()}
        if cpu_cfg:
            out["cpu_baseline"]["per_config"] = [{k: (round(v, 5) if isinstance(v, float) else v)
                                                 for k, v in c.items()} for c in cpu_cfg]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
