"""Decode-attention benchmark on one MI355X: KV HBM GB/s and sequences x steps / s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: kvc_block_table (paged
caches), kvc_append of every sequence's new rows, kvc_attn_partition and
kvc_attn_reduce.  The prepared step reads its lengths and free-list head from
buffers it never writes, so replaying it K times does identical work each
time; the cache and all inputs are resident in HBM before the timed region.

Printed: one JSON line.  value = KV bytes attended per step / the median time
of a step timed alone behind a 1 GiB write (no KV row comes from the
last-level caches), over --flush-iters steps; roofline.achieved = the same
bytes / the median of those steps' partition launches, HIP events on the
stream the kernels run on.  The K steps of the timed region (back to back,
between two synchronisations) are reported as 'steady'.  The same protocol
is applied to the other target workloads ('configs'), the paged and
contiguous forms of the 16 x 2048 layer are compared, a streaming-read probe
gives the device's read ceiling, and the oracle is timed on the host (one
thread, and every core).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV HBM GB/s (% of peak) + sequences·steps/sec at given ctx"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores
PREFILL_METRIC = "prefill attention TFLOP/s (causal visible pairs x 4 x head_dim x q heads)"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cached_decode_kvc_amd", "csrc")


def kernel_of(w, mfma: bool, stream_k: bool = False) -> tuple[str, list[str]]:
    """Name of the dominant kernel and the sources that define it (stream_k:
    the plan has no partition length)."""
    if w.dv:
        return "partition_mla", ["attn_mla.hip", "common.hpp"]
    if w.prefill:
        return "prefill_mfma", ["attn_prefill.hip", "common.hpp"]
    if mfma:
        return "partition_mfma", ["attn_mfma.hip", "common.hpp"]
    return ("partition_valu_sk" if stream_k else "partition_valu"), ["attn_valu.hip", "common.hpp"]


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != src_hash:
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rows(w, b):
    """Sequence b's attended rows as the oracle takes them, from the generator:
    (k, v) [Hkv, L, D] (MLA: the latent rows [L, Dk], None); an FP8 workload
    gets the oracle's own quantization of the rows, dequantized exactly."""
    import numpy as np

    import oracle
    from kv_cached_decode_kvc_amd import synth

    ref = oracle.get()
    cached = synth.cached_lengths(w)
    kv = []
    for x in (("k",) if w.dv else ("k", "v")):
        rows = np.concatenate([synth.cache_rows(w, x, b, int(cached[b])),
                               synth.new_rows(w, x, b)]).transpose(1, 0, 2).copy()
        if w.kv:
            rows = ref.dequantize_rows(*ref.quantize_rows(rows, w.kv), w.kv)
        kv.append(rows)
    if w.dv:
        return kv[0][0], None
    return kv[0], kv[1]


def cpu_baseline(w, seconds: float, gpu_out=None):
    """The oracle (float64) timed on this host, on a bounded sample of the same
    workload: the batch's whole sequences, cycled until `seconds` of oracle
    time per leg.  Two legs on the same rows: the single-threaded definition,
    and the many-sequence function (OpenMP over (sequence, query head) on every
    host core, the same arithmetic).  Row generation is not timed."""
    import numpy as np

    import oracle
    from kv_cached_decode_kvc_amd import metrics, synth

    ref = oracle.get()
    lens = synth.final_lengths(w)
    scale = 1.0 / math.sqrt(w.D)
    dt = "f64" if w.kv else w.dtype
    with ThreadPoolExecutor(max_workers=16) as ex:  # row generation, not timed
        rows = list(ex.map(lambda b: oracle_rows(w, b), range(w.B)))
    qs = [synth.queries(w, b) for b in range(w.B)]
    if w.kv:
        qs = [oracle.widen(q, "bf16") for q in qs]
    seq_bytes = [metrics.attended_cache_bytes([lens[b]], w.Hkv, w.kv_row_bytes, w.kv_tensors)
                 for b in range(w.B)]

    # single thread: one sequence per call, batch order, cycled
    spent, nbytes, nseq, worst = 0.0, 0, 0, 0.0
    b = 0
    while spent < seconds:
        k, v = rows[b]
        t0 = time.perf_counter()
        if w.dv:
            want = ref.mla_attention(qs[b], k, scale, w.dv)
        else:
            want = ref.attention(qs[b], k, v, scale, dt)
        spent += time.perf_counter() - t0
        nbytes += seq_bytes[b]
        nseq += 1
        if gpu_out is not None and nseq <= w.B:
            worst = max(worst, float(np.abs(gpu_out[b] - want).max()))
        b = (b + 1) % w.B
    single = {
        "value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
        "seq_steps_per_s": round(nseq / spent, 3),
        "sample": "%d whole sequences (batch order, cycled), %.1f s of oracle time" % (
            nseq, spent),
        "sample_max_abs_err_vs_gpu": worst if gpu_out is not None else None,
    }

    # every host core: the whole batch per call, cycled
    spent, nbytes, nseq, threads = 0.0, 0, 0, 0
    ks = [r[0] for r in rows]
    vs = None if w.dv else [r[1] for r in rows]
    while spent < seconds:
        t0 = time.perf_counter()
        _, threads = ref.attention_many(qs, ks, vs, scale, dt, dv=w.dv)
        spent += time.perf_counter() - t0
        nbytes += sum(seq_bytes)
        nseq += w.B
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {
        "value": round(nbytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "the batch's %d whole sequences per call, cycled %d times; float64; OpenMP over "
                  "(sequence, query head) on %d threads; %.1f s of oracle time; %.4g "
                  "sequence-steps/s" % (w.B, nseq // max(w.B, 1), threads, spent, nseq / spent),
        "seq_steps_per_s": round(nseq / spent, 3),
        "cpu_model": cpu_model(),
        "nproc": nproc,
        "single_thread": single,
    }


def pct(xs, q):
    import numpy as np
    return round(float(np.percentile(np.asarray(xs, dtype=np.float64), q)), 3)


def flushed_runs(run, iters: int, flush_bytes: int = 1 << 30):
    """Duration of `run` (launches on torch's current stream, the library's
    stream) with no KV row in the last-level caches, from HIP events.

    An event recorded just before a kernel adds the dispatch gap that follows
    it (about 5 us in the kernel trace, against none between two kernels), so
    a single run's event interval overstates it.  Each iteration therefore
    times, behind a 1 GiB write each: A = [run, 1 GiB write] and B = [run,
    1 GiB write, run].  B - A is one run that follows a 1 GiB write with no
    event before it -- a flushed run without the marker's gap.  Returns
    (durations B - A, single-run event intervals [run]), microseconds."""
    import torch
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    dur, single = [], []
    for i in range(iters):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        buf.fill_(float(i))
        e[0].record()
        run()
        e[1].record()
        buf.fill_(float(i) + 0.25)
        e[2].record()
        run()
        buf.fill_(float(i) + 0.5)
        e[3].record()
        buf.fill_(float(i) + 0.75)
        e[4].record()
        run()
        buf.fill_(float(i) + 0.125)
        run()
        e[5].record()
        torch.cuda.synchronize()
        single.append(e[0].elapsed_time(e[1]) * 1e3)
        dur.append((e[4].elapsed_time(e[5]) - e[2].elapsed_time(e[3])) * 1e3)
    del buf
    return dur, single


def attn_launch(lc):
    """The launch the roofline times: the attention call when it is one
    launch (the partition kernel combining its own partials, as the step
    runs it), else its partition launch alone (a reduce launch follows; MLA
    too); the prefill kernel."""
    from kv_cached_decode_kvc_amd import kvc
    if lc.w.dv or lc.w.prefill or kvc.kvc_attn_launches(lc.desc, lc.w.n_q) != 1:
        return lc.step_partition
    return lc.step_attn


def flushed_steps(lc, iters: int, flush_bytes: int = 1 << 30):
    """Whole steps and partition launches, each timed by flushed_runs.
    Returns (step us, partition us, step event intervals, partition event
    intervals)."""
    st, st_ev = flushed_runs(lc.step, iters, flush_bytes)
    pt, pt_ev = flushed_runs(attn_launch(lc), iters, flush_bytes)
    return st, pt, st_ev, pt_ev


class CallTimer:
    """HIP events between consecutive library calls on torch's current stream
    (the stream the binding launches on); per-call medians in microseconds.
    Each round starts behind a 1 GiB fill, which flushes the caches and keeps
    the device busy while the host enqueues the round, so that the events time
    the device and not the host's launch rate."""

    def __init__(self):
        import torch
        self.samples = {}
        self.pending = []
        self.lead = torch.empty((1 << 30) // 4, dtype=torch.float32, device="cuda")

    def start(self):
        import torch
        self.lead.fill_(1.0)
        self.pending = [(None, torch.cuda.Event(enable_timing=True))]
        self.pending[0][1].record()

    def mark(self, name):
        import torch
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pending.append((name, e))

    def collect(self):
        import torch
        torch.cuda.synchronize()
        for (_, a), (name, b) in zip(self.pending, self.pending[1:]):
            if name is not None:
                self.samples.setdefault(name, []).append(a.elapsed_time(b) * 1e3)
        self.pending = []

    def medians(self):
        return {k: pct(v, 50) for k, v in self.samples.items()}


def lifecycle_bench(iters: int, warmup: int):
    """Per-call device time of the block-lifecycle entry points in two
    replayable round trips, plus the block-copy bandwidth.

    speculative: the 5-row verify workload; each round runs copy-on-write,
      allocation and append of the 5 rows, attention, then truncation to the
      base length plus a seeded accepted count (0..5); an untimed truncation
      back to the base length restores the state.
    parallel sampling: 32 prompts (GQA 32/8, lengths 1024..4096) each forked
      into 4 samples (B = 128); each round forks, copies the shared partly
      filled last blocks, appends one token to every sample, attends, and
      releases the 96 forked samples (the timed truncation); an untimed
      truncation returns the prompts to their length.
    """
    import numpy as np
    import torch

    from kv_cached_decode_kvc_amd import kvc, metrics, runner, synth

    dev = "cuda"
    out = {"metric": "block-lifecycle call latency (us, median of HIP-event times)",
           "iters": iters, "warmup": warmup}

    # -- speculative rollback on the verify workload ----------------------
    w = synth.get("C5")
    lc = runner.build(w)
    refs = torch.zeros(lc.N, dtype=torch.int32, device=dev)
    src = torch.empty(w.B, dtype=torch.int32, device=dev)
    dst = torch.empty(w.B, dtype=torch.int32, device=dev)
    h = [torch.empty(1, dtype=torch.int32, device=dev) for _ in range(4)]
    l_t = torch.empty_like(lc.seq_lens)
    l_r = torch.empty_like(lc.seq_lens)
    rng = np.random.default_rng(55)
    accepted = [runner.i32(lc.s_len0.cpu().numpy() + rng.integers(0, w.n_q + 1, size=w.B), dev)
                for _ in range(8)]
    t = CallTimer()
    for it in range(warmup + iters):
        t.start()
        kvc.kvc_cow(lc.desc, lc.s_len0, lc.s_cu, lc.table, lc.free_list, lc.s_head0, h[0], refs,
                    lc.k, lc.v, src, dst, lc.status)
        t.mark("cow")
        kvc.kvc_block_table(lc.desc, lc.s_len0, lc.s_cu, lc.s_total, lc.table, lc.free_list,
                            h[0], h[1], lc.s_slots, lc.status)
        t.mark("block_table")
        kvc.kvc_append(lc.desc, lc.s_k, lc.s_v, lc.s_len0, lc.s_cu, lc.s_total, w.n_q,
                       lc.s_slots, lc.k, lc.v, lc.s_len1, lc.status)
        t.mark("append")
        lc.step_attn()
        t.mark("attention")
        kvc.kvc_truncate(lc.desc, lc.s_len1, accepted[it % 8], lc.table, lc.free_list, h[1],
                         h[2], refs, l_t, lc.status)
        t.mark("truncate")
        kvc.kvc_truncate(lc.desc, l_t, lc.s_len0, lc.table, lc.free_list, h[2], h[3], refs, l_r,
                         lc.status)
        if it >= warmup:
            t.collect()
        else:
            t.pending = []
    torch.cuda.synchronize()
    assert lc.dev_status() == 0, lc.dev_status()
    assert int(h[3].item()) == int(lc.s_head0.item())
    med = t.medians()
    step = sum(med.values())
    out["speculative"] = {
        "workload": w.name, "draft_rows": w.n_q, "calls_us": med, "round_us": round(step, 3),
        "lifecycle_share": round((med["cow"] + med["truncate"]) / step, 4),
        "verify_rows_per_s": round(w.B * w.n_q / (step * 1e-6), 1),
    }
    del lc

    # -- parallel sampling: fork + copy-on-write ---------------------------
    ws = synth.custom(name="parallel-sampling-32x4-gqa32x8-paged-ctx1024to4096", seed=6, B=128,
                      Hq=32, Hkv=8, D=128, dtype="bf16", block_size=16, n_q=1, len_lo=1024,
                      len_hi=4096)
    n_prompt = 32
    plen = synth.final_lengths(ws)[:n_prompt]
    pool = int(sum(-(-int(x) // 16) + 1 for x in plen) * 4 + ws.B)
    lc = runner.LayerCache(ws, block_size=16, capacity=4112, pool_blocks=pool)
    lengths = np.zeros(ws.B, np.int64)
    lengths[:n_prompt] = plen
    lc.prefill(lengths)
    lc.prepare_step(0)
    torch.cuda.synchronize()
    head0 = lc.head.clone()
    base = lc.seq_lens.clone()
    parents = runner.i32(np.repeat(np.arange(n_prompt), 3), dev)
    children = runner.i32(np.arange(n_prompt, ws.B), dev)
    zero_children = base.clone()  # prompts keep their length, samples go to 0
    refs = torch.zeros(lc.N, dtype=torch.int32, device=dev)
    src = torch.empty(ws.B, dtype=torch.int32, device=dev)
    dst = torch.empty(ws.B, dtype=torch.int32, device=dev)
    l_a = torch.empty_like(lc.seq_lens)
    l_b = torch.empty_like(lc.seq_lens)
    prompt_only = runner.i32(np.where(np.arange(ws.B) < n_prompt, lengths + 1, 0), dev)
    t = CallTimer()
    for it in range(warmup + iters):
        lens = base.clone()
        t.start()
        kvc.kvc_fork(lc.desc, parents, children, ws.B - n_prompt, lens, lc.table, refs, lc.status)
        t.mark("fork")
        kvc.kvc_cow(lc.desc, lens, lc.s_cu, lc.table, lc.free_list, lc.head, lc.head, refs, lc.k,
                    lc.v, src, dst, lc.status)
        t.mark("cow")
        kvc.kvc_block_table(lc.desc, lens, lc.s_cu, lc.s_total, lc.table, lc.free_list, lc.head,
                            lc.head, lc.s_slots, lc.status)
        t.mark("block_table")
        kvc.kvc_append(lc.desc, lc.s_k, lc.s_v, lens, lc.s_cu, lc.s_total, 1, lc.s_slots, lc.k,
                       lc.v, l_a, lc.status)
        t.mark("append")
        kvc.kvc_decode_attn(lc.desc, lc.s_q, lc.k, lc.v, l_a, lc.table, lc.scale, lc.s_out,
                            lc.s_ws, lc.status)
        t.mark("attention")
        kvc.kvc_truncate(lc.desc, l_a, prompt_only, lc.table, lc.free_list, lc.head, lc.head,
                         refs, l_b, lc.status)
        t.mark("truncate")
        kvc.kvc_truncate(lc.desc, l_b, zero_children, lc.table, lc.free_list, lc.head, lc.head,
                         refs, lens, lc.status)
        if it >= warmup:
            t.collect()
        else:
            t.pending = []
    torch.cuda.synchronize()
    assert lc.dev_status() == 0, lc.dev_status()
    assert int(lc.head.item()) == int(head0.item())
    assert int(refs.abs().sum().item()) == 0
    med = t.medians()
    step = sum(med.values())
    att_bytes = metrics.attended_kv_bytes(np.repeat(plen + 1, 4), ws.Hkv, ws.D, ws.esize)
    out["parallel_sampling"] = {
        "workload": ws.name, "prompts": n_prompt, "samples_per_prompt": 4,
        "calls_us": med, "round_us": round(step, 3),
        "lifecycle_share": round((med["fork"] + med["cow"] + med["truncate"]) / step, 4),
        "attention_gbs": round(att_bytes / (med["attention"] * 1e-6) / 1e9, 2),
    }
    blk_bytes = ws.Hkv * 16 * ws.D * ws.esize
    del lc

    # -- block copies: bandwidth -------------------------------------------
    n = 4096
    desc = kvc.cache_desc(1, ws.Hq, ws.Hkv, ws.D, "bf16", 16, max_blocks_per_seq=1,
                          num_blocks=2 * n)
    kp = torch.zeros((2 * n, ws.Hkv, 16, ws.D), dtype=torch.bfloat16, device=dev)
    vp = torch.zeros_like(kp)
    perm = np.random.default_rng(7).permutation(2 * n).astype(np.int32)
    s_d, d_d = runner.i32(perm[:n], dev), runner.i32(perm[n:], dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    t = CallTimer()
    for it in range(warmup + iters):
        t.start()
        kvc.kvc_copy_blocks(desc, s_d, d_d, n, kp, vp, status)
        t.mark("copy_blocks")
        if it >= warmup:
            t.collect()
        else:
            t.pending = []
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    us = t.medians()["copy_blocks"]
    moved = 2 * 2 * n * blk_bytes  # K and V, read and write
    out["copy_blocks"] = {
        "pairs": n, "block_bytes_k": blk_bytes, "us": us,
        "gbs": round(moved / (us * 1e-6) / 1e9, 2),
        "hbm_frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    return out


def graph_replay(w, lc, replays: int = 50):
    """The workload's whole multi-step loop (block table, append, attention per
    step) captured once as a HIP graph and replayed; also the same loop issued
    eagerly from Python, for comparison."""
    import time

    import torch

    from kv_cached_decode_kvc_amd import metrics, runner, synth

    loop = runner.DecodeLoop(lc)
    g = loop.capture()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    t_graph = (time.perf_counter() - t0) / replays
    t0 = time.perf_counter()
    for _ in range(replays):
        loop.run()
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / replays
    assert lc.dev_status() == 0
    final = synth.final_lengths(w)
    loop_bytes = sum(metrics.attended_cache_bytes(final + s * w.n_q, w.Hkv, w.kv_row_bytes,
                                                  w.kv_tensors)
                     for s in range(w.steps))
    return {
        "steps_per_replay": w.steps, "replays": replays,
        "us_per_step": round(t_graph / w.steps * 1e6, 3),
        "eager_us_per_step": round(t_eager / w.steps * 1e6, 3),
        "kv_bytes_per_loop": loop_bytes,
        "gbs": round(loop_bytes / t_graph / 1e9, 3),
        "seq_steps_per_s": round(w.B * w.steps / t_graph, 1),
    }


def calibrate_copy(nbytes: int, reps: int):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def stats(xs) -> dict:
    return {"p10": pct(xs, 10), "median": pct(xs, 50), "p90": pct(xs, 90)}


def steady_partition_us(lc, n: int) -> float:
    """Average of n back-to-back partition launches (HIP events)."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    run = attn_launch(lc)
    ev0.record()
    for _ in range(n):
        run()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / n * 1e3


def kv_bytes_of(w) -> int:
    from kv_cached_decode_kvc_amd import metrics, synth
    return metrics.attended_cache_bytes(synth.final_lengths(w), w.Hkv, w.kv_row_bytes,
                                        w.kv_tensors)


def config_result(name: str, warmup: int, iters: int, steady: int) -> dict:
    """One of the other target workloads: flushed step and partition times
    (median, p10, p90 over `iters` iterations behind a 1 GiB write), steady
    back-to-back partition time, and for multi-step workloads the HIP-graph
    replay of the whole loop."""
    import torch

    from kv_cached_decode_kvc_amd import runner, synth

    w = synth.get(name)
    print("# config %s (%s): building" % (name, w.name), file=sys.stderr, flush=True)
    lc = runner.build(w)
    for _ in range(warmup):
        lc.step()
    torch.cuda.synchronize()
    assert lc.dev_status() == 0
    kvb = kv_bytes_of(w)
    st_us, pt_us, _, _ = flushed_steps(lc, iters)
    sp = steady_partition_us(lc, steady)
    assert lc.dev_status() == 0
    step_med, part_med = pct(st_us, 50), pct(pt_us, 50)
    res = {
        "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
        "query_rows": w.n_q, "cache": w.cache_dtype, "block_size": w.block_size,
        "kv_bytes_per_step": kvb, "flushed_iters": iters,
        "flushed_step_us": stats(st_us), "flushed_partition_us": stats(pt_us),
        "gbs_step": round(kvb / (step_med * 1e-6) / 1e9, 2),
        "hbm_frac_step": round(kvb / (step_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "gbs_partition": round(kvb / (part_med * 1e-6) / 1e9, 2),
        "hbm_frac_partition": round(kvb / (part_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(w.B / (step_med * 1e-6), 1),
        "query_rows_per_s": round(w.B * w.n_q / (step_med * 1e-6), 1),
        "steady_partition_us": round(sp, 3),
        "steady_hbm_frac_partition": round(kvb / (sp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if w.steps > 1:
        res["graph_replay"] = graph_replay(w, lc)
    del lc
    torch.cuda.empty_cache()
    return res


def paged_vs_contiguous(iters: int) -> dict:
    """The 16 x 2048 Llama-2-13B-shaped layer as a paged cache (block 16, the
    seeded permuted pool, the same seed and rows) against the contiguous one:
    flushed partition times at the same partition length (1024 keys) isolate
    the block-table indirection; the paged cache's own default length is shown
    too."""
    import torch

    from kv_cached_decode_kvc_amd import kvc, runner, synth

    wc = synth.get("C2")
    wp = synth.custom(name="llama2-13b-layer-paged16-b16-ctx2048", seed=wc.seed, B=wc.B,
                      Hq=wc.Hq, Hkv=wc.Hkv, D=wc.D, dtype=wc.dtype, block_size=16, n_q=1,
                      len_lo=wc.len_lo, len_hi=wc.len_hi)
    kvb = kv_bytes_of(wc)
    res = {"workload": wp.name, "kv_bytes_per_step": kvb, "flushed_iters": iters}
    print("# paged vs contiguous: building", file=sys.stderr, flush=True)
    for label, w, P in (("contiguous_p1024", wc, 0), ("paged_p1024", wp, 1024),
                        ("paged_default", wp, 0)):
        lc = runner.build(w, partition_tokens=P)
        lc.step()
        torch.cuda.synchronize()
        us, _ = flushed_runs(lc.step_partition, iters)
        assert lc.dev_status() == 0
        res[label] = {"partition_tokens": kvc.kvc_attn_partition_tokens(lc.desc, 1),
                      "flushed_partition_us": stats(us),
                      "hbm_frac": round(kvb / (pct(us, 50) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del lc
        torch.cuda.empty_cache()
    c, p = res["contiguous_p1024"]["flushed_partition_us"]["median"], \
        res["paged_p1024"]["flushed_partition_us"]["median"]
    res["paged_over_contiguous_same_partition"] = round(p / c, 4)
    res["paged_default_over_contiguous"] = round(
        res["paged_default"]["flushed_partition_us"]["median"] / c, 4)
    return res


def probe(iters: int = 20, nbytes: int = 2 << 30) -> dict:
    """Plain streaming-read probe (libkvc_probe.so): a 2 GiB buffer read once
    per launch (8x the last-level cache), ordinary and non-temporal 16-byte
    loads, three grid sizes; average of `iters` back-to-back launches."""
    import torch

    from kv_cached_decode_kvc_amd import probe as pr

    buf = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"bytes_per_launch": nbytes, "launches": iters}
    best = 0.0
    for nt in (False, True):
        for wg in (1024, 2048, 4096):
            for _ in range(3):
                pr.stream_read(buf, nt, wg, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                pr.stream_read(buf, nt, wg, sink)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / iters * 1e3
            gbs = nbytes / (us * 1e-6) / 1e9
            res["%s_wg%d_gbs" % ("nontemporal" if nt else "ordinary", wg)] = round(gbs, 1)
            best = max(best, gbs)
    res["best_gbs"] = round(best, 1)
    res["best_frac"] = round(best / HBM_PEAK_GBS, 4)
    del buf
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="steady-state steps timed back to back between two synchronisations")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C2")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time of each CPU-baseline leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--flush-iters", type=int, default=100,
                    help="steps timed one at a time behind a 1 GiB write (the headline)")
    ap.add_argument("--configs", default="C1,C3,C4,C5",
                    help="other workloads measured with the same protocol ('none': skip)")
    ap.add_argument("--no-paged-compare", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--probe", action="store_true", help="run the streaming-read probe only")
    ap.add_argument("--lifecycle", action="store_true",
                    help="time the block-lifecycle calls instead (speculative rollback, "
                         "parallel sampling, block copies)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library's path runs on a single MI355X "
              "(sequences and KV heads shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cached_decode_kvc_amd import kvc, metrics, runner, synth

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return

    if args.probe:
        print(json.dumps({"probe": probe()}), flush=True)
        return

    if args.lifecycle:
        print(json.dumps(lifecycle_bench(max(args.steps, 10), args.warmup)), flush=True)
        return

    w = synth.get(args.workload)
    print("# building %s on the device" % w.name, file=sys.stderr, flush=True)
    lc = runner.build(w, partition_tokens=args.partition_tokens)
    torch.cuda.synchronize()
    P = (kvc.kvc_mla_partition_tokens(lc.desc, w.n_q, w.dv) if w.dv
         else kvc.kvc_attn_partition_tokens(lc.desc, w.n_q))
    mfma = w.dtype == "bf16" and w.G * w.n_q >= 2  # bf16 and FP8 caches

    for _ in range(args.warmup):
        lc.step()
    torch.cuda.synchronize()
    assert lc.dev_status() == 0, "device status %d" % lc.dev_status()

    # the timed region: K steady steps back to back, between synchronisations
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        lc.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert lc.dev_status() == 0
    print("# %d steady steps: %.2f us/step" % (K, wall / K * 1e6), file=sys.stderr, flush=True)

    # the headline: steps timed one at a time behind a 1 GiB write, so that no
    # KV row comes from the last-level caches
    F = max(1, args.flush_iters)
    st_us, pt_us, st_ev, pt_ev = flushed_steps(lc, F)
    assert lc.dev_status() == 0
    print("# %d flushed steps: median %.2f us" % (F, pct(st_us, 50)), file=sys.stderr, flush=True)

    lens = synth.final_lengths(w)
    kv_bytes = metrics.attended_cache_bytes(lens, w.Hkv, w.kv_row_bytes, w.kv_tensors)
    # score and value products, 2 FLOP per multiply-add, over every visible (row, key)
    flops = metrics.attention_flops(lens, w.n_q, w.Hq, w.D) // 2 + \
        metrics.attention_flops(lens, w.n_q, w.Hq, w.out_dim) // 2
    step_us, part_us = pct(st_us, 50), pct(pt_us, 50)
    value = kv_bytes / (step_us * 1e-6) / 1e9
    achieved = kv_bytes / (part_us * 1e-6) / 1e9
    steady_ms = wall / K * 1e3
    kname, ksrc = kernel_of(w, mfma, stream_k=P == 0)
    shash = source_hash(ksrc)
    traffic = stored_traffic(w.name, kname, shash)

    graph = graph_replay(w, lc) if w.steps > 1 else None
    gpu_out = lc.s_out.cpu().numpy()
    del lc
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype,
        "data": "synthetic (seeded N(0,1) rows; lengths and block permutation from the seed)",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
            "head_dim": w.D, "context": [int(lens.min()), int(lens.max())],
            "block_size": w.block_size, "query_rows": w.n_q, "partition_tokens": P,
            "accumulate": "f32", "cache": w.cache_dtype, "cache_row_bytes": w.kv_row_bytes,
            "cache_tensors": w.kv_tensors, "out_dim": w.out_dim,
        },
        "timing": "value and ms_per_step use the median of %d flushed step durations, roofline the "
                  "median of %d flushed partition-launch durations: per iteration, each behind a "
                  "1 GiB write that leaves no KV row in the last-level caches, HIP events around "
                  "A = [run, 1 GiB write] and B = [run, 1 GiB write, run]; B - A is one run after a "
                  "1 GiB write with no event marker (whose dispatch gap the single-run intervals in "
                  "'flushed' include); 'steady' is the timed region of %d back-to-back steps "
                  "between two synchronisations" % (F, F, K),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(w.B / (step_us * 1e-6), 1),
        "query_rows_per_s": round(w.B * w.n_q / (step_us * 1e-6), 1),
        "kv_bytes_per_step": kv_bytes,
        "flushed": {"iters": F, "flush_bytes": 1 << 30, "step_us": stats(st_us),
                    "partition_us": stats(pt_us),
                    "event_interval_step_us": stats(st_ev),
                    "event_interval_partition_us": stats(pt_ev)},
        "steady": {"steps": K, "ms_per_step": round(steady_ms, 5),
                   "gbs": round(kv_bytes / (steady_ms * 1e-3) / 1e9, 2),
                   "hbm_frac_step": round(kv_bytes / (steady_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "seq_steps_per_s": round(w.B / (steady_ms * 1e-3), 1)},
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_kernel_us": round(part_us, 3),
            "kernel_us": stats(pt_us),
            "algorithmic_bytes_per_launch": kv_bytes,
            "source_sha256": shash,
            "flops_per_launch": flops,
            "achieved_tflops": round(flops / (part_us * 1e-6) / 1e12, 2),
            "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        },
    }
    if w.prefill:  # compute-bound: the line reports FLOP/s against the matrix-core peak
        line["metric"] = PREFILL_METRIC
        line["value"] = round(flops / (step_us * 1e-6) / 1e12, 2)
        line["unit"] = "TFLOP/s"
        line["tokens_per_s"] = round(w.B * w.n_q / (step_us * 1e-6), 1)
        rf = line["roofline"]
        rf.update({"bound": "mfma", "achieved": rf["achieved_tflops"],
                   "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(rf["achieved_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                   "hbm_gbs": round(achieved, 2)})
    if graph is not None:
        line["graph_replay"] = graph

    configs = [c for c in args.configs.split(",") if c and c != "none"]
    if configs:
        line["configs"] = {c: config_result(c, min(args.warmup, 5), F, min(K, 50))
                           for c in configs}
    if not args.no_paged_compare and synth.get(args.workload).name == synth.get("C2").name:
        line["paged_vs_contiguous"] = paged_vs_contiguous(F)
    if not args.no_probe:
        print("# streaming-read probe", file=sys.stderr, flush=True)
        line["probe"] = probe()
    if args.no_cpu_baseline or w.prefill:  # prefill: the oracle takes minutes per sequence
        line["cpu_baseline"] = None
    else:
        print("# oracle timing on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, gpu_out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
