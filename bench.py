"""Benchmark: paged decode attention on one MI355X.

One step = one ``paged_decode_attn`` call (split-K partial kernel + merge
kernel) over the whole batch, inputs resident in HBM.  Default workload: the
long-context agentic batch (16 sequences, Llama-3.1-8B attention shape,
clipped log-normal context lengths with an 80K median, 512-token partitions).

Prints ONE JSON line:
  value          KV-read GB/s of the whole job: algorithmic K+V bytes of valid
                 tokens (sum_b ctx_b * 2 * Hkv * D * 2 B) / wall time per step
  roofline       the same bytes / the average call time measured with HIP
                 events on the launch stream, against the 8 TB/s HBM peak
  flushed        the headline call timed by events with 1 GiB of scratch read
                 before each call (the last-level cache then holds no K/V)
  also           the other decode workloads: the Llama-3.1-8B 4K batch, the ragged
                 256-sequence batch, the 32 x 128K batch as 4 range partials +
                 merge_partials (and its single pass), the agentic batch over an
                 FP8 cache, and at the Q48:KV8 and MHA Q40:KV40 head shapes
  multi_query_and_cascade
                 the other paths, fp16 and FP8 caches: speculative verification
                 (32 x 4096, 6 causal queries), chunked prefill (4 x 1024-query
                 chunks) and shared-prefix cascade decode (200 requests), each as
                 `--op multi_query` / `--op cascade` reports it (skip: --no-mq)
  cpu_baseline   the float64 CPU oracle: all cores (a process pool over every
                 sequence) and one core (a bounded sample)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0     # dense fp16 MFMA peak of MI355X
METRIC = "KV-read GB/s and % of HBM peak; decode-attn tokens/s at Llama-3.1-8B shape"
CSRC = os.path.join(ROOT, "decode_attention_paged_attn_amd", "csrc")
# the sources each timed kernel is built from (a counter record is valid only
# for the sources it was taken on)
KERNEL_SOURCES = {
    "attention": ("paged_attn.hip", "pda_common.h"),
    "multi_query": ("multi_query.hip", "pda_common.h"),
    "cascade": ("multi_query.hip", "paged_attn.hip", "pda_common.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def input_fingerprint(case):
    """SHA-256 of the small inputs (q, block table, context lengths) and a
    checksum of each K/V pool computed on the device (the sum of its 16-bit
    words as int64), so that a run's synthetic inputs can be compared."""
    import torch

    def sha(t):
        return hashlib.sha256(t.contiguous().cpu().numpy().tobytes()).hexdigest()[:16]

    def pool_sum(t):
        words = t.contiguous().view(torch.int16) if t.element_size() == 2 else \
            t.contiguous().view(torch.uint8)
        return int(words.to(torch.int64).sum().item()) if words.numel() < (1 << 28) else \
            int(sum(int(c.to(torch.int64).sum().item()) for c in words.view(-1).split(1 << 28)))

    return {"q_sha256_16": sha(case.q), "block_table_sha256_16": sha(case.block_table),
            "context_lens_sha256_16": sha(case.context_lens),
            "k_pool_word_sum": pool_sum(case.k_cache), "v_pool_word_sum": pool_sum(case.v_cache)}


def source_hash(op="attention"):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[op]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kv_bytes(lens, Hkv, D=128, elem=2):
    """Algorithmic K+V bytes of one call: valid tokens only."""
    return int(sum(int(n) for n in lens)) * 2 * Hkv * D * elem


def measured_traffic(key, op="attention"):
    """Counter-measured HBM bytes per call, if taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(op):
        return None
    return rec.get("bytes_per_call")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def _oracle_one(case, q, k, v, table, lens):
    import oracle.paged_attention as O
    if case["kv_dtype"] == "fp8":
        O.paged_decode_attention_fp8(q, k, v, table, lens, case["scale"], case["k_scale"],
                                     case["v_scale"])
    else:
        O.paged_decode_attention(q, k, v, table, lens, case["scale"])


def _pool_init():
    """A pool worker computes with one thread: BLAS limited before numpy loads."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"


def _pool_task(args):
    """One sequence in a worker: attach to the shared host copy, gather + attend."""
    from multiprocessing import shared_memory
    import numpy as np
    meta, shm_names = args
    shms = [shared_memory.SharedMemory(name=n) for n in shm_names]
    try:
        arrs = [np.ndarray(shape, dtype=np.dtype(dt), buffer=sh.buf)
                for (shape, dt), sh in zip(meta["arrays"], shms)]
        t0 = time.perf_counter()
        _oracle_one(meta["case"], *arrs, meta["lens"])
        return time.perf_counter() - t0
    finally:
        for sh in shms:
            sh.close()


def cpu_baseline(case, budget_s):
    """The float64 oracle as it stands, on host copies of whole sequences of the
    workload: (i) one core (one process, BLAS limited to one thread), sequences in
    a fixed random order until ``budget_s`` seconds of work; (ii) all cores: a
    process pool, one worker per core of this process's CPU share (at most 16),
    over every sequence of the workload, gathering from one host copy in shared
    memory.  Times cover gather + compute only."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    import numpy as np
    from decode_attention_paged_attn_amd import workloads as W
    meta_case = {"kv_dtype": case.kv_dtype, "scale": case.scale, "k_scale": case.k_scale,
                 "v_scale": case.v_scale}
    elem = case.kv_bytes_per_elem
    # (i) one core
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        one_thread = threadpool_limits(limits=1)
    except Exception:                                    # threadpoolctl missing
        one_thread = contextlib.nullcontext()
    order = np.random.default_rng(1).permutation(case.B)
    done, tokens, spent = [], 0, 0.0
    with one_thread:
        for b in order:
            q, k, v, table, lens = W.host_sequences(case, [int(b)])
            t0 = time.perf_counter()
            _oracle_one(meta_case, q, k, v, table, lens)
            spent += time.perf_counter() - t0
            done.append(int(b))
            tokens += int(lens[0])
            if spent >= budget_s:
                break
    one = kv_bytes([tokens], case.Hkv, elem=elem) / spent / 1e9
    # (ii) all cores of this process's share, one worker per core
    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:
        share = os.cpu_count() or 1
    workers = max(1, min(share, 16, case.B))
    tasks, shms = [], []
    try:
        for b in range(case.B):
            q, k, v, table, lens = W.host_sequences(case, [b])
            arrays, names = [], []
            for a in (q, k, v, table):
                a = np.ascontiguousarray(a)
                sh = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
                np.ndarray(a.shape, dtype=a.dtype, buffer=sh.buf)[...] = a
                shms.append(sh)
                arrays.append((a.shape, a.dtype.str))
                names.append(sh.name)
            tasks.append(({"case": meta_case, "arrays": arrays, "lens": lens}, names))
            del q, k, v
        with mp.get_context("spawn").Pool(workers, initializer=_pool_init) as pool:
            pool.map(_pool_task, tasks[:workers])          # workers up and numpy loaded
            t0 = time.perf_counter()
            pool.map(_pool_task, tasks, chunksize=1)
            wall = time.perf_counter() - t0
    finally:
        for sh in shms:
            sh.close()
            sh.unlink()
    all_tok = int(case.lens.sum())
    pool_gbs = kv_bytes([all_tok], case.Hkv, elem=elem) / wall / 1e9
    return {"value": round(pool_gbs, 4), "unit": "GB/s", "cores": int(workers), "kind": "oracle",
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "cpu_share": share,
            "sample": f"all {case.B} sequences ({all_tok} tokens, all {case.Hq} query heads), "
                      f"float64 numpy gather + two-pass softmax in a pool of {workers} "
                      f"single-threaded processes over one shared host copy, {wall:.1f} s wall",
            "one_core": {"value": round(one, 4), "unit": "GB/s", "cores": 1,
                         "sample": f"{len(done)} of {case.B} sequences ({tokens} tokens), "
                                   f"one process, BLAS limited to 1 thread, {spent:.1f} s"}}


def copy_calibration(mib, steps):
    """Plain copies of known size, the reference kernels for HBM byte counters.

    Each launch reads and writes ``mib`` MiB: first hipMemcpy's blit kernel
    (dst.copy_(src)), then an elementwise fp16 kernel (torch.neg into dst).
    """
    import torch
    n = mib << 20
    src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    res = {"bytes_read_per_launch": n, "bytes_written_per_launch": n}
    for name, fn in (("blit_copy", lambda: dst.copy_(src)),
                     ("elementwise_neg", lambda: torch.neg(src, out=dst))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        res[name] = {"launches": steps + 2, "ms": round(dt * 1e3, 4),
                     "GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}
    print(json.dumps(res), flush=True)


def measure(case, P, steps, warmup, flush_mib=0):
    """Time ``steps`` calls after ``warmup``; wall clock and HIP events on the stream."""
    import torch
    import decode_attention_paged_attn_amd as pda
    B, Hq, Hkv = case.B, case.Hq, case.Hkv
    width = case.block_table.shape[1]
    ws = torch.empty(max(pda.workspace_size(B, Hq, Hkv, width, P), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    unit = pda.workspace_layout(B, Hq, Hkv, width, P,
                                kv_fp8=case.kv_dtype == "fp8")["unit_tokens"]
    scratch = torch.ones(flush_mib << 20, dtype=torch.uint8, device="cuda") if flush_mib else None
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def flush():
        # read (ordinary loads, which allocate in L2 and the last-level cache)
        # a buffer four times the last-level cache: no K/V stays cached, and no
        # dirty lines are left to write back during the timed call
        pda.stream_read(scratch, sink, False)

    kw = case.attn_kwargs()

    def step():
        pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                              case.context_lens, case.scale, out=out, lse_out=lse,
                              partition_tokens=P, workspace=ws, **kw)

    _warm(step, warmup)
    # the timed pass: ``steps`` calls back to back, nothing else in the stream
    # but the optional cache flush
    t0 = time.perf_counter()
    for i in range(steps):
        if scratch is not None:
            flush()
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call durations for the roofline: a second pass, each call bracketed
    # by HIP events on the stream it is launched on
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if scratch is not None:
            flush()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ev_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    ev_mean = sum(ev_ms) / len(ev_ms)
    nbytes = kv_bytes(case.lens, Hkv, elem=case.kv_bytes_per_elem)
    ms_per_step = wall / steps * 1e3
    if scratch is not None:
        # the wall clock also ran the scratch reads: the rate of a flushed
        # call is the event-bracketed one
        ms_per_step = ev_mean
    return {
        "kv_bytes": nbytes,
        "unit_tokens": unit,
        "ms_per_step": round(ms_per_step, 5),
        "value": round(nbytes / (ms_per_step / 1e3) / 1e9, 2),
        "achieved": round(nbytes / (ev_mean / 1e3) / 1e9, 2),
        "tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "event_ms": {"mean": round(ev_mean, 5), "p10": round(ev_ms[len(ev_ms) // 10], 5),
                     "p50": round(ev_ms[len(ev_ms) // 2], 5),
                     "p90": round(ev_ms[(9 * len(ev_ms)) // 10], 5)},
    }


MIN_WARM_S = 0.2


def _warm(step, warmup):
    """``warmup`` untimed calls, then more until MIN_WARM_S of them have run: a
    GPU left idle (the CPU baseline runs seconds) needs that long to be back at
    its working clock, far longer than a few calls of a 100-us workload."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < MIN_WARM_S:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def _time_events(step, steps, warmup):
    """Mean ms per step: the wall clock of ``steps`` back-to-back calls, then the
    per-call durations of a second pass of ``steps`` calls, each bracketed by HIP
    events on torch's current stream (the events stay out of the wall-clock pass:
    recorded around every call they cost a short call up to 9% of its rate)."""
    import torch
    _warm(step, warmup)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) / steps * 1e3
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ev = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    return wall_ms, sum(ev) / len(ev), ev[len(ev) // 2]


def platform_info():
    """Device and software versions for the record."""
    import torch
    props = torch.cuda.get_device_properties(0)
    rocm = ""
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"device": props.name, "arch": getattr(props, "gcnArchName", ""),
            "compute_units": props.multi_processor_count, "rocm": rocm,
            "torch": torch.__version__, "torch_hip": torch.version.hip}


def stream_read_ceiling(gib=4, steps=10):
    """Read bandwidth of a plain streaming kernel (pda_stream_read) over ``gib``
    GiB: ordinary and non-temporal 16-byte loads, the better mean by events."""
    import torch
    import decode_attention_paged_attn_amd as pda
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"bytes": buf.numel()}
    for name, nt in (("ordinary_GBps", False), ("nontemporal_GBps", True)):
        _, ev_ms, _ = _time_events(lambda: pda.stream_read(buf, sink, nt), steps, 2)
        res[name] = round(buf.numel() / (ev_ms / 1e3) / 1e9, 1)
    res["GBps"] = max(res["ordinary_GBps"], res["nontemporal_GBps"])
    del buf
    torch.cuda.empty_cache()
    return res


LDS_PROBE_FORMS = (("ds_read_b128", 1024), ("ds_read_b64", 512), ("ds_read_b64_tr_b16", 512),
                   ("ds_read_b32", 256))


def bench_lds_probe(steps, iters=4096):
    """The LDS read forms of the multi-query kernels (pda_lds_probe), one at a
    time: two 256-thread work-groups per CU (their 64 KiB stages fill 128 of the
    CU's 160 KiB), ``iters`` passes of 16 reads per wave; mean kernel time by
    events, and per CU the time and bytes of one wave-wide read."""
    import torch
    import decode_attention_paged_attn_amd as pda
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs_per_cu = 2
    out = torch.empty(wgs_per_cu * cus * 256, dtype=torch.int32, device="cuda")
    reads_per_cu = wgs_per_cu * 4 * iters * 16            # 4 waves per work-group
    forms = {}
    for form, (name, nbytes) in enumerate(LDS_PROBE_FORMS):
        _, ev_ms, _ = _time_events(lambda: pda.lds_probe(form, out, iters), steps, 2)
        ns = ev_ms * 1e6 / reads_per_cu
        forms[name] = {"form": form, "ms": round(ev_ms, 4), "ns_per_wave_read_per_cu": round(ns, 4),
                       "bytes_per_ns_per_cu": round(nbytes / ns, 1)}
    print(json.dumps({"op": "lds_probe", "work_groups": wgs_per_cu * cus, "iters": iters,
                      "reads_per_wave": iters * 16, "steps": steps, "forms": forms,
                      "device": platform_info()}), flush=True)


def mq_work(case):
    """(unique K/V bytes, algorithmic FLOPs) of one multi-query call.

    Bytes: every cached token of a sequence that some query sees, K and V, all
    KV heads, once (2 bytes an element, 1 for an FP8 cache).  FLOPs: 4 * D per
    (query, query head, visible token): the q.k dot product and the p.v
    accumulation, 2 * D each.
    """
    Hkv, Hq, D = case.Hkv, case.Hq, 128
    elem = 1 if case.kv_dtype == "fp8" else 2
    nbytes = flops = 0
    for n, nq in zip(case.lens, case.n_queries):
        n, nq = int(n), int(nq)
        if nq == 0:
            continue
        if case.causal:
            vis = [max(0, n - nq + i + 1) for i in range(nq)]
        else:
            vis = [n] * nq
        nbytes += max(vis) * 2 * Hkv * D * elem
        flops += 4 * D * Hq * sum(vis)
    return nbytes, flops


def bench_multi_query(case, P, steps, warmup):
    print(json.dumps(measure_multi_query(case, P, steps, warmup)), flush=True)


def measure_multi_query(case, P, steps, warmup):
    import torch
    import decode_attention_paged_attn_amd as pda
    ws = torch.empty(max(pda.multi_query_workspace_size(case.S, case.T, case.Hq, case.Hkv,
                                                        case.block_table.shape[1], P), 1),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((case.T, case.Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((case.T, case.Hq), dtype=torch.float32, device="cuda")

    def step():
        pda.paged_multi_query_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                                   case.context_lens, case.query_start, case.scale,
                                   causal=case.causal, out=out, lse_out=lse,
                                   partition_tokens=P, workspace=ws, **case.attn_kwargs())

    wall_ms, ev_ms, ev_med = _time_events(step, steps, warmup)
    nbytes, flops = mq_work(case)
    # the bound: HBM for the unique K/V bytes, or the fp16 MFMA peak for the flops
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_FP16_PEAK_TFLOPS * 1e12)
    hbm_bound = t_hbm >= t_mfma
    roof = ({"bound": "hbm", "achieved": round(nbytes / (ev_ms / 1e3) / 1e9, 2),
             "peak": HBM_PEAK_GBS, "unit": "GB/s"} if hbm_bound else
            {"bound": "mfma", "achieved": round(flops / (ev_ms / 1e3) / 1e12, 2),
             "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s"})
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = "paged_multi_query_attn call (plan + tile + merge kernels)"
    roof["traffic"] = measured_traffic(f"multi_query:{case.name}", "multi_query")
    value = roof["achieved"] * ev_ms / wall_ms
    return {
        "metric": "multi-query paged attention: " + ("KV-read GB/s" if hbm_bound else "TFLOP/s"),
        "op": "paged_multi_query_attn", "value": round(value, 2), "unit": roof["unit"],
        "ms_per_step": round(wall_ms, 5), "event_ms": {"mean": round(ev_ms, 5),
                                                        "p50": round(ev_med, 5)},
        "query_tokens_per_s": round(case.T / (wall_ms / 1e3), 1),
        "kv_bytes_unique": nbytes, "flops": flops,
        "tflops": round(flops / (ev_ms / 1e3) / 1e12, 2),
        "kv_GBps": round(nbytes / (ev_ms / 1e3) / 1e9, 2),
        "roofline": roof, "steps": steps, "warmup": warmup, "min_warm_s": MIN_WARM_S, "dtype": case.kv_dtype,
        "data": "synthetic", "kernel_source_sha256_16": source_hash("multi_query"),
        "config": {"workload": case.name, "sequences": case.S, "query_tokens": case.T,
                   "q_heads": case.Hq, "kv_heads": case.Hkv, "head_dim": 128,
                   "causal": case.causal, "partition_tokens": P, "kv_dtype": case.kv_dtype,
                   "context_tokens": int(case.lens.sum())}}


def bench_cascade(case, steps, warmup):
    print(json.dumps(measure_cascade(case, steps, warmup)), flush=True)


def measure_cascade(case, steps, warmup):
    """Cascade (prefix pass + suffix pass + merge) against naive decode of the same batch."""
    import torch
    import decode_attention_paged_attn_amd as pda
    B, Hq = case.B, case.Hq
    o_parts = torch.empty((2, B, Hq, 128), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((2, B, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")

    def step():
        pda.cascade_decode_attn(case.q, case.k_cache, case.v_cache, case.prefix_table,
                                case.prefix_lens, case.group_start, case.suffix_table,
                                case.suffix_lens, case.scale, out=out,
                                partials=(o_parts, l_parts), **case.attn_kwargs())

    wall_ms, ev_ms, ev_med = _time_events(step, steps, warmup)
    table, lens = case.naive_table()
    naive_out = torch.empty_like(out)

    def naive():
        pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, table, lens, case.scale,
                              out=naive_out, **case.attn_kwargs())

    n_wall, n_ev, _ = _time_events(naive, steps, warmup)
    row = 2 * case.Hkv * 128 * (1 if case.kv_dtype == "fp8" else 2)   # K and V bytes a token
    # tokens read: naive decode reads each group's prefix once per request,
    # cascade once per group; both read every suffix once
    naive_tok, unique_tok = 0, 0
    for r in range(len(case.prefix_lens_host)):
        lo, hi = int(case.group_start_host[r]), int(case.group_start_host[r + 1])
        suffix = int(case.suffix_lens_host[lo:hi].sum())
        naive_tok += (hi - lo) * int(case.prefix_lens_host[r]) + suffix
        unique_tok += int(case.prefix_lens_host[r]) + suffix
    return {
        "metric": "cascade decode: requests/s (unique KV-read GB/s in roofline)",
        "op": "cascade_decode_attn", "value": round(B / (wall_ms / 1e3), 1), "unit": "requests/s",
        "ms_per_step": round(wall_ms, 5), "event_ms": {"mean": round(ev_ms, 5),
                                                        "p50": round(ev_med, 5)},
        "naive_decode_ms": round(n_ev, 5), "speedup_vs_naive_decode": round(n_ev / ev_ms, 3),
        "naive_kv_bytes": naive_tok * row, "unique_kv_bytes": unique_tok * row,
        "naive_decode_GBps": round(naive_tok * row / (n_ev / 1e3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(unique_tok * row / (ev_ms / 1e3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(unique_tok * row / (ev_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel": "cascade call (prefix pass + suffix pass + merge)",
                     "traffic": measured_traffic(f"cascade:{case.name}", "cascade")},
        "steps": steps, "warmup": warmup, "min_warm_s": MIN_WARM_S, "dtype": case.kv_dtype, "data": "synthetic",
        "config": {"workload": case.name, "requests": B, "kv_dtype": case.kv_dtype,
                   "groups": len(case.prefix_lens_host),
                   "prefix_tokens": [int(x) for x in case.prefix_lens_host],
                   "suffix_tokens_total": int(case.suffix_lens_host.sum()),
                   "q_heads": Hq, "kv_heads": case.Hkv, "head_dim": 128}}


def measure_partial_merge(case, steps, warmup, single_pass=True):
    """R range partials (paged_decode_attn_partial on block-table column slices)
    + merge_partials per step, and (single_pass) the single pass over the same
    batch."""
    import torch
    import decode_attention_paged_attn_amd as pda
    from decode_attention_paged_attn_amd import workloads as W
    R = case.ranges
    views = W.range_views(case, R)
    B, Hq = case.B, case.Hq
    o_parts = torch.empty((R, B, Hq, 128), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((R, B, Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(pda.workspace_size(B, Hq, case.Hkv, case.block_table.shape[1], 0), 1),
                     dtype=torch.uint8, device="cuda")
    kw = case.attn_kwargs()

    def split_path():
        for r, (bt, ln) in enumerate(views):
            pda.paged_decode_attn_partial(case.q, case.k_cache, case.v_cache, bt, ln, case.scale,
                                          o=o_parts[r], lse=l_parts[r], workspace=ws, **kw)
        pda.merge_partials(o_parts, l_parts, out=out, lse_out=lse)

    def single():
        pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                              case.context_lens, case.scale, out=out, lse_out=lse, workspace=ws,
                              **kw)

    wall_ms, ev_ms, _ = _time_events(split_path, steps, warmup)
    s_ev = _time_events(single, steps, warmup)[1] if single_pass else float("nan")
    nbytes = kv_bytes(case.lens, case.Hkv, elem=case.kv_bytes_per_elem)
    return {"value": round(nbytes / (wall_ms / 1e3) / 1e9, 2), "unit": "GB/s",
            "traffic": measured_traffic(f"disagg_merge_partial/{case.kv_dtype}"),
            "pct_hbm_peak": round(100.0 * nbytes / (wall_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
            "event_GBps": round(nbytes / (ev_ms / 1e3) / 1e9, 2),
            "ms_per_step": round(wall_ms, 5), "event_ms": round(ev_ms, 5),
            "decode_attn_tokens_per_s": round(B / (wall_ms / 1e3), 1),
            "kv_bytes_per_step": nbytes, "ranges": R,
            "step": f"{R} x paged_decode_attn_partial + merge_partials",
            "single_pass_event_ms": round(s_ev, 5),
            "single_pass_event_GBps": round(nbytes / (s_ev / 1e3) / 1e9, 2),
            "split_over_single_time": round(ev_ms / s_ev, 4)}


def bench_partial_merge(case, steps, warmup, single_pass=True):
    """R range partials (paged_decode_attn_partial over block-table column slices)
    plus merge_partials, against single-pass attention over the same batch."""
    m = measure_partial_merge(case, steps, warmup, single_pass)
    nbytes = m["kv_bytes_per_step"]
    ev_ms = m["event_ms"]
    print(json.dumps({
        "metric": "disaggregated partial merge: KV-read GB/s (R range partials + merge_partials)",
        "op": "paged_decode_attn_partial x R + merge_partials", "unit": "GB/s",
        "value": m["value"], "event_GBps": m["event_GBps"], "ms_per_step": m["ms_per_step"],
        "event_ms": ev_ms, "single_pass_event_ms": m["single_pass_event_ms"],
        "single_pass_event_GBps": m["single_pass_event_GBps"],
        "split_over_single_time": m["split_over_single_time"],
        "roofline": {"bound": "hbm", "achieved": m["event_GBps"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(m["event_GBps"] / HBM_PEAK_GBS, 4),
                     "kernel": "R partial calls + merge_partials",
                     "traffic": m["traffic"]},
        "steps": steps, "warmup": warmup, "min_warm_s": MIN_WARM_S, "dtype": case.kv_dtype,
        "data": "synthetic",
        "config": {"workload": case.name, "batch": case.B, "q_heads": case.Hq,
                   "kv_heads": case.Hkv, "head_dim": 128, "ranges": case.ranges,
                   "tokens_per_sequence": int(case.lens[0]), "kv_bytes_per_step": nbytes}}),
        flush=True)


def bench_append(case, steps, warmup):
    """paged_kv_append of one token per sequence (reads 2*B*Hkv*D fp16 and writes
    them in the cache's element type), and a decode step both ways: append then
    attention (two launches) against paged_decode_attn_append (one launch)."""
    import torch
    import decode_attention_paged_attn_amd as pda
    g = torch.Generator(device="cuda").manual_seed(1)
    kn = torch.randn((case.B, case.Hkv, 128), generator=g, device="cuda").half()
    vn = torch.randn((case.B, case.Hkv, 128), generator=g, device="cuda").half()
    ws = torch.empty(max(pda.workspace_size(case.B, case.Hq, case.Hkv, case.block_table.shape[1]),
                         1), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.B, case.Hq, 128), dtype=torch.float16, device="cuda")
    sc = case.attn_kwargs()

    def append():
        pda.paged_kv_append(case.k_cache, case.v_cache, kn, vn, case.block_table,
                            case.context_lens, **sc)

    def separate():
        append()
        pda.paged_decode_attn(case.q, case.k_cache, case.v_cache, case.block_table,
                              case.context_lens, case.scale, out=out, workspace=ws, **sc)

    def fused():
        pda.paged_decode_attn_append(case.q, kn, vn, case.k_cache, case.v_cache,
                                     case.block_table, case.context_lens, case.scale, out=out,
                                     workspace=ws, **sc)

    a_wall, a_ev, _ = _time_events(append, steps, warmup)
    s_wall, s_ev, _ = _time_events(separate, steps, warmup)
    f_wall, f_ev, _ = _time_events(fused, steps, warmup)
    elem = 1 if case.kv_dtype == "fp8" else 2
    nbytes = 2 * case.B * case.Hkv * 128 * (2 + elem)     # K and V rows, read + write
    kvb = kv_bytes(case.lens, case.Hkv, elem=case.kv_bytes_per_elem)
    print(json.dumps({"metric": "KV append GB/s; decode step with the append fused",
                      "op": "paged_kv_append / paged_decode_attn_append", "unit": "GB/s",
                      "value": round(nbytes / (a_wall / 1e3) / 1e9, 2),
                      "event_GBps": round(nbytes / (a_ev / 1e3) / 1e9, 2),
                      "us_per_call_events": round(a_ev * 1e3, 3), "bytes_per_call": nbytes,
                      "decode_step": {
                          "append_then_attend_us": round(s_ev * 1e3, 2),
                          "fused_us": round(f_ev * 1e3, 2),
                          "fused_KV_read_GBps": round(kvb / (f_ev / 1e3) / 1e9, 2),
                          "separate_KV_read_GBps": round(kvb / (s_ev / 1e3) / 1e9, 2),
                          "fused_over_separate_time": round(f_ev / s_ev, 4)},
                      "steps": steps, "dtype": case.kv_dtype,
                      "config": {"workload": case.name, "batch": case.B, "kv_heads": case.Hkv,
                                 "kv_dtype": case.kv_dtype}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="agentic_80k")
    ap.add_argument("--partition-tokens", type=int, default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read ceiling measured beside the headline")
    ap.add_argument("--also", default="llama8b_4k,ragged_mixed,disagg_merge:partial,agentic_80k:fp8,"
                                      "agentic_80k_q48kv8,agentic_80k_q40kv40",
                    help="comma-separated extra workloads reported under 'also': a workload "
                         "name, ':fp8' for its FP8 cache, ':partial' for its R range partials "
                         "+ merge_partials (disagg_merge)")
    ap.add_argument("--flush-record-mib", type=int, default=1024,
                    help="also time the headline with this many MiB of scratch read before "
                         "each call (event-timed; 0: skip)")
    ap.add_argument("--op", default="attention",
                    choices=["attention", "append", "multi_query", "cascade", "partial_merge",
                             "lds_probe"],
                    help="attention (default): paged_decode_attn; append: paged_kv_append of "
                         "one token per sequence; multi_query: paged_multi_query_attn on "
                         "--config spec_verify or chunked_prefill; cascade: "
                         "cascade_decode_attn on --config shared_prefix; partial_merge: 4 range "
                         "partials + merge_partials on disagg_merge, against single pass; "
                         "lds_probe: the LDS read forms of the multi-query kernels, timed alone")
    ap.add_argument("--no-mq", action="store_true",
                    help="skip the multi-query (speculative verification, chunked prefill) "
                         "and cascade records of the default run")
    ap.add_argument("--partial-only", action="store_true",
                    help="--op partial_merge: time only the partials + merge (no single pass)")
    ap.add_argument("--kv-dtype", default="fp16", choices=["fp16", "fp8"],
                    help="element type of the K/V cache (fp8: E4M3 codes with per-tensor scales)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="read this many MiB of scratch before each timed call (outside the "
                         "event pair; the headline is then event-timed)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead: time a plain device copy of MIB MiB (the reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU sharding of "
                          "the path is described in the design notes, not built",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import decode_attention_paged_attn_amd as pda
    from decode_attention_paged_attn_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    pda.load_library()
    if args.op == "lds_probe":
        bench_lds_probe(args.steps)
        return
    if args.op == "multi_query":
        name = args.config if args.config in W.MQ_CONFIGS else "spec_verify"
        case = W.MQ_CONFIGS[name](device="cuda", kv_dtype=args.kv_dtype)
        bench_multi_query(case, args.partition_tokens or 0, args.steps, args.warmup)
        return
    if args.op == "cascade":
        case = W.CASCADE_CONFIGS["shared_prefix"](device="cuda", kv_dtype=args.kv_dtype)
        bench_cascade(case, args.steps, args.warmup)
        return
    if args.op == "partial_merge":
        bench_partial_merge(W.disagg_merge(device="cuda", kv_dtype=args.kv_dtype), args.steps,
                            args.warmup, single_pass=not args.partial_only)
        return
    case = W.CONFIGS[args.config](device="cuda", kv_dtype=args.kv_dtype)
    if args.op == "append":
        bench_append(case, args.steps, args.warmup)
        return
    # the extra workloads get their memory now, while it is fresh: built after
    # the headline's pools were freed, a workload measured 4% slower than in a
    # process of its own
    also_cases = []
    for spec in [x for x in args.also.split(",") if x]:
        parts = spec.split(":")
        kv = "fp8" if "fp8" in parts[1:] else args.kv_dtype
        partial = "partial" in parts[1:]
        if parts[0] == args.config and kv == args.kv_dtype and not partial:
            continue
        also_cases.append((spec, partial, W.CONFIGS[parts[0]](device="cuda", kv_dtype=kv)))
    P = case.partition_tokens if args.partition_tokens is None else args.partition_tokens
    m = measure(case, P, args.steps, args.warmup, args.flush_mib)
    nbytes = m["kv_bytes"]
    B, Hq, Hkv = case.B, case.Hq, case.Hkv
    traffic = measured_traffic(f"{args.config}/{case.kv_dtype}")
    rec = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "min_warm_s": MIN_WARM_S,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": case.name,
            "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128, "block_size": 16,
            "kv_dtype": case.kv_dtype,
            "partition_tokens": m["unit_tokens"], "tokens": int(case.lens.sum()),
            "min_ctx": int(case.lens.min()), "max_ctx": int(case.lens.max()),
            "kv_bytes_per_step": nbytes, "seed": case.seed,
        },
        "pct_hbm_peak": round(100.0 * m["value"] / HBM_PEAK_GBS, 2),
        "decode_attn_tokens_per_s": m["tokens_per_s"],
        "attn_only_tokens_per_s_32_layer_step": round(m["tokens_per_s"] / 32, 1),
        "event_ms": m["event_ms"],
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_attn call (split_kernel + merge_kernel)",
            "achieved": m["achieved"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(m["achieved"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "kernel_source_sha256_16": source_hash(),
        "inputs": input_fingerprint(case),
        "platform": platform_info(),
    }
    if args.flush_mib:
        rec["flush_mib_between_steps"] = args.flush_mib
        rec["value_timing"] = "events (each call bracketed; the scratch reads outside)"
    if args.flush_record_mib:
        fm = measure(case, P, args.steps, 0, args.flush_record_mib)
        rec["flushed"] = {"flush_mib_before_each_call": args.flush_record_mib,
                          "event_GBps": fm["achieved"],
                          "pct_hbm_peak": round(100.0 * fm["achieved"] / HBM_PEAK_GBS, 2),
                          "event_ms": fm["event_ms"]}
    if not args.no_stream_read:
        ceiling = stream_read_ceiling()
        rec["stream_read_ceiling"] = ceiling
        rec["frac_of_stream_read_ceiling"] = round(m["achieved"] / ceiling["GBps"], 4)
    also = {}
    for spec, partial, acase in also_cases:
        key = acase.name + ("_4partials_merge" if partial else "")
        if partial:
            also[key] = measure_partial_merge(acase, args.steps, args.warmup)
        else:
            mm = measure(acase, acase.partition_tokens, args.steps, args.warmup, args.flush_mib)
            also[key] = {"value": mm["value"], "unit": "GB/s",
                         "pct_hbm_peak": round(100.0 * mm["value"] / HBM_PEAK_GBS, 2),
                         "event_GBps": mm["achieved"],
                         "event_pct_hbm_peak": round(100.0 * mm["achieved"] / HBM_PEAK_GBS, 2),
                         "ms_per_step": mm["ms_per_step"], "event_ms": mm["event_ms"],
                         "decode_attn_tokens_per_s": mm["tokens_per_s"],
                         "kv_bytes_per_step": mm["kv_bytes"], "partition_tokens": mm["unit_tokens"],
                         "traffic": measured_traffic(f"{spec.split(':')[0]}/{acase.kv_dtype}")}
        also[key]["kv_dtype"] = acase.kv_dtype
        also[key]["workload"] = spec
    if also:
        rec["also"] = also
    del also_cases
    if not args.no_mq:
        # the other paths of the call set, fp16 and FP8: one record each, as
        # `--op multi_query` / `--op cascade` print them
        keep = ("value", "unit", "ms_per_step", "event_ms", "roofline", "kv_GBps", "tflops",
                "query_tokens_per_s", "naive_decode_ms", "speedup_vs_naive_decode")
        mq = {}
        for name in ("spec_verify", "chunked_prefill", "shared_prefix"):
            for kv in ("fp16", "fp8"):
                if name == "shared_prefix":
                    c = W.CASCADE_CONFIGS[name](device="cuda", kv_dtype=kv)
                    r = measure_cascade(c, args.steps, args.warmup)
                else:
                    c = W.MQ_CONFIGS[name](device="cuda", kv_dtype=kv)
                    r = measure_multi_query(c, 0, args.steps, args.warmup)
                mq[r["config"]["workload"]] = dict({k: r[k] for k in keep if k in r},
                                                   metric=r["metric"], kv_dtype=kv)
                del c
                torch.cuda.empty_cache()
        rec["multi_query_and_cascade"] = mq
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
