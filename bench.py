#!/usr/bin/env python3
"""Paged decode attention on one MI355X: KV-read HBM GB/s (and % of peak) plus decode tokens/s.

One step = one decode step of the whole batch through every layer: the plan (block tables and
lengths -> wavefront shares, once per step since all layers share them), then per layer the
new tokens' slot write and the paged attention (decode kernel + log-sum-exp merge).  Where
the batch allows it (one query row per sequence, 16- or 32-bit cache) the slot write runs
inside the decode launch (pa_decode_write_attend); otherwise it is its own launch
(pa_write_kv, then pa_decode_attend).  Every layer has its own KV pool in HBM, so no layer's reads are served
from cache.  Inputs are synthetic, seeded, already resident in HBM when timing starts.

Prints one JSON line.  `value` is the KV bytes the attention reads per step (each attended
token's K and V once, per KV head, per layer) over the measured step time, in GB/s.
`roofline` reports the dominant kernel alone, timed with HIP events around its launches (the
library's profiling hooks record them on the launch stream): the decode kernel against HBM
bandwidth on the decode rows' KV bytes, or, when chunked-prefill rows dominate, the chunk
kernel against the dense MFMA peak on its FLOPs.  `cpu_baseline` is the fp64 CPU oracle
timed on the host cores on a bounded sample of the same workload.

The default run measures two shapes. The OPT-13B shape gives the
line's `value`, `roofline` and `cpu_baseline`, and the Qwen3-8B / Mistral-7B GQA shape is
measured after it with the same steps and reported under the key "gqa" with its own value,
roofline (kernel named as dispatched), counter traffic and CPU baseline.

In the parallel-sampling workload each layer's step also carries out the copy-on-write
copies of the first decode step after the fork (pa_copy_blocks) before the slot write; the
copy kernel is reported in `roofline_copy`.

  python bench.py [--steps K] [--warmup W]
                  [--workload opt13b|gqa|prefix_mixed|swa|parallel_sampling|tiny]
                  [--also W,...|none] [--kv native|q8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV-read HBM GB/s (% of peak) + decode tokens/s"
# 8-bit variants keep each workload's 16-bit activation type
Q8_DTYPE = {"opt13b": "q8_f16", "gqa": "q8_bf16", "swa": "q8_f16", "prefix_mixed": "q8_bf16",
            "parallel_sampling": "q8_f16"}
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense matrix peak, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
# The sources each kernel is built from (the launch code in decode.hip and the plan
# included): a committed counter record stays valid while they are unchanged.
COMMON_SOURCES = ["pa_device.h", "pa_internal.h", "plan.hip", "decode.hip"]
KERNEL_SOURCES = {
    "decode_kernel": ["decode_impl.h", *COMMON_SOURCES],
    "decode_mfma_kernel": ["decode_impl.h", "decode_mfma.h", *COMMON_SOURCES],
    "decode_group_kernel": ["decode_impl.h", "decode_group.h", *COMMON_SOURCES],
}
CHUNK_SOURCES = ["chunk_impl.h", *COMMON_SOURCES]

DESCRIPTIONS = {
    "opt13b": "OPT-13B-shaped paged decode: 64 seqs, 40 q heads = 40 KV heads, d=128, fp16 KV, "
              "16-token blocks, lengths U[64,2048], permuted blocks, 40 layers",
    "gqa": "Qwen3-8B/Mistral-7B-shaped GQA decode: 256 seqs, 32 q / 8 KV heads, d=128, bf16 KV, "
           "lengths log-normal(median 1024, sigma 1) clipped [16,32768], 36 layers",
    "prefix_mixed": "shared 512-token prefix (32 blocks, refcount 128) + private suffixes U[1,512], "
                    "128 decode seqs + 4 chunked-prefill queries of 512 causal rows over 1-4K "
                    "contexts, 32 q / 8 KV heads, d=128, bf16, 36 layers",
    "swa": "Gemma-3-4B-shaped sliding-window decode: 32 seqs, 8 q / 4 KV heads, d=256, fp16 KV, "
           "window 1024, lengths U[4096,131072], 29 sliding layers",
    "tiny": "tiny paged decode: 4 seqs, lengths {1,17,100,33}, 4 heads, d=64, fp32, 1 layer",
    "parallel_sampling": "OPT-13B-shaped parallel sampling, first decode step after the fork: "
                         "16 prompts of U[64,2048] tokens x 4 samples (64 seqs), 40 q = 40 KV "
                         "heads, d=128, fp16 KV, 16-token blocks; 3 of the 4 samples of a "
                         "prompt copy its partly filled last block (copy-on-write), 40 layers",
}


def kernel_source_hash(files) -> str:
    """Hash of the code in a kernel's sources: line comments and blank lines are left out
    (the sources hold no block comments and no "//" inside literals), so that an edit of
    comments alone leaves the counter records valid."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_144_amd", "csrc", f),
                  encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(key: str, files):
    """HBM bytes per launch of one kernel from the committed rocprofv3 counter runs (entry
    `key`: the workload, or the workload + "_chunk" for the chunk-row kernel), or None when
    there is none or that kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return e.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ work accounting
def kv_bytes_read(seq_lens, q_rows, window, num_kv_heads, head_dim, elem_bytes) -> int:
    """Algorithmic KV bytes one attention layer reads: every attended position once, K and V,
    per KV head (a sliding window caps the positions a row can see).  elem_bytes is the
    cache's bytes per element: 4, 2, or 17/16 for an 8-bit cache (a 2-byte scale per 32
    one-byte codes)."""
    import numpy as np
    total = 0
    for L, n in zip(np.asarray(seq_lens).tolist(), np.asarray(q_rows).tolist()):
        first = L - n                       # position of the first query row
        lo = max(0, first - window + 1) if window > 0 else 0
        total += max(0, L - lo)
    return int(round(2 * num_kv_heads * head_dim * elem_bytes * total))


def chunk_flops(seq_lens, q_rows, window, num_q_heads, head_dim) -> int:
    """Algorithmic FLOPs of the chunk rows (sequences with more than one query row): per row,
    per query head, per attended token, 2 * head_dim for q.K and 2 * head_dim for p.V."""
    import numpy as np
    total = 0
    for L, n in zip(np.asarray(seq_lens).tolist(), np.asarray(q_rows).tolist()):
        if n < 2:
            continue
        for r in range(n):
            p = L - n + r
            lo = max(0, p - window + 1) if window > 0 else 0
            total += max(0, p - lo + 1)
    return 4 * head_dim * num_q_heads * total


def step_rows(w):
    """Value rows of each sequence's newest q_rows tokens (this step's writes)."""
    import numpy as np

    from workloads import Append
    last = {}
    for op in w.script:
        if isinstance(op, Append) and op.nv > 0:
            last[op.seq] = (op.off, op.nv)
    rows = []
    for s in range(w.num_seqs):
        off, nv = last[s]
        n = int(w.q_rows[s])
        rows.extend(range(off + nv - n, off + nv))
    return np.asarray(rows, np.int64)


def cpu_baseline(w, n_layers, seconds):
    """The fp64 oracle on the same workload: sequences of one layer in a seeded order, eight
    at a time, cycling until `seconds` pass.  Rates come from what was processed."""
    import numpy as np

    import oracle
    ref = oracle.Reference(w, poison=False)
    threads = len(os.sched_getaffinity(0))
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done_bytes = done_rows = 0
    passes = 0
    t0 = time.perf_counter()
    i = 0
    while True:
        chunk = order[i:i + 8]
        ref.attention(seqs=chunk)
        done_bytes += kv_bytes_read(w.seq_lens[chunk], w.q_rows[chunk], w.window,
                                    w.num_kv_heads, w.head_dim, w.elem_bytes)
        done_rows += int(w.q_rows[chunk].sum())
        i += 8
        if i >= w.num_seqs:
            i = 0
            passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    frac = passes + i / w.num_seqs
    # the same oracle on one thread, over a shorter sample
    ref.threads = 1
    one_bytes, t1 = 0, time.perf_counter()
    j = 0
    while time.perf_counter() - t1 < min(3.0, seconds):
        chunk = order[j:j + 1]
        ref.attention(seqs=chunk)
        one_bytes += kv_bytes_read(w.seq_lens[chunk], w.q_rows[chunk], w.window,
                                   w.num_kv_heads, w.head_dim, w.elem_bytes)
        j = (j + 1) % w.num_seqs
    one_el = time.perf_counter() - t1
    ref.threads = 0
    return ref, {
        "value": round(done_bytes / el / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 oracle on {frac:.2f} layer(s) of the same workload "
                  f"({done_rows} query rows, {done_bytes / 1e9:.3f} GB of KV) in {el:.1f} s",
        "tokens_per_s": round(done_rows / el / n_layers, 3),
        "tokens_per_s_note": f"one layer's rate scaled to {n_layers} layers",
        "value_one_thread": round(one_bytes / one_el / 1e9, 3),
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def read_ceiling(pa, gib=4, launches=5):
    """The plain read rate of this device: pa_stream_read over a dedicated buffer of `gib`
    GiB (far beyond the 256 MB MALL), two untimed launches, then `launches` timed ones."""
    import torch
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        pa.stream_read(buf, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]
    for a, b in ev:
        a.record()
        pa.stream_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / launches
    del buf
    return {"kernel": "stream_read_kernel", "achieved": round(buf_bytes(gib) / (ms / 1e3) / 1e9, 2),
            "unit": "GB/s", "bytes_per_launch": buf_bytes(gib), "launches_timed": launches,
            "note": "one contiguous read of a buffer with 16-byte non-temporal loads, this box"}


def buf_bytes(gib):
    return gib << 30


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction, published


def time_swap(pa, dw, pools, n_seqs):
    """Evict the n_seqs sequences that arrived last (all of their blocks, every layer) to
    pinned host memory, then bring them back into free blocks; GB/s of each direction over
    the host link, next to a plain contiguous hipMemcpy of the same bytes."""
    import numpy as np
    import torch
    pool = dw.pool
    pool.take_copies()
    victims, outs = [], []
    blocks = sum(1 for s in range(dw.w.num_seqs) for b in pool.block_table(s) if b >= 0)
    pool.set_host_blocks(blocks)
    for _ in range(n_seqs):
        v = pool.latest_resident()
        if v is None:
            break
        victims.append(v)
        outs.append(pool.swap_out(v))
    pool.take_copies()
    ins = [pool.swap_in(v) for v in victims]
    pool.take_copies()
    out_p = torch.from_numpy(np.concatenate(outs)).cuda()
    in_p = torch.from_numpy(np.concatenate(ins)).cuda()
    kc = pools[0][0]
    nh = int(out_p.shape[0])
    host = [(torch.empty((nh,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True),
             torch.empty((nh,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True))
            for _ in pools]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    tile_bytes = kc[0].numel() * kc.element_size()          # all heads of one block
    moved = 2 * nh * tile_bytes * len(pools)                 # K and V, every layer

    def timed(fn):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3

    def out_all():
        for (k, v), (hk, hv) in zip(pools, host):
            pa.swap_blocks(k, v, hk, hv, out_p, err)

    def in_all():
        for (k, v), (hk, hv) in zip(pools, host):
            pa.swap_blocks(hk, hv, k, v, in_p, err)

    out_all()
    in_all()                                                  # warm-up
    t_out = timed(out_all)
    t_in = timed(in_all)
    # the same bytes as one contiguous copy each way
    hbuf = torch.empty(moved // len(pools), dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty_like(hbuf, device="cuda")
    dbuf.fill_(1)
    t_d2h = timed(lambda: [hbuf.copy_(dbuf, non_blocking=True) for _ in pools])
    t_h2d = timed(lambda: [dbuf.copy_(hbuf, non_blocking=True) for _ in pools])
    return {
        "seqs": len(victims),
        "blocks": nh,
        "layers": len(pools),
        "bytes_each_way": moved,
        "out_GBps": round(moved / t_out / 1e9, 2),
        "in_GBps": round(moved / t_in / 1e9, 2),
        "out_ms": round(t_out * 1e3, 3),
        "in_ms": round(t_in * 1e3, 3),
        "memcpy_d2h_GBps": round(moved / t_d2h / 1e9, 2),
        "memcpy_h2d_GBps": round(moved / t_h2d / 1e9, 2),
        "bound": "host link",
        "peak": HOST_LINK_PEAK_GBS,
        "unit": "GB/s",
        "frac_out": round(moved / t_out / 1e9 / HOST_LINK_PEAK_GBS, 4),
        "frac_in": round(moved / t_in / 1e9 / HOST_LINK_PEAK_GBS, 4),
        "error_bits": int(err.item()),
    }


# keys of the contract line that a secondary workload's record does not repeat
CONTRACT_KEYS = ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling",
                 "vs_baseline", "data")


def measure(args, name, kv="native", block_size=16, swap_seqs=0, cpu_seconds=None):
    """Build one workload on the device, time args.steps steps after args.warmup, and return
    its result record (the contract keys included) and the decode kernel's GB/s."""
    import numpy as np
    import torch

    import paged_kv_cache_144_amd as pa
    import workloads
    from paged_kv_cache_144_amd.runner import DeviceWorkload

    over = {}
    if block_size != 16:
        over["block_size"] = block_size
    if kv == "q8":
        over["dtype"] = Q8_DTYPE[name]
    w = workloads.make(name, **over)
    L = args.layers or w.n_layers
    print(f"[bench] building {name}: {w.num_seqs} seqs, {w.total_q_rows} rows, "
          f"{w.num_blocks} blocks/layer, {L} layers", file=sys.stderr, flush=True)
    dw = DeviceWorkload(w, "cuda")
    pools = [(dw.k_cache, dw.v_cache)]
    for _ in range(L - 1):
        pools.append((dw.k_cache.clone(), dw.v_cache.clone()))
    rows = torch.from_numpy(step_rows(w)).cuda()
    k_step = dw.k_new.index_select(0, rows).contiguous()
    v_step = dw.v_new.index_select(0, rows).contiguous()
    slot_step = dw.slot_mapping.index_select(0, rows).contiguous()
    out = torch.empty((w.total_q_rows, w.num_q_heads, w.head_dim), dtype=torch.float32,
                      device="cuda")
    kv_layer = kv_bytes_read(w.seq_lens, w.q_rows, w.window, w.num_kv_heads, w.head_dim,
                             w.elem_bytes)
    held = sum(len([b for b in dw.pool.block_table(s) if b >= 0]) for s in range(w.num_seqs))
    waste = 1.0 - min(int(w.seq_lens.sum()), held * w.block_size) / max(1, held * w.block_size)
    qsl = dw.qsl if dw.uses_rows else None
    common = dict(max_seq_len=dw.max_seq_len, query_start_loc=qsl, window=w.window,
                  workspace=dw.workspace)

    has_chunks = bool((w.q_rows > 1).any()) and w.dtype in MFMA_PEAK_TFLOPS
    copies = dw.step_copies
    # the one-launch step (slot write inside the decode launch) where it applies: one query
    # row per sequence and a cache that takes new rows as they are (not 8-bit)
    fused = (args.step == "fused" and bool((w.q_rows == 1).all())
             and w.dtype in ("f32", "f16", "bf16"))

    # layers whose launches are timed: about three per step, in the middle of each group of
    # `every` layers (an event pair costs the GPU a few microseconds, about a tenth of a
    # sliding-window layer, so fewer pairs keep the step close to an untimed one)
    every = max(1, args.event_every or -(-L // 3))
    sampled = list(range(every // 2, L, every))
    slot = {li: si for si, li in enumerate(sampled)}
    # Where a layer is exactly one launch (the one-launch step in group mode: no merge, no
    # copy, no chunk rows), one event pair brackets a run of consecutive layers instead, so
    # that the pair's own cost (a few microseconds, a sixth of a sliding-window kernel) is
    # shared by the run; the per-launch time then includes the short gaps between launches.
    kernel = pa.decode_kernel_name(dw.k_cache, w.num_q_heads, dw.q.dtype, w.num_seqs,
                                   w.window if bool((w.q_rows == 1).all()) else 0)
    run = 1
    if (fused and kernel == "decode_group_kernel" and copies is None and not has_chunks
            and args.event_every is None and every >= 4):
        run = every - 2
        sampled = list(range(1, L - run + 1, every))
        slot = {li: si for si, li in enumerate(sampled)}
    run_end = {li + run - 1: si for si, li in enumerate(sampled)}

    def step(events=None, cevents=None, xevents=None, wevents=None):
        pa.decode(dw.q, pools[0][0], pools[0][1], dw.block_tables, dw.seq_lens, float(w.scale),
                  step="plan", **common)
        for li, (kc, vc) in enumerate(pools):
            timed_layer = li in slot
            si = slot.get(li, 0)
            if copies is not None:
                if xevents is not None and timed_layer:
                    xevents[si][0].record()
                pa.copy_blocks(kc, vc, copies)
                if xevents is not None and timed_layer:
                    xevents[si][1].record()
            if not fused:
                if wevents is not None and timed_layer:
                    wevents[si][0].record()
                pa.write_kv(k_step, v_step, slot_step, kc, vc)
                if wevents is not None and timed_layer:
                    wevents[si][1].record()
            if events is not None and run == 1:
                pa.set_decode_profile_events(*(events[si] if timed_layer else (None, None)))
            elif events is not None and timed_layer:
                events[si][0].record()
            if cevents is not None:
                pa.set_chunk_profile_events(*(cevents[si] if timed_layer else (None, None)))
            if fused:
                pa.decode_write_attend(dw.q, k_step, v_step, kc, vc, dw.block_tables,
                                       dw.seq_lens, float(w.scale), max_seq_len=dw.max_seq_len,
                                       window=w.window, workspace=dw.workspace, out=out)
            else:
                pa.decode(dw.q, kc, vc, dw.block_tables, dw.seq_lens, float(w.scale), out=out,
                          step="attend", **common)
            if events is not None and run > 1 and li in run_end:
                events[run_end[li]][1].record()
        if events is not None:
            pa.set_decode_profile_events(None, None)
        if cevents is not None:
            pa.set_chunk_profile_events(None, None)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()

    # one pair of events per timed launch (every N-th layer) in the timed region
    def event_pairs():
        e = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in sampled] for _ in range(args.steps)]
        for per in e:
            for a, b in per:
                a.record()
                b.record()
        return e

    evs = event_pairs()
    cevs = event_pairs() if has_chunks else None
    xevs = event_pairs() if copies is not None else None
    wevs = None if fused else event_pairs()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(evs[k], cevs[k] if cevs else None, xevs[k] if xevs else None,
             wevs[k] if wevs else None)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    dec_avg_ms = float(np.mean([a.elapsed_time(b) for per in evs for a, b in per])) / run
    chunk_avg_ms = (float(np.mean([a.elapsed_time(b) for per in cevs for a, b in per]))
                    if cevs else 0.0)
    copy_avg_ms = (float(np.mean([a.elapsed_time(b) for per in xevs for a, b in per]))
                   if xevs else 0.0)
    write_avg_ms = (float(np.mean([a.elapsed_time(b) for per in wevs for a, b in per]))
                    if wevs else 0.0)
    err_bits = pa.device_error_bits(dw.workspace)

    step_s = total_ms / 1e3 / args.steps
    value = kv_layer * L / step_s / 1e9
    tokens_per_s = w.total_q_rows / step_s
    dec = w.q_rows == 1
    kv_decode = kv_bytes_read(w.seq_lens[dec], w.q_rows[dec], w.window, w.num_kv_heads,
                              w.head_dim, w.elem_bytes)
    achieved = kv_decode / (dec_avg_ms / 1e3) / 1e9
    traffic = (measured_traffic(name + ("_q8" if kv == "q8" else ""), KERNEL_SOURCES[kernel])
               if block_size == 16 else None)
    decode_roof = {
        "kernel": kernel,
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": int(kv_decode),
        "decode_kernel_avg_us": round(dec_avg_ms * 1e3, 2),
        "launches_timed": args.steps * len(sampled) * run,
        "timing": ("hipEvents around each timed launch" if run == 1 else
                   f"hipEvents around runs of {run} consecutive one-launch layers"),
    }
    chunk_roof = None
    if has_chunks:
        flops = chunk_flops(w.seq_lens, w.q_rows, w.window, w.num_q_heads, w.head_dim)
        tflops = flops / (chunk_avg_ms / 1e3) / 1e12
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        # the chunks' K/V, each (token, KV head) once: what the kernel must read at least
        chunk_kv = sum(2 * w.num_kv_heads * w.head_dim * w.elem_bytes * int(n_)
                       for n_, r_ in zip(w.seq_lens, w.q_rows) if r_ > 1)
        chunk_roof = {
            "kernel": "chunk_kernel",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": (measured_traffic(name + "_chunk", CHUNK_SOURCES)
                        if block_size == 16 else None),
            "chunk_kv_bytes_per_launch": int(chunk_kv),
            "algorithmic_flops_per_launch": int(flops),
            "chunk_kernel_avg_us": round(chunk_avg_ms * 1e3, 2),
            "launches_timed": args.steps * len(sampled),
        }

    copy_roof = None
    if copies is not None:
        # each copied row of K and of V, per KV head, is read once and written once
        cbytes = (4 * int(copies[:, 2].sum().item()) * w.num_kv_heads * w.head_dim
                  * w.elem_bytes)
        gbs = cbytes / (copy_avg_ms / 1e3) / 1e9
        copy_roof = {
            "kernel": "copy_blocks_kernel",
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": int(cbytes),
            "copies_per_launch": int(copies.shape[0]),
            "copy_kernel_avg_us": round(copy_avg_ms * 1e3, 2),
            "launches_timed": args.steps * len(sampled),
        }

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(tokens_per_s, 1),
        "config": {
            "workload": DESCRIPTIONS[name] + (
                "; 8-bit KV cache, one fp16 scale per 32 values" if kv == "q8" else "") + (
                f"; {block_size}-token blocks" if block_size != 16 else ""),
            "block_size": w.block_size,
            # slots allocated but empty (last blocks) over slots allocated
            "internal_waste": round(float(waste), 5),
            "batch": w.num_seqs,
            "query_rows": w.total_q_rows,
            "layers": L,
            "seq_len_total": int(w.seq_lens.sum()),
            "kv_bytes_per_layer": int(kv_layer),
            "seed": w.seed,
            "slot_write": "inside the decode launch" if fused else "own launch",
        },
        "roofline": chunk_roof if chunk_roof and chunk_avg_ms > dec_avg_ms else decode_roof,
        "write_kv": ({
            "fused": True,
            "note": "each new row is read and written inside the decode launch "
                    "(pa_decode_write_attend): no launch of its own",
            # each new row of K and of V is read once and written once
            "bytes_per_layer": int(4 * k_step.numel() * k_step.element_size()),
        } if fused else {
            "fused": False,
            "avg_us": round(write_avg_ms * 1e3, 2),
            "bytes_per_launch": int(4 * k_step.numel() * k_step.element_size()),
            "launches_timed": args.steps * len(sampled),
        }),
        "device_error_bits": err_bits,
    }
    if chunk_roof:
        result["roofline_decode"] = decode_roof
        result["roofline_chunk"] = chunk_roof
    if copy_roof:
        result["roofline_copy"] = copy_roof
    if swap_seqs > 0:
        result["swap"] = time_swap(pa, dw, pools, swap_seqs)
    if cpu_seconds:
        print(f"[bench] cpu baseline (oracle) on {name}", file=sys.stderr, flush=True)
        ref, cb = cpu_baseline(w, L, cpu_seconds)
        # the GPU output of the last layer (same values in every layer) on a few decode rows
        dec = np.nonzero(w.q_rows == 1)[0][:16]
        if dec.size:
            got = out.cpu().numpy().astype(np.float64)[w.query_start_loc()[dec]]
            cb["gpu_max_abs_err_vs_oracle"] = float(np.abs(got - ref.attention(seqs=dec)).max())
        result["cpu_baseline"] = cb
    # release this workload's pools before anything else is built
    del pools, dw, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return result, achieved


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="opt13b", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--also", default=None, metavar="W[,W...]",
                    help="workloads measured after the main one, each reported under its own "
                         "key with its own roofline and CPU baseline (default: gqa when the "
                         "main workload is the default OPT-13B shape with 16-bit KV, else none; "
                         "'none' for none)")
    ap.add_argument("--layers", type=int, default=None, help="default: the workload's")
    ap.add_argument("--block-size", type=int, choices=[8, 16, 32], default=16,
                    help="tokens per KV block (8 and 32: OPT-13B and GQA shapes, 16-bit KV)")
    ap.add_argument("--kv", choices=["native", "q8"], default="native",
                    help="q8: 8-bit KV cache (one fp16 scale per 32 values), same workload")
    ap.add_argument("--event-every", type=int, default=None, metavar="N",
                    help="kernel durations come from hipEvents recorded around the launches "
                         "of every N-th layer of each timed step (each recorded event adds a "
                         "few microseconds of queue gap, which N = 1 would add to every layer); "
                         "default: about three layers per step")
    ap.add_argument("--step", choices=["fused", "separate"], default="fused",
                    help="fused: each layer's slot write runs inside its decode launch "
                         "(pa_decode_write_attend) where the batch allows it (one query row "
                         "per sequence, 16- or 32-bit cache); separate: pa_write_kv, then "
                         "pa_decode_attend")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--swap-seqs", type=int, default=0, metavar="N",
                    help="after the timed steps, also time evicting the N sequences that "
                         "arrived last to pinned host memory and bringing them back")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only; run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_144_amd as pa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)
        return

    if args.block_size != 16 and (args.workload not in ("opt13b", "gqa") or args.kv == "q8"):
        print("bench.py: 8- and 32-token blocks are built for the OPT-13B and GQA "
              "shapes with 16-bit KV", file=sys.stderr)
        sys.exit(2)
    if args.kv == "q8" and args.workload not in Q8_DTYPE:
        print(f"bench.py: no 8-bit variant of {args.workload}", file=sys.stderr)
        sys.exit(2)
    if args.also is None:
        default = (args.workload == "opt13b" and args.kv == "native" and args.block_size == 16
                   and not args.layers)
        also = ["gqa"] if default else []
    else:
        also = [a for a in args.also.split(",") if a and a != "none"]
    for a in also:
        if a not in DESCRIPTIONS:
            print(f"bench.py: unknown workload {a!r}", file=sys.stderr)
            sys.exit(2)

    cpu = None if args.no_cpu_baseline else args.cpu_seconds
    result, achieved = measure(args, args.workload, args.kv, args.block_size, args.swap_seqs,
                               cpu)
    extra = {}
    for a in also:
        r, a_achieved = measure(args, a, args.kv if a in Q8_DTYPE else "native", 16, 0, cpu)
        extra[a] = (r, a_achieved)
    ceiling = read_ceiling(pa)
    ceiling["decode_kernel_frac_of_ceiling"] = round(achieved / ceiling["achieved"], 4)
    result["hbm_read_ceiling"] = ceiling
    for a, (r, a_achieved) in extra.items():
        r["decode_kernel_frac_of_ceiling"] = round(a_achieved / ceiling["achieved"], 4)
        result[a] = {k: v for k, v in r.items() if k not in CONTRACT_KEYS}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
