#!/usr/bin/env python3
"""Decode-step benchmark of the block-quantized KV cache on one MI355X.

Headline step = one decode step of the whole hot path on the 8K int4 workload (batch 8,
32 heads, head_dim 128, context 8192 per sequence, 4-bit block codes, 64-token blocks):
decode_step_qkv quantizes one new token per (sequence, head) into its row's tail block
and attends one fp16 query per (sequence, head) over the whole compressed cache,
including that token. With one split per row (256 rows fill the GPU) that is one
kernel launch: each row's workgroup appends, then attends. --separate times the same
step as two calls, kv_append then decode_attn_qkv.

Inputs are synthetic and seeded (decode_attention_block_amd.workloads), already
resident in HBM when timing starts. Steps rotate over enough copies of the cache
(>= 1 GiB in all) that the 256 MB Infinity Cache cannot hold them, so every step
reads its cache from HBM. Each copy gains one token per use, so the context grows
from 8192 by at most ceil(steps / copies) tokens; bytes are counted from the actual
lengths. Warm-up steps (the GPU takes a few milliseconds of load to reach steady
clocks) run first, from the same prefill lengths, which are restored before timing.

The same run also measures the other workloads (unless --headline-only) and reports
them under "workloads":
  * the 8K uint8 and FP8 E4M3 workloads, with the same step and rotation;
  * the 32K workload (batch 16, context 32768): its 64-step decode loop of
    decode_step_qkv, repeated from the same prefill (lengths reset between loops,
    outside the timed region);
  * the 32-layer ragged workload: one step is decode_attn_qkv over each of the 32
    layers' caches (per-sequence lengths 1024..8192, no append in this workload).
  * the grouped-query workload (64 query heads over 8 cached heads, batch 8, context
    8192): one step is decode_attn_gqa over one of the rotated cache copies;
  * the headline decode step again on paged caches (shuffled page pools).

Prints one JSON line. --profile-loop runs only the timed loop of --workload (for
rocprofv3), --copy-probe times a plain device copy of known size (the calibration
kernel for the FETCH_SIZE / WRITE_SIZE counters).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_int4_b8h32d128_ctx8k_traffic.json")
CACHE_BYTES_TARGET = 1 << 30   # total bytes of rotated cache copies
EVENT_STRIDE = 8               # HIP events around every 8th attention launch when a step
                               # has several launches: a pair of events around a launch
                               # adds ~5 us to its step
HEADLINE = "llama7b_b8_h32_d128_ctx8k_int4"
KV_FORMATS = {0: "int4 block-64 symmetric", 1: "uint8 block-64 asymmetric",
              2: "fp8 e4m3 block-64 scaled"}
OTHERS = ("llama7b_b8_h32_d128_ctx8k_uint8", "llama7b_b8_h32_d128_ctx8k_fp8",
          "long_b16_h32_d128_ctx32k_append64_int4",
          "llama7b_32layer_b8_h32_d128_ragged1k-8k_t3_int4", "llama70b_gqa8_b8_h8_d128_ctx8k_int4")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--blocks-per-split", type=int, default=0)
    p.add_argument("--separate", action="store_true",
                   help="time the step as kv_append + decode_attn_qkv (two calls)")
    p.add_argument("--paged", action="store_true",
                   help="time --workload on a paged cache (shuffled page pool)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate host time spent timing the oracle")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="measure only --workload, not the other workloads")
    p.add_argument("--profile-loop", action="store_true",
                   help="only the timed loop of --workload (for rocprofv3); no oracle, "
                        "no other workloads")
    p.add_argument("--copy-probe", action="store_true",
                   help="only a 1 GiB device-to-device copy (counter calibration)")
    return p.parse_args()


def code_bytes_per_token(w):
    return w.head_dim // 2 if w.scheme == 0 else w.head_dim


def attention_bytes(w, lens):
    """Algorithmic bytes of one decode_attn_qkv (decode_attn_gqa) call: K and V codes of
    the valid tokens, their block scales (and zero points for uint8), q and out (one
    row per query head)."""
    per_block_scalars = 2 * (2 if w.scheme == 1 else 1) * 4
    total = 0
    for n in lens:
        nb = (int(n) + 63) // 64
        total += w.heads * (2 * int(n) * code_bytes_per_token(w) + nb * per_block_scalars)
    total += 2 * w.batch * w.heads * w.group * w.head_dim * 2  # q in, out
    return total


def append_bytes(w):
    """Algorithmic bytes of one kv_append: the new K and V tokens in (fp16), their
    staged fp16 copy and their codes out."""
    rows = w.batch * w.heads
    return rows * 2 * (w.head_dim * 2 * 2 + code_bytes_per_token(w))


def measured_traffic():
    """HBM bytes per launch of the headline step kernel from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (scaled by the counters' reading for a 1 GiB copy), or None once the kernel's
    sources differ from the ones the counters were taken on."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    reps = 10
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"copy_bytes": n, "copy_ms": ms, "copy_gbs_read_plus_write": 2 * n / ms / 1e6}


def cpu_baseline(w, host_cache, q, lens, budget_s):
    """The oracle (single-threaded C++, fp64 attention over the dequantized cache) timed
    on the host: whole passes over all (sequence, head) rows of the workload's attention,
    repeated until about budget_s seconds have passed."""
    import oracle
    sm = float(np.float32(1) / np.sqrt(np.float32(w.head_dim)))
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention(host_cache, q, lens, sm)
        passes += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s:
            break
    gbs = passes * attention_bytes(w, lens) / elapsed / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full passes of the decode attention (all {w.batch * w.heads} "
                      f"sequence-head rows, context {int(lens[0])}) of {w.name} by the fp64 "
                      f"oracle on one host thread, {elapsed:.1f} s; kv_append not included",
            "tokens_per_s": w.batch * passes / elapsed}


def cpu_baseline_all_cores(w, host_cache, q, lens, budget_s):
    """The same unchanged oracle routine with the rows of each pass partitioned over all
    host cores this process may use (threads; the C++ routine runs outside the GIL)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    sm = float(np.float32(1) / np.sqrt(np.float32(w.head_dim)))
    n_rows = w.batch * w.heads
    cores = max(1, min(len(os.sched_getaffinity(0)), n_rows))
    bounds = [(n_rows * i // cores, n_rows * (i + 1) // cores) for i in range(cores)]
    passes = 0
    with ThreadPoolExecutor(cores) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(lambda r: oracle.attention(host_cache, q, lens, sm, rows=r), bounds))
            passes += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= budget_s:
                break
    gbs = passes * attention_bytes(w, lens) / elapsed / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} full passes of the same decode attention, rows split over "
                      f"{cores} host threads, {elapsed:.1f} s",
            "tokens_per_s": w.batch * passes / elapsed}


class Timer:
    """HIP events around sampled kernel launches (every EVENT_STRIDE-th) and around
    each timed segment, all on the current stream (the one the library's kernels are
    queued on). An event pair measures the launch including its dispatch."""

    def __init__(self, torch):
        self.torch = torch
        self.kernel = []     # (start, end) event pairs
        self.segments = []

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def kernel_ms(self):
        return [a.elapsed_time(b) for a, b in self.kernel]

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.segments)


def quantized_copies(kvq, torch, w, layer, lens, max_blocks, n_copies, device_inputs,
                     paged=False):
    """n_copies caches holding the quantized prefill of one layer; returns them and the
    prefill kernel times (ms). device_inputs: draw K and V with the device-side recipe
    (same distributions, other values) instead of the host recipe. paged: each copy is a
    paged cache whose block table scatters the blocks over its pool in a seeded random
    order."""
    n = int(np.max(lens))
    wl = wl_mod()
    if device_inputs:
        k = wl.prefill_batch_device(w, layer, 0, n_tokens=n)
        v = wl.prefill_batch_device(w, layer, 1, n_tokens=n)
    else:
        k = torch.from_numpy(wl.prefill_batch(w, layer, 0, n_tokens=n)).cuda()
        v = torch.from_numpy(wl.prefill_batch(w, layer, 1, n_tokens=n)).cuda()
    caches, ms = [], []
    for i in range(n_copies):
        if paged:
            n_pages = w.batch * max_blocks
            c = kvq.KVCache(w.scheme, w.batch, w.heads, w.head_dim, max_blocks,
                            num_pages=n_pages)
            perm = np.random.default_rng([w.index, i]).permutation(n_pages).astype(np.int32)
            c.block_table.copy_(torch.from_numpy(perm.reshape(w.batch, max_blocks)))
        else:
            c = kvq.KVCache(w.scheme, w.batch, w.heads, w.head_dim, max_blocks)
        c.seq_lens.copy_(torch.from_numpy(np.asarray(lens, np.int32)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.kv_quantize_blocks(c, k, v, n)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        caches.append(c)
    del k, v
    return caches, ms


def wl_mod():
    from decode_attention_block_amd import workloads
    return workloads


def workspace(kvq, torch, cache, lengths, bps):
    n = max(kvq.decode_attn_workspace_bytes(cache, int(L), bps) for L in lengths)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")   # counters start at zero


def run_append_attention(kvq, torch, w, steps, warmup, bps, keep_host, device_inputs,
                         separate=False, paged=False):
    """Single-layer fixed-length workloads; step = decode_step_qkv (or, with separate,
    kv_append + decode_attn_qkv; the sampled kernel is then the attention alone).

    Steps run in segments that start from the prefill lengths (reset between segments,
    untimed): the 32K workload's segments are its 64-step decode loop on one cache; the
    8K workloads rotate over cache copies, each gaining one token per use. Warm-up steps
    are whole steps too, in segments of their own."""
    wl = wl_mod()
    B, H, D = w.batch, w.heads, w.head_dim
    per_cache = 2 * B * H * w.context * code_bytes_per_token(w)
    if w.decode_steps:
        copies, growth = 1, w.decode_steps
    else:
        copies = max(1, math.ceil(CACHE_BYTES_TARGET / per_cache))
        growth = math.ceil(steps / copies)
    seg_cap = copies * growth                # steps before lengths must be reset
    max_blocks = (w.context + growth + 63) // 64
    t_setup = time.perf_counter()
    caches, prefill_ms = quantized_copies(kvq, torch, w, 0, wl.lengths(w), max_blocks, copies,
                                          device_inputs, paged)
    kn = np.stack([wl.appended_kv(w, 0, s, 0, growth) for s in range(B)], axis=1)
    vn = np.stack([wl.appended_kv(w, 0, s, 1, growth) for s in range(B)], axis=1)
    k_new = torch.from_numpy(kn).cuda()          # [growth][B][H][D]
    v_new = torch.from_numpy(vn).cuda()
    queries = torch.from_numpy(np.stack([wl.query(w, 0, s) for s in range(seg_cap)])).cuda()
    host_cache = caches[0].host_arrays() if keep_host else None
    ws = workspace(kvq, torch, caches[0], range(w.context, w.context + growth + 1), bps)
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    timer = Timer(torch)
    kernel_bytes, step_bytes = [], []
    # One launch per step: the kernel's average duration is the timed segments' total
    # over the steps (HIP events bracket the segments); several launches per step: HIP
    # events around every EVENT_STRIDE-th launch of the attention kernel.
    bps_eff, n_split = kvq.decode_attn_plan(caches[0], w.context + growth, bps)
    one_launch = not separate and n_split == 1

    def step(j, timed):
        """Step j of a segment: copy j % copies gains its (j // copies)-th token."""
        c = caches[j % copies]
        used = j // copies
        L = w.context + used + 1
        if separate:
            kvq.kv_append(c, k_new[used], v_new[used], L)
        sample = timed and not one_launch and j % EVENT_STRIDE == 0
        if sample:
            e0 = timer.event()
        if separate:
            kvq.decode_attn_qkv(c, queries[j], sm, out, ws, L, bps)
        else:
            kvq.decode_step_qkv(c, k_new[used], v_new[used], queries[j], sm, out, ws, L, bps)
        if sample:
            timer.kernel.append((e0, timer.event()))
            kernel_bytes.append(attention_bytes(w, [L] * B) +
                                (0 if separate else append_bytes(w)))
        if timed:
            step_bytes.append(attention_bytes(w, [L] * B) + append_bytes(w))
            if one_launch:
                kernel_bytes.append(step_bytes[-1])

    def run(n_steps, timed):
        done = 0
        while done < n_steps:
            for c in caches:
                c.seq_lens.fill_(w.context)
            torch.cuda.synchronize()
            n = min(seg_cap, n_steps - done)
            t0 = timer.event() if timed else None
            for j in range(n):
                step(j, timed)
            if timed:
                timer.segments.append((t0, timer.event()))
            done += n
        torch.cuda.synchronize()

    run(warmup, False)
    wall0 = time.perf_counter()
    run(steps, True)
    wall_s = time.perf_counter() - wall0
    total_ms = timer.total_ms()
    kernel_ms = [total_ms / steps] if one_launch else timer.kernel_ms()
    res = {
        "workload": w.name,
        "step": ("kv_append + decode_attn_qkv" if separate else
                 "decode_step_qkv (%s)" % ("append and attention in one launch" if one_launch
                                           else "append, then attention")),
        "kernel": kernel_name(w, fused=one_launch, paged=paged),
        "layout": "paged (block table over a shuffled page pool)" if paged else "dense",
        "steps": steps, "warmup": warmup,
        "ms_per_step": total_ms / steps,
        "gbs": sum(step_bytes) / (total_ms / 1e3) / 1e9,
        "tokens_per_s": B * steps / (total_ms / 1e3),
        "kernel_avg_us": float(np.mean(kernel_ms)) * 1e3,
        "kernel_gbs": float(np.mean(kernel_bytes)) / (float(np.mean(kernel_ms)) / 1e3) / 1e9,
        "kernel_bytes_per_launch": float(np.mean(kernel_bytes)),
        "kernel_timing": ("timed segments / steps (one launch per step)" if one_launch else
                          f"HIP event pairs around every {EVENT_STRIDE}th attention launch"),
        "context": [w.context + 1, w.context + growth],
        "cache_copies_rotated": copies, "blocks_per_split": bps_eff, "splits_per_row": n_split,
        "prefill_quantize_ms": float(np.median(prefill_ms)),
        "prefill_quantize_gbs": (2 * B * w.context * H * D * 2 + per_cache)
        / (float(np.median(prefill_ms)) / 1e3) / 1e9,
        "host_wall_s": wall_s, "setup_s": setup_s,
    }
    res["kernel_frac"] = res["kernel_gbs"] / HBM_PEAK_GBS
    return res, host_cache


def run_gqa(kvq, torch, w, steps, warmup, bps, paged=False):
    """Grouped-query workload: one step is decode_attn_gqa (w.group query heads per
    cached head) over one of enough cache copies (>= CACHE_BYTES_TARGET in all) that the
    Infinity Cache cannot hold them; lengths fixed at the context (no append)."""
    wl = wl_mod()
    B, H, D, G = w.batch, w.heads, w.head_dim, w.group
    lens = wl.lengths(w)
    L = int(lens.max())
    per_cache = 2 * B * H * L * code_bytes_per_token(w)
    copies = max(1, math.ceil(CACHE_BYTES_TARGET / per_cache))
    t_setup = time.perf_counter()
    caches, prefill_ms = quantized_copies(kvq, torch, w, 0, lens, w.max_blocks, copies, False,
                                          paged)
    q = torch.from_numpy(wl.query(w, 0)).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(kvq.decode_attn_gqa_workspace_bytes(caches[0], G, L, bps), 16),
                     dtype=torch.uint8, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    timer = Timer(torch)

    def run(n):
        for j in range(n):
            kvq.decode_attn_gqa(caches[j % copies], q, G, sm, out, ws, L, bps)

    run(warmup)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0 = timer.event()
    run(steps)
    timer.segments.append((t0, timer.event()))
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    total_ms = timer.total_ms()
    per_launch = attention_bytes(w, lens)
    bps_eff, n_split = kvq.decode_attn_gqa_plan(caches[0], G, L, bps)
    res = {
        "workload": w.name,
        "step": f"decode_attn_gqa ({G} query heads per cached head)",
        "kernel": f"attn_split_int4_gqa_kernel<{D}, {G}, {'true' if paged else 'false'}>",
        "layout": "paged (block table over a shuffled page pool)" if paged else "dense",
        "steps": steps, "warmup": warmup,
        "ms_per_step": total_ms / steps,
        "gbs": per_launch * steps / (total_ms / 1e3) / 1e9,
        "tokens_per_s": B * steps / (total_ms / 1e3),
        "kernel_avg_us": total_ms / steps * 1e3,
        "kernel_gbs": per_launch / (total_ms / steps / 1e3) / 1e9,
        "kernel_bytes_per_launch": float(per_launch),
        "kernel_timing": "timed segment / launches (one launch per step)",
        "context": [L, L], "cache_copies_rotated": copies,
        "blocks_per_split": bps_eff, "splits_per_row": n_split,
        "prefill_quantize_ms": float(np.median(prefill_ms)),
        "host_wall_s": wall_s, "setup_s": setup_s,
    }
    res["kernel_frac"] = res["kernel_gbs"] / HBM_PEAK_GBS
    return res


def run_layers(kvq, torch, w, steps, warmup, bps, device_inputs):
    """The 32-layer ragged workload: one step is decode_attn_qkv over every layer's
    cache, each layer with its own K, V and query."""
    wl = wl_mod()
    B, H, D = w.batch, w.heads, w.head_dim
    lens = wl.lengths(w)
    L = int(lens.max())
    plan_note = "automatic"
    if bps == 0 and w.ragged is not None:
        # a ragged batch: the caller, who knows it, splits rows at about half the
        # longest one, so the longest rows share their blocks between workgroups
        bps = ((L + 63) // 64 + 1) // 2
        plan_note = "half the longest row (chosen by the caller for a ragged batch)"
    t_setup = time.perf_counter()
    caches, prefill_ms, queries = [], [], []
    for layer in range(w.layers):
        c, ms = quantized_copies(kvq, torch, w, layer, lens, w.max_blocks, 1, device_inputs)
        caches += c
        prefill_ms += ms
        queries.append(torch.from_numpy(wl.query(w, layer)).cuda())
    ws = workspace(kvq, torch, caches[0], [L], bps)
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    timer = Timer(torch)

    def step(timed):
        # one launch per layer and nothing else: the kernel's average duration is the
        # timed segment over the launches
        for layer in range(w.layers):
            kvq.decode_attn_qkv(caches[layer], queries[layer], sm, out, ws, L, bps)

    wall0 = time.perf_counter()
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = timer.event()
    for _ in range(steps):
        step(True)
    timer.segments.append((t0, timer.event()))
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    total_ms = timer.total_ms()
    per_launch = attention_bytes(w, lens)
    kernel_ms = [total_ms / (steps * w.layers)]
    bps_eff, n_split = kvq.decode_attn_plan(caches[0], L, bps)
    res = {
        "workload": w.name,
        "step": f"decode_attn_qkv over {w.layers} layers",
        "kernel": kernel_name(w, fused=False),
        "steps": steps, "warmup": warmup,
        "ms_per_step": total_ms / steps,
        "gbs": per_launch * w.layers * steps / (total_ms / 1e3) / 1e9,
        "tokens_per_s": B * steps / (total_ms / 1e3),
        "kernel_avg_us": float(np.mean(kernel_ms)) * 1e3,
        "kernel_gbs": per_launch / (float(np.mean(kernel_ms)) / 1e3) / 1e9,
        "kernel_bytes_per_launch": float(per_launch),
        "kernel_timing": "timed segment / launches (one launch per layer)",
        "context": [int(lens.min()), L], "mean_context": float(lens.mean()),
        "blocks_per_split": bps_eff, "splits_per_row": n_split, "plan": plan_note,
        "prefill_quantize_ms_per_layer": float(np.median(prefill_ms)),
        "host_wall_s": wall_s, "setup_s": setup_s,
    }
    res["kernel_frac"] = res["kernel_gbs"] / HBM_PEAK_GBS
    res.update(graph_step(torch, w, caches, queries, sm, steps, warmup, bps, step))
    return res


def graph_step(torch, w, caches, queries, sm, steps, warmup, bps, eager_step):
    """The same 32-layer step captured once as a HIP graph (one replay per step) against
    the eager calls: GPU time per step (HIP events around the timed segment) and host
    time to queue one step."""
    from decode_attention_block_amd.graph import DecodeGraph
    dg = DecodeGraph(caches, sm, append=False, blocks_per_split=bps)
    for i, q in enumerate(queries):
        dg.q[i].copy_(q)
    for _ in range(warmup):
        dg.replay()
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("graph", dg.replay), ("eager", lambda: eager_step(True))):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        host = 0.0
        e0.record()
        for _ in range(steps):
            h0 = time.perf_counter()
            fn()
            host += time.perf_counter() - h0
        e1.record()
        torch.cuda.synchronize()
        res[f"{name}_ms_per_step"] = e0.elapsed_time(e1) / steps
        res[f"{name}_host_us_per_step"] = host / steps * 1e6
    res["graph"] = (f"{w.layers} decode_attn_qkv calls captured as one HIP graph "
                    f"(host bound fixed at the capacity, {caches[0].capacity} tokens)")
    return res


def kernel_name(w, fused, paged=False):
    """The timed kernel as rocprofv3 lists it (template arguments: head_dim, whether the
    workgroup also appends the row's token, whether the cache is paged)."""
    f, p = ("true" if fused else "false"), ("true" if paged else "false")
    if w.scheme == 0:
        return f"attn_split_int4_kernel<{w.head_dim}, {f}, {p}>"
    return f"attn_split_kernel<{w.scheme}, {w.head_dim}, {f}, {p}>"


def measure(kvq, torch, w, steps, warmup, bps, keep_host=False, device_inputs=False,
            separate=False, paged=False):
    if w.layers > 1:
        res = run_layers(kvq, torch, w, steps, warmup, bps, device_inputs), None
    elif w.group > 1:
        res = run_gqa(kvq, torch, w, steps, warmup, bps, paged), None
    else:
        res = run_append_attention(kvq, torch, w, steps, warmup, bps, keep_host, device_inputs,
                                   separate, paged)
    res[0]["inputs"] = ("K/V drawn on the device (torch generator, same distributions)"
                        if device_inputs else "K/V from the seeded host recipe")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path "
              f"shards by sequence or head with no communication; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_block_amd as kvq

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_probe:
        print(json.dumps(copy_probe()), flush=True)
        return

    wl = wl_mod()
    w = wl.BY_NAME[args.workload]
    with_cpu = not (args.no_cpu or args.profile_loop)
    print(f"[bench] {w.name}: {args.steps} steps after {args.warmup} warm-up",
          file=sys.stderr, flush=True)
    big = w.decode_steps > 0 or w.layers > 1
    res, host_cache = measure(kvq, torch, w, args.steps, args.warmup, args.blocks_per_split,
                              keep_host=with_cpu and not big, device_inputs=big,
                              separate=args.separate, paged=args.paged)
    if args.profile_loop:
        print(json.dumps(res), flush=True)
        return

    B, H, D = w.batch, w.heads, w.head_dim
    fused = ", true," in res["kernel"]
    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tokens/s, int4 KV, B=8 ctx 8K",
        "value": res["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; see decode_attention_block_amd/workloads.py)",
        "pct_of_hbm_peak": 100.0 * res["gbs"] / HBM_PEAK_GBS,
        "tokens_per_s": res["tokens_per_s"],
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": D,
                   "context": w.context, "context_range_timed": res["context"],
                   "kv_format": KV_FORMATS[w.scheme],
                   "step": res["step"], "layout": res.get("layout", "dense"),
                   "cache_copies_rotated": res.get("cache_copies_rotated"),
                   "blocks_per_split": res["blocks_per_split"],
                   "splits_per_row": res["splits_per_row"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": res["kernel"] + (" (decode_step_qkv: append + attention)"
                                                if fused else f" ({res['step']})"),
                     "achieved": res["kernel_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": res["kernel_gbs"] / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if w.name == HEADLINE and fused else None,
                     "avg_kernel_us": res["kernel_avg_us"], "timing": res["kernel_timing"],
                     "algorithmic_bytes_per_launch": res["kernel_bytes_per_launch"]},
        "graph_step": {k: res[k] for k in res if k.startswith(("graph", "eager"))} or None,
        "prefill_quantize": {"ms": res.get("prefill_quantize_ms"),
                             "gbs": res.get("prefill_quantize_gbs")},
        "host_wall_s": res["host_wall_s"],
        "setup_s": res["setup_s"],
    }
    if with_cpu and host_cache is not None:
        lens0 = np.full(B, w.context, np.int32)
        result["cpu_baseline"] = cpu_baseline(w, host_cache, wl.query(w, 0), lens0,
                                              args.cpu_seconds)
        result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(
            w, host_cache, wl.query(w, 0), lens0, args.cpu_seconds / 2)
        del host_cache
    if not args.headline_only:
        others = []
        for name in OTHERS:
            if name == w.name:
                continue
            ow = wl.BY_NAME[name]
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            steps = 64 * 3 if ow.decode_steps else (20 if ow.layers > 1 else args.steps)
            warm = 10 if ow.layers > 1 else args.warmup
            r, _ = measure(kvq, torch, ow, steps, warm, args.blocks_per_split,
                           device_inputs=ow.decode_steps > 0 or ow.layers > 1,
                           separate=args.separate)
            others.append(r)
            torch.cuda.empty_cache()
        if not args.paged and w.layers == 1:
            print(f"[bench] {w.name} paged", file=sys.stderr, flush=True)
            r, _ = measure(kvq, torch, w, args.steps, args.warmup, args.blocks_per_split,
                           device_inputs=big, separate=args.separate, paged=True)
            others.append(r)
            torch.cuda.empty_cache()
        result["workloads"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
