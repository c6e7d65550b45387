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
lengths.

Timing. The steps run in segments that start from the prefill lengths (restored
between segments, outside the timed region). Each segment's launches are captured once
as a HIP graph and the timed region replays them, bracketed by HIP events on the launch
stream: the GPU then runs the steps back to back, and the time is the kernels' own,
not the host's pace of queueing them (queued one by one from Python, a step of the
headline takes the host about as long as the GPU, so eager timing measures the host).
The eager time of the same steps is reported beside it. Per-step times (p10, p50, p90)
come from a separate sampling pass: HIP event pairs around each eagerly queued step,
all queued behind a few large device copies so that the host is ahead of the GPU.
Warm-up steps (the given number) run first through the same graphs. The other
workloads below, and the read probes, then keep warming up until WARMUP_MS_OTHERS of
wall time has passed, whatever --warmup says: timed right after their setup (and after
the host-side oracle legs of the workload before), with the GPU idle meanwhile, their
first milliseconds run slower, and their lines are meant to show the kernels. Each line
records the warm-up steps it ran; --warmup applies to the headline step as given.

Beside the HBM peak, every one-launch line is set against two streaming-read rates of
the same GPU (kvq_probe_stream_read, one contiguous slab per workgroup): over 2 GiB
(read_ceiling, the practical rate of long streams) and at the line's own bytes per
launch, replayed back to back over rotated copies as the steps are
(read_ceiling_same_size, which pays the same start-up and drain per launch).

The same run measures the other workloads (unless --headline-only) and reports them
under "workloads": the tiny workload (call latency), the 8K uint8 and FP8 E4M3
workloads, the 32K workload (its 64-step decode loop from the same prefill), the
32-layer ragged workload (one step = decode_attn_qkv over the 32 layers' caches), the
grouped-query workload (64 query heads over 8 cached heads), and the headline step on
paged caches. Beside every workload the CPU oracle (the plain C++ implementation the
tests check against) is timed on the host's cores on a sample of the same inputs: the
prefill quantization and one decode step (append + attention), on one thread and with
the sample's heads split over every host thread.

Prints one JSON line. --profile-loop runs only the timed loop of --workload (for
rocprofv3), --prefill-loop only its prefill quantization, --copy-probe times a plain
device copy of known size (the calibration kernel for the FETCH_SIZE / WRITE_SIZE
counters).
"""
import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_int4_b8h32d128_ctx8k_traffic.json")
CACHE_BYTES_TARGET = 1 << 30   # total bytes of rotated cache copies
SAMPLED_STEPS = 32             # steps timed one by one for the percentiles
COMPARE_ROUNDS = 3             # alternating eager / graph rounds for their comparison
HOLD_US = 200                  # stream hold before a timed graph segment (kvq_probe_hold)
WARMUP_MS_OTHERS = 30.0        # untimed GPU work before the other workloads' and probes' timing
HEADLINE = "llama7b_b8_h32_d128_ctx8k_int4"
KV_FORMATS = {0: "int4 block-64 symmetric", 1: "uint8 block-64 asymmetric",
              2: "fp8 e4m3 block-64 scaled"}
DTYPES = {0: "int4 codes x fp16 query -> fp32 accumulate (matrix cores)",
          1: "uint8 codes x fp16 query -> fp32 accumulate",
          2: "fp8 e4m3 codes x fp16 query -> fp32 accumulate"}
OTHERS = ("tiny_b1_h2_d64_ctx256_int4", "llama7b_b8_h32_d128_ctx8k_uint8",
          "llama7b_b8_h32_d128_ctx8k_fp8", "long_b16_h32_d128_ctx32k_append64_int4",
          "llama7b_32layer_b8_h32_d128_ragged1k-8k_t3_int4", "llama70b_gqa8_b8_h8_d128_ctx8k_int4",
          "llama70b_gqa8_b8_h8_d128_ctx8k_fp8")


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
    p.add_argument("--eager", action="store_true",
                   help="time the steps as queued one by one from the host (no graph)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate host time spent timing the oracle's headline decode step")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="measure only --workload, not the other workloads")
    p.add_argument("--profile-loop", action="store_true",
                   help="only the timed loop of --workload (for rocprofv3); no oracle, "
                        "no other workloads")
    p.add_argument("--prefill-loop", action="store_true",
                   help="only the prefill quantization of --workload, repeated (for rocprofv3)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only a 1 GiB device-to-device copy (counter calibration)")
    return p.parse_args()


def wl_mod():
    from decode_attention_block_amd import workloads
    return workloads


# ---- algorithmic bytes ----------------------------------------------------------------
def code_bytes_per_token(w):
    return w.head_dim // 2 if w.scheme == 0 else w.head_dim


def attention_bytes(w, lens, heads=None):
    """Algorithmic bytes of one decode_attn_qkv (decode_attn_gqa) call over the given
    per-sequence lengths: K and V codes of the valid tokens, their block scales (and zero
    points for uint8), q and out (one row per query head)."""
    H = w.heads if heads is None else heads
    per_block_scalars = 2 * (2 if w.scheme == 1 else 1) * 4
    total = 0
    for n in lens:
        nb = (int(n) + 63) // 64
        total += H * (2 * int(n) * code_bytes_per_token(w) + nb * per_block_scalars)
    total += 2 * len(lens) * H * w.group * w.head_dim * 2  # q in, out
    return total


def append_bytes(w, seqs=None, heads=None):
    """Algorithmic bytes of one kv_append: the new K and V tokens in (fp16), their staged
    fp16 copy and their codes out."""
    rows = (w.batch if seqs is None else seqs) * (w.heads if heads is None else heads)
    return rows * 2 * (w.head_dim * 2 * 2 + code_bytes_per_token(w))


def prefill_bytes(w, lens, heads=None):
    """Algorithmic bytes of kv_quantize_blocks over the given lengths: fp16 K and V in,
    codes and block scales (zero points) out."""
    H = w.heads if heads is None else heads
    per_block_scalars = 2 * (2 if w.scheme == 1 else 1) * 4
    total = 0
    for n in lens:
        nb = (int(n) + 63) // 64
        total += H * (2 * int(n) * (2 * w.head_dim + code_bytes_per_token(w)) +
                      nb * per_block_scalars)
    return total


def measured_traffic():
    """HBM bytes per launch of the headline step kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by the counters' reading for a 1 GiB copy), or
    None once the kernel's sources differ from the ones the counters were taken on."""
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


def pct(xs):
    xs = np.asarray(xs, np.float64)
    return {"p10": float(np.percentile(xs, 10)), "p50": float(np.percentile(xs, 50)),
            "p90": float(np.percentile(xs, 90))}


# ---- probes ---------------------------------------------------------------------------
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


def read_ceiling_at(kvq, torch, nbytes):
    """The streaming-read rate at one launch's size: kvq_probe_stream_read of `nbytes`,
    launches replayed back to back from a HIP graph over enough copies (>=
    CACHE_BYTES_TARGET in all) that the Infinity Cache cannot hold them, as the steps
    are timed, at 256, 512 and 1024 workgroups (one contiguous slab each); the best
    counts. A launch of a given size pays the same start-up and drain as the kernels
    compared with it, which the 2 GiB ceiling hides. Some slab sizes read far slower than
    their neighbours (in one run, 134.5 MB in 256 slabs: 52% of peak, with half the
    bytes 65% and twice the bytes 80%), hence the several counts."""
    n = (int(nbytes) + 4095) // 4096 * 4096
    copies = max(1, math.ceil(CACHE_BYTES_TARGET / n))
    reps = max(32, copies)
    buf = torch.empty(copies * n, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    views = [buf[i * n:(i + 1) * n] for i in range(copies)]
    by = {}
    for wg in (256, 512, 1024):
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(reps):
                kvq.kvq_probe_stream_read(views[j % copies], wg, sink)
        torch.cuda.synchronize()
        t_warm = time.perf_counter()
        while (time.perf_counter() - t_warm) * 1e3 < (WARMUP_MS_OTHERS if wg == 256 else 2.0):
            g.replay()
            torch.cuda.synchronize()
        us = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) / reps * 1e3)
        by[str(wg)] = float(np.median(us))
        del g
    del views, buf, sink
    torch.cuda.empty_cache()
    best = min(by, key=by.get)
    t = by[best]
    return {"bytes": n, "us_per_launch": t, "gbs": n / t / 1e3,
            "frac_of_peak": n / t / 1e3 / HBM_PEAK_GBS, "workgroups": int(best),
            "us_by_workgroups": by, "launches_per_replay": reps, "copies": copies}


def with_same_size_ceiling(kvq, torch, res):
    """Adds the read ceiling at the workload's bytes per launch (one-launch steps)."""
    per_launch = res.get("kernel_bytes_per_launch")
    if not per_launch:
        return res
    c = read_ceiling_at(kvq, torch, per_launch)
    res["read_ceiling_same_size"] = c
    res["kernel_frac_of_same_size_read_ceiling"] = res["kernel_gbs"] / c["gbs"]
    return res


def read_ceiling(kvq, torch):
    """The GPU's practical streaming-read rate: kvq_probe_stream_read over 2 GiB (8x the
    Infinity Cache), at several workgroup counts; the best is the ceiling."""
    n = 2 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(7)
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < WARMUP_MS_OTHERS:
        kvq.kvq_probe_stream_read(buf, 256, sink)
        torch.cuda.synchronize()
    by = {}
    for wg in (256, 512, 1024, 2048, 4096):
        for _ in range(2):
            kvq.kvq_probe_stream_read(buf, wg, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            kvq.kvq_probe_stream_read(buf, wg, sink)
        e1.record()
        torch.cuda.synchronize()
        by[str(wg)] = n / (e0.elapsed_time(e1) / reps / 1e3) / 1e9
    best = max(by.values())
    del buf, sink
    torch.cuda.empty_cache()
    return {"gbs": best, "frac_of_peak": best / HBM_PEAK_GBS, "bytes": n,
            "kernel": "kvq_probe_stream_read (contiguous slab per 256-thread workgroup, "
                      "16-byte non-temporal loads)", "gbs_by_workgroups": by}


# ---- timing machinery -----------------------------------------------------------------
class Stepper:
    """Times steps of a workload. queue(j) queues step j of a segment (0 <= j < seg_cap;
    the caller's inputs for step j are fixed); reset() restores the state a segment
    starts from (queued on the stream, outside any timed region). Segments of n steps
    are captured once as HIP graphs (torch's graph capture of the library's launches)
    and replayed."""

    def __init__(self, torch, queue, seg_cap, reset=None):
        self.torch, self.queue, self.seg_cap, self.reset = torch, queue, seg_cap, reset
        self.graphs = {}

    def _graph(self, n):
        if n not in self.graphs:
            torch = self.torch
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(n):
                    self.queue(j)
            torch.cuda.synchronize()
            self.graphs[n] = g
        return self.graphs[n]

    def prepare(self, *step_counts):
        """Captures every segment graph that runs of these step counts will replay, so
        that no capture (host work with the GPU idle) falls between the warm-up and the
        timed steps."""
        for n_steps in step_counts:
            for n in self._segments(n_steps):
                self._graph(n)

    def _segments(self, n_steps):
        done = 0
        while done < n_steps:
            n = min(self.seg_cap, n_steps - done)
            yield n
            done += n

    def run(self, n_steps, timed, graph=True):
        """n_steps steps; returns their total GPU time in ms (HIP events around every
        segment) when timed. A timed graph segment is queued behind a short hold of the
        stream (kvq_probe_hold), so that its start event is taken when the GPU reaches
        the segment, not when the host begins to submit it: the events then bracket the
        GPU's execution of the steps without the graph launch's submission latency."""
        torch = self.torch
        total = 0.0
        for n in self._segments(n_steps):
            if graph:
                g = self._graph(n)
            if self.reset:
                self.reset()
            torch.cuda.synchronize()
            if timed and graph:
                import decode_attention_block_amd as kvq
                kvq.kvq_probe_hold(HOLD_US)
            if timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            if graph:
                g.replay()
            else:
                for j in range(n):
                    self.queue(j)
            if timed:
                e1.record()
            torch.cuda.synchronize()
            if timed:
                total += e0.elapsed_time(e1)
        return total

    def sample(self, n):
        """Per-step GPU times (ms) of the first n steps of a segment: HIP event pairs
        around each step, all queued behind about 4 ms of device copies."""
        torch = self.torch
        n = min(n, self.seg_cap)
        if self.reset:
            self.reset()
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(32):
            b.copy_(a)
        pairs = []
        for j in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            self.queue(j)
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        del a, b
        return [e0.elapsed_time(e1) for e0, e1 in pairs]


# ---- the oracle beside the GPU --------------------------------------------------------
def _repeat(fn, budget_s, min_reps=1):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if reps >= min_reps and el >= budget_s:
            return el / reps, reps


def oracle_legs(w, k_s, v_s, q_s, length, budget_s, label, new_kv=None):
    """The CPU oracle on a sample of the workload: k_s, v_s float16 [1][>=length][Hs][D]
    (one sequence, Hs heads of the same inputs the GPU quantized) and q_s
    [1][Hs * group][D]. Times, on one host thread and with the heads split over all host
    threads: the prefill quantization of the sample (oracle.quantize_cache over `length`
    tokens) and one decode step: with new_kv = (k, v) [1][Hs][D], oracle.append of that
    token then oracle.attention over length + 1 tokens, as the GPU's decode step does;
    without, oracle.attention over `length` tokens (workloads whose step is attention
    only), once per query head of a group."""
    import oracle
    Hs, D, G = k_s.shape[2], w.head_dim, w.group
    if new_kv is not None:
        hk = np.concatenate([k_s[:, :length], new_kv[0][:, None]], axis=1)
        hv = np.concatenate([v_s[:, :length], new_kv[1][:, None]], axis=1)
        n_attn = length + 1
    else:
        hk, hv, n_attn = k_s[:, :length], v_s[:, :length], length
    mb = (length + 1 + 63) // 64
    l0, l1 = np.array([length], np.int32), np.array([n_attn], np.int32)
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    qg = [np.ascontiguousarray(q_s.reshape(1, Hs, G, D)[:, :, g]) for g in range(G)]

    def quant(h0, h1):
        return oracle.quantize_cache(w.scheme, hk[:, :, h0:h1], hv[:, :, h0:h1], l0, mb)

    def step_fn(h0, h1):
        c = quant(h0, h1)
        qs = [np.ascontiguousarray(q[:, h0:h1]) for q in qg]

        def step():
            if new_kv is not None:
                oracle.append(c, hk[:, :, h0:h1], hv[:, :, h0:h1], l1)
            for q in qs:
                oracle.attention(c, q, l1, sm)
        return step

    q_bytes = prefill_bytes(w, [length], heads=Hs)
    s_bytes = attention_bytes(w, [n_attn], heads=Hs)
    if new_kv is not None:
        s_bytes += append_bytes(w, seqs=1, heads=Hs)
    cores = max(1, min(len(os.sched_getaffinity(0)), Hs))
    parts = [(Hs * i // cores, Hs * (i + 1) // cores) for i in range(cores)]
    res = {"sample": f"{label}: sequence 0, heads 0..{Hs - 1} of the workload's inputs, "
                     f"context {length}" + (" + 1 appended token" if new_kv is not None
                                             else ""),
           "step": ("oracle.append + oracle.attention" if new_kv is not None else
                    "oracle.attention" + (f" x {G} (query heads per cached head)"
                                          if G > 1 else "")),
           "host_threads_available": len(os.sched_getaffinity(0))}
    t, n = _repeat(lambda: quant(0, Hs), budget_s * 0.25)
    res["prefill_quantize_1core"] = {"ms": t * 1e3, "gbs": q_bytes / t / 1e9, "reps": n,
                                     "cores": 1}
    step1 = step_fn(0, Hs)
    t, n = _repeat(step1, budget_s * 0.35)
    res["decode_step_1core"] = {"ms": t * 1e3, "gbs": s_bytes / t / 1e9, "reps": n, "cores": 1,
                                "tokens_per_s": 1.0 / t}
    with ThreadPoolExecutor(cores) as ex:
        t, n = _repeat(lambda: list(ex.map(lambda p: quant(*p), parts)), budget_s * 0.15)
        res["prefill_quantize_all_cores"] = {"ms": t * 1e3, "gbs": q_bytes / t / 1e9,
                                             "reps": n, "cores": cores}
        steps = list(ex.map(lambda p: step_fn(*p), parts))
        t, n = _repeat(lambda: list(ex.map(lambda s: s(), steps)), budget_s * 0.25)
        res["decode_step_all_cores"] = {"ms": t * 1e3, "gbs": s_bytes / t / 1e9, "reps": n,
                                        "cores": cores, "tokens_per_s": 1.0 / t}
    return res


def ratios(gpu_step_gbs, gpu_prefill_gbs, legs):
    if not legs:
        return None
    return {"decode_step_gpu_over_1core": gpu_step_gbs / legs["decode_step_1core"]["gbs"],
            "decode_step_gpu_over_all_cores": gpu_step_gbs / legs["decode_step_all_cores"]["gbs"],
            "prefill_gpu_over_1core": (gpu_prefill_gbs / legs["prefill_quantize_1core"]["gbs"]
                                       if gpu_prefill_gbs else None),
            "prefill_gpu_over_all_cores": (gpu_prefill_gbs /
                                           legs["prefill_quantize_all_cores"]["gbs"]
                                           if gpu_prefill_gbs else None)}


def host_sample(t, heads):
    """Sequence 0, the first `heads` heads of a [B][S][H][D] fp16 tensor (torch or
    numpy), on the host."""
    x = t[0:1, :, :heads]
    if hasattr(x, "cpu"):
        x = x.contiguous().cpu().numpy()
    return np.ascontiguousarray(x)


def sample_heads(w):
    """Heads of sequence 0 the oracle leg takes: all of them, except at 32K context
    (a quarter, so that one single-threaded prefill quantization stays near 2 s)."""
    return max(1, min(w.heads, w.heads * 8192 // max(w.context, 1)))


# ---- workloads ------------------------------------------------------------------------
def prefill_inputs(torch, w, layer, n, device_inputs):
    wl = wl_mod()
    if device_inputs:
        return (wl.prefill_batch_device(w, layer, 0, n_tokens=n),
                wl.prefill_batch_device(w, layer, 1, n_tokens=n))
    return (torch.from_numpy(wl.prefill_batch(w, layer, 0, n_tokens=n)).cuda(),
            torch.from_numpy(wl.prefill_batch(w, layer, 1, n_tokens=n)).cuda())


def quantized_copies(kvq, torch, w, k, v, lens, max_blocks, n_copies, paged=False):
    """n_copies caches holding the quantized prefill k, v (device tensors); returns them
    and the prefill kernel times (ms). paged: each copy is a paged cache whose block table
    scatters the blocks over its pool in a seeded random order."""
    n = int(np.max(lens))
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
    return caches, ms


def prefill_loop(kvq, torch, w, steps, warmup):
    """Only the prefill quantization of --workload (kv_quantize_blocks of its whole
    context into one cache), warmup + steps times, for rocprofv3; HIP events around the
    timed calls."""
    wl = wl_mod()
    lens = wl.lengths(w)
    n = int(lens.max())
    k, v = prefill_inputs(torch, w, 0, n, w.decode_steps > 0 or w.layers > 1)
    c = kvq.KVCache(w.scheme, w.batch, w.heads, w.head_dim, w.max_blocks)
    c.seq_lens.copy_(torch.from_numpy(np.asarray(lens, np.int32)))
    for _ in range(warmup):
        kvq.kv_quantize_blocks(c, k, v, n)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        kvq.kv_quantize_blocks(c, k, v, n)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": w.name, "call": "kv_quantize_blocks (whole prefill)",
            "kernel": f"quantize_blocks_kernel<{w.scheme}, {w.head_dim}>", "steps": steps,
            "warmup": warmup, "ms_per_call": ms,
            "gbs": prefill_bytes(w, lens) / (ms / 1e3) / 1e9,
            "bytes_per_call": prefill_bytes(w, lens)}


def kernel_name(w, fused, paged=False):
    """The timed kernel as rocprofv3 lists it (template arguments: head_dim, whether the
    workgroup also appends the row's token, whether the cache is paged)."""
    f, p = ("true" if fused else "false"), ("true" if paged else "false")
    if w.scheme == 0:
        return f"attn_split_int4_kernel<{w.head_dim}, {f}, {p}>"
    return f"attn_split_kernel<{w.scheme}, {w.head_dim}, {f}, {p}>"


def timing_fields(stepper, steps, warmup, eager, launches_per_step, step_bytes_fn,
                  per_launch_bytes, warmup_ms=0.0):
    """Warm-up, the timed steps (graph replays, or eager), the eager comparison and the
    per-step percentiles; step_bytes_fn(total steps) = algorithmic bytes of the timed
    steps. The timed steps follow the warm-up directly (their graphs are captured before
    it, so no capture leaves the GPU idle between them); the comparison rounds come after
    them, and their graph figure is reported as the later rounds' rate. With warmup_ms,
    the warm-up goes on (in runs of `steps` steps) until that much wall time has passed."""
    if not eager:
        stepper.prepare(warmup, steps)
    stepper.run(warmup, timed=False, graph=not eager)
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < warmup_ms:
        stepper.run(steps, timed=False, graph=not eager)
        warmup += steps
    wall0 = time.perf_counter()
    total_ms = stepper.run(steps, timed=True, graph=not eager)
    wall_s = time.perf_counter() - wall0
    # graph replay against eager calls of the same steps, in alternating rounds (the
    # first pass after a pause runs slower while the GPU ramps up, so neither may always
    # go first); medians of the rounds
    g_ms, e_ms = [], []
    for _ in range(COMPARE_ROUNDS):
        e_ms.append(stepper.run(steps, timed=True, graph=False))
        g_ms.append(stepper.run(steps, timed=True, graph=True))
    eager_ms = float(np.median(e_ms))
    samples = stepper.sample(SAMPLED_STEPS)
    bytes_ = step_bytes_fn(steps)
    launch_us = total_ms / (steps * launches_per_step) * 1e3
    return {
        "steps": steps, "warmup": warmup,
        "timing": ("eager calls, HIP events around each segment" if eager else
                   "HIP graph replay of each segment's steps, HIP events around each segment "
                   f"(queued behind a {HOLD_US} us hold of the stream)"),
        "ms_per_step": total_ms / steps,
        "gbs": bytes_ / (total_ms / 1e3) / 1e9,
        "eager_ms_per_step": eager_ms / steps,
        "eager_gbs": bytes_ / (eager_ms / 1e3) / 1e9,
        "graph_vs_eager": {"graph_ms_per_step": float(np.median(g_ms)) / steps,
                           "eager_ms_per_step": eager_ms / steps,
                           "rounds": COMPARE_ROUNDS,
                           "note": "alternating rounds after the timed steps, medians"},
        "later_ms_per_step": float(np.median(g_ms)) / steps,
        "later_gbs": bytes_ / (float(np.median(g_ms)) / 1e3) / 1e9,
        "step_us": {k: v * 1e3 for k, v in pct(samples).items()},
        "step_us_sampling": (f"HIP event pairs around each of {len(samples)} steps queued "
                             "behind device copies (includes the events' own time)"),
        "kernel_avg_us": launch_us,
        "kernel_gbs": per_launch_bytes / (launch_us / 1e6) / 1e9,
        "kernel_bytes_per_launch": float(per_launch_bytes),
        "host_wall_s": wall_s,
    }


def run_append_attention(kvq, torch, w, steps, warmup, bps, device_inputs, separate=False,
                         paged=False, eager=False, with_cpu=False, cpu_budget=4.0,
                         warmup_ms=0.0):
    """Single-layer fixed-length workloads; step = decode_step_qkv (or, with separate,
    kv_append + decode_attn_qkv). The 32K workload's segments are its 64-step decode
    loop on one cache; the 8K workloads rotate over cache copies, each gaining one
    token per use; the tiny workload runs on one cache (it is far smaller than the
    caches, and its line is the call latency)."""
    wl = wl_mod()
    B, H, D = w.batch, w.heads, w.head_dim
    per_cache = 2 * B * H * w.context * code_bytes_per_token(w)
    tiny = per_cache < (1 << 20)
    if w.decode_steps:
        copies, growth = 1, w.decode_steps
    elif tiny:
        copies, growth = 1, min(steps, 64)
    else:
        copies = max(1, math.ceil(CACHE_BYTES_TARGET / per_cache))
        growth = math.ceil(steps / copies)
    seg_cap = copies * growth                # steps before lengths must be reset
    max_blocks = (w.context + growth + 63) // 64
    t_setup = time.perf_counter()
    lens0 = wl.lengths(w)
    k, v = prefill_inputs(torch, w, 0, w.context, device_inputs)
    caches, prefill_ms = quantized_copies(kvq, torch, w, k, v, lens0, max_blocks, copies, paged)
    Hs = sample_heads(w)
    ks = host_sample(k, Hs) if with_cpu else None
    vs = host_sample(v, Hs) if with_cpu else None
    del k, v
    torch.cuda.empty_cache()
    kn = np.stack([wl.appended_kv(w, 0, s, 0, growth) for s in range(B)], axis=1)
    vn = np.stack([wl.appended_kv(w, 0, s, 1, growth) for s in range(B)], axis=1)
    k_new = torch.from_numpy(kn).cuda()          # [growth][B][H][D]
    v_new = torch.from_numpy(vn).cuda()
    q_host = [wl.query(w, 0, s) for s in range(seg_cap)]
    queries = torch.from_numpy(np.stack(q_host)).cuda()
    ws = torch.zeros(max(kvq.decode_attn_workspace_bytes(caches[0], L, bps)
                         for L in range(w.context, w.context + growth + 1)),
                     dtype=torch.uint8, device="cuda")          # counters start at zero
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    bps_eff, n_split = kvq.decode_attn_plan(caches[0], w.context + growth, bps)
    one_launch = not separate and kvq.decode_step_launches(caches[0], w.context + growth,
                                                           bps) == 1

    def queue(j):
        """Step j of a segment: copy j % copies gains its (j // copies)-th token."""
        c = caches[j % copies]
        used = j // copies
        L = w.context + used + 1
        if separate:
            kvq.kv_append(c, k_new[used], v_new[used], L)
            kvq.decode_attn_qkv(c, queries[j], sm, out, ws, L, bps)
        else:
            kvq.decode_step_qkv(c, k_new[used], v_new[used], queries[j], sm, out, ws, L, bps)

    def reset():
        for c in caches:
            c.seq_lens.fill_(w.context)

    def step_bytes(n):
        tot = 0
        for j in range(n):
            L = w.context + (j % seg_cap) // copies + 1
            tot += attention_bytes(w, [L] * B) + append_bytes(w)
        return tot

    stepper = Stepper(torch, queue, seg_cap, reset)
    launches = 1 if one_launch else 2
    per_launch = step_bytes(steps) / steps
    res = timing_fields(stepper, steps, warmup, eager, launches, step_bytes,
                        per_launch if one_launch else 0.0, warmup_ms)
    res.update({
        "workload": w.name,
        "step": ("kv_append + decode_attn_qkv" if separate else
                 "decode_step_qkv (%s)" % ("append and attention in one launch" if one_launch
                                           else "append, then attention")),
        "kernel": kernel_name(w, fused=one_launch, paged=paged),
        "layout": "paged (block table over a shuffled page pool)" if paged else "dense",
        "tokens_per_s": B * steps / (res["ms_per_step"] * steps / 1e3),
        "context": [w.context + 1, w.context + growth],
        "cache_copies_rotated": copies, "blocks_per_split": bps_eff, "splits_per_row": n_split,
        "prefill_quantize_ms": float(np.median(prefill_ms)),
        "prefill_quantize_gbs": prefill_bytes(w, lens0) / (float(np.median(prefill_ms)) / 1e3)
        / 1e9,
        "setup_s": setup_s,
    })
    if not one_launch:
        res.pop("kernel_gbs")
        res.pop("kernel_bytes_per_launch")
        res["kernel_avg_us"] = None
    res["kernel_frac"] = res.get("kernel_gbs", 0.0) / HBM_PEAK_GBS
    if tiny:
        # the call latency a host sees: one eager decode_step_qkv, then a synchronize
        lat = []
        reset()
        torch.cuda.synchronize()
        for j in range(min(seg_cap, 64)):
            t0 = time.perf_counter()
            queue(j)
            torch.cuda.synchronize()
            lat.append((time.perf_counter() - t0) * 1e6)
        res["host_call_latency_us"] = pct(lat)
    if with_cpu:
        kn_s = np.ascontiguousarray(kn[0, 0:1, :Hs])
        vn_s = np.ascontiguousarray(vn[0, 0:1, :Hs])
        qs = np.ascontiguousarray(q_host[0][0:1, :Hs * w.group])
        res["oracle"] = oracle_legs(w, ks, vs, qs, int(lens0[0]), cpu_budget, w.name,
                                    new_kv=(kn_s, vn_s))
        res["gpu_over_oracle"] = ratios(res["gbs"], res["prefill_quantize_gbs"], res["oracle"])
    return res


def run_gqa(kvq, torch, w, steps, warmup, bps, paged=False, eager=False, with_cpu=False,
            cpu_budget=4.0, warmup_ms=0.0):
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
    k, v = prefill_inputs(torch, w, 0, L, False)
    caches, prefill_ms = quantized_copies(kvq, torch, w, k, v, lens, w.max_blocks, copies, paged)
    Hs = sample_heads(w)
    ks = host_sample(k, Hs) if with_cpu else None
    vs = host_sample(v, Hs) if with_cpu else None
    del k, v
    q_host = wl.query(w, 0)
    q = torch.from_numpy(q_host).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(kvq.decode_attn_gqa_workspace_bytes(caches[0], G, L, bps), 16),
                     dtype=torch.uint8, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    per_launch = attention_bytes(w, lens)

    def queue(j):
        kvq.decode_attn_gqa(caches[j % copies], q, G, sm, out, ws, L, bps)

    stepper = Stepper(torch, queue, max(steps, warmup, SAMPLED_STEPS))
    res = timing_fields(stepper, steps, warmup, eager, 1, lambda n: n * per_launch, per_launch,
                        warmup_ms)
    bps_eff, n_split = kvq.decode_attn_gqa_plan(caches[0], G, L, bps)
    res.update({
        "workload": w.name,
        "step": f"decode_attn_gqa ({G} query heads per cached head)",
        "kernel": (f"attn_split_int4_gqa_kernel<{D}, {G}, {'true' if paged else 'false'}>"
                   if w.scheme == 0 else
                   f"attn_split_gqa8_kernel<{w.scheme}, {D}, {G}, {'true' if paged else 'false'}>"),
        "layout": "paged (block table over a shuffled page pool)" if paged else "dense",
        "tokens_per_s": B * steps / (res["ms_per_step"] * steps / 1e3),
        "context": [L, L], "cache_copies_rotated": copies,
        "blocks_per_split": bps_eff, "splits_per_row": n_split,
        "prefill_quantize_ms": float(np.median(prefill_ms)),
        "prefill_quantize_gbs": prefill_bytes(w, lens) / (float(np.median(prefill_ms)) / 1e3)
        / 1e9,
        "setup_s": setup_s,
    })
    res["kernel_frac"] = res["kernel_gbs"] / HBM_PEAK_GBS
    if with_cpu:
        res["oracle"] = oracle_legs(w, ks, vs, np.ascontiguousarray(q_host[0:1, :Hs * G]), L,
                                    cpu_budget, w.name)
        # the step is attention alone on both sides
        res["gpu_over_oracle"] = ratios(res["gbs"], res["prefill_quantize_gbs"], res["oracle"])
    return res


def run_layers(kvq, torch, w, steps, warmup, bps, eager=False, with_cpu=False, cpu_budget=4.0,
               warmup_ms=0.0):
    """The 32-layer ragged workload: one step is decode_attn_qkv over every layer's
    cache, each layer with its own K, V and query (no append in this workload)."""
    wl = wl_mod()
    B, H, D = w.batch, w.heads, w.head_dim
    lens = wl.lengths(w)
    L = int(lens.max())
    t_setup = time.perf_counter()
    caches, prefill_ms, queries = [], [], []
    ks = vs = None
    Hs = sample_heads(w)
    for layer in range(w.layers):
        k, v = prefill_inputs(torch, w, layer, L, True)
        c, ms = quantized_copies(kvq, torch, w, k, v, lens, w.max_blocks, 1)
        if with_cpu and layer == 0:
            ks, vs = host_sample(k, Hs), host_sample(v, Hs)
        del k, v
        caches += c
        prefill_ms += ms
        queries.append(torch.from_numpy(wl.query(w, layer)).cuda())
    torch.cuda.empty_cache()
    ws = torch.zeros(max(kvq.decode_attn_workspace_bytes(caches[0], L, bps), 16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    sm = wl.softmax_scale(w)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    per_launch = attention_bytes(w, lens)

    def queue(j):
        for layer in range(w.layers):
            kvq.decode_attn_qkv(caches[layer], queries[layer], sm, out, ws, L, bps)

    stepper = Stepper(torch, queue, max(steps, warmup, SAMPLED_STEPS))
    res = timing_fields(stepper, steps, warmup, eager, w.layers,
                        lambda n: n * w.layers * per_launch, per_launch, warmup_ms)
    bps_eff, n_split = kvq.decode_attn_plan(caches[0], L, bps)
    res.update({
        "workload": w.name,
        "step": f"decode_attn_qkv over {w.layers} layers",
        "kernel": kernel_name(w, fused=False),
        "tokens_per_s": B * steps / (res["ms_per_step"] * steps / 1e3),
        "context": [int(lens.min()), L], "mean_context": float(lens.mean()),
        "blocks_per_split": bps_eff, "splits_per_row": n_split,
        "plan": ("automatic (each row's split chosen on the device from the lengths)"
                 if bps == 0 else f"{bps} blocks per split (caller's choice)"),
        "prefill_quantize_ms_per_layer": float(np.median(prefill_ms)),
        "prefill_quantize_gbs": prefill_bytes(w, lens) / (float(np.median(prefill_ms)) / 1e3)
        / 1e9,
        "setup_s": setup_s,
    })
    res["kernel_frac"] = res["kernel_gbs"] / HBM_PEAK_GBS
    if with_cpu:
        res["oracle"] = oracle_legs(w, ks, vs, np.ascontiguousarray(wl.query(w, 0)[0:1, :Hs]),
                                    int(lens[0]), cpu_budget, w.name + " layer 0")
        res["gpu_over_oracle"] = ratios(res["gbs"], res["prefill_quantize_gbs"], res["oracle"])
    return res


def measure(kvq, torch, w, steps, warmup, bps, separate=False, paged=False, eager=False,
            with_cpu=False, cpu_budget=4.0, warmup_ms=0.0):
    big = w.decode_steps > 0 or w.layers > 1
    if w.layers > 1:
        res = run_layers(kvq, torch, w, steps, warmup, bps, eager, with_cpu, cpu_budget,
                         warmup_ms)
    elif w.group > 1:
        res = run_gqa(kvq, torch, w, steps, warmup, bps, paged, eager, with_cpu, cpu_budget,
                      warmup_ms)
    else:
        res = run_append_attention(kvq, torch, w, steps, warmup, bps, big, separate, paged,
                                   eager, with_cpu, cpu_budget, warmup_ms)
    res["inputs"] = ("K/V drawn on the device (torch generator, same distributions)"
                     if big else "K/V from the seeded host recipe")
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
    if args.prefill_loop:
        print(json.dumps(prefill_loop(kvq, torch, w, args.steps, args.warmup)), flush=True)
        return
    with_cpu = not (args.no_cpu or args.profile_loop)
    print(f"[bench] {w.name}: {args.steps} steps after {args.warmup} warm-up",
          file=sys.stderr, flush=True)
    res = measure(kvq, torch, w, args.steps, args.warmup, args.blocks_per_split,
                  separate=args.separate, paged=args.paged, eager=args.eager,
                  with_cpu=with_cpu, cpu_budget=args.cpu_seconds)
    if args.profile_loop:
        print(json.dumps(res), flush=True)
        return
    print("[bench] stream-read ceiling", file=sys.stderr, flush=True)
    ceiling = read_ceiling(kvq, torch)
    with_same_size_ceiling(kvq, torch, res)

    B, H, D = w.batch, w.heads, w.head_dim
    fused = ", true," in res["kernel"]
    achieved = res.get("kernel_gbs")
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
        "dtype": DTYPES[w.scheme],
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
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS if achieved else None,
                     "traffic": measured_traffic() if w.name == HEADLINE and fused else None,
                     "avg_kernel_us": res["kernel_avg_us"],
                     "timing": res["timing"] + " / launches",
                     "algorithmic_bytes_per_launch": res.get("kernel_bytes_per_launch"),
                     "frac_of_read_ceiling": achieved / ceiling["gbs"] if achieved else None,
                     "frac_of_same_size_read_ceiling":
                         res.get("kernel_frac_of_same_size_read_ceiling")},
        "read_ceiling": ceiling,
        "read_ceiling_same_size": res.get("read_ceiling_same_size"),
        "step_us": res["step_us"],
        "step_us_sampling": res["step_us_sampling"],
        "eager": {"ms_per_step": res["eager_ms_per_step"], "gbs": res["eager_gbs"],
                  "note": "the same steps queued one by one from the host"},
        "graph_vs_eager": res["graph_vs_eager"],
        "later_rounds": {"ms_per_step": res["later_ms_per_step"], "gbs": res["later_gbs"],
                         "pct_of_hbm_peak": 100.0 * res["later_gbs"] / HBM_PEAK_GBS,
                         "note": ("the same steps replayed in the comparison rounds right "
                                  "after the timed ones (median): the timed steps come first "
                                  "after setup and the warm-up, in the GPU's first "
                                  "milliseconds of continuous work; these rounds fall in the "
                                  "next few, where it runs slower, before it settles (the "
                                  "steady rate is the one bench.py --profile-loop times after "
                                  "300 warm-up steps)")},
        "prefill_quantize": {"ms": res.get("prefill_quantize_ms"),
                             "gbs": res.get("prefill_quantize_gbs")},
        "host_wall_s": res["host_wall_s"],
        "setup_s": res["setup_s"],
    }
    if with_cpu and "oracle" in res:
        legs = res["oracle"]
        one, allc = legs["decode_step_1core"], legs["decode_step_all_cores"]
        result["cpu_baseline"] = {
            "value": one["gbs"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": legs["sample"] + f"; one decode step (oracle.append + oracle.attention) "
                      f"repeated {one['reps']} times on one host thread, "
                      f"{one['ms'] * one['reps'] / 1e3:.1f} s",
            "tokens_per_s": one["tokens_per_s"]}
        result["cpu_baseline_all_cores"] = {
            "value": allc["gbs"], "unit": "GB/s", "cores": allc["cores"], "kind": "oracle",
            "sample": legs["sample"] + f"; heads split over {allc['cores']} host threads",
            "tokens_per_s": allc["tokens_per_s"]}
        result["oracle"] = legs
        result["gpu_over_oracle"] = res["gpu_over_oracle"]
    if not args.headline_only:
        others = []
        for name in OTHERS:
            if name == w.name:
                continue
            ow = wl.BY_NAME[name]
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            if ow.decode_steps:
                st, warm = 64 * 3, 64
            elif ow.layers > 1:
                st, warm = max(5, min(args.steps, 20)), max(2, min(args.warmup, 10))
            else:
                st, warm = args.steps, args.warmup
            r = measure(kvq, torch, ow, st, warm, args.blocks_per_split,
                        separate=args.separate, eager=args.eager, with_cpu=with_cpu,
                        cpu_budget=4.0, warmup_ms=WARMUP_MS_OTHERS)
            others.append(with_same_size_ceiling(kvq, torch, r))
            torch.cuda.empty_cache()
        if not args.paged and w.layers == 1 and w.group == 1:
            print(f"[bench] {w.name} paged", file=sys.stderr, flush=True)
            r = measure(kvq, torch, w, args.steps, args.warmup, args.blocks_per_split,
                        separate=args.separate, paged=True, eager=args.eager,
                        warmup_ms=WARMUP_MS_OTHERS)
            others.append(with_same_size_ceiling(kvq, torch, r))
            torch.cuda.empty_cache()
        result["workloads"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
