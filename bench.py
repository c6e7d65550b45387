#!/usr/bin/env python3
"""Decode-step benchmark of the block-quantized KV cache on one MI355X.

One step = one decode step of the whole hot path on the 8K int4 workload (batch 8,
32 heads, head_dim 128, context 8192 per sequence, 4-bit block codes, 64-token blocks):
kv_append quantizes one new token per sequence into its row's tail block (one kernel),
then decode_attn_qkv attends one fp16 query per (sequence, head) over the whole
compressed cache (one kernel: split-K over the context, the last workgroup of each row
merges its splits).

Inputs are synthetic and seeded (decode_attention_block_amd.workloads), already
resident in HBM when timing starts. Steps rotate over enough copies of the cache
(>= 1 GiB in all) that the 256 MB Infinity Cache cannot hold them, so every step
reads its cache from HBM. Each copy gains one token per use, so the context grows
from 8192 by at most ceil((warmup + steps) / copies) tokens; bytes are counted from
the actual lengths.

Prints one JSON line (see the keys below). --profile-loop runs only the timed loop
(for rocprofv3), --copy-probe times a plain device copy of known size (the
calibration kernel for the FETCH_SIZE / WRITE_SIZE counters).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_split_int4_b8h32d128_ctx8k_traffic.json")
CACHE_BYTES_TARGET = 1 << 30   # total bytes of rotated cache copies
HEADLINE = "llama7b_b8_h32_d128_ctx8k_int4"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--blocks-per-split", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate host time spent timing the oracle")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--profile-loop", action="store_true",
                   help="only the timed loop (for rocprofv3); no oracle, no copy probe")
    p.add_argument("--copy-probe", action="store_true",
                   help="only a 1 GiB device-to-device copy (counter calibration)")
    return p.parse_args()


def code_bytes_per_token(w):
    return w.head_dim // 2 if w.scheme == 0 else w.head_dim


def attention_bytes(w, lens):
    """Algorithmic bytes of one decode_attn_qkv call: K and V codes of the valid
    tokens, their block scales (and zero points for uint8), q and out."""
    per_block_scalars = 2 * (2 if w.scheme == 1 else 1) * 4
    total = 0
    for n in lens:
        nb = (int(n) + 63) // 64
        total += w.heads * (2 * int(n) * code_bytes_per_token(w) + nb * per_block_scalars)
    total += 2 * w.batch * w.heads * w.head_dim * 2  # q in, out
    return total


def append_bytes(w):
    """Algorithmic bytes of one kv_append: the new K and V tokens in (fp16), their
    staged fp16 copy and their codes out."""
    rows = w.batch * w.heads
    return rows * 2 * (w.head_dim * 2 * 2 + code_bytes_per_token(w))


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (this path "
              f"shards by sequence or head with no communication; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_block_amd as kvq
    from decode_attention_block_amd import workloads as wl

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_probe:
        print(json.dumps(copy_probe()), flush=True)
        return

    w = wl.BY_NAME[args.workload]
    if w.ragged is not None or w.layers != 1:
        sys.exit("bench.py times single-layer, fixed-length workloads")
    B, H, D = w.batch, w.heads, w.head_dim
    per_cache = 2 * B * H * w.context * code_bytes_per_token(w)
    copies = max(1, math.ceil(CACHE_BYTES_TARGET / per_cache))
    total_steps = args.warmup + args.steps
    growth = math.ceil(total_steps / copies)
    max_blocks = (w.context + growth + 63) // 64

    # ---- untimed setup: inputs, prefill quantization into every copy ----------------
    t_setup = time.perf_counter()
    k = torch.from_numpy(wl.prefill_batch(w, 0, 0)).cuda()
    v = torch.from_numpy(wl.prefill_batch(w, 0, 1)).cuda()
    kn = np.stack([wl.appended_kv(w, 0, s, 0, growth) for s in range(B)], axis=1)
    vn = np.stack([wl.appended_kv(w, 0, s, 1, growth) for s in range(B)], axis=1)
    k_new = torch.from_numpy(kn).cuda()          # [growth][B][H][D]
    v_new = torch.from_numpy(vn).cuda()
    queries = torch.from_numpy(np.stack([wl.query(w, 0, s) for s in range(total_steps)])).cuda()
    caches = []
    prefill_ms = []
    for _ in range(copies):
        c = kvq.KVCache(w.scheme, B, H, D, max_blocks)
        c.seq_lens.fill_(w.context)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        kvq.kv_quantize_blocks(c, k, v, w.context)
        e1.record()
        torch.cuda.synchronize()
        prefill_ms.append(e0.elapsed_time(e1))
        caches.append(c)
    del k, v
    host_cache = caches[0].host_arrays() if not (args.no_cpu or args.profile_loop) else None
    max_len_all = w.context + growth
    ws_bytes = max(kvq.decode_attn_workspace_bytes(caches[0], L, args.blocks_per_split)
                   for L in range(w.context, max_len_all + 1))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")  # counters start at zero
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    sm = wl.softmax_scale(w)
    lens_host = [w.context] * copies
    uses = [0] * copies
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    ev_attn = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    step_bytes, step_attn_bytes = [], []

    def step(i, timed_index):
        ci = i % copies
        c = caches[ci]
        kvq.kv_append(c, k_new[uses[ci]], v_new[uses[ci]], lens_host[ci] + 1)
        uses[ci] += 1
        lens_host[ci] += 1
        L = lens_host[ci]
        if timed_index is not None:
            ev_attn[timed_index][0].record()
        kvq.decode_attn_qkv(c, queries[i], sm, out, ws, L, args.blocks_per_split)
        if timed_index is not None:
            ev_attn[timed_index][1].record()
            lens = [L] * B
            step_attn_bytes.append(attention_bytes(w, lens))
            step_bytes.append(attention_bytes(w, lens) + append_bytes(w))

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for j in range(args.steps):
        step(args.warmup + j, j)
    t1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    attn_ms = [a.elapsed_time(b) for a, b in ev_attn]
    avg_attn_ms = float(np.mean(attn_ms))

    ms_per_step = total_ms / args.steps
    value = sum(step_bytes) / (total_ms / 1e3) / 1e9
    achieved = float(np.mean(step_attn_bytes)) / (avg_attn_ms / 1e3) / 1e9
    bps, n_split = kvq.decode_attn_plan(caches[0], max_len_all, args.blocks_per_split)
    result = {
        "metric": "decode-attn effective HBM GB/s (% of peak) + tokens/s, int4 KV, B=8 ctx 8K",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) K/V with 0.1% x20 outliers, N(0,1) queries)",
        "pct_of_hbm_peak": 100.0 * value / HBM_PEAK_GBS,
        "tokens_per_s": B * args.steps / (total_ms / 1e3),
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": D,
                   "context": w.context, "context_growth_max": growth,
                   "kv_format": "int4 block-64 symmetric" if w.scheme == 0
                   else "uint8 block-64 asymmetric",
                   "step": "kv_append + decode_attn_qkv",
                   "cache_copies_rotated": copies, "blocks_per_split": bps,
                   "splits_per_row": n_split, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "attn_split_int4_kernel<128> (decode_attn_qkv)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if w.name == HEADLINE else None,
                     "avg_kernel_us": avg_attn_ms * 1e3,
                     "algorithmic_bytes_per_launch": float(np.mean(step_attn_bytes))},
        "prefill_quantize": {"ms": float(np.median(prefill_ms)),
                             "gbs": (2 * B * w.context * H * D * 2 + per_cache)
                             / (float(np.median(prefill_ms)) / 1e3) / 1e9},
        "host_wall_s": wall_s,
        "setup_s": setup_s,
    }
    if not (args.no_cpu or args.profile_loop):
        lens0 = np.full(B, w.context, np.int32)
        host_cache["B"] = B
        result["cpu_baseline"] = cpu_baseline(w, host_cache, wl.query(w, 0), lens0,
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
