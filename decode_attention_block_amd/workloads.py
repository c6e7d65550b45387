"""The synthetic decode workloads and their seeded input generators.

This module draws random numbers and nothing else: it holds no quantization or
attention arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any of the method.

Shapes follow the workloads on the pages: Llama-2-7B-shaped heads (32 heads of 128
channels, 32 layers) as in page "DeepSeek-R1推理延迟骤降41.8%？…" §2.1; batch 8 at
context 8192 as in page "第一章：DeepSeek R1推理模型性能跃迁全景概览" chapter 1's deployment
table; batch 16 at 32K context as in that page's §2.3 table. The grouped-query workload
(64 query heads over 8 cached heads) stands for decoding with shared cached heads
(page "DeepSeek R1性能优化有哪些技巧" §二: MLA decodes as multi-query attention).

Recipe (every draw from numpy PCG64 seeded by SeedSequence([SEED, workload index,
layer, stream id, sequence])):
  * normal_outliers: x ~ N(0, 1) drawn in binary32; a Binomial(n, 0.001) number of
    distinct positions, uniform over the n elements (drawn without replacement), is
    multiplied by 20 (so 0.1% of entries on average are outliers, each scaled once);
    then rounded to fp16 (nearest-even). Normals are drawn in binary32 rather than
    binary64: the fp16 values then go through two roundings instead of one, which moves
    a value to a neighbouring fp16 number only where the binary32 draw lands exactly on
    an fp16 rounding tie (about one draw in 2^13), and halves the host's drawing time.
  * normal(mu): x ~ N(mu, 1) in binary32, rounded to fp16.
  * student_t3_half: x = 0.5 * Z / sqrt(2G/3), Z ~ N(0,1), G ~ Gamma(1.5, 1)
    (2G ~ chi-square with 3 degrees of freedom), binary32, rounded to fp16.
  * the query is N(0, 1) for every workload, one token per sequence and head.
  * ragged lengths: integers uniform on [1024, 8192] inclusive, one per sequence,
    shared by all layers.
Streams: 0 = prefill K, 1 = prefill V, 2 = query, 3 = lengths, 4 = appended K,
5 = appended V.
"""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 20261202
BLOCK = 64
INT4_SYM = 0
UINT8_ASYM = 1
FP8_E4M3 = 2

STREAM_K, STREAM_V, STREAM_Q, STREAM_LENS, STREAM_K_APPEND, STREAM_V_APPEND = range(6)


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    heads: int
    head_dim: int
    context: int            # prefill length (upper bound for ragged lengths)
    scheme: int
    k_dist: str
    v_dist: str
    layers: int = 1
    decode_steps: int = 0   # tokens appended per sequence, one per decode step
    ragged: tuple = None    # (lo, hi) inclusive range of per-sequence lengths
    group: int = 1          # query heads per cached head (grouped-query attention)

    @property
    def max_len(self):
        return self.context + self.decode_steps

    @property
    def max_blocks(self):
        return (self.max_len + BLOCK - 1) // BLOCK


WORKLOADS = [
    Workload(0, "tiny_b1_h2_d64_ctx256_int4", 1, 2, 64, 256, INT4_SYM,
             "normal_outliers", "normal_outliers"),
    Workload(1, "llama7b_b8_h32_d128_ctx8k_int4", 8, 32, 128, 8192, INT4_SYM,
             "normal_outliers", "normal_outliers"),
    Workload(2, "llama7b_b8_h32_d128_ctx8k_uint8", 8, 32, 128, 8192, UINT8_ASYM,
             "normal0", "normal0.5"),
    Workload(3, "long_b16_h32_d128_ctx32k_append64_int4", 16, 32, 128, 32768, INT4_SYM,
             "normal_outliers", "normal_outliers", decode_steps=64),
    Workload(4, "llama7b_32layer_b8_h32_d128_ragged1k-8k_t3_int4", 8, 32, 128, 8192,
             INT4_SYM, "student_t3_half", "student_t3_half", layers=32,
             ragged=(1024, 8192)),
    # grouped-query decode: 64 query heads over 8 cached heads (a Llama-2-70B-shaped
    # layer), the cache of the 8K workloads' shape otherwise
    Workload(5, "llama70b_gqa8_b8_h8_d128_ctx8k_int4", 8, 8, 128, 8192, INT4_SYM,
             "normal_outliers", "normal_outliers", group=8),
    # the 8K shape with the FP8 E4M3 cache (page "DeepSeek R1性能优化有哪些技巧" §一)
    Workload(6, "llama7b_b8_h32_d128_ctx8k_fp8", 8, 32, 128, 8192, FP8_E4M3,
             "normal_outliers", "normal_outliers"),
    # grouped-query decode over the FP8 cache (the pages pair the FP8 KV cache with
    # shared-head decode: page "DeepSeek R1性能优化有哪些技巧" §一, §二)
    Workload(7, "llama70b_gqa8_b8_h8_d128_ctx8k_fp8", 8, 8, 128, 8192, FP8_E4M3,
             "normal_outliers", "normal_outliers", group=8),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def rng(workload, layer, stream, seq):
    ss = np.random.SeedSequence([SEED, workload.index, layer, stream, seq])
    return np.random.Generator(np.random.PCG64(ss))


def outlier_positions(g, n):
    """Binomial(n, 0.001) distinct positions in [0, n), uniform (drawn without
    replacement)."""
    k = int(g.binomial(n, 0.001)) if n else 0
    return g.choice(n, size=k, replace=False) if k else np.empty(0, np.int64)


def draw(g, dist, shape):
    """float16 samples of `dist` with the given shape from generator g."""
    n = int(np.prod(shape))
    if dist == "normal_outliers":
        x = g.standard_normal(n, dtype=np.float32)
        x[outlier_positions(g, n)] *= np.float32(20.0)
    elif dist.startswith("normal"):
        mu = np.float32(float(dist[len("normal"):] or 0.0))
        x = g.standard_normal(n, dtype=np.float32)
        if mu != 0:
            x += mu
    elif dist == "student_t3_half":
        z = g.standard_normal(n, dtype=np.float32)
        gam = g.standard_gamma(1.5, n, dtype=np.float32)
        x = np.float32(0.5) * z / np.sqrt(np.float32(2.0 / 3.0) * gam)
    else:
        raise ValueError(dist)
    return x.astype(np.float16).reshape(shape)


def prefill_kv(w, layer, seq, which, n_tokens=None):
    """float16 [n_tokens][H][D] prefill K (which=0) or V (which=1) of one sequence."""
    n = w.context if n_tokens is None else n_tokens
    dist = w.k_dist if which == 0 else w.v_dist
    stream = STREAM_K if which == 0 else STREAM_V
    return draw(rng(w, layer, stream, seq), dist, (n, w.heads, w.head_dim))


def appended_kv(w, layer, seq, which, n_steps=None):
    """float16 [n_steps][H][D]: the tokens appended one per decode step."""
    n = w.decode_steps if n_steps is None else n_steps
    dist = w.k_dist if which == 0 else w.v_dist
    stream = STREAM_K_APPEND if which == 0 else STREAM_V_APPEND
    return draw(rng(w, layer, stream, seq), dist, (n, w.heads, w.head_dim))


def query(w, layer, step=0):
    """float16 [B][H * group][D] query for one decode step of one layer."""
    g = rng(w, layer, STREAM_Q, step)
    return draw(g, "normal0", (w.batch, w.heads * w.group, w.head_dim))


def lengths(w):
    """int32 [B] context lengths (ragged workloads draw them; others use `context`)."""
    if w.ragged is None:
        return np.full(w.batch, w.context, dtype=np.int32)
    lo, hi = w.ragged
    g = rng(w, 0, STREAM_LENS, 0)
    return g.integers(lo, hi + 1, size=w.batch).astype(np.int32)


def prefill_batch(w, layer, which, n_tokens=None, seqs=None):
    """float16 [B][S][H][D] prefill tensor for all (or the listed) sequences. Each
    sequence has its own stream, so drawing them on parallel threads changes nothing."""
    seqs = list(range(w.batch) if seqs is None else seqs)
    n = w.context if n_tokens is None else n_tokens
    out = np.empty((len(seqs), n, w.heads, w.head_dim), np.float16)

    def fill(i):
        out[i] = prefill_kv(w, layer, seqs[i], which, n)

    workers = max(1, min(len(seqs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(len(seqs))))
    return out


def softmax_scale(w):
    """binary32 1/sqrt(head_dim), the query scaling the workloads use."""
    return float(np.float32(1.0) / np.sqrt(np.float32(w.head_dim)))


def device_seed(w, layer, stream, seq):
    """63-bit seed of the device-side generator for one (workload, layer, stream,
    sequence)."""
    ss = np.random.SeedSequence([SEED, w.index, layer, stream, seq, 1 << 20])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def prefill_batch_device(w, layer, which, n_tokens=None, device="cuda"):
    """float16 torch tensor [B][S][H][D] drawn on the device with torch's seeded
    generator, one stream per sequence: the same distributions as prefill_batch
    (outliers as an independent 0.1% mask; Student-t(3) as
    Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)), different random streams, so different values.
    Used where drawing on the host would take minutes (timing the 32K and 32-layer
    workloads); the parity tests use the host recipe."""
    import torch
    n = w.context if n_tokens is None else n_tokens
    shape = (n, w.heads, w.head_dim)
    dist = w.k_dist if which == 0 else w.v_dist
    stream = STREAM_K if which == 0 else STREAM_V
    out = torch.empty((w.batch,) + shape, dtype=torch.float16, device=device)
    g = torch.Generator(device=device)
    for b in range(w.batch):
        g.manual_seed(device_seed(w, layer, stream, b))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if dist == "normal_outliers":
            u = torch.rand(shape, generator=g, device=device)
            x.mul_(torch.where(u < 0.001, 20.0, 1.0))
        elif dist.startswith("normal"):
            mu = float(dist[len("normal"):] or 0.0)
            if mu:
                x += mu
        elif dist == "student_t3_half":
            chi2 = torch.zeros_like(x)
            for _ in range(3):
                z = torch.randn(shape, generator=g, device=device)
                chi2.addcmul_(z, z)
            x.mul_(0.5).div_(torch.sqrt(chi2 / 3.0))
        else:
            raise ValueError(dist)
        out[b] = x
    return out
