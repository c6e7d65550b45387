"""Shared test helpers: run the HIP path and the oracle on the same seeded inputs."""
import sys

import numpy as np

import oracle

ATTN_TOL = 2e-3  # max over rows of ||o_gpu - o_ref||_inf / ||o_ref||_inf


def say(*args):
    """Names the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *args, file=sys.stderr, flush=True)


def torch_mod():
    import torch
    return torch


def to_gpu(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_quantize(scheme, k, v, lens, max_blocks, max_len=None, with_tail=True):
    """Quantizes host fp16 [B][S][H][D] k, v on the GPU; returns the KVCache."""
    import decode_attention_block_amd as kvq
    torch = torch_mod()
    B, S, H, D = k.shape
    c = kvq.KVCache(scheme, B, H, D, max_blocks, with_tail=with_tail)
    c.seq_lens.copy_(torch.from_numpy(np.asarray(lens, np.int32)))
    kt, vt = to_gpu(k), to_gpu(v)
    kvq.kv_quantize_blocks(c, kt, vt, int(np.max(lens)) if max_len is None else max_len)
    torch.cuda.synchronize()
    return c


def assert_cache_equal(gpu, ref, lens, rows=None):
    """Bitwise equality of codes, scales and zero points over every quantized block of
    the listed (b, h) rows (all rows by default)."""
    B, H = ref["B"], ref["H"]
    rows = [(b, h) for b in range(B) for h in range(H)] if rows is None else rows
    for b, h in rows:
        nb = (int(lens[b]) + 63) // 64
        for key in ("k_codes", "v_codes"):
            g, r = gpu[key][b, h, :nb], ref[key][b, h, :nb]
            if not np.array_equal(g, r):
                bad = np.argwhere(g != r)[:5]
                raise AssertionError(f"{key} row ({b},{h}) differs at {bad.tolist()}")
        for key in ("k_scale", "v_scale") + (("k_zero", "v_zero") if ref["scheme"] else ()):
            g = gpu[key][b, h, :nb].view(np.uint32)
            r = ref[key][b, h, :nb].view(np.uint32)
            if not np.array_equal(g, r):
                bad = np.argwhere(g != r)[:5]
                raise AssertionError(f"{key} row ({b},{h}) differs at {bad.tolist()}")


# The outputs are fp16: below 2^-14 its values are spaced 2^-24 apart, so an exact result
# there is delivered with an absolute error of up to 2^-25 whatever the arithmetic (a row
# whose values are all that small cannot meet a relative bound). Differences are counted
# beyond that floor; above 2^-14 fp16 rounds to within 2^-11 relative, well inside the
# tolerance.
FP16_HALF_SUBNORMAL_STEP = 2.0 ** -25


def attn_errors(o_gpu, o_ref, rows=None):
    """(max over rows of the normwise relative error, max elementwise error relative to
    max(|ref|, 1e-3 * ||ref_row||_inf)), differences counted beyond fp16's absolute
    resolution near zero (FP16_HALF_SUBNORMAL_STEP)."""
    g = np.asarray(o_gpu, np.float64)
    r = np.asarray(o_ref, np.float64)
    B, H, D = r.shape
    rows = [(b, h) for b in range(B) for h in range(H)] if rows is None else rows
    norm_err, elem_err = 0.0, 0.0
    for b, h in rows:
        ref = r[b, h]
        scale = np.abs(ref).max()
        if scale == 0:
            assert np.abs(g[b, h]).max() == 0, (b, h)
            continue
        diff = np.maximum(np.abs(g[b, h] - ref) - FP16_HALF_SUBNORMAL_STEP, 0.0)
        norm_err = max(norm_err, diff.max() / scale)
        elem_err = max(elem_err, (diff / np.maximum(np.abs(ref), 1e-3 * scale)).max())
    return norm_err, elem_err


def gpu_attention(cache, q, sm_scale, max_len, blocks_per_split=0):
    import decode_attention_block_amd as kvq
    torch = torch_mod()
    B, H, D = q.shape
    qt = to_gpu(q)
    out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    ws = kvq.make_workspace(cache, max_len, blocks_per_split)
    kvq.decode_attn_qkv(cache, qt, sm_scale, out, ws, max_len, blocks_per_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_cache(scheme, k, v, lens, max_blocks):
    return oracle.quantize_cache(scheme, k, v, np.asarray(lens, np.int32), max_blocks)
