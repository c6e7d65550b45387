"""Seeded random shapes through the whole path, each case against the oracle: batch
sizes up to 80 (past the 64 sequences the automatic plan pairs), 1 to 40 heads, head_dim
64 or 128, lengths drawn over empty, one-token, block-edge and long rows, the automatic
split plan or a caller's, every cache format. Per case: prefill bit-exact, two appends
bit-exact, attention within 2e-3 of the oracle, split + combine bitwise the fused call,
the workspace's arrival counters back at zero."""
import numpy as np
import pytest

import oracle
from helpers import (ATTN_TOL, assert_cache_equal, attn_errors, gpu_quantize, oracle_cache,
                     say, to_gpu)

pytestmark = pytest.mark.gpu

SCHEMES = (oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3)


def _case(seed):
    rs = np.random.default_rng(1000 + seed)
    scheme = SCHEMES[seed % 3]
    D = (64, 128)[(seed // 3) % 2]
    B = int(rs.choice([1, 3, 8, 33, 64, 65, 80]))
    H = int(rs.choice([1, 2, 5, 8, 13, 40]))
    while B * H * D > 400000:  # keep the oracle's work to seconds
        H = max(1, H // 2)
    MB = int(rs.integers(2, 7))
    cap = MB * 64
    pool = [0, 1, 63, 64, 65, 127, 128, cap - 2]
    lens = np.where(rs.random(B) < 0.5, rs.choice(pool, B), rs.integers(0, cap - 1, B))
    lens = np.minimum(lens, cap - 2).astype(np.int32)
    bps = 0 if rs.random() < 0.6 else int(rs.integers(1, MB + 1))
    if seed % 4 in (1, 2):  # the automatic plan on the larger batches
        bps = 0
    return rs, scheme, D, B, H, MB, lens, bps


@pytest.mark.parametrize("seed", range(12))
def test_random_shape_end_to_end(seed):
    import decode_attention_block_amd as kvq
    import torch
    rs, scheme, D, B, H, MB, lens, bps = _case(seed)
    say("random shape", seed, "scheme", scheme, "D", D, "B", B, "H", H, "MB", MB, "bps", bps)
    S = MB * 64
    dist_v = 1.0 if scheme != oracle.UINT8_ASYM else 0.5
    k = rs.standard_normal((B, S, H, D)).astype(np.float16)
    v = (rs.standard_normal((B, S, H, D)) * dist_v).astype(np.float16)
    c = gpu_quantize(scheme, k, v, lens, MB)
    assert_cache_equal(c.host_arrays(), oracle_cache(scheme, k, v, lens, MB), lens)
    for _ in range(2):
        kn = np.ascontiguousarray(k[np.arange(B), lens])
        vn = np.ascontiguousarray(v[np.arange(B), lens])
        kvq.kv_append(c, to_gpu(kn), to_gpu(vn), int(lens.max()) + 1)
        torch.cuda.synchronize()
        lens = (lens + 1).astype(np.int32)
        assert list(c.seq_lens.cpu().numpy()) == lens.tolist()
        assert_cache_equal(c.host_arrays(), oracle_cache(scheme, k, v, lens, MB), lens)
    q = rs.standard_normal((B, H, D)).astype(np.float16)
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    L = int(lens.max())
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L, bps)
    fused = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, sm, fused, ws, L, bps)
    torch.cuda.synchronize()
    o = fused.cpu().numpy()
    assert not ws[:4 * B * H].any()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"random shape {seed}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    assert not o[lens == 0].any()
    split = torch.full_like(qt, 7.0)
    kvq.decode_attn_split(c, qt, sm, ws, L, bps)
    kvq.decode_attn_combine(c, split, ws, L, bps)
    torch.cuda.synchronize()
    assert np.array_equal(split.cpu().numpy(), o)


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_grouped_query(seed):
    """decode_attn_gqa on seeded random shapes (group 2, 4 or 8; batches up to 80; the
    automatic plan or a caller's; every format) against the oracle's attention over the
    cache with every cached head repeated G times (query head h * G + g reads cached head
    h); the workspace's arrival counters back at zero."""
    import decode_attention_block_amd as kvq
    import torch
    rs = np.random.default_rng(2000 + seed)
    scheme = SCHEMES[seed % 3]
    D = (64, 128)[(seed // 3) % 2]
    G = int(rs.choice([2, 4, 8]))
    B = int(rs.choice([1, 5, 8, 40, 80]))
    H = int(rs.choice([1, 2, 3, 8]))
    while B * H * D * G > 600000:
        H = max(1, H // 2)
        if B * H * D * G > 600000 and H == 1:
            B = max(1, B // 2)
    MB = int(rs.integers(2, 6))
    cap = MB * 64
    lens = np.where(rs.random(B) < 0.4, rs.choice([0, 1, 63, 64, 65, cap], B),
                    rs.integers(0, cap + 1, B)).astype(np.int32)
    bps = 0 if seed % 2 == 0 else int(rs.integers(1, MB + 1))
    say("random gqa", seed, "scheme", scheme, "D", D, "G", G, "B", B, "H", H, "MB", MB, "bps", bps)
    S = cap
    dist_v = 1.0 if scheme != oracle.UINT8_ASYM else 0.5
    k = rs.standard_normal((B, S, H, D)).astype(np.float16)
    v = (rs.standard_normal((B, S, H, D)) * dist_v).astype(np.float16)
    q = rs.standard_normal((B, H * G, D)).astype(np.float16)
    c = gpu_quantize(scheme, k, v, lens, MB)
    L = max(int(lens.max()), 1)
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    out = torch.full((B, H * G, D), 7.0, dtype=torch.float16, device="cuda")
    ws = kvq.make_workspace(c, L, bps, group=G)
    kvq.decode_attn_gqa(c, to_gpu(q), G, sm, out, ws, L, bps)
    torch.cuda.synchronize()
    assert not ws[:4 * B * H].any()
    o = out.cpu().numpy()
    host = c.host_arrays()
    rep = dict(host)
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        if host.get(key) is not None:
            rep[key] = np.ascontiguousarray(np.repeat(host[key], G, axis=1))
    rep["H"] = H * G
    ref = oracle.attention(rep, q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"random gqa {seed}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    assert not o[lens == 0].any()


@pytest.mark.parametrize("seed", range(6))
def test_random_shape_decode_steps(seed):
    """decode_step_qkv on seeded random shapes, dense or paged (a shuffled page pool 1.5
    times the blocks), one launch (the rows fill the GPU) or two: three steps, after each
    the lengths and the whole cache bit-exact against the oracle's quantization of the
    history and the output within 2e-3 of the oracle's attention over the new length."""
    import decode_attention_block_amd as kvq
    import torch
    rs = np.random.default_rng(3000 + seed)
    scheme = SCHEMES[seed % 3]
    D = (64, 128)[(seed // 3) % 2]
    B, H = [(8, 32), (3, 5), (20, 13), (1, 40), (70, 4), (6, 7)][seed]
    paged = seed % 2 == 1
    MB = int(rs.integers(2, 5))
    cap = MB * 64
    lens = np.where(rs.random(B) < 0.4, rs.choice([0, 1, 63, 64, 65], B),
                    rs.integers(0, cap - 3, B))
    lens = np.minimum(lens, cap - 3).astype(np.int32)
    say("random steps", seed, "scheme", scheme, "D", D, "B", B, "H", H, "MB", MB,
        "paged", paged, "launches", "1" if B * H >= 256 else "2")
    S = cap
    dist_v = 1.0 if scheme != oracle.UINT8_ASYM else 0.5
    k = rs.standard_normal((B, S, H, D)).astype(np.float16)
    v = (rs.standard_normal((B, S, H, D)) * dist_v).astype(np.float16)
    if paged:
        n_pages = (3 * B * MB) // 2
        c = kvq.KVCache(scheme, B, H, D, MB, num_pages=n_pages)
        perm = rs.permutation(n_pages)[: B * MB].astype(np.int32)
        c.block_table.copy_(torch.from_numpy(perm.reshape(B, MB)))
    else:
        c = kvq.KVCache(scheme, B, H, D, MB)
    c.seq_lens.copy_(torch.from_numpy(lens))
    kvq.kv_quantize_blocks(c, to_gpu(k), to_gpu(v), max(int(lens.max()), 1))
    torch.cuda.synchronize()
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    for step in range(3):
        after = int(lens.max()) + 1
        kn = to_gpu(np.ascontiguousarray(k[np.arange(B), lens]))
        vn = to_gpu(np.ascontiguousarray(v[np.arange(B), lens]))
        q = rs.standard_normal((B, H, D)).astype(np.float16)
        out = torch.full((B, H, D), 7.0, dtype=torch.float16, device="cuda")
        kvq.decode_step_qkv(c, kn, vn, to_gpu(q), sm, out, kvq.make_workspace(c, after), after)
        torch.cuda.synchronize()
        lens = (lens + 1).astype(np.int32)
        assert list(c.seq_lens.cpu().numpy()) == lens.tolist()
        host = c.host_arrays()
        assert_cache_equal(host, oracle_cache(scheme, k, v, lens, MB), lens)
        norm_err, _ = attn_errors(out.cpu().numpy(), oracle.attention(host, q, lens, sm))
        print(f"random steps {seed} step {step}: normwise {norm_err:.3e}")
        assert norm_err <= ATTN_TOL
