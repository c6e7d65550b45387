"""GPU parity of the paged cache layout: with a block table that scatters every
sequence's blocks over a shuffled page pool, every call (prefill quantization, append,
attention, decode step) must give bitwise the results of the dense layout on the same
data, and the pool pages no table entry names must stay untouched."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import assert_cache_equal, oracle_cache, say, to_gpu

pytestmark = pytest.mark.gpu

INT4, UINT8, FP8 = oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3
SENTINEL = 0xA5


def _history(scheme, B, H, D, S, seed):
    g = wl.rng(wl.WORKLOADS[0], 120 + seed, scheme, D)
    dist_v = "normal0.5" if scheme == UINT8 else "normal_outliers"
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, dist_v, (B, S, H, D))
    return k, v, g


def _pair(scheme, B, H, D, MB, lens, k, v, seed):
    """A dense cache and a paged one (pool 1.5x the blocks, shuffled pages, unused
    pages filled with a sentinel), both quantized from the same prefill."""
    import decode_attention_block_amd as kvq
    import torch
    n_pages = (3 * B * MB) // 2
    dense = kvq.KVCache(scheme, B, H, D, MB)
    paged = kvq.KVCache(scheme, B, H, D, MB, num_pages=n_pages)
    perm = np.random.default_rng(seed).permutation(n_pages)[: B * MB].astype(np.int32)
    paged.block_table.copy_(torch.from_numpy(perm.reshape(B, MB)))
    unused = np.setdiff1d(np.arange(n_pages), perm)
    for t in (paged.k_codes, paged.v_codes):
        t[torch.from_numpy(unused).long()] = SENTINEL
    for c in (dense, paged):
        c.seq_lens.copy_(torch.from_numpy(np.asarray(lens, np.int32)))
        kvq.kv_quantize_blocks(c, to_gpu(k), to_gpu(v), int(np.max(lens)))
    torch.cuda.synchronize()
    return dense, paged, unused


def _assert_pool_untouched(paged, unused):
    import torch
    idx = torch.from_numpy(unused).long()
    for t in (paged.k_codes, paged.v_codes):
        assert bool((t[idx] == SENTINEL).all()), "an unmapped page was written"


def _assert_same_cache(dense, paged, lens):
    d, p = dense.host_arrays(natural=False), paged.host_arrays(natural=False)
    B, H = d["B"], d["H"]
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        for b in range(B):
            nb = (int(lens[b]) + 63) // 64
            x, y = d[key][b, :, :nb], p[key][b, :, :nb]
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (key, b)


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_prefill_and_attention_equal_dense(scheme, D):
    import decode_attention_block_amd as kvq
    import torch
    say("paged prefill+attention", scheme, D)
    B, H, MB, S = 4, 3, 6, 384
    lens = np.array([384, 1, 200, 0], np.int32)
    k, v, g = _history(scheme, B, H, D, S, seed=D + scheme)
    dense, paged, unused = _pair(scheme, B, H, D, MB, lens, k, v, seed=7)
    _assert_same_cache(dense, paged, lens)
    assert_cache_equal(paged.host_arrays(), oracle_cache(scheme, k, v, lens, MB), lens)
    _assert_pool_untouched(paged, unused)
    q = to_gpu(wl.draw(g, "normal0", (B, H, D)))
    for bps in (0, 2):
        outs = []
        for c in (dense, paged):
            out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
            ws = kvq.make_workspace(c, S, bps)
            kvq.decode_attn_qkv(c, q, 1.0 / np.sqrt(D), out, ws, S, bps)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), bps


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("BH", [(8, 32), (3, 5)])
def test_paged_appends_and_decode_steps_equal_dense(scheme, BH):
    """kv_append and decode_step_qkv (one launch for 8 x 32 rows, two launches for
    3 x 5) on both layouts, across block boundaries."""
    import decode_attention_block_amd as kvq
    import torch
    B, H = BH
    D, MB, S = 128, 5, 320
    say("paged appends+steps", scheme, B, H)
    lens = np.array([0, 1, 63, 64, 100, 127, 5, 250][:B], np.int32)
    k, v, g = _history(scheme, B, H, D, S, seed=B + 3 * scheme)
    dense, paged, unused = _pair(scheme, B, H, D, MB, lens, k, v, seed=11)
    q = to_gpu(wl.draw(g, "normal0", (B, H, D)))
    sm = 1.0 / np.sqrt(D)
    cur = lens.copy()
    for step in range(4):
        after = int(cur.max()) + 1
        kn, vn = to_gpu(k[np.arange(B), cur]), to_gpu(v[np.arange(B), cur])
        outs = []
        for c in (dense, paged):
            if step % 2 == 0:
                kvq.kv_append(c, kn, vn, after)
                outs.append(None)
            else:
                out = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
                kvq.decode_step_qkv(c, kn, vn, q, sm, out, kvq.make_workspace(c, after), after)
                outs.append(out)
        cur = cur + 1
        torch.cuda.synchronize()
        assert np.array_equal(dense.seq_lens.cpu().numpy(), cur)
        assert np.array_equal(paged.seq_lens.cpu().numpy(), cur)
        _assert_same_cache(dense, paged, cur)
        if outs[0] is not None:
            assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), step
    assert_cache_equal(paged.host_arrays(), oracle_cache(scheme, k, v, cur, MB), cur)
    _assert_pool_untouched(paged, unused)
