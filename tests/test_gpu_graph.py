"""A multi-layer decode step captured as a HIP graph (decode_attention_block_amd.graph)
must give, replay after replay, bitwise what the same calls give eagerly: caches,
lengths and outputs of every layer, with eager work between the replays. After the last
replay every layer's cache must also equal the oracle's quantization of the whole
history bit for bit, and every layer's output must be within the attention tolerance
of the oracle's fp64 attention over that cache."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import ATTN_TOL, assert_cache_equal, attn_errors, gpu_quantize, say, to_gpu

pytestmark = pytest.mark.gpu

INT4, UINT8, FP8 = oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3


def _layers(scheme, n_layers, B, H, D, S, lens, MB, seed):
    k_all, v_all, eager, graphed = [], [], [], []
    for layer in range(n_layers):
        g = wl.rng(wl.WORKLOADS[0], 160 + seed, layer, D)
        dist_v = "normal0.5" if scheme == UINT8 else "normal_outliers"
        k = wl.draw(g, "normal_outliers", (B, S, H, D))
        v = wl.draw(g, dist_v, (B, S, H, D))
        k_all.append(k)
        v_all.append(v)
        eager.append(gpu_quantize(scheme, k, v, lens, MB))
        graphed.append(gpu_quantize(scheme, k, v, lens, MB))
    return k_all, v_all, eager, graphed


def _same(a, b):
    import torch
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("append", [True, False])
@pytest.mark.parametrize("bps", [0, 1])  # one split per row (one launch), or four per row
def test_graph_replays_equal_eager_steps(scheme, append, bps):
    import decode_attention_block_amd as kvq
    from decode_attention_block_amd.graph import DecodeGraph
    import torch
    say("graph", scheme, append, bps)
    L, B, H, D, MB, S = 3, 8, 32, 64, 4, 256
    lens = np.array([0, 1, 63, 64, 100, 127, 5, 200], np.int32)
    k_all, v_all, eager, graphed = _layers(scheme, L, B, H, D, S, lens, MB, seed=scheme)
    sm = 1.0 / np.sqrt(D)
    dg = DecodeGraph(graphed, sm, append=append, blocks_per_split=bps)
    cap = MB * 64
    ws = [kvq.make_workspace(c, cap, bps) for c in eager]
    out = [torch.empty((B, H, D), dtype=torch.float16, device="cuda") for _ in range(L)]
    cur = lens.copy()
    rs = np.random.default_rng(5)
    q_host = [None] * L
    for step in range(4):
        for i in range(L):
            q_host[i] = rs.standard_normal((B, H, D)).astype(np.float16)
            q = to_gpu(q_host[i])
            dg.q[i].copy_(q)
            if append:
                kn = to_gpu(k_all[i][np.arange(B), cur])
                vn = to_gpu(v_all[i][np.arange(B), cur])
                dg.k_new[i].copy_(kn)
                dg.v_new[i].copy_(vn)
                kvq.decode_step_qkv(eager[i], kn, vn, q, sm, out[i], ws[i], cap, bps)
            else:
                kvq.decode_attn_qkv(eager[i], q, sm, out[i], ws[i], cap, bps)
        dg.replay()
        torch.cuda.synchronize()
        if append:
            cur = cur + 1
        for i in range(L):
            assert np.array_equal(eager[i].seq_lens.cpu().numpy(), cur)
            assert np.array_equal(graphed[i].seq_lens.cpu().numpy(), cur)
            assert _same(out[i], dg.out[i]), (step, i)
            for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_tail", "v_tail"):
                assert _same(getattr(eager[i], key), getattr(graphed[i], key)), (step, i, key)
    # the replayed state against the oracle: caches bit for bit, outputs within tolerance
    for i in range(L):
        ref = oracle.quantize_cache(scheme, k_all[i], v_all[i], cur, MB)
        assert_cache_equal(graphed[i].host_arrays(), ref, cur)
        o_ref = oracle.attention(ref, q_host[i], cur, sm)
        norm_err, _ = attn_errors(dg.out[i].cpu().numpy(), o_ref)
        assert norm_err <= ATTN_TOL, (i, norm_err)
