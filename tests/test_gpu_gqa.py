"""GPU parity of decode_attn_gqa (grouped-query decode attention) against the oracle:
grouped-query attention is multi-head attention in which cached head h serves query
heads h * G .. h * G + G - 1, so the oracle's reference is its fp64 attention over the
cache with every head repeated G times (a copy, no arithmetic). Tolerance as for
decode_attn_qkv; group 1 must be decode_attn_qkv itself (bitwise). Every scheme: int4 on
the matrix cores, uint8 and FP8 on the vector ALUs."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import ATTN_TOL, attn_errors, gpu_quantize, say, to_gpu

pytestmark = pytest.mark.gpu

INT4, UINT8, FP8 = oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3


def repeat_heads(host, G):
    """The cache dict with each head's arrays repeated G times (query head h*G + g
    reads cached head h)."""
    out = dict(host)
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        if host.get(key) is not None:
            out[key] = np.ascontiguousarray(np.repeat(host[key], G, axis=1))
    out["H"] = host["H"] * G
    return out


def _case(D, G, B=3, H=2, S=600, lens=(600, 1, 333), seed=0, scheme=INT4):
    g = wl.rng(wl.WORKLOADS[0], 140 + seed, G, D)
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, "normal0.5" if scheme == UINT8 else "normal_outliers", (B, S, H, D))
    q = wl.draw(g, "normal0", (B, H * G, D))
    return k, v, q, np.asarray(lens, np.int32)


def _gqa(c, q, G, sm, max_len, bps=0):
    import decode_attention_block_amd as kvq
    import torch
    B, HG, D = q.shape
    out = torch.empty((B, HG, D), dtype=torch.float16, device="cuda")
    ws = kvq.make_workspace(c, max_len, bps, group=G)
    kvq.decode_attn_gqa(c, to_gpu(q), G, sm, out, ws, max_len, bps)
    torch.cuda.synchronize()
    assert not ws[: 4 * c.batch * c.heads].any().item()   # counters left zero
    return out.cpu().numpy()


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bps", [0, 2])
def test_gqa_matches_oracle(scheme, G, D, bps):
    say("gqa", scheme, G, D, bps)
    k, v, q, lens = _case(D, G, seed=D + G, scheme=scheme)
    MB = 10
    c = gpu_quantize(scheme, k, v, lens, MB)
    sm = 1.0 / np.sqrt(D)
    o = _gqa(c, q, G, sm, int(lens.max()), bps)
    ref = oracle.attention(repeat_heads(c.host_arrays(), G), q, lens, sm)
    norm_err, elem_err = attn_errors(o, ref)
    print(f"scheme={scheme} G={G} D={D} bps={bps}: normwise {norm_err:.3e} "
          f"elementwise {elem_err:.3e}")
    assert norm_err <= ATTN_TOL


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
def test_gqa_empty_rows_and_paged_layout(scheme):
    """Rows of length 0 give zeros; on a paged cache (shuffled pool) the result is
    bitwise the dense one."""
    import decode_attention_block_amd as kvq
    import torch
    say("gqa empty+paged", scheme)
    G, D, B, H, MB = 4, 128, 4, 3, 6
    k, v, q, lens = _case(D, G, B=B, H=H, S=384, lens=(384, 0, 65, 200), seed=9, scheme=scheme)
    dense = gpu_quantize(scheme, k, v, lens, MB)
    paged = kvq.KVCache(scheme, B, H, D, MB, num_pages=B * MB + 5)
    perm = np.random.default_rng(3).permutation(B * MB + 5)[: B * MB].astype(np.int32)
    paged.block_table.copy_(torch.from_numpy(perm.reshape(B, MB)))
    paged.seq_lens.copy_(torch.from_numpy(lens))
    kvq.kv_quantize_blocks(paged, to_gpu(k), to_gpu(v), 384)
    sm = 1.0 / np.sqrt(D)
    o_d = _gqa(dense, q, G, sm, 384)
    o_p = _gqa(paged, q, G, sm, 384)
    assert np.array_equal(o_d.view(np.uint16), o_p.view(np.uint16))
    assert not o_d[1].any()
    ref = oracle.attention(repeat_heads(dense.host_arrays(), G), q, lens, sm)
    rows = [(b, h) for b in (0, 2, 3) for h in range(H * G)]
    assert attn_errors(o_d, ref, rows)[0] <= ATTN_TOL


@pytest.mark.parametrize("scheme", [INT4, FP8])
def test_group_one_is_decode_attn_qkv(scheme):
    import decode_attention_block_amd as kvq
    import torch
    say("gqa group 1", scheme)
    k, v, q, lens = _case(128, 1, seed=4, scheme=scheme)
    c = gpu_quantize(scheme, k, v, lens, 10)
    sm = 1.0 / np.sqrt(128)
    o1 = _gqa(c, q, 1, sm, 600)
    out = torch.empty(q.shape, dtype=torch.float16, device="cuda")
    kvq.decode_attn_qkv(c, to_gpu(q), sm, out, kvq.make_workspace(c, 600), 600)
    assert np.array_equal(o1.view(np.uint16), out.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("scheme", [INT4, FP8])
def test_gqa_workload_full_size_sampled(scheme):
    """The grouped-query workload (64 query heads over 8 cached heads, batch 8, context
    8192) in the launch configuration bench.py times (int4; and the same shape over an
    FP8 cache); sequences 0 and 7, all query heads, against the oracle."""
    w = wl.BY_NAME["llama70b_gqa8_b8_h8_d128_ctx8k_int4"]
    say("gqa workload", w.name, scheme)
    lens = wl.lengths(w)
    k = wl.prefill_batch(w, 0, 0)
    v = wl.prefill_batch(w, 0, 1)
    q = wl.query(w, 0)
    c = gpu_quantize(scheme, k, v, lens, w.max_blocks)
    sm = wl.softmax_scale(w)
    o = _gqa(c, q, w.group, sm, int(lens.max()))
    seqs = [0, 7]
    host = repeat_heads(c.host_arrays(seqs=seqs), w.group)
    ref = oracle.attention(host, q[seqs], lens[seqs], sm)
    norm_err, _ = attn_errors(o[seqs], ref)
    print(f"{w.name}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
