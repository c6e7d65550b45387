"""GPU parity of decode_attn_qkv against the oracle's fp64 attention over the same
dequantized cache (max over rows of ||o_gpu - o_ref||_inf / ||o_ref||_inf <= 2e-3),
plus the properties that hold at any size: split-count invariance, padding-poison
invariance, determinism and empty rows."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import (ATTN_TOL, attn_errors, gpu_attention, gpu_quantize, oracle_cache, say,
                     to_gpu)

pytestmark = pytest.mark.gpu

INT4, UINT8, FP8 = oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3


def _workload_case(index, layer=0, seqs=None):
    w = wl.WORKLOADS[index]
    lens = wl.lengths(w)
    n = int(lens.max())
    k = wl.prefill_batch(w, layer, 0, n_tokens=n)
    v = wl.prefill_batch(w, layer, 1, n_tokens=n)
    q = wl.query(w, layer)
    return w, k, v, q, lens


@pytest.mark.parametrize("index", [0, 1, 2, 6])
def test_workload_attention_all_rows(index):
    w, k, v, q, lens = _workload_case(index)
    say("attention", w.name)
    c = gpu_quantize(w.scheme, k, v, lens, w.max_blocks)
    sm = wl.softmax_scale(w)
    o = gpu_attention(c, q, sm, int(lens.max()))
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, elem_err = attn_errors(o, ref)
    print(f"{w.name}: normwise {norm_err:.3e} elementwise(floored) {elem_err:.3e}")
    assert norm_err <= ATTN_TOL


def test_ragged_32_layer_attention_sampled_layers():
    w = wl.WORKLOADS[4]
    for layer in (0, 13, 31):
        _, k, v, q, lens = _workload_case(4, layer)
        say("attention", w.name, "layer", layer)
        c = gpu_quantize(w.scheme, k, v, lens, w.max_blocks)
        sm = wl.softmax_scale(w)
        o = gpu_attention(c, q, sm, int(lens.max()))
        ref = oracle.attention(c.host_arrays(), q, lens, sm)
        norm_err, _ = attn_errors(o, ref)
        print(f"{w.name} layer {layer}: normwise {norm_err:.3e}")
        assert norm_err <= ATTN_TOL


def _small_case(scheme, D, seed=7, B=4, H=3, S=700, lens=(700, 1, 333, 64)):
    g = wl.rng(wl.WORKLOADS[0], 60 + seed, scheme, D)
    dist_v = "normal0.5" if scheme == UINT8 else "normal_outliers"
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, dist_v, (B, S, H, D))
    q = wl.draw(g, "normal0", (B, H, D))
    return k, v, q, np.array(lens, np.int32)


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("D", [64, 128])
def test_split_counts_all_agree_with_oracle(scheme, D):
    """Every split size (1 block .. one split for the whole row, and the automatic
    plan) is within tolerance of the oracle and within 1e-5 of each other."""
    k, v, q, lens = _small_case(scheme, D)
    MB = 11
    c = gpu_quantize(scheme, k, v, lens, MB)
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    outs = []
    for bps in (0, 1, 2, 3, 4, 8, 11, 64):
        say("split", scheme, D, "bps", bps)
        o = gpu_attention(c, q, sm, int(lens.max()), bps)
        norm_err, _ = attn_errors(o, ref)
        assert norm_err <= ATTN_TOL, (bps, norm_err)
        outs.append(o.astype(np.float64))
    spread = max(np.abs(a - outs[0]).max() for a in outs)
    assert spread <= 1e-5 * max(1.0, np.abs(outs[0]).max()) + 2 ** -10 * np.abs(outs[0]).max()


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
def test_padding_poison_and_determinism(scheme):
    """Garbage in the padding bytes of each last block changes nothing (bitwise), and
    repeated calls are bitwise identical."""
    import torch
    k, v, q, lens = _small_case(scheme, 128, seed=3, lens=(699, 5, 130, 64))
    MB = 11
    c = gpu_quantize(scheme, k, v, lens, MB)
    sm = 0.08838834764831845
    say("poison", scheme)
    base = gpu_attention(c, q, sm, int(lens.max()))
    for _ in range(3):
        assert np.array_equal(gpu_attention(c, q, sm, int(lens.max())), base)
    from decode_attention_block_amd import layout
    rs = np.random.default_rng(1)
    for b, n in enumerate(lens):
        j, t = divmod(int(n), 64)
        if t:
            for which, codes in (("k", c.k_codes), ("v", c.v_codes)):
                blk = codes[b, :, j].cpu().numpy()          # [H][64][row bytes] as stored
                if scheme == INT4:
                    blk = layout.int4_to_natural(blk, which)
                blk[:, t:] = rs.integers(0, 256, blk[:, t:].shape, dtype=np.uint8)
                if scheme == INT4:
                    blk = layout.int4_from_natural(blk, which)
                codes[b, :, j] = torch.from_numpy(blk).cuda()
    torch.cuda.synchronize()
    assert np.array_equal(gpu_attention(c, q, sm, int(lens.max())), base)


def test_empty_and_single_token_rows():
    k, v, q, lens = _small_case(INT4, 128, seed=5, B=3, S=70, lens=(0, 1, 70))
    c = gpu_quantize(INT4, k, v, lens, 2)
    say("empty rows")
    o = gpu_attention(c, q, 0.0883883476, 70)
    ref = oracle.attention(c.host_arrays(), q, lens, 0.0883883476)
    assert not o[0].any()
    norm_err, _ = attn_errors(o, ref, rows=[(1, h) for h in range(3)] + [(2, h) for h in range(3)])
    assert norm_err <= ATTN_TOL


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("bps", [2, 0])
def test_split_and_combine_phases_equal_fused_call(scheme, bps):
    """decode_attn_split + decode_attn_combine give bitwise the fused result (several
    splits per row, and the automatic plan), and the fused call leaves the workspace's
    arrival counters at zero after every call."""
    import decode_attention_block_amd as kvq
    import torch
    k, v, q, lens = _small_case(scheme, 64, seed=8)
    c = gpu_quantize(scheme, k, v, lens, 11)
    say("phases", scheme, bps)
    L = int(lens.max())
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L, bps)
    fused = torch.empty_like(qt)
    for _ in range(3):
        kvq.decode_attn_qkv(c, qt, 0.125, fused, ws, L, bps)
        torch.cuda.synchronize()
        assert not ws[:4 * c.batch * c.heads].any()
    out = torch.empty_like(qt)
    kvq.decode_attn_split(c, qt, 0.125, ws, L, bps)
    kvq.decode_attn_combine(c, out, ws, L, bps)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), fused.cpu().numpy())


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bps", [0, 3])
def test_ragged_rows(scheme, D, bps):
    """Ragged rows in one batch: empty, one-token, block-edge and long rows (one split or
    several). All rows within tolerance of the oracle; split + combine bitwise equal to
    the fused call; counters back at zero; repeated calls identical."""
    import decode_attention_block_amd as kvq
    import torch
    B, H, S = 13, 3, 700
    lens = np.array([0, 1, 63, 64, 65, 700, 0, 333, 129, 2, 640, 17, 511], np.int32)
    k, v, q, _ = _small_case(scheme, D, seed=21, B=B, H=H, S=S, lens=lens)
    c = gpu_quantize(scheme, k, v, lens, 11)
    L = int(lens.max())
    say("ragged", scheme, D, "plan", kvq.decode_attn_plan(c, L, bps))
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L, bps)
    fused = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, sm, fused, ws, L, bps)
    torch.cuda.synchronize()
    o = fused.cpu().numpy()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"ragged scheme {scheme} D {D} bps {bps}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    assert not o[0].any() and not o[6].any()                  # empty rows are zeros
    assert not ws[:4 * B * H].any()
    for _ in range(2):
        again = torch.empty_like(qt)
        kvq.decode_attn_qkv(c, qt, sm, again, ws, L, bps)
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy(), o)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_split(c, qt, sm, ws, L, bps)
    kvq.decode_attn_combine(c, out, ws, L, bps)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), o)


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
def test_automatic_plan_with_more_rows_than_cus(scheme):
    """The automatic plan over a batch of more rows (320) than compute units, with random
    lengths (empty rows included), so the device cuts the long rows and leaves the
    others whole. Every row within tolerance of the oracle; split + combine bitwise equal
    to the fused call; counters back at zero; repeated calls identical."""
    import decode_attention_block_amd as kvq
    import torch
    B, H, S, D = 40, 8, 700, 64
    lens = np.random.default_rng(77).integers(0, S + 1, B).astype(np.int32)
    lens[[3, 17]] = 0
    lens[5] = S
    k, v, q, _ = _small_case(scheme, D, seed=31, B=B, H=H, S=S, lens=lens)
    c = gpu_quantize(scheme, k, v, lens, 11)
    L = int(lens.max())
    say("automatic plan, 320 rows", scheme, lens.tolist())
    sm = 0.125
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L)
    fused = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, sm, fused, ws, L)
    torch.cuda.synchronize()
    o = fused.cpu().numpy()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"automatic plan, 320 rows, scheme {scheme}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    assert not o[3].any() and not o[17].any()
    assert not ws[:4 * B * H].any()
    again = torch.empty_like(qt)
    kvq.decode_attn_qkv(c, qt, sm, again, ws, L)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy(), o)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_split(c, qt, sm, ws, L)
    kvq.decode_attn_combine(c, out, ws, L)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), o)


@pytest.mark.parametrize("B", [64, 65])
def test_automatic_plan_pairing_limit(B):
    """Three split columns under the automatic plan with a ragged batch of 64 sequences
    (the later pieces of cut rows are streamed by the workgroups of other sequences'
    positions) and of 65 (each row's pieces by its own positions): within tolerance of
    the oracle, and bitwise the split + combine of the same plan."""
    import decode_attention_block_amd as kvq
    import torch
    H, S, D = 4, 600, 64
    lens = np.random.default_rng(5 + B).integers(1, S + 1, B).astype(np.int32)
    lens[[0, B - 1]] = (S, 1)
    k, v, q, _ = _small_case(INT4, D, seed=37, B=B, H=H, S=S, lens=lens)
    c = gpu_quantize(INT4, k, v, lens, 10)
    L = int(lens.max())
    assert kvq.decode_attn_plan(c, L) == (0, 3)
    say("pairing limit", B)
    sm = 0.125
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, sm, out, ws, L)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"pairing limit B={B}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    split = torch.full_like(qt, 7.0)
    kvq.decode_attn_split(c, qt, sm, ws, L)
    kvq.decode_attn_combine(c, split, ws, L)
    torch.cuda.synchronize()
    assert np.array_equal(split.cpu().numpy(), o)


@pytest.mark.parametrize("lens", [(5, 70), (0, 0, 0), (0, 130, 0)])
def test_lengths_below_the_launch_bound(lens):
    """max_len well above every length (the launch sizes for capacity, the rows are
    shorter), and batches with empty rows only."""
    import decode_attention_block_amd as kvq
    import torch
    lens = np.array(lens, np.int32)
    B, H, S = len(lens), 2, 130
    k, v, q, _ = _small_case(INT4, 128, seed=23, B=B, H=H, S=S, lens=lens)
    c = gpu_quantize(INT4, k, v, lens, 4, max_len=S)
    say("short rows", lens.tolist())
    sm = 0.0883883476
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, 256)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, sm, out, ws, 256)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    rows = [(b, h) for b in range(B) for h in range(H) if lens[b] > 0]
    for b in range(B):
        if lens[b] == 0:
            assert not o[b].any()
    if rows:
        norm_err, _ = attn_errors(o, ref, rows=rows)
        assert norm_err <= ATTN_TOL
    assert not ws[:4 * B * H].any()


def test_zero_context_call_writes_zeros():
    import decode_attention_block_amd as kvq
    import torch
    k, v, q, lens = _small_case(INT4, 128, seed=9, B=2, S=64, lens=(0, 0))
    c = gpu_quantize(INT4, k, v, lens, 1, max_len=0)
    say("zero context")
    qt = to_gpu(q)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_qkv(c, qt, 0.1, out, None, 0)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()


@pytest.mark.parametrize("scheme", [INT4, UINT8])
@pytest.mark.parametrize("bps", [1, 2, 5])
def test_many_splits_per_row(scheme, bps):
    """Rows cut into many splits (up to 41, several chunks of partial states in the
    merge, and a last chunk partly past the row's splits): fused call within tolerance
    of the oracle, bitwise equal to split + combine and to itself on a repeat; counters
    back at zero."""
    import decode_attention_block_amd as kvq
    import torch
    B, H, S = 3, 2, 2600
    lens = np.array([2600, 577, 1], np.int32)
    k, v, q, _ = _small_case(scheme, 64, seed=31, B=B, H=H, S=S, lens=lens)
    c = gpu_quantize(scheme, k, v, lens, 41)
    L = int(lens.max())
    say("many splits", scheme, "plan", kvq.decode_attn_plan(c, L, bps))
    assert kvq.decode_attn_plan(c, L, bps)[1] == (41 + bps - 1) // bps
    sm = 0.125
    qt = to_gpu(q)
    ws = kvq.make_workspace(c, L, bps)
    fused = torch.empty_like(qt)
    kvq.decode_attn_qkv(c, qt, sm, fused, ws, L, bps)
    torch.cuda.synchronize()
    o = fused.cpu().numpy()
    ref = oracle.attention(c.host_arrays(), q, lens, sm)
    norm_err, _ = attn_errors(o, ref)
    print(f"many splits scheme {scheme} bps {bps}: normwise {norm_err:.3e}")
    assert norm_err <= ATTN_TOL
    assert not ws[:4 * B * H].any()
    again = torch.empty_like(qt)
    kvq.decode_attn_qkv(c, qt, sm, again, ws, L, bps)
    out = torch.full_like(qt, 7.0)
    kvq.decode_attn_split(c, qt, sm, ws, L, bps)
    kvq.decode_attn_combine(c, out, ws, L, bps)
    torch.cuda.synchronize()
    assert np.array_equal(again.cpu().numpy(), o)
    assert np.array_equal(out.cpu().numpy(), o)


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
def test_device_plan_cuts_the_long_rows_of_a_full_batch(scheme):
    """blocks_per_split = 0 on 8 x 32 rows (the rows fill the GPU): each row's split is
    chosen on the device from all the lengths. With one long sequence (10 blocks) among
    one-block ones the batch holds 32 * 17 blocks, chunks of ceil(544 / 256) = 3 blocks,
    so the long rows are cut, in pieces of about ceil(544 / 384) = 2 blocks, at most 3:
    3 pieces of ceil(10 / 3) = 4 blocks (4, 4, 2), and the others stay whole: bitwise
    the output of the caller's plan of 4 blocks per split (the pieces of the cut rows
    are streamed by the workgroups of other sequences' positions). With all rows equal
    (10 blocks each) every row stays whole: bitwise the plan of 10. Both within
    tolerance of the oracle."""
    import decode_attention_block_amd as kvq
    import torch
    B, H, D, S = 8, 32, 64, 640
    for lens, same_as in (((64, 600, 64, 64, 64, 64, 64, 64), 4), ((600,) * 8, 10)):
        say("device plan", scheme, lens[:2], same_as)
        k, v, q, lens = _small_case(scheme, D, seed=31, B=B, H=H, S=S, lens=lens)
        c = gpu_quantize(scheme, k, v, lens, 10)
        L = int(lens.max())
        assert kvq.decode_attn_plan(c, L) == (0, 3)
        sm = float(np.float32(1) / np.sqrt(np.float32(D)))
        qt = to_gpu(q)
        outs = []
        for bps in (0, same_as):
            out = torch.full_like(qt, 7.0)
            kvq.decode_attn_qkv(c, qt, sm, out, kvq.make_workspace(c, L, bps), L, bps)
            torch.cuda.synchronize()
            outs.append(out)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
        ref = oracle.attention(c.host_arrays(), q, lens, sm)
        norm_err, _ = attn_errors(outs[0].cpu().numpy(), ref)
        assert norm_err <= ATTN_TOL, norm_err
