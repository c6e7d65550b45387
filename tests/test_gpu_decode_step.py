"""GPU parity of decode_step_qkv: one decode step (append, then attention over the
lengths after it) must leave the cache and seq_lens bitwise equal to kv_append followed
by decode_attn_qkv, and its output equal to theirs up to the attention's summation
order (bitwise on the two-launch path, which is those two calls; on the single-launch
path the new token's block is summed last, so the fp16 outputs may differ in the last
place), and its attention must match the oracle's over the appended history."""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from helpers import ATTN_TOL, attn_errors, gpu_quantize, oracle_cache, say, to_gpu

pytestmark = pytest.mark.gpu

INT4, UINT8, FP8 = oracle.INT4_SYM, oracle.UINT8_ASYM, oracle.FP8_E4M3


def _history(scheme, B, H, D, S, seed):
    g = wl.rng(wl.WORKLOADS[0], 80 + seed, scheme, D)
    dist_v = "normal0.5" if scheme == UINT8 else "normal_outliers"
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, dist_v, (B, S, H, D))
    q = wl.draw(g, "normal0", (B, H, D))
    return k, v, q


def _state(c):
    torch = __import__("torch")
    torch.cuda.synchronize()
    arrays = c.host_arrays(natural=False)
    arrays["k_tail"] = c.k_tail.cpu().numpy()
    arrays["v_tail"] = c.v_tail.cpu().numpy()
    arrays["seq_lens"] = c.seq_lens.cpu().numpy()
    return arrays


def _assert_same_state(a, b):
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero", "k_tail",
                "v_tail", "seq_lens"):
        if a.get(key) is None:
            assert b.get(key) is None, key
            continue
        x, y = np.asarray(a[key]), np.asarray(b[key])
        assert x.shape == y.shape, key
        if not np.array_equal(x.view(np.uint8), y.view(np.uint8)):
            raise AssertionError(f"{key} differs")


def _assert_same_output(out, out_ref, bitwise):
    torch = __import__("torch")
    if bitwise:
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
        return
    # one fp16 unit in the last place of the row's largest output at most
    norm_err, _ = attn_errors(out.cpu().numpy(), out_ref.cpu().numpy())
    assert norm_err <= 2.0 ** -10, norm_err


# (B, H): 8 x 32 = 256 rows -> one piece per row (single launch); 20 x 13 = 260 rows ->
# single launch with heads not a multiple of the ticket's groups of 8 (8 + 5); 3 x 5 ->
# several splits per row (append and attention as two launches, bitwise equal to the two
# calls).
@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("BH", [(8, 32), (20, 13), (3, 5)])
def test_step_equals_append_then_attention(scheme, D, BH):
    import decode_attention_block_amd as kvq
    import torch
    B, H = BH
    say("decode step", scheme, D, B, H)
    MB, S = 5, 320
    k, v, q = _history(scheme, B, H, D, S, seed=D + B)
    start = np.resize(np.array([0, 1, 63, 64, 100, 127, 5, 250], np.int32), B)
    ref_c = gpu_quantize(scheme, k, v, start, MB)
    c = gpu_quantize(scheme, k, v, start, MB)
    sm = 1.0 / np.sqrt(D)
    lens = start.copy()
    qt = to_gpu(q)
    out_ref = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(out_ref)
    for step in range(3):
        max_after = int(lens.max()) + 1
        ws_ref = kvq.make_workspace(ref_c, max_after)
        ws = kvq.make_workspace(c, max_after)
        kn = to_gpu(k[np.arange(B), lens])
        vn = to_gpu(v[np.arange(B), lens])
        kvq.kv_append(ref_c, kn, vn, max_after)
        kvq.decode_attn_qkv(ref_c, qt, sm, out_ref, ws_ref, max_after)
        kvq.decode_step_qkv(c, kn, vn, qt, sm, out, ws, max_after)
        lens = lens + 1
        a, b = _state(ref_c), _state(c)
        assert np.array_equal(b["seq_lens"], lens)
        _assert_same_state(a, b)
        _assert_same_output(out, out_ref, kvq.decode_step_launches(c, max_after) == 2)
        # the workspace counters are left zero for the next call
        n_rows = B * H
        assert not ws[: 4 * n_rows].any().item()
    # the last step against the oracle: cache bit-exact, attention within tolerance
    ref = oracle_cache(scheme, k, v, lens, MB)
    oracle_out = oracle.attention(ref, q, lens, sm)
    norm_err, _ = attn_errors(out.cpu().numpy(), oracle_out)
    assert norm_err <= ATTN_TOL


def test_step_on_full_rows_attends_without_appending():
    """A row at capacity is left unchanged by the append and attended at full length;
    the other rows of the batch still append."""
    import decode_attention_block_amd as kvq
    import torch
    say("decode step capacity")
    B, H, D, MB = 8, 32, 64, 2
    k, v, q = _history(INT4, B, H, D, 129, seed=3)
    start = np.array([128, 10, 127, 64, 128, 0, 1, 100], np.int32)
    ref_c = gpu_quantize(INT4, k, v, start, MB)
    c = gpu_quantize(INT4, k, v, start, MB)
    before = _state(c)
    sm = 1.0 / np.sqrt(D)
    idx = np.minimum(start, 128)
    kn, vn, qt = to_gpu(k[np.arange(B), idx]), to_gpu(v[np.arange(B), idx]), to_gpu(q)
    out_ref = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(out_ref)
    assert kvq.decode_step_launches(c, 128) == 1   # the single-launch path
    kvq.kv_append(ref_c, kn, vn, 128)
    kvq.decode_attn_qkv(ref_c, qt, sm, out_ref, kvq.make_workspace(ref_c, 128), 128)
    kvq.decode_step_qkv(c, kn, vn, qt, sm, out, kvq.make_workspace(c, 128), 128)
    after = _state(c)
    _assert_same_state(_state(ref_c), after)
    _assert_same_output(out, out_ref, False)
    assert list(after["seq_lens"]) == [128, 11, 128, 65, 128, 1, 2, 101]
    for b in (0, 4):
        assert np.array_equal(after["k_codes"][b], before["k_codes"][b])
        assert np.array_equal(after["v_scale"][b], before["v_scale"][b])


@pytest.mark.parametrize("scheme", [INT4, UINT8, FP8])
def test_step_with_lengths_beyond_the_bound(scheme):
    """Rows longer than max_len_after still append, and are attended over their first
    max_len_after tokens (as decode_attn_qkv clamps): the new token's block is then cut
    (row 0), or not attended at all (row 1)."""
    import decode_attention_block_amd as kvq
    import torch
    say("decode step clamp", scheme)
    B, H, D, MB = 8, 32, 128, 5
    k, v, q = _history(scheme, B, H, D, 320, seed=5)
    start = np.array([100, 200, 10, 64, 69, 0, 63, 5], np.int32)
    ref_c = gpu_quantize(scheme, k, v, start, MB)
    c = gpu_quantize(scheme, k, v, start, MB)
    sm = 1.0 / np.sqrt(D)
    bound = 70
    kn = to_gpu(k[np.arange(B), start])
    vn = to_gpu(v[np.arange(B), start])
    qt = to_gpu(q)
    out_ref = torch.empty((B, H, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(out_ref)
    assert kvq.decode_step_launches(c, bound) == 1
    kvq.kv_append(ref_c, kn, vn, bound)
    kvq.decode_attn_qkv(ref_c, qt, sm, out_ref, kvq.make_workspace(ref_c, bound), bound)
    kvq.decode_step_qkv(c, kn, vn, qt, sm, out, kvq.make_workspace(c, bound), bound)
    after = _state(c)
    _assert_same_state(_state(ref_c), after)
    assert np.array_equal(after["seq_lens"], start + 1)
    _assert_same_output(out, out_ref, False)
    lens = start + 1
    ref = oracle_cache(scheme, k, v, lens, MB)
    oracle_out = oracle.attention(ref, q, np.minimum(lens, bound), sm)
    norm_err, _ = attn_errors(out.cpu().numpy(), oracle_out)
    assert norm_err <= ATTN_TOL
