"""Pins of the oracle's fp64 decode attention.

The plain definition (scaled dot-product attention of one query over the dequantized
cache, textbook form; the pages never write it out) is checked against closed forms,
special cases and an independent library routine (torch's CPU scaled_dot_product_attention
in float64 over K^/V^ decoded here from the cache bytes).
"""
import math

import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl

INT4, UINT8 = oracle.INT4_SYM, oracle.UINT8_ASYM


def test_two_token_closed_form():
    """K block scale 1 (absmax 7.5), q = 8 e0, sm = 1/8 -> scores 0 and 1, so
    o = (v0 + e v1) / (1 + e)."""
    D = 64
    k = np.zeros((1, 64, 1, D), np.float16)
    v = np.zeros((1, 64, 1, D), np.float16)
    k[0, 1, 0, 0] = 1.0
    k[0, 1, 0, 1] = 7.5     # sets absmax 7.5 -> s = 1; q_1 = 0 so it adds nothing
    v[0, 1, 0, 0] = 2.0
    v[0, 0, 0, 1] = 7.5
    lens = np.array([2], np.int32)
    c = oracle.quantize_cache(INT4, k, v, lens, 1)
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 0] = 8.0
    o = oracle.attention(c, q, lens, 0.125)[0, 0]
    e = math.e
    assert abs(o[0] - 2 * e / (1 + e)) < 1e-14
    assert abs(o[1] - 7 / (1 + e)) < 1e-14       # 7.5 encodes as code 7
    assert np.all(o[2:] == 0)


@pytest.mark.parametrize("scheme", [INT4, UINT8, oracle.FP8_E4M3])
def test_length_one_returns_first_value_row(scheme):
    rs = np.random.default_rng(2)
    x = rs.standard_normal((1, 64, 2, 128)).astype(np.float16)
    lens = np.array([1], np.int32)
    c = oracle.quantize_cache(scheme, x, x[:, ::-1].copy(), lens, 1)
    q = rs.standard_normal((1, 2, 128)).astype(np.float16)
    o = oracle.attention(c, q, lens, 0.1)
    for h in range(2):
        _, vh = oracle.dequantize(c, 0, h, 1)
        assert np.array_equal(o[0, h], vh[0])


@pytest.mark.parametrize("scheme", [INT4, UINT8])
def test_zero_query_and_constant_keys_give_mean(scheme):
    rs = np.random.default_rng(3)
    B, S, H, D = 2, 150, 2, 64
    k = rs.standard_normal((B, S, H, D)).astype(np.float16)
    v = rs.standard_normal((B, S, H, D)).astype(np.float16)
    lens = np.array([150, 77], np.int32)
    c = oracle.quantize_cache(scheme, k, v, lens, 3)
    o = oracle.attention(c, np.zeros((B, H, D), np.float16), lens, 0.125)
    c0 = oracle.quantize_cache(scheme, np.zeros_like(k), v, lens, 3)
    q = rs.standard_normal((B, H, D)).astype(np.float16)
    o0 = oracle.attention(c0, q, lens, 0.125)
    for b in range(B):
        for h in range(H):
            _, vh = oracle.dequantize(c, b, h, lens[b])
            assert np.allclose(o[b, h], vh.mean(0), rtol=0, atol=1e-13)
            assert np.allclose(o0[b, h], vh.mean(0), rtol=0, atol=1e-13)


def test_empty_row_is_zero():
    x = np.ones((1, 64, 1, 64), np.float16)
    lens = np.array([0], np.int32)
    c = oracle.quantize_cache(INT4, x, x, lens, 1)
    o = oracle.attention(c, np.ones((1, 1, 64), np.float16), lens, 0.125)
    assert np.all(o == 0)


@pytest.mark.parametrize("scheme,dist", [(INT4, "normal_outliers"), (UINT8, "normal0.5"),
                                         (INT4, "student_t3_half"),
                                         (oracle.FP8_E4M3, "normal_outliers")])
def test_matches_torch_sdpa_fp64(scheme, dist):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    w = wl.WORKLOADS[0]
    g = wl.rng(w, 11, 0, 0)
    B, S, H, D = 2, 300, 3, 128
    k = wl.draw(g, dist, (B, S, H, D))
    v = wl.draw(g, dist, (B, S, H, D))
    lens = np.array([300, 129], np.int32)
    q = wl.draw(g, "normal0", (B, H, D))
    sm = float(np.float32(1) / np.sqrt(np.float32(D)))
    c = oracle.quantize_cache(scheme, k, v, lens, 5)
    o = oracle.attention(c, q, lens, sm)
    for b in range(B):
        for h in range(H):
            kh, vh = oracle.dequantize(c, b, h, lens[b])
            qt = torch.from_numpy(q[b, h].astype(np.float64)).view(1, 1, 1, D)
            ref = F.scaled_dot_product_attention(
                qt, torch.from_numpy(kh).view(1, 1, -1, D),
                torch.from_numpy(vh).view(1, 1, -1, D), scale=sm)
            ref = ref.view(D).numpy()
            assert np.max(np.abs(o[b, h] - ref)) <= 1e-12 * max(1.0, np.abs(ref).max())


def test_block_permutation_and_value_scaling():
    rs = np.random.default_rng(4)
    S, D = 256, 64
    k = rs.standard_normal((1, S, 1, D)).astype(np.float16)
    v = rs.standard_normal((1, S, 1, D)).astype(np.float16)
    lens = np.array([S], np.int32)
    q = rs.standard_normal((1, 1, D)).astype(np.float16)
    c = oracle.quantize_cache(INT4, k, v, lens, 4)
    o = oracle.attention(c, q, lens, 0.125)
    order = [2, 0, 3, 1]
    cp = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in c.items()}
    for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        cp[key][0, 0] = c[key][0, 0][order]
    op = oracle.attention(cp, q, lens, 0.125)
    assert np.allclose(op, o, rtol=0, atol=1e-13)
    c2 = {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in c.items()}
    c2["v_scale"] *= 2
    assert np.array_equal(oracle.attention(c2, q, lens, 0.125), 2 * o)


def test_rows_subset_matches_full():
    w = wl.WORKLOADS[0]
    k = wl.prefill_batch(w, 0, 0)
    v = wl.prefill_batch(w, 0, 1)
    lens = wl.lengths(w)
    c = oracle.quantize_cache(w.scheme, k, v, lens, w.max_blocks)
    q = wl.query(w, 0)
    full = oracle.attention(c, q, lens, wl.softmax_scale(w))
    part = oracle.attention(c, q, lens, wl.softmax_scale(w), rows=(1, 2))
    assert np.array_equal(part[0, 1], full[0, 1]) and np.isnan(part[0, 0]).all()


def test_fp8_dequantization_matches_torch_float8():
    """FP8 K^ = value(code) * s with value() as torch's float8_e4m3fn decodes the same
    byte (an independent decoder), for every element of a quantized cache."""
    torch = pytest.importorskip("torch")
    w = wl.WORKLOADS[0]
    g = wl.rng(w, 12, 0, 0)
    x = wl.draw(g, "normal_outliers", (1, 130, 2, 64))
    lens = np.array([130], np.int32)
    c = oracle.quantize_cache(oracle.FP8_E4M3, x, x, lens, 3)
    for h in range(2):
        kh, _ = oracle.dequantize(c, 0, h, 130)
        codes = c["k_codes"][0, h].reshape(-1, 64)[:130]
        vals = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
        s = np.repeat(c["k_scale"][0, h].astype(np.float64), 64)[:130]
        ref = vals.to(torch.float64).numpy() * s[:, None]
        assert np.array_equal(kh, ref)
