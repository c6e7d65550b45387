"""Pins of the oracle's quantizer against values the pages and arithmetic fix.

The quantizer is an encoding, so the oracle must reproduce it bit for bit: these tests
hold it to hand-worked examples (tests/golden/quant_examples.txt), to the fp16 format
definition, to closed-form invariants and to the round-trip error bound.
"""
import numpy as np
import pytest

import oracle
from decode_attention_block_amd import workloads as wl
from golden_io import read_sections

INT4, UINT8 = oracle.INT4_SYM, oracle.UINT8_ASYM


def f32bits(x):
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def unpack_int4(row_bytes):
    """Signed int4 codes from packed bytes: channel 2k = low nibble of byte k, each
    nibble the offset-binary value code + 8."""
    b = np.asarray(row_bytes, dtype=np.uint8)
    out = np.empty(2 * b.size, np.int64)
    out[0::2] = (b & 0x0F).astype(np.int64) - 8
    out[1::2] = (b >> 4).astype(np.int64) - 8
    return out


def single_block(values, D=64, fill=None, ntok=1):
    """float16 [1][64][1][D]: token 0 carries the example, other tokens zero."""
    x = np.zeros((1, 64, 1, D), np.float16)
    if fill is not None:
        x[0, :ntok, 0, :] = np.float16(fill)
    else:
        x[0, 0, 0, :len(values)] = np.asarray(values, np.float16)
    return x


def test_fp16_decoder_matches_format_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_float(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("name", list(read_sections("quant_examples.txt")))
def test_golden_example(name):
    ex = read_sections("quant_examples.txt")[name]
    scheme = {"int4": INT4, "uint8": UINT8, "fp8": oracle.FP8_E4M3}[ex["scheme"]]
    fill = float(ex["fill"]) if "fill" in ex else None
    xs = [float(t) for t in ex["x"].split()] if "x" in ex else []
    x = single_block(xs, fill=fill)
    c = oracle.quantize_cache(scheme, x, x.copy(), np.array([1], np.int32), 1)
    for which in ("k", "v"):
        assert f32bits(c[which + "_scale"][0, 0, 0]) == int(ex["scale"], 16), which
        assert f32bits(c[which + "_zero"][0, 0, 0]) == int(ex["zero"], 16), which
        row = c[which + "_codes"][0, 0, 0, 0]
        codes = unpack_int4(row) if scheme == INT4 else row.astype(np.int64)
        want = [int(t) for t in ex["codes"].split()]
        if fill is not None:
            assert (codes == want[0]).all()
        else:
            assert list(codes[:len(want)]) == want
            # channels holding 0.0 take the code of zero: 0 (int4, FP8) or zp (uint8)
            zero_code = int(c[which + "_zero"][0, 0, 0]) if scheme == UINT8 else 0
            assert (codes[len(want):] == zero_code).all()
        if "packed" in ex:
            packed = [int(t, 16) for t in ex["packed"].split()]
            assert list(row[:len(packed)]) == packed
        # tokens 1..63 are padding: code byte 0
        assert not c[which + "_codes"][0, 0, 0, 1:].any()


@pytest.mark.parametrize("scheme", [INT4, UINT8])
def test_padding_and_untouched_blocks(scheme):
    rs = np.random.default_rng(1)
    B, S, H, D, MB = 2, 200, 3, 64, 5
    x = rs.standard_normal((B, S, H, D)).astype(np.float16)
    lens = np.array([130, 64], np.int32)
    c = oracle.empty_cache(scheme, B, H, D, MB)
    for k in ("k_codes", "v_codes"):
        c[k][:] = 0xAA
    for k in ("k_scale", "v_scale", "k_zero", "v_zero"):
        c[k][:] = -7.0
    oracle.quantize_cache(scheme, x, x, lens, MB, cache=c)
    # row b=0: blocks 0,1 full, block 2 holds 2 tokens; blocks 3,4 untouched
    assert not c["k_codes"][0, :, 2, 2:].any()
    assert (c["k_codes"][0, :, 3:] == 0xAA).all() and (c["k_scale"][0, :, 3:] == -7).all()
    assert (c["k_codes"][1, :, 1:] == 0xAA).all()
    assert (c["k_scale"][0, :, :3] > 0).all()


def _blocks(x, lens):
    """Yields (b, h, j, block values float32 [ntok][D])."""
    B, S, H, D = x.shape
    for b in range(B):
        for h in range(H):
            for j in range((lens[b] + 63) // 64):
                t1 = min(lens[b], 64 * j + 64)
                yield b, h, j, x[b, 64 * j:t1, h, :].astype(np.float32)


DISTS = ["normal_outliers", "normal0.5", "student_t3_half"]


@pytest.mark.parametrize("dist", DISTS)
@pytest.mark.parametrize("scheme", [INT4, UINT8])
def test_roundtrip_bound_and_invariants(scheme, dist):
    """|x - dequant(code(x))| <= s/2 for every element (the clamp never bites for these
    scales), the scale is the stated binary32 quotient, and the extreme elements map to
    the extreme codes."""
    w = wl.WORKLOADS[1]
    g = wl.rng(w, 99, 0, 0)
    B, S, H, D = 2, 300, 4, 128
    x = wl.draw(g, dist, (B, S, H, D))
    lens = np.array([300, 171], np.int32)
    c = oracle.quantize_cache(scheme, x, x, lens, 5)
    for b, h, j, blk in _blocks(x, lens):
        s = c["k_scale"][b, h, j]
        kh, _ = oracle.dequantize(c, b, h, lens[b])
        err = np.abs(blk.astype(np.float64) - kh[64 * j:64 * j + blk.shape[0]])
        assert err.max() <= 0.5 * float(s) * (1 + 1e-5)
        if scheme == INT4:
            a = np.abs(blk).max()
            assert f32bits(s) == f32bits(np.float32(a) / np.float32(7.5))
            codes = unpack_int4(c["k_codes"][b, h, j, :blk.shape[0]].ravel())
            codes = codes.reshape(blk.shape)
            assert (codes[blk == a] == 7).all()
            assert set(codes[blk == -a].tolist()) <= {-7, -8}
            assert codes.min() >= -8 and codes.max() <= 7
        else:
            codes = c["k_codes"][b, h, j, :blk.shape[0]].astype(np.int64)
            mn, mx = blk.min(), blk.max()
            assert f32bits(s) == f32bits(np.float32(mx - mn) / np.float32(255))
            assert (codes[blk == mn] == 0).all()
            assert set(codes[blk == mx].tolist()) <= {254, 255}


@pytest.mark.parametrize("scheme", [INT4, UINT8, oracle.FP8_E4M3])
def test_token_permutation_within_block(scheme):
    rs = np.random.default_rng(5)
    x = rs.standard_normal((1, 64, 1, 64)).astype(np.float16)
    perm = rs.permutation(64)
    xp = x[:, perm].copy()
    one = np.array([64], np.int32)
    c1 = oracle.quantize_cache(scheme, x, x, one, 1)
    c2 = oracle.quantize_cache(scheme, xp, xp, one, 1)
    assert c1["k_scale"][0, 0, 0] == c2["k_scale"][0, 0, 0]
    assert c1["k_zero"][0, 0, 0] == c2["k_zero"][0, 0, 0]
    assert np.array_equal(c1["k_codes"][0, 0, 0][perm], c2["k_codes"][0, 0, 0])


@pytest.mark.parametrize("scheme", [INT4, UINT8, oracle.FP8_E4M3])
def test_append_is_requantized_tail(scheme):
    """Appending token by token (oracle_append) ends in the same cache as quantizing the
    whole history at once, at every length crossed (0->1, 63->64, 64->65, ...)."""
    w = wl.WORKLOADS[0]
    B, H, D = 2, 2, 64
    S = 140
    g = wl.rng(w, 7, 0, 0)
    k = wl.draw(g, "normal_outliers", (B, S, H, D))
    v = wl.draw(g, "normal0.5", (B, S, H, D))
    MB = 3
    start = np.array([0, 61], np.int32)
    c = oracle.quantize_cache(scheme, k, v, start, MB)
    lens = start.copy()
    while lens.max() < S:
        lens = np.minimum(lens + 1, S)
        oracle.append(c, k, v, lens)
        ref = oracle.quantize_cache(scheme, k, v, lens, MB)
        for key in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
            assert np.array_equal(c[key], ref[key]), (key, lens)


# ---- FP8 E4M3 (pinned against torch's own float8_e4m3fn conversions) -------------------
FP8 = oracle.FP8_E4M3


def test_e4m3_values_match_torch_float8_on_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    finite = (codes & 0x7F) != 0x7F
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))
    # the format's landmarks: 2^-9 (smallest subnormal), 2^-6 (smallest normal), 1, 448
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0


def test_e4m3_code_matches_torch_rounding():
    """Nearest value, ties to even, sign kept: torch's float32 -> float8_e4m3fn cast on
    random values over the whole range, every exact value, and every exact midpoint."""
    torch = pytest.importorskip("torch")
    rs = np.random.default_rng(11)
    vals = np.concatenate([
        rs.standard_normal(20000).astype(np.float32) * np.float32(30),
        (rs.uniform(-1, 1, 20000) * 2.0 ** rs.integers(-14, 9, 20000)).astype(np.float32),
        np.float32([0.0, -0.0, 463.9, -463.0, 447.99, 1e-30, -1e-30]),
    ])
    finite = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = ((finite[1:] + finite[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([vals, finite.astype(np.float32), mids, -mids])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_code(vals), ref)


def test_e4m3_code_saturates_to_the_largest_finite_value():
    # the nearest finite value beyond 448 is 448 (torch's cast gives NaN from 480 on)
    big = np.float32([448.0, 464.0, 480.0, 1000.0, 3.0e38, -500.0])
    assert oracle.e4m3_code(big).tolist() == [0x7E] * 5 + [0xFE]


def test_fp8_block_scale_and_exact_grid():
    """A block whose values are exactly s times E4M3 values (s = absmax / 448 a power of
    two) is coded to those values; the scale is absmax / 448 in binary32."""
    rs = np.random.default_rng(2)
    codes = rs.integers(0, 0x7F, size=(64, 64)).astype(np.uint8)
    codes[0, 0] = 0x7E                                   # the block's absmax: 448 * s
    signs = rs.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes = codes | signs
    s = 2.0 ** -6
    vals = (oracle.e4m3_value(codes) * s).astype(np.float16)
    assert np.array_equal(vals.astype(np.float64), oracle.e4m3_value(codes) * s)  # exact
    x = vals.reshape(1, 64, 1, 64)
    c = oracle.quantize_cache(FP8, x, x, np.array([64], np.int32), 1)
    assert c["k_scale"][0, 0, 0] == np.float32(s)
    got = c["k_codes"][0, 0, 0]
    # -0 values (a zero code with the sign bit) keep their sign
    assert np.array_equal(got, codes)


@pytest.mark.parametrize("dist", DISTS)
def test_fp8_roundtrip_bound(dist):
    """Every element is within half a step of its E4M3 grid after scaling: |x/s - v| <=
    half the gap to the neighbouring values (relative 2^-4, absolute 2^-10 below 2^-6)."""
    w = wl.WORKLOADS[1]
    g = wl.rng(w, 98, 0, 0)
    B, S, H, D = 1, 200, 2, 64
    x = wl.draw(g, dist, (B, S, H, D))
    lens = np.array([200], np.int32)
    c = oracle.quantize_cache(FP8, x, x, lens, 4)
    for b, h, j, blk in _blocks(x, lens):
        s = np.float64(c["k_scale"][b, h, j])
        a = np.abs(blk).max()
        assert f32bits(c["k_scale"][b, h, j]) == f32bits(np.float32(a) / np.float32(448))
        kh, _ = oracle.dequantize(c, b, h, lens[b])
        q = blk.astype(np.float64) / s
        v = kh[64 * j:64 * j + blk.shape[0]] / s
        bound = np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
        assert (np.abs(q - v) <= bound).all()
