"""The clamp-and-add rule by which the int4 and uint8 kernels take their codes, checked on
the CPU against the oracle over about 10^6 values (workload-like blocks, blocks of exact
ties, blocks far from zero).

The kernels take q = RN(x * RN(1 / s)) in binary32, clamp it to the code range, add
1.5 * 2^23 + 8 (int4) or 1.5 * 2^23 + zp (uint8) and read the code from the low bits of
the sum's bit pattern; a value whose clamped quotient lies within 2^-17 (int4) or
2^-20 |q| (uint8) of a rounding boundary is divided out instead. This emulates that rule
with numpy binary32 arithmetic and requires, for every value the rule does not send to
the division, the oracle's code: rint(x / s) clamped (int4 stored as c + 8; uint8 plus
the zero point, clamped to 0..255). The scales and zero points are taken as the oracle
defines them and compared with its own first. The GPU parity tests check the kernels
themselves on the workloads; this checks the rule on inputs built to sit on its
boundaries."""
import numpy as np

import oracle

f32 = np.float32


def _blocks(rs, B=4, S=256, H=4, D=128):
    """[B][S][H][D] fp16: rows of normal values, normal values with outliers, values on
    int4 rounding boundaries (multiples of absmax / 15), and values far from zero."""
    x = rs.standard_normal((B, S, H, D)).astype(np.float16)
    x[1] = (x[1] * np.where(rs.random((S, H, D)) < 0.001, 20, 1)).astype(np.float16)
    ties = rs.integers(-15, 16, (S, H, D)) * 0.5                 # absmax 7.5: s = 1
    ties[::64, :, 0] = 7.5
    x[2] = ties.astype(np.float16)
    x[3, :, 0] = (1000 + 0.5 * rs.integers(0, 2, (S, D))).astype(np.float16)
    x[3, :, 1] = rs.uniform(100, 110, (S, D)).astype(np.float16)
    x[3, :, 2] = rs.uniform(-20, -10, (S, D)).astype(np.float16)
    x[3, :, 3] = (rs.integers(-60, 61, (S, D)) * 0.25).astype(np.float16)
    return x


def _int4_rule(blk):
    """Codes (c + 8) and near flags of one int4 block (float16 [64][D])."""
    x = blk.astype(f32)
    a = f32(np.abs(x).max())
    s = f32(a / f32(7.5)) if a != 0 else f32(0)
    if s == 0:
        return s, np.full(x.shape, 8, np.uint32), np.zeros(x.shape, bool)
    r = f32(f32(1) / s)
    qc = np.clip((x * r).astype(f32), f32(-8), f32(7)).astype(f32)
    magic = f32(12582920.0)                       # 1.5 * 2^23 + 8
    t = (qc + magic).astype(f32)
    dist = np.abs((qc - (t - magic).astype(f32)).astype(f32))
    near = ~(dist < f32(0.5 - 2.0 ** -17))
    return s, t.view(np.uint32) & 0xF, near


def _uint8_rule(blk):
    """Scale, zero point, codes and near flags of one uint8 block (float16 [64][D])."""
    x = blk.astype(f32)
    mn, mx = f32(x.min()), f32(x.max())
    if mx == mn:
        if mx == 0:
            return f32(0), f32(0), np.zeros(x.shape, np.uint32), np.zeros(x.shape, bool)
        mn, mx = f32(min(mn, f32(0))), f32(max(mx, f32(0)))
    s = f32(f32(mx - mn) / f32(255))
    zp = f32(np.rint(f32(-mn / s)) + f32(0))
    r = f32(f32(1) / s)
    qc = np.clip((x * r).astype(f32), -zp, f32(255) - zp).astype(f32)
    magic = f32(f32(12582912.0) + zp)             # 1.5 * 2^23 + zp
    t = (qc + magic).astype(f32)
    dist = np.abs((qc - (t - magic).astype(f32)).astype(f32))
    # fma(|qc|, 2^-20, dist) rounded once: the product is exact, the binary64 sum of two
    # binary32 values of these magnitudes is exact, and one rounding to binary32 follows
    test = (np.abs(qc).astype(np.float64) * 2.0 ** -20 + dist.astype(np.float64)).astype(f32)
    near = ~(test < f32(0.5))
    return s, zp, t.view(np.uint32) & 0xFF, near


def test_int4_clamp_and_add_rule_matches_oracle():
    x = _blocks(np.random.default_rng(11))
    B, S, H, D = x.shape
    lens = np.full(B, S, np.int32)
    ref = oracle.quantize_cache(oracle.INT4_SYM, x, x, lens, S // 64)
    checked, flagged = 0, np.zeros(B, np.int64)
    for b in range(B):
        for h in range(H):
            for j in range(S // 64):
                blk = x[b, 64 * j:64 * (j + 1), h]
                s, code, near = _int4_rule(blk)
                assert s.view(np.uint32) == ref["k_scale"][b, h, j].view(np.uint32)
                packed = ref["k_codes"][b, h, j]                       # [64][D/2]
                want = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(64, D)
                assert np.array_equal(code[~near], want[~near].astype(np.uint32)), (b, h, j)
                checked += int((~near).sum())
                flagged[b] += int(near.sum())
    per_row = S * H * D
    assert checked > 400000
    assert flagged[0] < per_row // 1000 and flagged[1] < per_row // 1000  # rare on normal values
    assert flagged[2] > per_row // 4  # the planted ties are all sent to the division


def test_uint8_clamp_and_add_rule_matches_oracle():
    x = _blocks(np.random.default_rng(12))
    B, S, H, D = x.shape
    lens = np.full(B, S, np.int32)
    ref = oracle.quantize_cache(oracle.UINT8_ASYM, x, x, lens, S // 64)
    checked, flagged = 0, np.zeros(B, np.int64)
    zps = []
    for b in range(B):
        for h in range(H):
            for j in range(S // 64):
                blk = x[b, 64 * j:64 * (j + 1), h]
                s, zp, code, near = _uint8_rule(blk)
                assert s.view(np.uint32) == ref["k_scale"][b, h, j].view(np.uint32)
                assert zp.view(np.uint32) == ref["k_zero"][b, h, j].view(np.uint32)
                want = ref["k_codes"][b, h, j].astype(np.uint32)       # [64][D]
                assert np.array_equal(code[~near], want[~near]), (b, h, j)
                checked += int((~near).sum())
                flagged[b] += int(near.sum())
                zps.append(float(zp))
    assert min(zps) < -500000 and max(zps) > 255   # zero points outside the code range
    per_row = S * H * D
    assert checked > 400000
    assert flagged[0] < per_row // 100 and flagged[1] < per_row // 100
