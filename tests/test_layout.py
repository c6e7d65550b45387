"""The host-side description of the int4 storage order (decode_attention_block_amd.layout)
against the formula in its docstring, worked by hand for single nibbles."""
import numpy as np
import pytest

from decode_attention_block_amd import layout


def one_hot_natural(D, t, d, value=0xB):
    nat = np.zeros((64, D // 2), np.uint8)
    nat[t, d // 2] = value << (4 * (d % 2))
    return nat


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("which", ["k", "v"])
def test_round_trip(D, which):
    rs = np.random.default_rng(0)
    nat = rs.integers(0, 256, (2, 3, 64, D // 2), dtype=np.uint8)
    st = layout.int4_from_natural(nat, which)
    assert np.array_equal(layout.int4_to_natural(st, which), nat)
    assert sorted(st.ravel().tolist()) != [] and st.shape == nat.shape


def test_k_nibble_position_by_hand():
    # D=128, token 37, channel 77: nt = 2, lane%16 = 5; ks = 2, lane//16 = (77-64)//8 = 1,
    # q = 13 - 8 = 5 -> lane 21, f = 2*4 + 2 = 10 -> byte ((10//4)*64 + 21)*16 + (10%4)*4 + 2
    # = (128 + 21)*16 + 8 + 2 = 2394, high nibble (q odd).
    st = layout.int4_from_natural(one_hot_natural(128, 37, 77), "k").ravel()
    assert np.flatnonzero(st).tolist() == [2394] and st[2394] == 0xB0


def test_v_nibble_position_by_hand():
    # D=128, token 45, channel 100: nt = 6, lane%16 = 4; ks = 1, lane//16 = (45-32)//8 = 1,
    # q = 5 -> lane 20, f = 2*6 + 1 = 13 -> byte ((13//4)*64 + 20)*16 + (13%4)*4 + 2
    # = (192 + 20)*16 + 4 + 2 = 3398, high nibble.
    st = layout.int4_from_natural(one_hot_natural(128, 45, 100), "v").ravel()
    assert np.flatnonzero(st).tolist() == [3398] and st[3398] == 0xB0


def test_v_first_dword_holds_eight_tokens_of_channel_zero():
    D = 64
    nat = np.zeros((64, D // 2), np.uint8)
    for t in range(8):
        nat[t, 0] = t + 1            # channel 0 of tokens 0..7 (low nibble)
    st = layout.int4_from_natural(nat, "v").ravel()
    assert st[:4].tolist() == [0x21, 0x43, 0x65, 0x87]


def _brute_force_to_natural(region, D, which):
    """One nibble at a time, straight from the storage formula: dword f of lane l at
    byte ((f//4)*64 + l)*16 + (f%4)*4, nibble q in bits 4q..4q+3 of that dword."""
    nat = np.zeros((64, D), np.uint8)
    F, ks_k = D // 8, D // 32
    for lane in range(64):
        for f in range(F):
            for q in range(8):
                byte = ((f // 4) * 64 + lane) * 16 + (f % 4) * 4 + q // 2
                val = (int(region[byte]) >> (4 * (q % 2))) & 0xF
                if which == "k":
                    t, d = 16 * (f // ks_k) + lane % 16, 32 * (f % ks_k) + 8 * (lane // 16) + q
                else:
                    t, d = 32 * (f % 2) + 8 * (lane // 16) + q, 16 * (f // 2) + lane % 16
                nat[t, d] = val
    return nat[:, 0::2] | (nat[:, 1::2] << 4)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("which", ["k", "v"])
def test_converters_match_nibble_by_nibble_formula(D, which):
    rs = np.random.default_rng(D + len(which))
    st = rs.integers(0, 256, (2, 64, D // 2), dtype=np.uint8)
    nat = layout.int4_to_natural(st, which)
    for i in range(2):
        assert np.array_equal(nat[i], _brute_force_to_natural(st[i].ravel(), D, which))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("which", ["k", "v"])
def test_c_abi_converters_match_the_stored_order(D, which):
    """kvq_int4_to_natural / kvq_int4_from_natural (host C ABI) give the converters above
    on several regions of random bytes, and invert each other."""
    import ctypes

    import decode_attention_block_amd as kvq
    L = kvq.load_library()
    n = 5
    rs = np.random.default_rng(D + (which == "v"))
    stored = rs.integers(0, 256, size=(n, 64, D // 2), dtype=np.uint8)
    nat = np.empty_like(stored)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.kvq_int4_to_natural(ptr(stored), ptr(nat), D, which == "v", n) == 0
    assert np.array_equal(nat, layout.int4_to_natural(stored, which))
    back = np.empty_like(stored)
    assert L.kvq_int4_from_natural(ptr(nat), ptr(back), D, which == "v", n) == 0
    assert np.array_equal(back, stored)
    assert L.kvq_int4_to_natural(ptr(stored), ptr(nat), 96, 0, 1) == -2
    assert L.kvq_int4_to_natural(None, ptr(nat), D, 0, 1) == -1
