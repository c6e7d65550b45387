"""The stored order of the int4 cache, as host-side numpy converters.

The library keeps uint8 codes in natural order ([token][channel] per 64-token block)
and int4 codes in the operand order of the gfx950 matrix cores (kvq_device.h):

  each block region (K or V of one block of one row, 64 tokens x D channels, 32*D
  bytes) is 64 lanes x F = D/8 dwords; dword f of lane l sits at byte
  ((f // 4) * 64 + l) * 16 + (f % 4) * 4 and holds 8 offset-binary nibbles (code + 8),
  nibble q in bits 4q..4q+3 (even q in the low nibble of byte q // 2):
    K: f = nt * (D/32) + ks; nibble q = channel 32*ks + 8*(l//16) + q of token 16*nt + l%16
    V: f = 2 * nt + ks;      nibble q = token 32*ks + 8*(l//16) + q of channel 16*nt + l%16

Natural order packs channel 2k of a token in the low nibble of byte k. These helpers
only move nibbles (reading a cache back, or writing test patterns into it); no part
of the computation runs here.
"""
import numpy as np

BLOCK = 64


def _unpack(b):
    """uint8 [..., n] -> nibbles [..., n, 2] (low nibble first)."""
    return np.stack([b & 0xF, b >> 4], axis=-1)


def _pack(n):
    """nibbles [..., n, 2] -> uint8 [..., n]."""
    return (n[..., 0] | (n[..., 1] << 4)).astype(np.uint8)


def _stored_to_fl(stored, D):
    """[..., 64, D/2] stored bytes -> nibbles [..., F, 64 lanes, 8]: dword f of lane l."""
    F = D // 8
    lead = stored.shape[:-2]
    # byte ((f//4)*64 + l)*16 + (f%4)*4 + q//2  ->  [f//4][l][f%4][q]
    nib = _unpack(stored.reshape(lead + (F // 4, 64, 4, 4))).reshape(lead + (F // 4, 64, 4, 8))
    n = len(lead)
    nib = nib.transpose(tuple(range(n)) + (n, n + 2, n + 1, n + 3))   # [g][r][l][q]
    return nib.reshape(lead + (F, 64, 8))


def _fl_to_stored(fl, D):
    F = D // 8
    lead = fl.shape[:-3]
    n = len(lead)
    nib = fl.reshape(lead + (F // 4, 4, 64, 8))
    nib = nib.transpose(tuple(range(n)) + (n, n + 2, n + 1, n + 3))   # [g][l][r][q]
    return _pack(nib.reshape(lead + (F // 4, 64, 4, 4, 2))).reshape(lead + (BLOCK, D // 2))


# Axis orders. K: dword f = nt*(D/32) + ks and lane l = 16*lh + ll give the 5-d index
# [nt][ks][lh][ll][q]; token 16*nt + ll, channel 32*ks + 8*lh + q, so natural order
# [token][channel] = [nt][ll][ks][lh][q]. V: f = 2*nt + ks gives [nt][ks][lh][ll][q];
# token 32*ks + 8*lh + q, channel 16*nt + ll, so natural order = [ks][lh][q][nt][ll].
_K_TO_NAT = (0, 3, 1, 2, 4)
_V_TO_NAT = (1, 2, 4, 0, 3)


def _split_shape(which, D):
    return (4, D // 32, 4, 16, 8) if which == "k" else (D // 16, 2, 4, 16, 8)


def int4_to_natural(stored, which):
    """stored: uint8 [..., 64, D/2] int4 codes as the library keeps them (each trailing
    [64, D/2] is one block region); which: 'k' or 'v'. Returns the same codes in
    natural order."""
    stored = np.asarray(stored, np.uint8)
    D = stored.shape[-1] * 2
    lead = stored.shape[:-2]
    n = len(lead)
    fl = _stored_to_fl(stored, D).reshape(lead + _split_shape(which, D))
    perm = _K_TO_NAT if which == "k" else _V_TO_NAT
    nat = fl.transpose(tuple(range(n)) + tuple(n + p for p in perm))
    return _pack(nat.reshape(lead + (BLOCK, D // 2, 2)))


def int4_from_natural(natural, which):
    """Inverse of int4_to_natural."""
    natural = np.asarray(natural, np.uint8)
    D = natural.shape[-1] * 2
    lead = natural.shape[:-2]
    n = len(lead)
    perm = _K_TO_NAT if which == "k" else _V_TO_NAT
    split = _split_shape(which, D)
    nat = _unpack(natural).reshape(lead + tuple(split[p] for p in perm))
    inv = tuple(int(i) for i in np.argsort(perm))
    fl = nat.transpose(tuple(range(n)) + tuple(n + p for p in inv))
    return _fl_to_stored(np.ascontiguousarray(fl).reshape(lead + (D // 8, 64, 8)), D)
