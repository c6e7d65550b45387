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
import functools

import numpy as np

BLOCK = 64


@functools.lru_cache(maxsize=None)
def _maps(D):
    """For one region: stored byte, nibble-in-byte and natural (token, channel) of every
    stored nibble, each shaped [64 lanes][F dwords][8 nibbles]."""
    F = D // 8
    ks_k = D // 32
    lane = np.arange(64).reshape(64, 1, 1)
    f = np.arange(F).reshape(1, F, 1)
    q = np.arange(8).reshape(1, 1, 8)
    byte = ((f // 4) * 64 + lane) * 16 + (f % 4) * 4 + q // 2
    nib = np.broadcast_to(q % 2, byte.shape)
    t_k = np.broadcast_to(16 * (f // ks_k) + lane % 16, byte.shape)
    d_k = 32 * (f % ks_k) + 8 * (lane // 16) + q
    d_v = np.broadcast_to(16 * (f // 2) + lane % 16, byte.shape)
    t_v = 32 * (f % 2) + 8 * (lane // 16) + q
    return byte, nib, (t_k, d_k), (t_v, d_v)


def int4_to_natural(stored, which):
    """stored: uint8 [..., 64, D/2] int4 codes as the library keeps them (each trailing
    [64, D/2] is one block region); which: 'k' or 'v'. Returns the same codes in
    natural order."""
    stored = np.asarray(stored, np.uint8)
    D = stored.shape[-1] * 2
    lead = stored.shape[:-2]
    region = stored.reshape(lead + (32 * D,))
    byte, nib, kmap, vmap = _maps(D)
    t, d = kmap if which == "k" else vmap
    nibbles = (region[..., byte] >> (4 * nib).astype(np.uint8)) & 0xF
    nat = np.zeros(lead + (BLOCK, D), np.uint8)
    nat[..., t, d] = nibbles
    return (nat[..., 0::2] | (nat[..., 1::2] << 4)).astype(np.uint8)


def int4_from_natural(natural, which):
    """Inverse of int4_to_natural."""
    natural = np.asarray(natural, np.uint8)
    D = natural.shape[-1] * 2
    lead = natural.shape[:-2]
    nat = np.empty(lead + (BLOCK, D), np.uint8)
    nat[..., 0::2] = natural & 0xF
    nat[..., 1::2] = natural >> 4
    byte, nib, kmap, vmap = _maps(D)
    t, d = kmap if which == "k" else vmap
    nibbles = nat[..., t, d]                      # [..., 64, F, 8]
    region = np.zeros(lead + (32 * D,), np.uint8)
    region[..., byte[..., 0::2]] = nibbles[..., 0::2] | (nibbles[..., 1::2] << 4)
    return region.reshape(lead + (BLOCK, D // 2))
