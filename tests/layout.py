"""Readers of the packed cache layout documented in include/kivi.h, for tests.

Codes: one 1024-byte tile per 32-token group.  In a tile, 16-byte chunk ((u*8+q)*4+h)
holds the 8 code bytes of channel quarter h (channels 32h..32h+31) of token 4q+2u, then
of token 4q+2u+1; those 8 bytes are two 32-bit words (channels 32h..+15 and 32h+16..+31)
and in a word channel 4i+b sits in byte b at bits 2i, 2i+1.
Value pairs: per 32-token group, [channel group][token in group][scale, zero].
"""
import numpy as np

D, G = 128, 32


def code_pos(t, j):
    """(byte offset within the row, bit shift) of token t, channel j."""
    t, j = np.asarray(t), np.asarray(j)
    tt = t % 32
    q, u, t1 = tt // 4, (tt % 4) // 2, tt % 2
    h, w, c = j // 32, (j % 32) // 16, j % 16
    byte = (t // 32) * 1024 + ((u * 8 + q) * 4 + h) * 16 + t1 * 8 + w * 4 + (c % 4)
    return byte, 2 * (c // 4)


def unpack_codes(tiles):
    """[..., n_tiles, 1024] uint8 -> [..., n_tiles*32, 128] codes (token-major)."""
    tiles = np.asarray(tiles)
    lead = tiles.shape[:-2]
    flat = tiles.reshape(*lead, -1)
    T = tiles.shape[-2] * 32
    t = np.arange(T)[:, None]
    j = np.arange(D)[None, :]
    byte, shift = code_pos(t, j)
    return (flat[..., byte] >> shift.astype(np.uint8)) & 3


def value_pairs(v_sz):
    """[..., n_tiles, 4, 32, 2] -> [..., n_tiles*32, 4, 2] (token-major)."""
    v = np.asarray(v_sz)
    v = np.swapaxes(v, -3, -2)                      # [..., tiles, 32, 4, 2]
    return v.reshape(*v.shape[:-4], -1, v.shape[-2], 2)


def token_quarter_bytes(tiles_row, t, h):
    """The 8 code bytes of token t, channel quarter h, from one row's tiles [n, 1024]."""
    flat = np.asarray(tiles_row).reshape(-1)
    start, _ = code_pos(t, 32 * h)
    return flat[start:start + 8]
