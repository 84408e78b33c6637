"""Readers of the packed cache layout documented in include/kivi.h, for tests.

Codes: one 1024-byte tile per 32-token group.
Key tiles: a little-endian 32-bit word holds the 16 channels 16w..16w+15 of one token,
channel 16w + 4i + b in byte b at bits 2i, 2i+1; 16-byte chunk (16k+n) holds words k and
4+k of token n, then of token 16+n.
Value tiles: a byte holds one channel's codes for four consecutive tokens, token 4a+i at
bits 2i, 2i+1; 16-byte chunk (16k+n) covers tokens 8k..8k+7 and its byte 4p+2h+e holds
channel n+16(2p+e) for tokens 8k+4h..8k+4h+3.
Value pairs: [token][channel group][scale, zero].
"""
import numpy as np

D = 128          # codes are stored in 32-token tiles whatever the group size is


def value_code_pos(t, j):
    """(byte offset within the row, bit shift) of value token t, channel j."""
    t, j = np.asarray(t), np.asarray(j)
    tt = t % 32
    v, n = j // 16, j % 16
    chunk = (tt // 8) * 16 + n
    byte = (t // 32) * 1024 + chunk * 16 + (v // 2) * 4 + ((tt % 8) // 4) * 2 + v % 2
    return byte, 2 * (tt % 4)


def key_code_pos(t, j):
    """(byte offset within the row, bit shift) of key token t, channel j."""
    t, j = np.asarray(t), np.asarray(j)
    tt = t % 32
    w, c = j // 16, j % 16
    chunk = (w % 4) * 16 + tt % 16
    byte = (t // 32) * 1024 + chunk * 16 + (tt // 16) * 8 + (w // 4) * 4 + (c % 4)
    return byte, 2 * (c // 4)


def _unpack(tiles, pos):
    tiles = np.asarray(tiles)
    lead = tiles.shape[:-2]
    flat = tiles.reshape(*lead, -1)
    T = tiles.shape[-2] * 32
    t = np.arange(T)[:, None]
    j = np.arange(D)[None, :]
    byte, shift = pos(t, j)
    return (flat[..., byte] >> shift.astype(np.uint8)) & 3


def unpack_value_codes(tiles):
    """[..., n_tiles, 1024] uint8 -> [..., n_tiles*32, 128] codes (token-major)."""
    return _unpack(tiles, value_code_pos)


def unpack_key_codes(tiles):
    """[..., n_tiles, 1024] uint8 -> [..., n_tiles*32, 128] codes (token-major)."""
    return _unpack(tiles, key_code_pos)


def value_pairs(v_sz):
    """[..., tokens, D/G, 2] value pairs (stored token-major already)."""
    return np.asarray(v_sz)


def key_word_bytes(tiles_row, t, w):
    """The 4 key-code bytes of word w (channels 16w..16w+15) of token t, from one row's tiles."""
    flat = np.asarray(tiles_row).reshape(-1)
    start, _ = key_code_pos(t, 16 * w)
    return flat[start:start + 4]
