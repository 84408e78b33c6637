"""The 2-bit packed tile layout against bytes worked out by hand (tests/golden/layout_tiles.txt).

The pages fix only that four 2-bit codes share a byte (record kv-efficiency/kivi-2bit-llama2-13b-
mha-4k, "KV bytes basis"); the tile order is this library's own, stated in include/kivi.h.  The
fixture's offsets and bytes were derived by hand from that prose, so they pin both the oracle's
packing and tests/layout.py (the reader the other tests use) independently of either.
"""
import numpy as np
import pytest

import layout
from golden_io import layout_tiles
from oracle import ref

D = 128
ONEHOT = [e for e in layout_tiles() if e[0] == "onehot"]
PATTERN = [e for e in layout_tiles() if e[0] == "pattern"]
F16 = {0: 0x0000, 1: 0x3C00, 2: 0x4000, 3: 0x4200}


def pattern_code(t, j):
    """The fixture's input: code(t, j) = (t + t//4 + j + j//4 + j//16) mod 4."""
    return (t + t // 4 + j + j // 4 + j // 16) % 4


def _quantized_row(src, kind):
    rc = ref.RefCache(1, 1, D, 32, 128, src.shape[1])
    (rc.quantize_k if kind == "key" else rc.quantize_v)(src, src.shape[1])
    codes = rc.k_codes if kind == "key" else rc.v_codes
    pairs = rc.k_sz if kind == "key" else rc.v_sz
    return codes[0].reshape(-1), pairs


def test_fixture_covers_every_index_component():
    keys = [e for e in ONEHOT if e[1] == "key"]
    vals = [e for e in ONEHOT if e[1] == "value"]
    # keys: both tiles, both token halves, every word slot k, both word halves, every byte b, every i
    assert {t // 32 for _, _, t, _, _, _ in keys} == {0, 1}
    assert {(t % 32) // 16 for _, _, t, _, _, _ in keys} == {0, 1}
    assert {(j // 16) % 4 for _, _, _, j, _, _ in keys} == {0, 1, 2, 3}
    assert {j // 64 for _, _, _, j, _, _ in keys} == {0, 1}
    assert {j % 4 for _, _, _, j, _, _ in keys} == {0, 1, 2, 3}
    assert {(j % 16) // 4 for _, _, _, j, _, _ in keys} == {0, 1, 2, 3}
    # values: both tiles, every 8-token block, both 4-token halves, every p and e, every shift
    assert {t // 32 for _, _, t, _, _, _ in vals} == {0, 1}
    assert {(t % 32) // 8 for _, _, t, _, _, _ in vals} == {0, 1, 2, 3}
    assert {(t % 8) // 4 for _, _, t, _, _, _ in vals} == {0, 1}
    assert {(j // 16) // 2 for _, _, _, j, _, _ in vals} == {0, 1, 2, 3}
    assert {(j // 16) % 2 for _, _, _, j, _, _ in vals} == {0, 1}
    assert {t % 4 for _, _, t, _, _, _ in vals} == {0, 1, 2, 3}


@pytest.mark.parametrize("entry", ONEHOT, ids=lambda e: f"{e[1]}-t{e[2]}-j{e[3]}")
def test_oracle_one_hot_tile(entry):
    _, kind, t, j, offset, shift = entry
    src = np.zeros((1, 64, D), np.uint16)
    src[0, t, j] = 0x4200                        # 3.0
    codes, _ = _quantized_row(src, kind)
    nz = np.flatnonzero(codes)
    assert nz.tolist() == [offset], f"nonzero bytes at {nz.tolist()}, hand-worked {offset}"
    assert codes[offset] == 3 << shift


@pytest.mark.parametrize("entry", ONEHOT, ids=lambda e: f"{e[1]}-t{e[2]}-j{e[3]}")
def test_layout_reader_one_hot(entry):
    _, kind, t, j, offset, shift = entry
    pos = layout.key_code_pos if kind == "key" else layout.value_code_pos
    byte, sh = pos(t, j)
    assert (int(byte), int(sh)) == (offset, shift)


@pytest.mark.parametrize("kind", ["key", "value"])
def test_oracle_pattern_tile(kind):
    t = np.arange(32)[:, None]
    j = np.arange(D)[None, :]
    src = np.vectorize(F16.get)(pattern_code(t, j)).astype(np.uint16)[None]
    codes, pairs = _quantized_row(src, kind)
    assert np.all(pairs[..., 0] == 0x3C00) and np.all(pairs[..., 1] == 0)   # scale 1, zero 0
    for _, k, offset, byte in PATTERN:
        if k == kind:
            assert codes[offset] == byte, f"{kind} byte {offset}: {codes[offset]:#04x}, hand-worked {byte:#04x}"


@pytest.mark.parametrize("kind", ["key", "value"])
def test_layout_reader_pattern_bytes(kind):
    """Each hand-worked byte, read back through tests/layout.py, gives the input's codes."""
    pos = layout.key_code_pos if kind == "key" else layout.value_code_pos
    t = np.arange(32)[:, None].repeat(D, 1)
    j = np.arange(D)[None, :].repeat(32, 0)
    byte, sh = pos(t, j)
    checked = 0
    for _, k, offset, value in PATTERN:
        if k != kind:
            continue
        at = np.argwhere(byte == offset)
        assert len(at) == 4, f"the reader puts {len(at)} codes in byte {offset}"
        for tt, jj in at:
            assert (value >> int(sh[tt, jj])) & 3 == pattern_code(tt, jj)
            checked += 1
    assert checked == 32
