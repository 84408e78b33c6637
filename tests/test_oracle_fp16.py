"""Pins of the oracle's own binary32 -> binary16 rounding (RNE, subnormals kept).

Checked exhaustively against torch's CPU conversion (an IEEE round-to-nearest-even
library routine) over every positive binary32 value below the overflow threshold,
on a strided sample of negatives, and against numpy on a second sample.
"""
import numpy as np
import pytest
import torch

from oracle import ref


def _torch_f16_bits(x):
    return torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.slow
def test_f32_to_f16_exhaustive_positive():
    # all positive finite binary32 whose biased exponent is <= 142 (|x| < 65536): this
    # covers zero, every fp16 subnormal and normal, and the round-to-infinity edge
    chunk = 1 << 24
    top = 143 << 23
    for start in range(0, top, chunk):
        bits = np.arange(start, min(start + chunk, top), dtype=np.uint32)
        x = bits.view(np.float32)
        got = ref.f32_to_f16(x)
        want = _torch_f16_bits(x)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (hex(int(bits[bad[0]])), hex(int(got[bad[0]])), hex(int(want[bad[0]])))


def test_f32_to_f16_negative_sample():
    bits = (np.arange(0, 143 << 23, 4099, dtype=np.uint64).astype(np.uint32)) | np.uint32(0x80000000)
    x = bits.view(np.float32)
    assert np.array_equal(ref.f32_to_f16(x), _torch_f16_bits(x))


def test_f32_to_f16_numpy_sample():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(2_000_000) * rng.choice([1e-7, 1e-5, 1e-2, 1, 1e3, 1e4], 2_000_000)).astype(np.float32)
    x = x[np.abs(x) < 65504]
    assert np.array_equal(ref.f32_to_f16(x), x.astype(np.float16).view(np.uint16))


def test_f32_to_f16_specials():
    vals = np.array([np.inf, -np.inf, 65504.0, 65519.996, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
                     1.5 * 2.0 ** -25, 2.0 ** -26, -0.0, 0.0], np.float32)
    got = ref.f32_to_f16(vals)
    assert [hex(v) for v in got] == [hex(v) for v in _torch_f16_bits(vals)]
    assert got[0] == 0x7C00 and got[4] == 0x7C00 and got[2] == 0x7BFF
    assert got[7] == 0x0001 and got[8] == 0x0000 and got[9] == 0x0001 and got[11] == 0x8000
    nan = ref.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_f16_to_f32_every_pattern():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([ref.f16_to_f32_scalar(b) for b in bits[::7]], np.float32)
    w = want[::7]
    finite = np.isfinite(w)
    assert np.array_equal(got[finite].view(np.uint32), w[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(w))
