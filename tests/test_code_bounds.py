"""The G = 32 prefill quantizers' code rule on the fp16 inputs themselves, checked against the
correctly rounded division it replaces.

For a group with minimum mn (fp16) and fp16 scale s, the code of x is min(rint(fl(d / s)), 3),
d = fl(x - mn).  The prefill quantizers compare x with three fp16 bounds instead, so that a
pair of codes is three packed fp16 subtractions (the sign of V - x) and no conversion:
  V1 = the largest fp16 at or below mn + s/2 + ulp(s/2)/2,
  V2 = the largest fp16 below      mn + 3s/2 - ulp(3s/2)/2,
  V3 = the largest fp16 at or below mn + 5s/2 + ulp(5s/2)/2,
(ulp of the binary32 value; the sums in binary64, rounded to fp16 through binary32 and moved
one step down where that overshoots), and code = [x > V1] + [x > V2] + [x > V3].
The rule is restated here in numpy and compared, for every positive finite fp16 scale and a
spread of minima (every 37th fp16 value and the special ones), with the division at each
bound, one fp16 step either side of it, and at random x of the group's range.  The same
comparison over all 63,488 finite fp16 minima (2.0e9 (mn, s) pairs) found no difference; it
takes about five minutes and is not repeated here.  The GPU quantizers' codes are compared
bit for bit with the oracle's by the GPU tests."""
import numpy as np

S16 = np.arange(1, 0x7C00, dtype=np.uint16)
S = S16.view(np.float16).astype(np.float32)


def _half_ulp(v):
    _, e = np.frexp(v.astype(np.float64))
    return np.ldexp(1.0, (e - 25).astype(np.int32))


def _prev16(h):
    h = h.astype(np.int32)
    r = np.where((h & 0x8000) != 0, h + 1, h - 1)
    return np.where((h & 0x7FFF) == 0, 0x8001, r).astype(np.uint16)


def _next16(h):
    h = h.astype(np.int32)
    r = np.where((h & 0x8000) != 0, h - 1, h + 1)
    r = np.where(h == 0x8000, 1, r)
    return np.where(h == 0x8001, 0, r).astype(np.uint16)


def _floor16(x, strict):
    with np.errstate(over="ignore"):
        h = x.astype(np.float32).astype(np.float16).view(np.uint16)
    hd = h.view(np.float16).astype(np.float64)
    return np.where((hd >= x) if strict else (hd > x), _prev16(h), h).astype(np.uint16)


def _bounds(mn):
    m = np.float64(mn)
    s1, s2, s3 = S * np.float32(0.5), S * np.float32(1.5), S * np.float32(2.5)
    return (_floor16(m + (s1.astype(np.float64) + _half_ulp(s1)), False),
            _floor16(m + (s2.astype(np.float64) - _half_ulp(s2)), True),
            _floor16(m + (s3.astype(np.float64) + _half_ulp(s3)), False))


def _by_division(xbits, mn):
    x = xbits.view(np.float16).astype(np.float32)
    with np.errstate(all="ignore"):
        d = x - np.float32(mn)
        return np.minimum(np.rint((d / S).astype(np.float32)), 3).astype(np.int64)


def _by_bounds(xbits, v):
    x = xbits.view(np.float16).astype(np.float64)
    return sum((x > b.view(np.float16).astype(np.float64)).astype(np.int64) for b in v)


def _minima():
    finite = [m for m in range(0, 0x10000, 37) if (m & 0x7FFF) < 0x7C00]
    special = [0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0xFBFF, 0xF800, 0xC000]
    return sorted(set(finite + special))


def test_bounds_against_the_division():
    rng = np.random.default_rng(5)
    for mb in _minima():
        mn = np.uint16(mb).view(np.float16).astype(np.float32)
        v = _bounds(mn)
        assert not any((b == 0x8000).any() for b in v)          # never -0
        top = np.float64(mn) + 3.5 * S.astype(np.float64)     # the group's range, with margin
        inside = top <= 65504.0
        for b in v:
            for x in (b, _next16(b), _prev16(b)):
                live = inside & ((x & 0x7FFF) < 0x7C00) & (x.view(np.float16).astype(np.float64) >= mn)
                assert np.array_equal(_by_division(x, mn)[live], _by_bounds(x, v)[live]), hex(mb)
        xr = (np.float64(mn) + rng.random(S.size) * 3.0 * S.astype(np.float64))
        xr = np.minimum(xr, 65504.0).astype(np.float16).view(np.uint16)
        live = inside & (xr.view(np.float16).astype(np.float64) >= mn)
        assert np.array_equal(_by_division(xr, mn)[live], _by_bounds(xr, v)[live]), hex(mb)


def test_thresholds_are_the_exact_multiples():
    # the binary32 neighbours of (0.5 + 2^-25)s, (1.5 - 2^-24)s, (2.5 + 2^-23)s that the
    # division-free rule uses are s/2, 3s/2 and 5s/2 themselves for every fp16 scale
    sd = S.astype(np.float64)
    t1 = (sd * (0.5 + 2.0 ** -25)).astype(np.float32)
    t1 = np.where(t1.astype(np.float64) > sd * (0.5 + 2.0 ** -25), np.nextafter(t1, np.float32(0)), t1)
    t2 = (sd * (1.5 - 2.0 ** -24)).astype(np.float32)
    t2 = np.where(t2.astype(np.float64) < sd * (1.5 - 2.0 ** -24), np.nextafter(t2, np.float32(np.inf)), t2)
    t3 = (sd * (2.5 + 2.0 ** -23)).astype(np.float32)
    t3 = np.where(t3.astype(np.float64) > sd * (2.5 + 2.0 ** -23), np.nextafter(t3, np.float32(0)), t3)
    assert np.array_equal(t1, S * np.float32(0.5))
    assert np.array_equal(t2, S * np.float32(1.5))
    assert np.array_equal(t3, S * np.float32(2.5))


def test_sign_of_the_fp16_difference():
    # x > V iff fl16(V - x) has its sign bit set, for V never -0: every fp16 pair on a grid
    rng = np.random.default_rng(9)
    fin = np.array([h for h in range(0x10000) if (h & 0x7FFF) < 0x7C00 and h != 0x8000], dtype=np.uint16)
    xs = np.concatenate([fin, [0x8000]]).astype(np.uint16)
    vs = rng.choice(fin, 512)
    vs = np.concatenate([vs, np.array([0x0000, 0x0001, 0x8001, 0x7BFF, 0xFBFF, 0x7C00], np.uint16)])
    x = xs.view(np.float16)
    for vb in vs:
        vv = np.uint16(vb).view(np.float16)
        with np.errstate(over="ignore"):
            diff = (np.float16(vv) - x).view(np.uint16)   # rounded to fp16: the sign of the exact difference
        assert np.array_equal((diff >> 15) == 1, x.astype(np.float64) > np.float64(vv)), hex(vb)
