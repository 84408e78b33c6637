"""The 2-bit quantizers' division-free code rule, checked against the division it replaces.

The GPU quantizers give a value x of a group with minimum mn and fp16 scale s the code
min(rint(fl(d / s)), 3), d = fl(x - mn), without dividing: per group they form three binary32
thresholds, RD((0.5 + 2^-25) s), RU((1.5 - 2^-24) s) and RD((2.5 + 2^-23) s) (RD, RU the
binary32 neighbours below and above the exact binary64 product), and count
[d > t1] + [d >= t2] + [d > t3].  Here that rule is restated in numpy and compared with the
correctly rounded binary32 division and ties-to-even rint, for every positive finite fp16
scale, at the binary32 values within 8 ulps of s times each rounding boundary and of the
integers between them, and at random d in [0, 4s).  (The GPU quantizers themselves are
checked bit for bit against the oracle by the GPU tests.)"""
import numpy as np

S = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)


def _rd(x):
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(0)), f)


def _ru(x):
    f = x.astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)


def _thresholds(s):
    sd = s.astype(np.float64)
    return _rd(sd * (0.5 + 2.0 ** -25)), _ru(sd * (1.5 - 2.0 ** -24)), _rd(sd * (2.5 + 2.0 ** -23))


def _by_division(d, s):
    with np.errstate(all="ignore"):
        return np.minimum(np.rint((d / s).astype(np.float32)), 3).astype(np.int64)


def _by_thresholds(d, t):
    return (d > t[0]).astype(np.int64) + (d >= t[1]) + (d > t[2])


def test_near_every_boundary_for_every_scale():
    t = _thresholds(S)
    for m in (0.5, 1.0, 1.5, 2.0, 2.5, 3.0):
        base = (S.astype(np.float64) * m).astype(np.float32)
        for direction in (np.float32(0), np.float32(np.inf)):
            d = base.copy()
            for _ in range(9):
                assert np.array_equal(_by_division(d, S), _by_thresholds(d, t)), (m, direction)
                d = np.nextafter(d, direction)


def test_random_values():
    rng = np.random.default_rng(11)
    i = rng.integers(0, S.size, 1_000_000)
    d = (rng.random(i.size) * 4.0 * S[i]).astype(np.float32)
    t = tuple(x[i] for x in _thresholds(S))
    assert np.array_equal(_by_division(d, S[i]), _by_thresholds(d, t))


def test_the_boundaries_are_where_rounding_says():
    # at the exact boundary products the division rounds to the half-integer itself and
    # rint sends it to the even code: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2
    s = np.float32(3.0)
    d = np.array([1.5, 4.5, 7.5], dtype=np.float32)
    assert _by_division(d, s).tolist() == [0, 2, 2]
    assert _by_thresholds(d, _thresholds(np.array([s] * 3, dtype=np.float32))).tolist() == [0, 2, 2]
