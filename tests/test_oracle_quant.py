"""Pins of the oracle's 2-bit asymmetric group quantizer and its packed layout.

What fixes the oracle here (none of it reuses the oracle's own formula):
  * hand-derived vectors (tests/golden/quant_vectors.txt, working shown there);
  * brute force: every code is the nearest of the four levels zero + c*scale, in exact
    integer arithmetic (fp16 values are integers in units of 2^-24), on ~10^6 groups;
  * the scale is the fp16 value nearest to (max - min)/3, the zero point is the minimum;
  * invariants: reconstruction error <= scale/2, constant groups exact, the minimum
    reconstructs exactly, codes do not depend on the order of a group's elements.
"""
import numpy as np
import pytest

from golden_io import quant_vectors
from layout import key_word_bytes, unpack_key_codes, unpack_value_codes, value_pairs
from oracle import ref

D, G = 128, 32


def _units(bits):
    """fp16 bit patterns -> exact int64 value in units of 2^-24."""
    return (bits.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)


def _ulp_units(s_bits):
    e = ((s_bits >> 10) & 0x1F).astype(np.int64)
    return np.where(e == 0, 1, 2 ** np.maximum(e - 1, 0))   # ulp of fp16 in 2^-24 units


# ------------------------------------------------------------------ vectors ----
@pytest.mark.parametrize("vec", quant_vectors(), ids=lambda v: v["name"])
def test_hand_vectors_group(vec):
    s, z, codes = ref.quant_group(np.array(vec["input"], np.uint16))
    assert (s, z) == (vec["scale"], vec["zero"])
    assert codes.tolist() == vec["codes"]


@pytest.mark.parametrize("vec", quant_vectors(), ids=lambda v: v["name"])
def test_hand_vectors_as_value_token(vec):
    """The group as channels 32..63 of one value token: pair and codes at their documented places."""
    c = ref.RefCache(1, 1, D, G, 128, token_cap=G)
    src = np.zeros((1, 1, D), np.uint16)
    src[0, 0, 32:64] = vec["input"]
    c.quantize_v(src, 1)
    assert value_pairs(c.v_sz[0])[0, 1].tolist() == [vec["scale"], vec["zero"]]
    assert unpack_value_codes(c.v_codes[0])[0, 32:64].tolist() == vec["codes"]


@pytest.mark.parametrize("vec", quant_vectors(), ids=lambda v: v["name"])
def test_hand_vectors_as_key_channel(vec):
    """The group as channel 5 of 32 key tokens: channel 5 = 4*1 + 1 is byte 1, bits 2-3 of
    each token's first code word."""
    c = ref.RefCache(1, 1, D, G, 128, token_cap=2 * G)
    src = np.zeros((1, 2 * G, D), np.uint16)
    src[0, G:, 5] = vec["input"]
    c.quantize_k(src, 2 * G)
    assert c.k_sz[0, 1, 5].tolist() == [vec["scale"], vec["zero"]]
    byte1 = np.array([key_word_bytes(c.k_codes[0], t, 0)[1] for t in range(G, 2 * G)])
    assert (byte1 >> 2 & 3).tolist() == vec["codes"]
    assert (byte1 & 0xF3).tolist() == [0] * G   # channels 1, 9, 13 are zero groups


# ------------------------------------------------------------ random groups ----
def _groups(kind, n, rng, g=G):
    if kind == "normal":
        x = rng.standard_normal((n, g))
    elif kind == "wide":
        x = rng.standard_normal((n, g)) * 10.0 ** rng.uniform(-7.5, 4.6, (n, 1))
    elif kind == "grid":      # small dyadic grid: many exact ties
        x = rng.integers(-12, 13, (n, g)) / 8.0
    elif kind == "levels":    # zero + multiples of a step, incl. half levels
        step = 2.0 ** rng.integers(-20, 8, (n, 1))
        x = rng.uniform(-100, 100, (n, 1)).round() * step + rng.integers(0, 7, (n, g)) * step / 2
    elif kind == "outlier":
        x = rng.standard_normal((n, g)) * np.exp(rng.uniform(np.log(100), np.log(7000), (n, 1)))
        x[:, 0] = rng.choice([-65504.0, 65504.0, 0.0], n)
    elif kind == "tiny":      # subnormal ranges
        x = rng.integers(0, 9, (n, g)) * 2.0 ** -24 + rng.integers(-3, 3, (n, 1)) * 2.0 ** -14
    else:
        raise ValueError(kind)
    return np.clip(x, -65504, 65504).astype(np.float16).view(np.uint16)


KINDS = ["normal", "wide", "grid", "levels", "outlier", "tiny"]


def _quantize_as_values(x_bits):
    """Run groups [n, g] (g = 32, 64 or 128) through the per-token value quantizer with
    value groups of g channels (128 / g groups per token)."""
    n, g = x_bits.shape
    per_tok = D // g
    tokens = n // per_tok
    tokens -= tokens % 128                        # whole token groups (cache tiles) for any g
    c = ref.RefCache(1, 1, D, g, 128, token_cap=tokens)
    c.quantize_v(x_bits[: tokens * per_tok].reshape(1, tokens, D), tokens)
    vp = value_pairs(c.v_sz[0])                    # [tokens, per_tok, 2]
    s = vp[:, :, 0].reshape(-1)
    z = vp[:, :, 1].reshape(-1)
    codes = unpack_value_codes(c.v_codes[0]).reshape(-1, g)
    return s, z, codes


GROUPS = [32, 64, 128]


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("kind", KINDS)
def test_brute_force_nearest_level(kind, g):
    rng = np.random.default_rng(100 + KINDS.index(kind) + g)
    x = _groups(kind, 160_000 * 32 // g, rng, g)
    s, z, codes = _quantize_as_values(x)
    x = x[: codes.shape[0]]
    X, S, Z = _units(x), _units(s)[:, None], _units(z)[:, None]
    levels = Z[..., None] + S[..., None] * np.arange(4)            # [n, 1, 4]
    err = np.abs(X[..., None] - levels)                             # [n, G, 4]
    best = err.min(-1)
    mine = np.take_along_axis(err, codes[..., None].astype(np.int64), -1)[..., 0]
    # a code other than the nearest level is allowed only inside a 2^-20-wide tie band
    tol = (S * 2.0 ** -19).astype(np.int64) + (S > 0)
    ok = (mine <= best + tol) & ((S > 0) | (codes == 0))
    assert ok.all(), np.argwhere(~ok)[:5]
    # exact ties are broken towards the even code
    t2 = 2 * (X - Z)
    exact_tie = (S > 0) & (t2 % np.maximum(S, 1) == 0) & ((t2 // np.maximum(S, 1)) % 2 == 1) \
        & (t2 < 7 * S)
    assert (codes[exact_tie] % 2 == 0).all()


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("kind", KINDS)
def test_scale_is_nearest_fp16_of_range_over_3_and_zero_is_min(kind, g):
    rng = np.random.default_rng(200 + KINDS.index(kind) + g)
    x = _groups(kind, 80_000 * 32 // g, rng, g)
    s, z, _ = _quantize_as_values(x)
    x = x[: s.shape[0]]
    X = _units(x)
    mn, mx = X.min(1), X.max(1)
    S = _units(s)
    # |s - range/3| <= half an fp16 ulp of s (plus the binary32 intermediate rounding)
    dev = np.abs(3 * S - (mx - mn)).astype(np.float64)
    bound = 3 * _ulp_units(s) / 2.0 + (mx - mn) * 2.0 ** -23
    assert (dev <= bound).all()
    # zero point: the minimum value, with -0 stored as +0
    zf = z.view(np.float16).astype(np.float64)
    assert np.array_equal(zf, x.view(np.float16).astype(np.float64).min(1))
    assert not (z == 0x8000).any()


@pytest.mark.parametrize("g", GROUPS)
@pytest.mark.parametrize("kind", KINDS)
def test_reconstruction_invariants(kind, g):
    rng = np.random.default_rng(300 + KINDS.index(kind) + g)
    x = _groups(kind, 80_000 * 32 // g, rng, g)
    s, z, codes = _quantize_as_values(x)
    x = x[: codes.shape[0]]
    xf = x.view(np.float16).astype(np.float64)
    sf = s.view(np.float16).astype(np.float64)[:, None]
    zf = z.view(np.float16).astype(np.float64)[:, None]
    xhat = zf + codes * sf
    rng_ = xf.max(1, keepdims=True) - xf.min(1, keepdims=True)
    err = np.abs(xf - xhat)
    # general bound (clamp can bite when the fp16 scale rounds below range/3)
    bound = 0.5 * sf * (1 + 2.0 ** -20) + 3 * np.maximum(0.0, rng_ / 3 - sf)
    assert (err <= bound).all()
    normal_s = sf[:, 0] >= 2.0 ** -14
    assert (err[normal_s] <= 0.5 * sf[normal_s] * (1 + 2.0 ** -20) + 3 * np.maximum(0, rng_[normal_s] / 3 - sf[normal_s])).all()
    # the minimum reconstructs exactly; constant groups are exact
    amin = xf.argmin(1)
    assert np.array_equal(xhat[np.arange(len(xf)), amin], xf[np.arange(len(xf)), amin])
    const = rng_[:, 0] == 0
    assert np.array_equal(xhat[const], xf[const])


def test_codes_do_not_depend_on_element_order():
    rng = np.random.default_rng(5)
    x = np.concatenate([_groups(k, 4096, rng) for k in KINDS])
    perm = rng.permutation(G)
    s1, z1, c1 = _quantize_as_values(x)
    s2, z2, c2 = _quantize_as_values(np.ascontiguousarray(x[:, perm]))
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
    assert np.array_equal(c1[:, perm], c2)


def test_signed_zeros_do_not_depend_on_order():
    rng = np.random.default_rng(6)
    x = rng.choice(np.array([0x8000, 0x0000, 0x3C00, 0xBC00], np.uint16), (20480, G), p=[.45, .45, .05, .05])
    s1, z1, c1 = _quantize_as_values(x)
    s2, z2, c2 = _quantize_as_values(np.ascontiguousarray(x[:, ::-1]))
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2) and np.array_equal(c1[:, ::-1], c2)
    assert not (s1 == 0x8000).any() and not (z1 == 0x8000).any()


@pytest.mark.parametrize("Gs", GROUPS)
def test_keys_per_channel_values_per_token_axes(Gs):
    """Keys group along tokens for each channel (Gs tokens), values along channels for each
    token (Gs channels), for every supported group size Gs; each stored pair and code is the
    group quantizer applied to exactly that group."""
    rng = np.random.default_rng(9 + Gs)
    T = 2 * Gs
    k = rng.standard_normal((1, T, D)).astype(np.float16).view(np.uint16)
    c = ref.RefCache(1, 1, D, Gs, 128, token_cap=T)
    c.quantize_k(k, T)
    c.quantize_v(k, T)
    kf = k.view(np.float16).astype(np.float64)[0]
    kcodes, vcodes = unpack_key_codes(c.k_codes[0]), unpack_value_codes(c.v_codes[0])
    for g in range(2):
        for j in range(D):
            s, z, codes = ref.quant_group(k[0, g * Gs:(g + 1) * Gs, j])
            assert c.k_sz[0, g, j].tolist() == [s, z]
            assert np.array_equal(kcodes[g * Gs:(g + 1) * Gs, j], codes)
            assert np.uint16(z).view(np.float16) == kf[g * Gs:(g + 1) * Gs, j].min()
    for t in range(T):
        for kk in range(D // Gs):
            s, z, codes = ref.quant_group(k[0, t, kk * Gs:(kk + 1) * Gs])
            assert value_pairs(c.v_sz[0])[t, kk].tolist() == [s, z]
            assert np.array_equal(vcodes[t, kk * Gs:(kk + 1) * Gs], codes)


def test_per_channel_keys_isolate_outlier_channels():
    """Direction reported by the article (paragraph 2): per-channel key groups isolate the
    fixed outlier channels, so the ordinary channels keep a small error; per-token groups
    stretch every token's levels over the outlier and the ordinary channels pay for it.
    Synthetic model: four channels with a large offset (150..7000) and a 2% spread, the
    other channels N(0, 1); the error is measured on the ordinary channels."""
    rng = np.random.default_rng(3)
    kf = rng.standard_normal((G * 8, D))
    off = np.array([150.0, -900.0, 3000.0, -7000.0])
    kf[:, [3, 40, 77, 100]] = off * (1 + 0.02 * rng.standard_normal((G * 8, 4)))
    k = kf.astype(np.float16).view(np.uint16)[None]
    c = ref.RefCache(1, 1, D, G, 128, token_cap=G * 8)
    c.quantize_k(k, G * 8)
    c.quantize_v(k, G * 8)         # the same tensor grouped per token
    c.set_state(G * 8, 0, 0)
    K_chan, K_tok = c.dequant_row(0)
    x = k[0].view(np.float16).astype(np.float64)
    ordinary = np.setdiff1d(np.arange(D), [3, 40, 77, 100])
    e_chan = np.mean((K_chan - x)[:, ordinary] ** 2)
    e_tok = np.mean((K_tok - x)[:, ordinary] ** 2)
    assert e_chan < 0.1 * e_tok
