"""Pins of the oracle's 4-bit member of the quantizer family and of its 4-bit cache layout.

The 4-bit quantizer keeps the 2-bit scheme's rules with sixteen levels: zero = group
minimum, scale = fp16((max - min)/15), code = clamp(round-half-even((x - zero)/scale), 0, 15),
computed against the stored fp16 scale.  Fixed here without reusing the oracle's formula:
hand cases with exact levels and ties, brute force over ~10^6 groups in exact integer
arithmetic (every code is the nearest level, exact ties to the even code), the scale rule,
reconstruction bounds, the axes (keys per channel, values per token) against direct group
quantization, the token-major nibble layout read back by hand, the cache's state machine,
and attention over the dequantized cache against dense fp64 attention.
"""
import numpy as np
import pytest

from oracle import ref

D = 128
KINDS = ["normal", "wide", "grid", "levels", "outlier", "tiny"]


def _units(bits):
    return (bits.view(np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)


def _ulp_units(s_bits):
    e = ((s_bits >> 10) & 0x1F).astype(np.int64)
    return np.where(e == 0, 1, 2 ** np.maximum(e - 1, 0))


def _f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def unpack4(codes):
    """[..., T, D/2] uint8 -> [..., T, D] codes: channel j in byte j/2, even channel low."""
    codes = np.asarray(codes)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


# ------------------------------------------------------------------ hand cases ----
@pytest.mark.parametrize("x,scale,codes", [
    # sixteen evenly spaced values: the step is exact, each value is its own level
    ([i * 0.25 for i in range(16)], 0.25, list(range(16))),
    # min 0, max 15: scale 1; 0.5 and 1.5 are ties, to the even codes 0 and 2; 14.5 -> 14
    ([0.0, 15.0, 0.5, 1.5, 2.5, 14.5, 7.25, 7.75], 1.0, [0, 15, 0, 2, 2, 14, 7, 8]),
    # negative zero point
    ([-7.5, 0.0, 7.5, -3.75], 1.0, [0, 8, 15, 4]),
    # a constant group: scale 0, every code 0
    ([3.0, 3.0, 3.0], 0.0, [0, 0, 0]),
])
def test_hand_cases(x, scale, codes):
    s, z, c = ref.quant_group(_f16(x), bits=4)
    assert float(np.uint16(s).view(np.float16)) == scale
    assert float(np.uint16(z).view(np.float16)) == min(x)
    assert c.tolist() == codes


def test_two_bit_member_is_the_two_bit_quantizer():
    rng = np.random.default_rng(5)
    for _ in range(200):
        x = _f16(rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3))
        assert ref.quant_group(x, bits=2)[0] == ref.quant_group(x)[0]
        assert np.array_equal(ref.quant_group(x, bits=2)[2], ref.quant_group(x)[2])


# --------------------------------------------------------------- random groups ----
def _groups(kind, n, rng, g):
    if kind == "normal":
        x = rng.standard_normal((n, g))
    elif kind == "wide":
        x = rng.standard_normal((n, g)) * 10.0 ** rng.uniform(-7.5, 4.6, (n, 1))
    elif kind == "grid":      # dyadic grid: many exact ties
        x = rng.integers(-40, 41, (n, g)) / 16.0
    elif kind == "levels":    # zero + multiples of half a step
        step = 2.0 ** rng.integers(-20, 6, (n, 1))
        x = rng.uniform(-100, 100, (n, 1)).round() * step + rng.integers(0, 31, (n, g)) * step / 2
    elif kind == "outlier":
        x = rng.standard_normal((n, g)) * np.exp(rng.uniform(np.log(100), np.log(7000), (n, 1)))
        x[:, 0] = rng.choice([-65504.0, 65504.0, 0.0], n)
    elif kind == "tiny":
        x = rng.integers(0, 33, (n, g)) * 2.0 ** -24 + rng.integers(-3, 3, (n, 1)) * 2.0 ** -14
    else:
        raise ValueError(kind)
    return np.clip(x, -65504, 65504).astype(np.float16).view(np.uint16)


def _as_values(x_bits, g):
    """Groups [n, g] through a 4-bit cache's per-token value quantizer (D/g groups a token)."""
    n = x_bits.shape[0]
    per_tok = D // g
    tokens = n // per_tok
    tokens -= tokens % 128
    c = ref.RefCache(1, 1, D, g, 128, token_cap=tokens, bits=4)
    c.quantize_v(x_bits[: tokens * per_tok].reshape(1, tokens, D), tokens)
    s = c.v_sz[0, :, :, 0].reshape(-1)
    z = c.v_sz[0, :, :, 1].reshape(-1)
    codes = unpack4(c.v_codes[0]).reshape(-1, g)
    return s, z, codes


@pytest.mark.parametrize("g", [32, 128])
@pytest.mark.parametrize("kind", KINDS)
def test_brute_force_nearest_level(kind, g):
    rng = np.random.default_rng(400 + KINDS.index(kind) + g)
    x = _groups(kind, 120_000 * 32 // g, rng, g)
    s, z, codes = _as_values(x, g)
    x = x[: codes.shape[0]]
    X, S, Z = _units(x), _units(s)[:, None], _units(z)[:, None]
    levels = Z[..., None] + S[..., None] * np.arange(16)
    err = np.abs(X[..., None] - levels)
    best = err.min(-1)
    mine = np.take_along_axis(err, codes[..., None].astype(np.int64), -1)[..., 0]
    tol = (S * 2.0 ** -19).astype(np.int64) + (S > 0)   # binary32 quotient rounding near a tie
    ok = (mine <= best + tol) & ((S > 0) | (codes == 0))
    assert ok.all(), np.argwhere(~ok)[:5]
    t2 = 2 * (X - Z)
    exact_tie = (S > 0) & (t2 % np.maximum(S, 1) == 0) & ((t2 // np.maximum(S, 1)) % 2 == 1) & (t2 < 31 * S)
    assert (codes[exact_tie] % 2 == 0).all()
    assert codes.max() <= 15


@pytest.mark.parametrize("kind", KINDS)
def test_scale_is_nearest_fp16_of_range_over_15_and_zero_is_min(kind):
    rng = np.random.default_rng(500 + KINDS.index(kind))
    x = _groups(kind, 60_000, rng, 32)
    s, z, codes = _as_values(x, 32)
    x = x[: s.shape[0]]
    X = _units(x)
    mn, mx = X.min(1), X.max(1)
    S = _units(s)
    dev = np.abs(15 * S - (mx - mn)).astype(np.float64)
    assert (dev <= 15 * _ulp_units(s) / 2.0 + (mx - mn) * 2.0 ** -23).all()
    assert np.array_equal(z.view(np.float16).astype(np.float64), x.view(np.float16).astype(np.float64).min(1))
    xf = x.view(np.float16).astype(np.float64)
    sf = s.view(np.float16).astype(np.float64)[:, None]
    xhat = z.view(np.float16).astype(np.float64)[:, None] + codes * sf
    rng_ = xf.max(1, keepdims=True) - xf.min(1, keepdims=True)
    bound = 0.5 * sf * (1 + 2.0 ** -20) + 15 * np.maximum(0.0, rng_ / 15 - sf)
    assert (np.abs(xf - xhat) <= bound).all()
    amin = xf.argmin(1)
    assert np.array_equal(xhat[np.arange(len(xf)), amin], xf[np.arange(len(xf)), amin])


# -------------------------------------------------------------- axes and layout ----
@pytest.mark.parametrize("g", [32, 64, 128])
def test_keys_per_channel_values_per_token_in_the_nibble_layout(g):
    rng = np.random.default_rng(g)
    T = 2 * g
    k = _f16(rng.standard_normal((1, T, D)) * 5)
    v = _f16(rng.standard_normal((1, T, D)))
    c = ref.RefCache(1, 1, D, g, 128, token_cap=T, bits=4)
    c.quantize_k(k, T)
    c.quantize_v(v, T)
    kc, vc = unpack4(c.k_codes[0]), unpack4(c.v_codes[0])
    for grp in range(T // g):
        for j in (0, 1, 5, 64, 127):
            s, z, codes = ref.quant_group(k[0, grp * g:(grp + 1) * g, j], bits=4)
            assert (c.k_sz[0, grp, j, 0], c.k_sz[0, grp, j, 1]) == (s, z)
            assert np.array_equal(kc[grp * g:(grp + 1) * g, j], codes)
    for t in (0, 1, T - 1):
        for kk in range(D // g):
            s, z, codes = ref.quant_group(v[0, t, kk * g:(kk + 1) * g], bits=4)
            assert (c.v_sz[0, t, kk, 0], c.v_sz[0, t, kk, 1]) == (s, z)
            assert np.array_equal(vc[t, kk * g:(kk + 1) * g], codes)


def test_append_from_empty_matches_closed_form_and_prefill():
    B, H, T, G, R = 1, 2, 300, 32, 128
    rng = np.random.default_rng(9)
    k = _f16(rng.standard_normal((B * H, T, D)) * 3)
    v = _f16(rng.standard_normal((B * H, T, D)))
    c = ref.RefCache(B, H, D, G, R, token_cap=384, bits=4)
    for t in range(T):
        c.append(k[:, t], v[:, t])
        n = t + 1
        nq = 0 if n <= R else G * -(-(n - R) // G)
        assert (c.n_quant, c.n_res, c.res_head) == (nq, n - nq, nq % R)
    p = ref.RefCache(B, H, D, G, R, token_cap=384, bits=4)
    p.prefill(k, v, c.n_quant)
    nq = c.n_quant
    assert np.array_equal(c.k_codes[:, :nq], p.k_codes[:, :nq])
    assert np.array_equal(c.v_codes[:, :nq], p.v_codes[:, :nq])
    for row in range(B * H):
        Kc, Vc = c.dequant_row(row)
        Kp, Vp = p.dequant_row(row)
        assert np.array_equal(Kc, Kp) and np.array_equal(Vc, Vp)


def test_attention_is_dense_attention_over_the_dequantized_cache():
    """Dequantized values come from the nibble layout read back here, not from the oracle."""
    rng = np.random.default_rng(11)
    B, H, Hq, nq, nr = 1, 2, 4, 256, 40
    k = _f16(rng.standard_normal((B * H, nq + nr, D)) * 4)
    v = _f16(rng.standard_normal((B * H, nq + nr, D)))
    c = ref.RefCache(B, H, D, 32, 128, token_cap=nq, bits=4)
    c.prefill(k, v, nq)
    q = _f16(rng.standard_normal((B, Hq, D)))
    sm = float(np.float32(0.088))   # the oracle takes the softmax scale as binary32
    out, lse = c.decode_attn(q, sm)
    kc, vc = unpack4(c.k_codes), unpack4(c.v_codes)
    for hq in range(Hq):
        row = hq // (Hq // H)
        ks = c.k_sz[row].view(np.float16).astype(np.float64)       # [groups, D, 2]
        vs = c.v_sz[row].view(np.float16).astype(np.float64)       # [tokens, D/32, 2]
        K = ks[np.arange(nq) // 32, :, 1] + kc[row, :nq] * ks[np.arange(nq) // 32, :, 0]
        V = vs[:nq, np.arange(D) // 32, 1] + vc[row, :nq] * vs[:nq, np.arange(D) // 32, 0]
        K = np.concatenate([K, k[row, nq:].view(np.float16).astype(np.float64)])
        V = np.concatenate([V, v[row, nq:].view(np.float16).astype(np.float64)])
        qq = q[0, hq].view(np.float16).astype(np.float64)
        logits = (K @ qq) * sm
        m = logits.max()
        p = np.exp(logits - m)
        assert np.allclose(out[0, hq], (p @ V) / p.sum(), rtol=1e-12, atol=1e-12)
        assert abs(lse[0, hq] - (m + np.log(p.sum()))) < 1e-9
