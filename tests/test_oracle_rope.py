"""Pins of the oracle's rotary position embedding and of its attention over pre-RoPE keys.

The pages advise quantizing keys before RoPE ("Your KV cache doesn't have a bit problem...",
paragraph 4; the KVQuant summary on GrooveSquid) without writing RoPE out; the oracle takes
the rotate-half rotary embedding (channel i with i + d/2, frequency base^(-2i/d), angle
position * frequency).  Fixed here without reusing its code: RoPE as multiplication of the
complex numbers x_i + i*x_{i+d/2} by exp(i*pos*w_i) (numpy complex arithmetic), the
rotation's invariants (pair norms, inverse at -pos, dot products that depend only on the
position difference), each pair's frequency read back as an angle, and attention over a
cache whose keys numpy dequantizes-by-hand and turns at their sequence positions.
"""
import numpy as np
import pytest

from oracle import ref

D = 128


def _complex_rope(x, pos, base):
    """x [..., d] at positions pos [...]: (x_i + i x_{i+d/2}) * exp(i pos base^(-2i/d))."""
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    w = base ** (-2.0 * np.arange(h) / x.shape[-1])
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, np.float64)[..., None] * w)
    return np.concatenate([z.real, z.imag], -1)


def test_hand_case_and_position_zero():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    # d = 4, base 100: pairs (0, 2) at 1 rad per position, (1, 3) at 0.1 rad per position
    out = ref.rope(x, 3, 100.0)
    expect = [np.cos(3) - 3 * np.sin(3), 2 * np.cos(0.3) - 4 * np.sin(0.3),
              3 * np.cos(3) + np.sin(3), 4 * np.cos(0.3) + 2 * np.sin(0.3)]
    assert np.allclose(out, expect, rtol=0, atol=1e-15)
    assert np.array_equal(ref.rope(x, 0, 100.0), x)


@pytest.mark.parametrize("base", [10000.0, 500000.0, 7.5])
def test_matches_complex_multiplication(base):
    rng = np.random.default_rng(int(base))
    for pos in [1, 2, 31, 32, 1000, 4095, 131071, 1 << 20]:
        x = rng.standard_normal(D) * 10.0 ** rng.uniform(-2, 3)
        got = ref.rope(x, pos, base)
        want = _complex_rope(x, pos, base)
        assert np.allclose(got, want, rtol=0, atol=1e-12 * np.abs(x).max() * (1 + pos * 1e-4)), pos


def test_pair_norms_kept_and_inverse():
    rng = np.random.default_rng(3)
    for pos in [0, 7, 65535, 131072]:
        x = rng.standard_normal(D)
        y = ref.rope(x, pos, 10000.0)
        assert np.allclose(np.hypot(y[:64], y[64:]), np.hypot(x[:64], x[64:]), rtol=1e-14, atol=0)
        assert np.allclose(ref.rope(y, -pos, 10000.0), x, rtol=0, atol=1e-12)


def test_dot_products_depend_only_on_the_position_difference():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in [(5, 2), (100, 37), (131071, 0), (4096, 4096)]:
        ref_dot = ref.rope(q, m - n, 10000.0) @ k
        for s in (1, 333, 70000):
            assert abs(ref.rope(q, m + s, 10000.0) @ ref.rope(k, n + s, 10000.0) - ref_dot) < 1e-10


def test_each_pair_turns_at_its_frequency():
    base = 10000.0
    for i in range(D // 2):
        e = np.zeros(D)
        e[i] = 1.0
        y = ref.rope(e, 1, base)
        w = base ** (-2.0 * i / D)
        assert abs(np.arctan2(y[i + D // 2], y[i]) - w) < 1e-15
        assert np.count_nonzero(np.abs(y) > 1e-300) <= 2    # only the pair (i, i + d/2) moves


def _f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


@pytest.mark.parametrize("bits", [2, 4])
def test_attention_over_keys_turned_at_their_positions(bits):
    """Keys dequantized by hand from the documented layout, residual read oldest first from
    a wrapped ring, each turned at its sequence position by complex multiplication."""
    rng = np.random.default_rng(11 + bits)
    B, H, Hq, G, R = 1, 2, 4, 32, 64
    nq0, nr0 = 128, 40
    k = _f16(rng.standard_normal((B * H, nq0 + nr0, D)) * 4)
    v = _f16(rng.standard_normal((B * H, nq0 + nr0, D)))
    c = ref.RefCache(B, H, D, G, R, token_cap=512, bits=bits)
    c.prefill(k, v, nq0)
    for _ in range(50):                 # two flushes: the ring wraps and res_head moves
        c.append(_f16(rng.standard_normal((B * H, D)) * 4), _f16(rng.standard_normal((B * H, D))))
    assert c.res_head != 0
    q = _f16(rng.standard_normal((B, Hq, D)))
    sm = float(np.float32(0.088))
    out, lse = c.decode_attn_rope(q, sm, 10000.0)
    n = c.n_quant + c.n_res
    for hq in range(Hq):
        row = hq // (Hq // H)
        K, V = c.dequant_row(row)      # sequence order: history, then the ring oldest first
        assert K.shape[0] == n
        Kr = _complex_rope(K, np.arange(n), 10000.0)
        qq = q[0, hq].view(np.float16).astype(np.float64)
        logits = (Kr @ qq) * sm
        m = logits.max()
        p = np.exp(logits - m)
        assert np.allclose(out[0, hq], (p @ V) / p.sum(), rtol=1e-10, atol=1e-12)
        assert abs(lse[0, hq] - (m + np.log(p.sum()))) < 1e-9
    # without the rotation the result differs (the positions matter)
    plain, _ = c.decode_attn(q, sm)
    assert np.abs(plain - out).max() > 1e-3


def test_single_token_returns_its_value():
    """One cached token: softmax weight 1 whatever its rotation."""
    rng = np.random.default_rng(12)
    k = _f16(rng.standard_normal((1, 1, D)) * 3)
    v = _f16(rng.standard_normal((1, 1, D)))
    c = ref.RefCache(1, 1, D, 32, 128, token_cap=0)
    c.prefill(k, v, 0)
    q = _f16(rng.standard_normal((1, 1, D)))
    out, lse = c.decode_attn_rope(q, 0.1, 10000.0)
    assert np.array_equal(out[0, 0], v[0, 0].view(np.float16).astype(np.float64))
    logit = 0.1 * (k[0, 0].view(np.float16).astype(np.float64) @ q[0, 0].view(np.float16).astype(np.float64))
    assert abs(lse[0, 0] - np.float64(np.float32(0.1)) / 0.1 * logit) < 1e-9   # position 0: no turn
