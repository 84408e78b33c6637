"""Pins of the oracle's fp64 attention, split-K merge and query-head mapping.

Fixed against: torch's scaled_dot_product_attention in float64 on the CPU (a library
routine), closed forms (q = 0 gives the mean of V; one key gives its value; one
dominant logit gives that row), token-permutation invariance, and the log-sum-exp
merge equalling the unsplit result over arbitrary partitions.
"""
import numpy as np
import pytest
import torch

from oracle import ref

D = 128
SM = 0.08838834764831845


def _sdpa(q, K, V, sm):
    qt = torch.from_numpy(q)[None, None, None, :]
    Kt = torch.from_numpy(K)[None, None]
    Vt = torch.from_numpy(V)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=sm)[0, 0, 0].numpy()
    lse = torch.logsumexp(torch.from_numpy(K @ q * sm), 0).item()
    return out, lse


@pytest.mark.parametrize("n", [1, 2, 33, 300, 4100])
def test_dense_matches_torch_sdpa_fp64(n):
    rng = np.random.default_rng(n)
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)) * 3, rng.standard_normal((n, D))
    out, lse = ref.attn_dense(q, K, V, SM)
    o2, l2 = _sdpa(q, K, V, SM)
    assert np.max(np.abs(out - o2)) <= 1e-12 * np.max(np.abs(o2)) + 1e-15
    assert abs(lse - l2) <= 1e-12 * max(1, abs(l2))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((257, D)) * 50, rng.standard_normal((257, D))
    out, lse = ref.attn_dense(np.zeros(D), K, V, SM)
    assert np.allclose(out, V.mean(0), rtol=0, atol=1e-13)
    assert abs(lse - np.log(257)) < 1e-13


def test_single_key_gives_its_value():
    rng = np.random.default_rng(2)
    K, V = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    out, _ = ref.attn_dense(rng.standard_normal(D), K, V, SM)
    assert np.array_equal(out, V[0])


def test_dominant_logit_selects_its_row():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(D)
    K, V = rng.standard_normal((64, D)), rng.standard_normal((64, D))
    K[17] = q * (2000.0 / (q @ q) / SM)        # logit 2000 against O(1): exp(-1990) == 0
    out, lse = ref.attn_dense(q, K, V, SM)
    assert np.allclose(out, V[17], rtol=0, atol=1e-15)
    assert abs(lse - SM * (K[17] @ q)) < 1e-9


def test_token_order_is_irrelevant():
    rng = np.random.default_rng(4)
    q, K, V = rng.standard_normal(D), rng.standard_normal((500, D)), rng.standard_normal((500, D))
    p = rng.permutation(500)
    a, la = ref.attn_dense(q, K, V, SM)
    b, lb = ref.attn_dense(q, K[p], V[p], SM)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15) and abs(la - lb) < 1e-12


@pytest.mark.parametrize("parts", [1, 2, 7, 33])
def test_split_merge_equals_unsplit(parts):
    rng = np.random.default_rng(parts)
    n = 1000
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)) * 4, rng.standard_normal((n, D))
    cuts = np.sort(rng.choice(np.arange(1, n), parts - 1, replace=False)) if parts > 1 else np.array([], int)
    bounds = [0, *cuts.tolist(), n]
    bounds.insert(1, 0)                          # one empty part as well
    ms, ls, os_ = [], [], []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        m, l, o = ref.attn_partial(q, K, V, t0, t1, SM)
        ms.append(m), ls.append(l), os_.append(o)
    out, lse = ref.attn_merge(np.array(ms), np.array(ls), np.array(os_))
    o2, l2 = ref.attn_dense(q, K, V, SM)
    assert np.max(np.abs(out - o2)) <= 1e-12 * np.max(np.abs(o2))
    assert abs(lse - l2) <= 1e-12 * max(1.0, abs(l2))


def _random_cache(B, Hkv, n_quant, n_res, seed, res_head=0):
    rng = np.random.default_rng(seed)
    T = n_quant + n_res
    k = (rng.standard_normal((B * Hkv, T, D)) * 4).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((B * Hkv, T, D)).astype(np.float16).view(np.uint16)
    c = ref.RefCache(B, Hkv, D, 32, 128, token_cap=max(32, n_quant))
    c.prefill(k, v, n_quant)
    if res_head:          # rotate the ring: same logical residual, different slots
        order = [(i - res_head) % 128 for i in range(128)]
        c.k_res[:] = c.k_res[:, order]
        c.v_res[:] = c.v_res[:, order]
        c.set_state(n_quant, n_res, res_head)
    return c, k, v


def test_gqa_head_mapping_matches_torch_convention():
    """Query head hq reads kv head hq // (Hq/Hkv), as torch's enable_gqa does."""
    B, Hkv, Hq = 2, 2, 8
    c, _, _ = _random_cache(B, Hkv, 64, 40, 5)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16).view(np.uint16)
    out, lse = c.decode_attn(q, SM)
    Ks, Vs = zip(*[c.dequant_row(r) for r in range(B * Hkv)])
    Kt = torch.from_numpy(np.stack(Ks).reshape(B, Hkv, -1, D))
    Vt = torch.from_numpy(np.stack(Vs).reshape(B, Hkv, -1, D))
    qt = torch.from_numpy(q.view(np.float16).astype(np.float64))[:, :, None, :]
    sm32 = float(np.float32(SM))          # the decode call takes the scale as binary32
    want = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=sm32, enable_gqa=True)[:, :, 0]
    assert np.max(np.abs(out - want.numpy())) <= 1e-12 * np.max(np.abs(want.numpy()))


def test_context_is_quantized_history_then_residual():
    c, k, v = _random_cache(1, 1, 96, 50, 7)
    K, V = c.dequant_row(0)
    assert K.shape == (146, D)
    kf = k[0].view(np.float16).astype(np.float64)
    assert np.array_equal(K[96:], kf[96:146])                  # residual kept exactly
    assert np.max(np.abs(K[:96] - kf[:96])) <= np.abs(kf[:96]).max() # quantized part approximates


def test_ring_rotation_does_not_change_attention():
    q = np.random.default_rng(8).standard_normal((1, 1, D)).astype(np.float16).view(np.uint16)
    c0, _, _ = _random_cache(1, 1, 64, 128, 9)
    c1, _, _ = _random_cache(1, 1, 64, 128, 9, res_head=96)
    assert np.array_equal(c0.dequant_row(0)[0], c1.dequant_row(0)[0])
    o0, l0 = c0.decode_attn(q, SM)
    o1, l1 = c1.decode_attn(q, SM)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_no_quantized_history_is_plain_fp16_attention():
    c, k, v = _random_cache(1, 1, 0, 100, 10)
    q = np.random.default_rng(11).standard_normal((1, 1, D)).astype(np.float16).view(np.uint16)
    out, lse = c.decode_attn(q, SM)
    f = lambda a: a.view(np.float16).astype(np.float64)
    o2, l2 = _sdpa(f(q)[0, 0], f(k[0]), f(v[0]), float(np.float32(SM)))
    assert np.max(np.abs(out[0, 0] - o2)) <= 1e-12 * np.max(np.abs(o2))
    assert abs(lse[0, 0] - l2) < 1e-12 * abs(l2) + 1e-15


def test_sampled_rows_equal_full_rows():
    c, _, _ = _random_cache(2, 2, 64, 10, 12)
    q = np.random.default_rng(13).standard_normal((2, 4, D)).astype(np.float16).view(np.uint16)
    full, lf = c.decode_attn(q, SM)
    part, lp = c.decode_attn(q, SM, rows=np.array([5, 0, 7]))
    flat, pflat = full.reshape(8, D), part.reshape(8, D)
    for r in (5, 0, 7):
        assert np.array_equal(flat[r], pflat[r])
    assert np.isnan(pflat[1]).all()
