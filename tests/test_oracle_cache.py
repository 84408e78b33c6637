"""Pins of the oracle's cache state machine (residual append, group flush) and of the
byte accounting that the inference-research record prints.

The flush policy is a reading (the record only says the newest R tokens stay in full
precision and that only grouped history is quantized): when a token arrives and the
residual already holds R tokens, the oldest G residual tokens become the next key/value
group.  Pinned here by the closed form of the state after n appends, and by the fact
that appending tokens one by one must give exactly the cache that a prefill of the
same token sequence gives (so every flush took the oldest tokens, in order).
"""
import numpy as np
import pytest

from golden_io import key_values
from layout import value_pairs
from oracle import ref

D, G, R = 128, 32, 128


def _tokens(rows, T, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((rows, T, D)) * 3
    k[:, :, [5, 77]] *= 300
    k = k.astype(np.float16).view(np.uint16)
    v = rng.standard_normal((rows, T, D)).astype(np.float16).view(np.uint16)
    return k, v


def _closed_form_state(n_tokens, R=R, G=G):
    n_quant = 0 if n_tokens <= R else G * -(-(n_tokens - R) // G)
    return n_quant, n_tokens - n_quant, (n_quant % R)


@pytest.mark.parametrize("R,G", [(32, 32), (64, 32), (128, 32), (256, 32), (64, 64), (128, 64), (128, 128),
                                 (256, 128)])
def test_append_from_empty_matches_closed_form_and_prefill(R, G):
    """The residual length R and the group size G are parameters: for every pair, after n
    tokens the history holds the fewest whole groups of G that leave at most R tokens in
    the ring."""
    B, H, T = 2, 3, 300
    k, v = _tokens(B * H, T, 1)
    c = ref.RefCache(B, H, D, G, R, token_cap=384)
    flush_steps = []
    for t in range(T):
        if c.append(k[:, t], v[:, t]):
            flush_steps.append(t)
        assert (c.n_quant, c.n_res, c.res_head) == _closed_form_state(t + 1, R, G)
    # a flush happens exactly when the residual is full as the token arrives
    assert flush_steps == [R + i * G for i in range((T - R - 1) // G + 1)]
    p = ref.RefCache(B, H, D, G, R, token_cap=384)
    p.prefill(k, v, c.n_quant)
    nq = c.n_quant
    assert np.array_equal(c.k_codes[:, : nq // G], p.k_codes[:, : nq // G])
    assert np.array_equal(c.v_codes[:, : nq // G], p.v_codes[:, : nq // G])
    assert np.array_equal(c.k_sz[:, : nq // G], p.k_sz[:, : nq // G])
    assert np.array_equal(c.v_sz[:, :nq], p.v_sz[:, :nq])
    for row in range(B * H):
        Kc, Vc = c.dequant_row(row)
        Kp, Vp = p.dequant_row(row)
        assert np.array_equal(Kc, Kp) and np.array_equal(Vc, Vp)
    # the residual holds the newest tokens, oldest first from res_head
    for i in range(c.n_res):
        slot = (c.res_head + i) % R
        assert np.array_equal(c.k_res[:, slot], k[:, nq + i])
        assert np.array_equal(c.v_res[:, slot], v[:, nq + i])


def _closed_form_state_flush_all(n_tokens, R=R):
    """Flush of the whole residual: after n tokens the ring holds ((n - 1) mod R) + 1 of
    them (n >= 1) and the history the rest, always a whole number of residuals."""
    n_res = (n_tokens - 1) % R + 1 if n_tokens > 0 else 0
    return n_tokens - n_res, n_res, 0


@pytest.mark.parametrize("R,G", [(32, 32), (64, 32), (128, 32), (128, 64), (128, 128), (256, 64)])
def test_flush_all_from_empty_matches_closed_form_and_prefill(R, G):
    """The other flush policy: a full residual is quantized whole (R / G groups at once).
    The history grows by R at every flush, the ring's head stays at slot 0, and the cache
    equals a prefill of the same tokens with that history."""
    B, H, T = 2, 2, 700
    k, v = _tokens(B * H, T, 7)
    c = ref.RefCache(B, H, D, G, R, token_cap=768, flush_all=True)
    flush_steps = []
    for t in range(T):
        if c.append(k[:, t], v[:, t]):
            flush_steps.append(t)
        assert (c.n_quant, c.n_res, c.res_head) == _closed_form_state_flush_all(t + 1, R)
    assert flush_steps == list(range(R, T, R))
    p = ref.RefCache(B, H, D, G, R, token_cap=768)
    p.prefill(k, v, c.n_quant)
    nq = c.n_quant
    assert np.array_equal(c.k_codes[:, : nq // 32], p.k_codes[:, : nq // 32])
    assert np.array_equal(c.v_codes[:, : nq // 32], p.v_codes[:, : nq // 32])
    assert np.array_equal(c.k_sz[:, : nq // G], p.k_sz[:, : nq // G])
    assert np.array_equal(c.v_sz[:, :nq], p.v_sz[:, :nq])
    for i in range(c.n_res):
        assert np.array_equal(c.k_res[:, (c.res_head + i) % R], k[:, nq + i])
        assert np.array_equal(c.v_res[:, (c.res_head + i) % R], v[:, nq + i])


def test_flush_all_from_a_prefilled_state_moves_the_head_by_whole_residuals():
    """From a prefill whose ring does not start at slot 0 of a cycle: every flush moves R
    tokens, so the head comes back to the same slot and the history stays a multiple of G."""
    n_quant, n_res, steps = 96, 100, 300
    k, v = _tokens(1, n_quant + n_res + steps, 8)
    c = ref.RefCache(1, 1, D, G, R, token_cap=1024, flush_all=True)
    c.prefill(k[:, : n_quant + n_res], v[:, : n_quant + n_res], n_quant)
    flushes = [s for s in range(steps) if c.append(k[:, n_quant + n_res + s], v[:, n_quant + n_res + s])]
    assert flushes == [28, 28 + R, 28 + 2 * R]
    assert (c.n_quant, c.n_res, c.res_head) == (n_quant + 3 * R, n_res + steps - 3 * R, 0)
    p = ref.RefCache(1, 1, D, G, R, token_cap=1024)
    p.prefill(k, v, c.n_quant)
    for row in range(1):
        Kc, Vc = c.dequant_row(row)
        Kp, Vp = p.dequant_row(row)
        assert np.array_equal(Kc, Kp) and np.array_equal(Vc, Vp)


@pytest.mark.parametrize("n_quant,n_res,steps,flushes", [
    (3968, 128, 64, [0, 32]),            # Llama-2-7B layer workload: steps 1 and 33
    (8064, 128, 128, [0, 32, 64, 96]),   # GQA workload: steps 1, 33, 65, 97
    (64, 100, 70, [28, 60]),
])
def test_flush_schedule_from_a_prefilled_state(n_quant, n_res, steps, flushes):
    k, v = _tokens(1, n_quant + n_res + steps, 2)
    cap = n_quant + n_res + steps + G
    c = ref.RefCache(1, 1, D, G, R, token_cap=cap - cap % G)
    c.prefill(k[:, : n_quant + n_res], v[:, : n_quant + n_res], n_quant)
    got = [s for s in range(steps) if c.append(k[:, n_quant + n_res + s], v[:, n_quant + n_res + s])]
    assert got == flushes
    assert c.n_quant == n_quant + G * len(flushes)
    assert c.n_res == n_res + steps - G * len(flushes)
    assert R - G < c.n_res <= R or len(flushes) == 0


def test_prefill_layout_and_residual_slots():
    k, v = _tokens(2, 96 + 40, 3)
    c = ref.RefCache(1, 2, D, G, R, token_cap=96)
    c.prefill(k, v, 96)
    assert (c.n_quant, c.n_res, c.res_head) == (96, 40, 0)
    assert np.array_equal(c.k_res[:, :40], k[:, 96:])
    assert np.array_equal(c.v_res[:, :40], v[:, 96:])
    s, z, codes = ref.quant_group(k[1, 64:96, 9])
    assert c.k_sz[1, 2, 9].tolist() == [s, z]


def test_bytes_match_the_record():
    g = key_values("bytes_llama2_13b.txt")
    codes, meta, fp16 = ref.bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["group"])
    assert codes == g["codes_bytes_per_token"]
    assert fp16 == g["fp16_bytes_per_token"]
    res_total = g["residual"] * fp16
    assert res_total == g["residual_bytes_total"]
    assert res_total // g["context"] == g["residual_bytes_per_token_at_context"]
    assert codes + res_total // g["context"] == g["page_sum_bytes_per_token"]
    assert fp16 / (codes + res_total // g["context"]) == g["page_reduction_at_context"]
    assert fp16 * g["context"] / 2 ** 30 == g["fp16_sequence_gib_at_context"]
    # metadata the page leaves out: one fp16 (scale, zero) pair per 32 elements of K and V
    assert meta == codes // 2 == 51200
    # with metadata, 3,968 quantized + 128 residual tokens: 174,400 B/token, 4.70x
    per_tok = ((codes + meta) * (g["context"] - g["residual"]) + res_total) / g["context"]
    assert per_tok == 174400
    assert round(fp16 / per_tok, 2) == 4.70


def test_bytes_per_head_token():
    """One kv head, d = 128: 32 + 32 bytes of codes and 16 + 16 of pairs per token."""
    codes, meta, fp16 = ref.bytes_per_token(1, 1, 128, 32)
    assert (codes, meta, fp16) == (64, 32, 512)


def test_dequant_row_reconstructs_each_element_within_half_its_group_scale():
    """Every dequantized element lies within half its own group's scale of the input
    (keys: group = 32 tokens of one channel; values: 32 channels of one token)."""
    k, v = _tokens(2, 5 * G + 20, 4)
    c = ref.RefCache(2, 1, D, G, R, token_cap=5 * G)
    c.prefill(k, v, 5 * G)
    f = lambda a: a.view(np.float16).astype(np.float64)
    for row in range(2):
        K, V = c.dequant_row(row)
        ks = f(c.k_sz[row, :, :, 0])                  # [groups, D]
        vs = f(value_pairs(c.v_sz[row])[:, :, 0])     # [tokens, D/G]
        k_bound = np.repeat(ks, G, axis=0) * 0.5 * (1 + 2.0 ** -20)
        v_bound = np.repeat(vs, G, axis=1) * 0.5 * (1 + 2.0 ** -20)
        assert (np.abs(K[: 5 * G] - f(k[row, : 5 * G])) <= k_bound).all()
        assert (np.abs(V[: 5 * G] - f(v[row, : 5 * G])) <= v_bound).all()
        assert np.array_equal(K[5 * G:], f(k[row, 5 * G:])) and np.array_equal(V[5 * G:], f(v[row, 5 * G:]))
