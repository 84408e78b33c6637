"""GPU parity with group sizes G = 64 and 128 (the group size is a parameter of the cache;
the pages' ablation varies it): codes and pairs bit-exact against the oracle built with the
same G, attention within the attention bar, decode steps whose flushes move G tokens, and
ragged batches."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128
D = 128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _setup(w, dev):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, group=w.group, residual_cap=w.residual_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=w.residual_cap,
                   group=w.group)
    return cache, rc


@pytest.mark.parametrize("G", [64, 128])
def test_prefill_bit_exact(G):
    dev = gpu_or_skip()
    w = synth.small(seed=G, batch=2, q_heads=4, kv_heads=4, context=10 * G + 77, n_quant=10 * G, group=G)
    cache, rc = _setup(w, dev)
    assert_cache_equal(cache, rc)


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("tokens,off", [(1, 0), (33, 0), (100, 64), (129, 128)])
def test_value_tokens_ragged(G, tokens, off):
    """Per-token value groups of G channels for runs of tokens that start and end inside
    32-token code tiles (the codes of the tile's other tokens are kept)."""
    dev = gpu_or_skip()
    kivi = _kivi()
    T = 512
    rng = np.random.default_rng(G + tokens)
    x = torch.from_numpy(rng.standard_normal((2, tokens, D)).astype(np.float16)).to(dev)
    cache = kivi.Cache(1, 2, T, group=G, device=dev)
    kivi.kivi_quantize_v_per_token(x.view(1, 2, tokens, D), cache, dst_token_off=off)
    torch.cuda.synchronize()
    rc = ref.RefCache(1, 2, D, G, 128, token_cap=T)
    rc.quantize_v(bits(x), tokens, dst_off=off)
    assert np.array_equal(cache.v_codes.cpu().numpy(), rc.v_codes)
    assert np.array_equal(bits(cache.v_sz), rc.v_sz)


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("q_heads,kv_heads,splits", [(4, 4, 0), (8, 2, 0), (6, 2, 3), (4, 4, 5)])
def test_attention(G, q_heads, kv_heads, splits):
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=G + q_heads + splits, batch=2, q_heads=q_heads, kv_heads=kv_heads,
                    context=16 * G + 100, n_quant=16 * G, group=G)
    cache, rc = _setup(w, dev)
    q = synth.query(w, device=dev)
    out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = rc.decode_attn(bits(q), SM)
    assert_attn_close(out, ref_out, what=f"G={G} {q_heads}/{kv_heads} splits={splits}")
    assert_lse_close(lse, ref_lse)


@pytest.mark.parametrize("G,R,fused", [(64, 128, True), (64, 64, False), (128, 128, True), (128, 256, False)])
def test_decode_loop(G, R, fused):
    """Steps whose flushes move G ring tokens into one new key group and G value tokens."""
    dev = gpu_or_skip()
    kivi = _kivi()
    steps = 3 * G + 10
    w = synth.small(seed=G + R, batch=2, q_heads=8, kv_heads=2, context=2 * G + R - 3, n_quant=2 * G,
                    group=G, residual_cap=R, decode_steps=steps)
    cache, rc = _setup(w, dev)
    flushes = []
    for s in range(steps):
        kn, vn = synth.step_kv(w, s, device=dev)
        q = synth.query(w, step=s + 1, device=dev)
        if fused:
            out, lse, f = kivi.kivi_decode_step(cache, kn, vn, q, SM, lse=True)
        else:
            f = kivi.kivi_append_flush(cache, kn, vn)
            out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True)
        assert bool(f) == bool(rc.append(bits(kn).reshape(-1, D), bits(vn).reshape(-1, D))), s
        if f:
            flushes.append(s)
        torch.cuda.synchronize()
        if f or s % 8 == 0 or s == steps - 1:
            assert_cache_equal(cache, rc)
        ref_out, ref_lse = rc.decode_attn(bits(q), SM)
        assert_attn_close(out, ref_out, what=f"G={G} R={R} step {s}")
        assert_lse_close(lse, ref_lse)
    assert flushes == list(range(3, steps, G))


def test_ragged_group_64():
    """Ragged batch with G = 64: per-sequence flushes move 64 tokens."""
    dev = gpu_or_skip()
    kivi = _kivi()
    G, B, H = 64, 3, 2
    lengths = [(128, 127), (0, 128), (64, 3)]
    cache = kivi.Cache(B, H, 1024, group=G, device=dev)
    refs, states = [], []
    for b, (nq, nr) in enumerate(lengths):
        w = synth.small(seed=70 + b, batch=1, q_heads=4, kv_heads=H, context=nq + nr, n_quant=nq, group=G)
        k, v = synth.prefill_kv(w, device=dev)
        view = cache.sequence(b)
        kivi.kivi_prefill(k, v, nq, view)
        refs.append(ref_cache(1, H, 1024, k.cpu(), v.cpu(), nq, group=G))
        states.append(view.state)
    state = kivi.seq_state(states, device=dev)
    sw = synth.small(seed=99, batch=B, q_heads=4, kv_heads=H, context=1, n_quant=0, group=G)
    for s in range(80):
        kn, vn = synth.step_kv(sw, s, device=dev)
        q = synth.query(sw, step=s + 1, device=dev)
        kivi.kivi_append_flush_ragged(cache, state, kn, vn)
        out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True)
        torch.cuda.synchronize()
        host = state.cpu().numpy()
        for b, rc in enumerate(refs):
            rc.append(bits(kn[b]).reshape(-1, D), bits(vn[b]).reshape(-1, D))
            assert tuple(host[b, :3]) == (rc.n_quant, rc.n_res, rc.res_head), (s, b)
            ref_out, ref_lse = rc.decode_attn(bits(q[b:b + 1]), SM)
            assert_attn_close(out[b:b + 1], ref_out, what=f"ragged G=64 step {s} seq {b}")
            assert_lse_close(lse[b:b + 1], ref_lse)
    assert int(np.count_nonzero(state[:, 3].cpu().numpy())) == 0
