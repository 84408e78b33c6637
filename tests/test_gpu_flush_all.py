"""GPU parity of the second flush policy (KIVI_FLUSH_ALL: a full residual is quantized whole,
R/G groups at once) against the oracle with the same policy: caches bit-exact after every
flush, attention at every step, flushes exactly every R tokens, and ragged batches whose
sequences flush at their own steps."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128
D = 128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


@pytest.mark.parametrize("q_heads,kv_heads,G,R,fused", [
    (4, 4, 32, 128, True), (8, 2, 32, 128, False), (8, 2, 32, 64, True), (4, 4, 64, 128, False),
    (6, 2, 128, 256, True),
])
def test_decode_loop(q_heads, kv_heads, G, R, fused):
    dev = gpu_or_skip()
    kivi = _kivi()
    steps = 2 * R + 20
    w = synth.small(seed=R + G + q_heads, batch=2, q_heads=q_heads, kv_heads=kv_heads, context=4 * G + R - 5,
                    n_quant=4 * G, group=G, residual_cap=R, decode_steps=steps + R)
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, group=G, residual_cap=R, device=dev, flush_all=True)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=R, group=G,
                   flush_all=True)
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
        assert cache.state == (rc.n_quant, rc.n_res, rc.res_head), s
        if f:
            flushes.append(s)
        torch.cuda.synchronize()
        if f or s % 16 == 0 or s == steps - 1:
            assert_cache_equal(cache, rc)
        ref_out, ref_lse = rc.decode_attn(bits(q), SM)
        assert_attn_close(out, ref_out, what=f"flush-all G={G} R={R} step {s}")
        assert_lse_close(lse, ref_lse)
    assert flushes == list(range(5, steps, R))   # the ring starts 5 short of full


def test_ragged_batch():
    """Sequences with different ring fill levels flush whole rings at different steps."""
    dev = gpu_or_skip()
    kivi = _kivi()
    R, H, cap = 64, 2, 1024
    lengths = [(64, 63), (0, 10), (128, 64), (32, 1)]
    B = len(lengths)
    cache = kivi.Cache(B, H, cap, residual_cap=R, device=dev, flush_all=True)
    refs, states = [], []
    for b, (nq, nr) in enumerate(lengths):
        wb = synth.small(seed=90 + b, batch=1, q_heads=4, kv_heads=H, context=nq + nr, n_quant=nq, residual_cap=R)
        k, v = synth.prefill_kv(wb, device=dev)
        view = cache.sequence(b)
        kivi.kivi_prefill(k, v, nq, view)
        refs.append(ref_cache(1, H, cap, k.cpu(), v.cpu(), nq, residual_cap=R, flush_all=True))
        states.append(view.state)
    state = kivi.seq_state(states, device=dev)
    sw = synth.small(seed=97, batch=B, q_heads=4, kv_heads=H, context=1, n_quant=0)
    flushes = {b: [] for b in range(B)}
    for s in range(140):
        kn, vn = synth.step_kv(sw, s, device=dev)
        q = synth.query(sw, step=s + 1, device=dev)
        kivi.kivi_append_flush_ragged(cache, state, kn, vn)
        out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True)
        torch.cuda.synchronize()
        host = state.cpu().numpy()
        for b, rc in enumerate(refs):
            if rc.append(bits(kn[b]).reshape(-1, D), bits(vn[b]).reshape(-1, D)):
                flushes[b].append(s)
            assert tuple(host[b, :3]) == (rc.n_quant, rc.n_res, rc.res_head), (s, b)
            ref_out, ref_lse = rc.decode_attn(bits(q[b:b + 1]), SM)
            assert_attn_close(out[b:b + 1], ref_out, what=f"ragged flush-all step {s} seq {b}")
            assert_lse_close(lse[b:b + 1], ref_lse)
    assert flushes == {0: [1, 65, 129], 1: [54, 118], 2: [0, 64, 128], 3: [63, 127]}
    assert int(np.count_nonzero(state[:, 3].cpu().numpy())) == 0
    for b, rc in enumerate(refs):
        view = cache.sequence(b)
        view.set_state(rc.n_quant, rc.n_res, rc.res_head)
        assert_cache_equal(view, rc)
