"""GPU parity with residual rings other than R = 128 (the residual length is a parameter of
the cache; the pages' ablation varies it): decode steps with group flushes, caches compared
bit-exactly and attention every step against the oracle built with the same R."""
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128


@pytest.mark.parametrize("R,fused", [(32, True), (64, False), (96, True), (256, True), (256, False)])
def test_decode_loop_with_residual(R, fused):
    dev = gpu_or_skip()
    from kv_cache_bit_quantize_amd import kivi
    steps = 2 * R + 40
    w = synth.small(seed=R + fused, batch=2, q_heads=4, kv_heads=2, context=64 + R - 5, n_quant=64,
                    residual_cap=R, decode_steps=steps)
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, residual_cap=R, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=R)
    flushes = []
    for s in range(steps):
        kn, vn = synth.step_kv(w, s, device=dev)
        q = synth.query(w, step=s + 1, device=dev)
        if fused:
            out, lse, f = kivi.kivi_decode_step(cache, kn, vn, q, SM, lse=True)
        else:
            f = kivi.kivi_append_flush(cache, kn, vn)
            out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True)
        assert bool(f) == bool(rc.append(bits(kn).reshape(-1, 128), bits(vn).reshape(-1, 128))), s
        if f:
            flushes.append(s)
        torch.cuda.synchronize()
        if f or s % 16 == 0 or s == steps - 1:
            assert_cache_equal(cache, rc)
        ref_out, ref_lse = rc.decode_attn(bits(q), SM)
        assert_attn_close(out, ref_out, what=f"R={R} step {s}")
        assert_lse_close(lse, ref_lse)
    # the ring starts 5 short of full; afterwards one flush per 32 appends
    assert flushes == list(range(5, steps, 32))
