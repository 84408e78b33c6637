"""GPU parity of decode steps: append (with group flushes) followed by attention, step
after step, against the oracle's state machine and fp64 attention."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _steps(w, dev, steps, check_cache_every, attn_rows_every, bsel=None, fused=False):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    bsel = list(range(w.batch)) if bsel is None else bsel
    rc = ref_cache(len(bsel), w.kv_heads, w.token_cap, k[bsel].cpu(), v[bsel].cpu(), w.n_quant)
    rows = [b * w.kv_heads + h for b in bsel for h in range(w.kv_heads)]
    del k, v
    flushes = []
    for s in range(steps):
        kn, vn = synth.step_kv(w, s, device=dev)
        q = synth.query(w, step=s + 1, device=dev)
        if fused:
            out, lse, f_gpu = kivi.kivi_decode_step(cache, kn, vn, q, SM, lse=True)
        else:
            f_gpu = kivi.kivi_append_flush(cache, kn, vn)
            out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True)
        f_ref = rc.append(bits(kn[bsel]).reshape(-1, 128), bits(vn[bsel]).reshape(-1, 128))
        assert f_gpu == f_ref, s
        if f_gpu:
            flushes.append(s)
        torch.cuda.synchronize()
        if f_gpu or (check_cache_every and s % check_cache_every == 0) or s == steps - 1:
            class View:
                pass
            g = View()
            idx = torch.as_tensor(rows, device=dev)
            for name in ("k_codes", "v_codes", "k_sz", "v_sz", "k_res", "v_res"):
                setattr(g, name, getattr(cache, name).index_select(0, idx))
            g.state = cache.state
            assert_cache_equal(g, rc)
        if s % attn_rows_every == 0 or f_gpu or s == steps - 1:
            ref_out, ref_lse = rc.decode_attn(bits(q[bsel]), SM)
            assert_attn_close(out[bsel], ref_out, what=f"step {s}")
            assert_lse_close(lse[bsel], ref_lse)
    return flushes


def test_small_decode_loop_every_step():
    dev = gpu_or_skip()
    w = synth.small(seed=11, batch=2, q_heads=4, kv_heads=2, context=96 + 100, n_quant=96, decode_steps=100)
    flushes = _steps(w, dev, 100, check_cache_every=1, attn_rows_every=1)
    assert flushes == [28, 60, 92]


def test_empty_start_fills_then_flushes():
    dev = gpu_or_skip()
    w = synth.small(seed=12, batch=1, q_heads=2, kv_heads=2, context=1, n_quant=0, decode_steps=200)
    flushes = _steps(w, dev, 200, check_cache_every=5, attn_rows_every=3)
    assert flushes == [127, 159, 191]


def test_llama2_7b_layer_64_steps():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["llama2-7b-layer"]
    flushes = _steps(w, dev, 64, check_cache_every=0, attn_rows_every=8, bsel=[0, 7])
    assert flushes == [0, 32]


def test_gqa_mistral_128_steps_sampled():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["gqa-mistral-7b"]
    flushes = _steps(w, dev, 128, check_cache_every=0, attn_rows_every=8, bsel=[5])
    assert flushes == [0, 32, 64, 96]


# ---- the fused decode step (kivi_decode_step): same state machine and results, one launch
# when no group is flushed

@pytest.mark.parametrize("q_heads,kv_heads", [(4, 2), (3, 3), (8, 2)])
def test_fused_step_small_loop_every_step(q_heads, kv_heads):
    dev = gpu_or_skip()
    w = synth.small(seed=20 + q_heads, batch=2, q_heads=q_heads, kv_heads=kv_heads, context=96 + 100, n_quant=96,
                    decode_steps=70)
    flushes = _steps(w, dev, 70, check_cache_every=1, attn_rows_every=1, fused=True)
    assert flushes == [28, 60]


def test_fused_step_empty_start():
    dev = gpu_or_skip()
    w = synth.small(seed=21, batch=1, q_heads=2, kv_heads=1, context=1, n_quant=0, decode_steps=170)
    flushes = _steps(w, dev, 170, check_cache_every=7, attn_rows_every=3, fused=True)
    assert flushes == [127, 159]


def test_fused_step_gqa_mistral_sampled():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["gqa-mistral-7b"]
    flushes = _steps(w, dev, 40, check_cache_every=0, attn_rows_every=5, bsel=[9], fused=True)
    assert flushes == [0, 32]


def test_fused_step_long_context_sampled():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["long-128k"]
    _steps(w, dev, 3, check_cache_every=1, attn_rows_every=1, fused=True)
