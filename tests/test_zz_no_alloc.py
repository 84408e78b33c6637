"""kivi_decode_attn_noalloc (the library's static per-device scratch in place of a workspace)
against kivi_decode_attn (a caller workspace) on the same inputs, and both against the oracle.
Both calls launch the same kernel with the same split count.  The single-query kernel hands
tile pairs to its waves from a queue, so which wave sums which tokens (and the fp32 rounding)
changes from run to run: the two outputs are compared at the parity bar (per row 2e-3 of the
row's largest magnitude, lse within 2e-3 + 2^-18 |lse|), not bit for bit.  Calls in a row
change the shape (the second is smaller, then larger again, then the same shape repeated), so
the scratch's clearing on a shape change and its reuse within a shape are both exercised; a
shape whose workspace exceeds the scratch is refused."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _cache(w, dev, code_bits=2):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, residual_cap=w.residual_cap, device=dev, bits=code_bits)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    return cache, k, v


def _both(cache, q, splits=0):
    kivi = _kivi()
    B, Hq, _ = q.shape
    ref_out, ref_lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=splits)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    kivi.kivi_decode_attn_noalloc(cache, q, SM, out, lse, num_splits=splits)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def _gpu(t):
    return t.detach().cpu().numpy().astype(np.float64)


def _compare(w, cache, k, v, q, out, lse, ref_out, ref_lse, what, code_bits=2):
    # the scratch call against the workspace call ...
    assert_attn_close(out, _gpu(ref_out), what=f"{what}: noalloc vs workspace")
    assert_lse_close(lse, _gpu(ref_lse))
    # ... and against the oracle
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, bits=code_bits)
    o_ref, l_ref = rc.decode_attn(bits(q), SM)
    assert_attn_close(out, o_ref, what=f"{what}: noalloc vs oracle")
    assert_lse_close(lse, l_ref)


def test_matches_workspace_call_across_shapes():
    dev = gpu_or_skip()
    big = synth.small(seed=1001, batch=2, q_heads=32, kv_heads=8, context=8192 + 60, n_quant=8192)
    small = synth.small(seed=1002, batch=1, q_heads=4, kv_heads=4, context=4096 + 17, n_quant=4096)
    mha = synth.small(seed=1003, batch=1, q_heads=32, kv_heads=32, context=32768 + 32, n_quant=32768)
    caches = {w.seed: _cache(w, dev) for w in (big, small, mha)}
    order = [(big, 0), (small, 0), (big, 5), (big, 0), (mha, 0), (small, 3), (small, 3), (mha, 0)]
    for i, (w, s) in enumerate(order):
        cache, k, v = caches[w.seed]
        q = synth.query(w, step=i, device=dev)
        out, lse, ref_out, ref_lse = _both(cache, q, s)
        _compare(w, cache, k, v, q, out, lse, ref_out, ref_lse, f"call {i} ({w.seed}, splits {s})")


def test_4bit_cache_and_repeat_calls():
    dev = gpu_or_skip()
    w = synth.small(seed=1004, batch=2, q_heads=8, kv_heads=2, context=4096 + 100, n_quant=4096)
    cache, k, v = _cache(w, dev, code_bits=4)
    for i in range(3):
        q = synth.query(w, step=i, device=dev)
        out, lse, ref_out, ref_lse = _both(cache, q)
        _compare(w, cache, k, v, q, out, lse, ref_out, ref_lse, f"4-bit call {i}", code_bits=4)


def test_too_large_for_the_scratch_is_refused():
    dev = gpu_or_skip()
    kivi = _kivi()
    # 64 x 64 query rows at 4 splits need 64*64*4*130*8 bytes of partials (> 8 MiB)
    w = synth.small(seed=1005, batch=64, q_heads=64, kv_heads=64, context=64, n_quant=32)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    need = kivi.lib.kivi_decode_attn_workspace(kivi.C.byref(cache.c), 64, 4)
    assert need > kivi.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 64, 128), dtype=torch.float16, device=dev)
    out = torch.empty_like(q)
    cache.set_state(32, 0, 0)
    with pytest.raises(kivi.KiviError) as e:
        kivi.kivi_decode_attn_noalloc(cache, q, SM, out, num_splits=4)
    assert e.value.status == -5
