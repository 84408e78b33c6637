"""GPU parity with one attention workspace kept across many calls, as a serving loop keeps it.

Split partials carry a per-call tag (the merging workgroup of each row moves the row's epoch
on), so a partial left by an earlier call must never be taken for one of the current call.
Each test runs a sequence of calls on one workspace, changing the split count between calls
(more, fewer, one), and checks every call against the oracle."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128
D = 128
SPLITS = [8, 3, 16, 1, 5, 8, 16, 2, 0, 0, 16, 1, 1, 7]


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _setup(w, dev):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, residual_cap=w.residual_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=w.residual_cap)
    return cache, rc, k, v


def _workspace(kivi, cache, q_heads, max_splits, dev):
    need = max(kivi.lib.kivi_decode_attn_workspace(kivi.C.byref(cache.c), q_heads, s) for s in range(1, max_splits + 1))
    need = max(need, kivi.lib.kivi_decode_attn_workspace(kivi.C.byref(cache.c), q_heads, 0))
    return torch.zeros(need, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("q_heads,kv_heads", [(4, 4), (8, 2)])
def test_split_counts_change_between_calls(q_heads, kv_heads):
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=31 + q_heads, batch=2, q_heads=q_heads, kv_heads=kv_heads, context=2048 + 77,
                    n_quant=2048)
    cache, rc, _, _ = _setup(w, dev)
    ws = _workspace(kivi, cache, q_heads, 16, dev)
    for i, s in enumerate(SPLITS):
        q = synth.query(w, step=i, device=dev)
        out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        ref_out, ref_lse = rc.decode_attn(bits(q), SM)
        assert_attn_close(out, ref_out, what=f"call {i} splits={s}")
        assert_lse_close(lse, ref_lse)


def test_decode_steps_share_one_workspace():
    """Fused steps over several flushes (the automatic split count moves with the history)."""
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=44, batch=2, q_heads=8, kv_heads=2, context=256 + 60, n_quant=256, residual_cap=64,
                    decode_steps=200)
    cache, rc, _, _ = _setup(w, dev)
    ws = _workspace(kivi, cache, w.q_heads, 16, dev)
    for s in range(150):
        kn, vn = synth.step_kv(w, s, device=dev)
        q = synth.query(w, step=s + 1, device=dev)
        out, lse, f = kivi.kivi_decode_step(cache, kn, vn, q, SM, lse=True, workspace=ws,
                                            num_splits=(0 if s % 3 else 4))
        assert bool(f) == bool(rc.append(bits(kn).reshape(-1, D), bits(vn).reshape(-1, D))), s
        torch.cuda.synchronize()
        ref_out, ref_lse = rc.decode_attn(bits(q), SM)
        assert_attn_close(out, ref_out, what=f"step {s}")
        assert_lse_close(lse, ref_lse)
    assert_cache_equal(cache, rc)


def test_ragged_calls_share_one_workspace():
    dev = gpu_or_skip()
    kivi = _kivi()
    lengths = [(1024, 100), (0, 7), (2048, 128), (96, 0)]
    B, Hq, Hkv = len(lengths), 4, 2
    cache = kivi.Cache(B, Hkv, 4096, device=dev)
    refs, states = [], []
    for b, (nq, nr) in enumerate(lengths):
        wb = synth.small(seed=60 + b, batch=1, q_heads=Hq, kv_heads=Hkv, context=nq + nr, n_quant=nq)
        k, v = synth.prefill_kv(wb, device=dev)
        view = cache.sequence(b)
        kivi.kivi_prefill(k, v, nq, view)
        refs.append(ref_cache(1, Hkv, 4096, k.cpu(), v.cpu(), nq))
        states.append(view.state)
    state = kivi.seq_state(states, device=dev)
    sw = synth.small(seed=66, batch=B, q_heads=Hq, kv_heads=Hkv, context=1, n_quant=0)
    ws = _workspace(kivi, cache, Hq, 32, dev)
    ws = torch.zeros(max(ws.numel(), kivi.lib.kivi_decode_attn_workspace(
        kivi.C.byref(cache.c), Hq, kivi.kivi_decode_attn_ragged_splits(cache, Hq))), dtype=torch.uint8, device=dev)
    for i, s in enumerate([0, 3, 0, 1, 0, 8]):
        q = synth.query(sw, step=i, device=dev)
        out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True, num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        for b, rc in enumerate(refs):
            ref_out, ref_lse = rc.decode_attn(bits(q[b:b + 1]), SM)
            assert_attn_close(out[b:b + 1], ref_out, what=f"ragged call {i} splits={s} seq {b}")
            assert_lse_close(lse[b:b + 1], ref_lse)


def test_fp16_comparator_calls_share_one_workspace():
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=71, batch=2, q_heads=8, kv_heads=2, context=3000, n_quant=0)
    k, v = synth.prefill_kv(w, device=dev)
    need = max(kivi.lib.kivi_decode_attn_fp16_workspace(w.batch, w.kv_heads, w.context, w.q_heads, s)
               for s in range(0, 12))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for i, s in enumerate([0, 5, 11, 1, 0, 3]):
        q = synth.query(w, step=i, device=dev)
        out, lse = kivi.kivi_decode_attn_fp16(k, v, q, SM, lse=True, num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        Hq, ratio = w.q_heads, w.q_heads // w.kv_heads
        ref_out = np.zeros((w.batch * Hq, D))
        ref_lse = np.zeros(w.batch * Hq)
        for r in range(w.batch * Hq):
            b, hq = divmod(r, Hq)
            K = k[b, hq // ratio].double().cpu().numpy()
            V = v[b, hq // ratio].double().cpu().numpy()
            ref_out[r], ref_lse[r] = ref.attn_dense(q[b, hq].double().cpu().numpy(), K, V, SM)
        assert_attn_close(out, ref_out, what=f"fp16 call {i} splits={s}")
        assert_lse_close(lse, ref_lse)
