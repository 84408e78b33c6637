"""GPU parity of the fp16 comparator (kivi_decode_attn_fp16) against the oracle's fp64
dense attention over the same fp16 keys and values.

Bar: the attention bar of the 2-bit path, per output row max |o_gpu - o_ref| / max |o_ref|
<= 2e-3, and |exp(lse_gpu - lse_ref) - 1| <= 2e-3.  Padding tokens past `tokens` in each
row hold NaN, so a read outside the context would show in the output."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_lse_close, gpu_or_skip
from kv_cache_bit_quantize_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu
D = 128
SM = synth.SM_SCALE_D128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _inputs(w, stride, dev):
    k, v = synth.prefill_kv(w, device=dev)
    q = synth.query(w, device=dev)
    if stride > w.context:
        kp = torch.full((w.batch, w.kv_heads, stride, D), float("nan"), dtype=torch.float16, device=dev)
        vp = kp.clone()
        kp[:, :, :w.context] = k
        vp[:, :, :w.context] = v
        k, v = kp, vp
    return k.contiguous(), v.contiguous(), q


def _reference(k, v, q, tokens, rows):
    """fp64 attention of the listed query rows (b*Hq + hq) over the first `tokens` tokens."""
    B, Hkv = k.shape[:2]
    Hq = q.shape[1]
    ratio = Hq // Hkv
    out = np.zeros((B * Hq, D))
    lse = np.zeros(B * Hq)
    for r in rows:
        b, hq = divmod(int(r), Hq)
        K = k[b, hq // ratio, :tokens].double().cpu().numpy()
        V = v[b, hq // ratio, :tokens].double().cpu().numpy()
        out[r], lse[r] = ref.attn_dense(q[b, hq].double().cpu().numpy(), K, V, SM)
    return out, lse


def _check(w, stride, splits=0, rows=None, what=""):
    dev = gpu_or_skip()
    kivi = _kivi()
    k, v, q = _inputs(w, stride, dev)
    out, lse = kivi.kivi_decode_attn_fp16(k, v, q, SM, tokens=w.context, lse=True, num_splits=splits)
    torch.cuda.synchronize()
    all_rows = np.arange(w.batch * w.q_heads) if rows is None else np.asarray(rows)
    ref_out, ref_lse = _reference(k, v, q, w.context, all_rows)
    assert_attn_close(out, ref_out, rows=all_rows, what=what)
    assert_lse_close(lse, ref_lse, rows=all_rows)
    return out


def test_single_token():
    w = synth.small(seed=21, batch=1, q_heads=1, kv_heads=1, context=1, n_quant=0)
    _check(w, 1, what="fp16 one token")


@pytest.mark.parametrize("batch,q_heads,kv_heads,tokens,stride,splits", [
    (2, 4, 4, 100, 128, 0),       # one query per workgroup, padded rows
    (2, 8, 2, 1000, 1024, 3),     # query groups of 4, 3 splits
    (1, 6, 2, 333, 400, 0),       # groups of 3, ragged tail
    (3, 10, 2, 257, 257, 5),      # ratio 5: one query per workgroup
    (1, 4, 2, 2048, 2048, 0),     # groups of 2
    (2, 4, 1, 17, 32, 7),         # more splits than the context fills: empty splits
    (1, 2, 2, 5000, 5000, 1),     # one split: the output written without the merge
])
def test_shapes(batch, q_heads, kv_heads, tokens, stride, splits):
    w = synth.small(seed=batch * 1000 + tokens, batch=batch, q_heads=q_heads, kv_heads=kv_heads,
                    context=tokens, n_quant=0)
    _check(w, stride, splits=splits, what=f"fp16 {q_heads}/{kv_heads} T={tokens}")


def test_split_count_does_not_change_the_result():
    w = synth.small(seed=33, batch=1, q_heads=4, kv_heads=4, context=4096 + 50, n_quant=0, outliers=0)
    outs = [_check(w, w.context, splits=s, what=f"fp16 splits={s}").float() for s in (1, 2, 9, 64)]
    base = outs[0]
    for o in outs[1:]:
        rel = ((o - base).abs().max(-1).values / base.abs().max(-1).values).max().item()
        assert rel <= 1e-3, rel


def test_long_128k_sampled_rows():
    """The long-context shape (32 heads, 131,072 fp16 tokens per head), automatic splits."""
    w = synth.WORKLOADS["long-128k"]
    _check(w, w.context, rows=[0, 13, 31], what="fp16 long-128k")


def test_gqa_mistral_sampled_rows():
    """Batch 64, 32 query heads over 8 kv heads, 8,192 fp16 tokens, automatic splits."""
    w = synth.WORKLOADS["gqa-mistral-7b"]
    _check(w, w.context, rows=[0, 5, 777, 2047], what="fp16 gqa-mistral-7b")


def test_timed_launch_matches_untimed():
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=44, batch=2, q_heads=8, kv_heads=2, context=3000, n_quant=0)
    k, v, q = _inputs(w, w.context, dev)
    plain = kivi.kivi_decode_attn_fp16(k, v, q, SM)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    kivi.kivi_time_next_attention(*ev)
    timed = kivi.kivi_decode_attn_fp16(k, v, q, SM)
    torch.cuda.synchronize()
    assert torch.equal(timed, plain)
    assert 0.0 < ev[0].elapsed_time(ev[1]) < 1000.0
