"""GPU parity of the fused decode attention against the fp64 CPU oracle.

Bar: per output row, max |o_gpu - o_ref| / max |o_ref| <= 2e-3 (fp32 accumulation and
fp16 output against fp64), and |lse_gpu - lse_ref| <= 2e-3 + 2^-18 |lse_ref|: the absolute
part is the same 2e-3, the relative part allows for binary32 logits (each logit is a sum of
128 folded products whose terms can exceed the logit several-fold, so its rounding error is
a few 2^-24 of the terms' magnitude; with 10^2..7*10^3 outlier channels logits reach
thousands, where 2e-3 absolute would ask for ~8 binary32 ulps; kivi_testlib.LSE_REL)."""
import numpy as np
import pytest
import torch

from kivi_testlib import ATTN_TOL, assert_attn_close, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
D, G = 128, 32
SM = synth.SM_SCALE_D128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _setup(w, dev, rows=None, layer=0, k=None, v=None, q=None):
    """GPU cache + q for workload w; oracle cache over the kv rows the sampled q rows need."""
    kivi = _kivi()
    if k is None:
        k, v = synth.prefill_kv(w, layer=layer, device=dev)
    if q is None:
        q = synth.query(w, layer=layer, device=dev)
    k, v, q = k.to(dev), v.to(dev), q.to(dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant)
    return cache, rc, q


def _run(cache, q, lse=True, splits=0):
    out, l = _kivi().kivi_decode_attn(cache, q, SM, lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    return out, l


def _check(cache, rc, q, rows=None, splits=0, what=""):
    out, lse = _run(cache, q, splits=splits)
    ref_out, ref_lse = rc.decode_attn(bits(q), SM, rows=rows)
    err = assert_attn_close(out, ref_out, rows=rows, what=what)
    assert_lse_close(lse, ref_lse, rows=rows)
    return out, err


def test_tiny_workload():
    dev = gpu_or_skip()
    cache, rc, q = _setup(synth.WORKLOADS["tiny"], dev)
    _check(cache, rc, q, what="tiny")


@pytest.mark.parametrize("n_quant,n_res", [(0, 1), (0, 100), (32, 0), (32, 5), (96, 128), (640, 0),
                                           (640, 77), (1024, 128)])
def test_history_and_residual_sizes(n_quant, n_res):
    dev = gpu_or_skip()
    w = synth.small(seed=n_quant + n_res, batch=2, q_heads=3, kv_heads=3, context=n_quant + n_res,
                    n_quant=n_quant)
    cache, rc, q = _setup(w, dev)
    _check(cache, rc, q, what=f"nq={n_quant} r={n_res}")


def test_diffuse_attention_without_outliers():
    """No outlier channels and small logits: the softmax spreads over many tokens."""
    dev = gpu_or_skip()
    w = synth.small(seed=3, batch=2, q_heads=4, kv_heads=4, context=2048 + 64, n_quant=2048, outliers=0)
    k, v = synth.prefill_kv(w, device=dev)
    q = synth.query(w, device=dev) * 0.25
    cache, rc, q = _setup(w, dev, k=k, v=v, q=q.half())
    _check(cache, rc, q, what="diffuse")


def test_zero_query_gives_mean():
    dev = gpu_or_skip()
    w = synth.small(seed=4, context=992 + 40, n_quant=992)
    cache, rc, _ = _setup(w, dev)
    q = torch.zeros((w.batch, w.q_heads, D), dtype=torch.float16, device=dev)
    _check(cache, rc, q, what="q=0")


def test_extreme_values():
    """Keys and values at the fp16 extremes (+-65504) mixed with ordinary values."""
    dev = gpu_or_skip()
    w = synth.small(seed=5, batch=1, q_heads=2, kv_heads=2, context=256 + 20, n_quant=256)
    k, v = synth.prefill_kv(w, device="cpu")
    k[:, :, ::7, 3] = 65504.0
    k[:, :, 1::7, 3] = -65504.0
    v[:, :, ::5, 10] = 65504.0
    v[:, :, 2::5, 11] = -65504.0
    q = synth.query(w) * 1e-3
    cache, rc, q = _setup(w, dev, k=k, v=v, q=q.half())
    _check(cache, rc, q, what="extremes")


def test_gqa_ratio_four():
    dev = gpu_or_skip()
    w = synth.small(seed=6, batch=3, q_heads=8, kv_heads=2, context=1536 + 100, n_quant=1536)
    cache, rc, q = _setup(w, dev)
    _check(cache, rc, q, what="gqa")


@pytest.mark.parametrize("q_heads,kv_heads,n_quant,n_res,splits", [
    (4, 2, 1024, 37, 0),     # ratio 2: two queries per workgroup
    (6, 2, 640, 128, 0),     # ratio 3
    (16, 2, 512, 5, 3),      # ratio 8: two workgroups of 4 queries per kv head, 3 splits
    (10, 2, 320, 64, 0),     # ratio 5: one query per workgroup
    (12, 4, 96, 0, 1),       # ratio 3, one split (output written without the merge)
    (8, 1, 2048, 128, 5),    # ratio 8, one kv head, full residual ring
    (8, 2, 0, 77, 0),        # residual only
    (4, 1, 32, 1, 2),        # one group, one residual token, more splits than needed
])
def test_gqa_query_groups(q_heads, kv_heads, n_quant, n_res, splits):
    """Every query head of a group gets its own attention over the shared kv head, for the
    query-group sizes the kernels take together and the ones they split or run alone."""
    dev = gpu_or_skip()
    w = synth.small(seed=q_heads * 100 + n_quant + n_res, batch=2, q_heads=q_heads, kv_heads=kv_heads,
                    context=n_quant + n_res, n_quant=n_quant)
    cache, rc, q = _setup(w, dev)
    _check(cache, rc, q, splits=splits, what=f"gqa {q_heads}/{kv_heads}")


@pytest.mark.parametrize("q_heads,kv_heads", [(4, 4), (8, 2)])
def test_timed_launch_matches_untimed(q_heads, kv_heads):
    """kivi_time_next_attention: the timed launch (hipExtLaunchKernel with the caller's events)
    gives the same bytes as an untimed one and a positive kernel duration; the setting is
    used by one launch only."""
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=11, batch=2, q_heads=q_heads, kv_heads=kv_heads, context=1024 + 40, n_quant=1024)
    cache, rc, q = _setup(w, dev)
    plain, _ = _run(cache, q, lse=False)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    kivi.kivi_time_next_attention(*ev)
    timed, _ = _run(cache, q, lse=False)
    ms = ev[0].elapsed_time(ev[1])
    assert torch.equal(timed, plain)
    assert 0.0 < ms < 1000.0, ms
    again, _ = _run(cache, q, lse=False)   # not timed: the events keep the first launch's times
    assert torch.equal(again, plain)
    assert ev[0].elapsed_time(ev[1]) == ms
    with pytest.raises(ValueError):
        kivi.kivi_time_next_attention(torch.cuda.Event(enable_timing=True), ev[1])


def test_split_count_does_not_change_the_result():
    dev = gpu_or_skip()
    w = synth.small(seed=7, batch=1, q_heads=4, kv_heads=4, context=4096 + 50, n_quant=4096, outliers=0)
    cache, rc, q = _setup(w, dev)
    groups = w.n_quant // G
    outs = {s: _check(cache, rc, q, splits=s, what=f"splits={s}")[0].float() for s in (1, 2, 7, 40, groups, groups + 5)}
    base = outs[1]
    for s, o in outs.items():
        rel = ((o - base).abs().max(-1).values / base.abs().max(-1).values).max().item()
        assert rel <= 1e-3, (s, rel)


@pytest.mark.parametrize("batch,heads,splits", [(20, 16, 0), (20, 16, 3), (26, 16, 0), (40, 16, 1)])
def test_more_query_rows_than_cus(batch, heads, splits):
    """More query rows than the chip's 256 CUs: the single-query kernel runs 4-wave workgroups,
    three per CU (320 rows: 2 splits each; 416 and 640 rows: one), all rows against the oracle."""
    dev = gpu_or_skip()
    w = synth.small(seed=60 + batch, batch=batch, q_heads=heads, kv_heads=heads, context=1536 + 45, n_quant=1536)
    cache, rc, q = _setup(w, dev)
    _check(cache, rc, q, splits=splits, what=f"{batch * heads} rows splits={splits}")


def test_llama2_7b_layer_all_rows():
    dev = gpu_or_skip()
    cache, rc, q = _setup(synth.WORKLOADS["llama2-7b-layer"], dev)
    _check(cache, rc, q, what="llama2-7b-layer")


def test_long_128k_all_rows():
    dev = gpu_or_skip()
    cache, rc, q = _setup(synth.WORKLOADS["long-128k"], dev)
    _check(cache, rc, q, what="long-128k")


def test_gqa_mistral_sampled_rows():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["gqa-mistral-7b"]
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    q = synth.query(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    out, lse = _run(cache, q)
    # oracle over 3 batch rows (all their 32 query heads / 8 kv heads)
    bsel = [0, 31, 63]
    rc = ref_cache(len(bsel), w.kv_heads, w.token_cap, k[bsel].cpu(), v[bsel].cpu(), w.n_quant)
    ref_out, ref_lse = rc.decode_attn(bits(q[bsel]), SM)
    assert_attn_close(out[bsel], ref_out, what="gqa-mistral")
    assert_lse_close(lse[bsel], ref_lse)


def test_llama2_13b_cache_layers_sampled_rows():
    dev = gpu_or_skip()
    w = synth.WORKLOADS["llama2-13b-cache"]
    kivi = _kivi()
    for layer in (0, 39):
        k, v = synth.prefill_kv(w, layer=layer, device=dev)
        q = synth.query(w, layer=layer, device=dev)
        cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
        kivi.kivi_prefill(k, v, w.n_quant, cache)
        out, lse = _run(cache, q)
        bsel = [0, 15]
        rc = ref_cache(len(bsel), w.kv_heads, w.token_cap, k[bsel].cpu(), v[bsel].cpu(), w.n_quant)
        ref_out, ref_lse = rc.decode_attn(bits(q[bsel]), SM)
        assert_attn_close(out[bsel], ref_out, what=f"13b layer {layer}")
        assert_lse_close(lse[bsel], ref_lse)
        del k, v, cache
