"""GPU parity of attention over pre-RoPE keys (kivi_decode_attn_rope) against the oracle's
kivi_ref_decode_attn_rope: keys dequantized, turned by the rotary embedding at their
sequence positions, dense fp64 attention.  Bar: per row max |o_gpu - o_ref| / max |o_ref|
<= 2e-3, lse within 2e-3 + 2^-18 |lse|.  Covers both code widths, the three group sizes,
MHA and GQA (ratios 4, 3 and 2, whose calls take a kv head's query heads in one workgroup),
explicit split counts, caches with only history or only residual, a decode
loop whose flushes move the residual ring, another rotary base, the 131,072-token shape
(angles past 10^5 radians) on sampled rows, the whole gqa-mistral-7b cache in both widths,
and ragged batches (each sequence turned at its own positions)."""
import numpy as np
import pytest
import torch

from kivi_testlib import SlicedRef, assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth
from oracle import ref

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128
D = 128
BASE = 10000.0


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _setup(w, dev, code_bits=2, flush_all=False):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, group=w.group, residual_cap=w.residual_cap, device=dev,
                       bits=code_bits, flush_all=flush_all)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=w.residual_cap,
                   group=w.group, bits=code_bits, flush_all=flush_all)
    return cache, rc


def _check(cache, rc, q, base=BASE, splits=0, rows=None, what=""):
    out, lse = _kivi().kivi_decode_attn_rope(cache, q, SM, base, lse=True, num_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = rc.decode_attn_rope(bits(q), SM, base, rows=rows)
    assert_attn_close(out, ref_out, rows=rows, what=what)
    assert_lse_close(lse, ref_lse, rows=rows)


@pytest.mark.parametrize("code_bits", [2, 4])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("q_heads,kv_heads,splits", [(4, 4, 0), (8, 2, 0), (6, 2, 3), (2, 2, 7), (4, 2, 5), (3, 1, 0)])
def test_attention(code_bits, G, q_heads, kv_heads, splits):
    dev = gpu_or_skip()
    w = synth.small(seed=600 + G + q_heads + splits, batch=2, q_heads=q_heads, kv_heads=kv_heads,
                    context=16 * G + 77, n_quant=16 * G, group=G)
    cache, rc = _setup(w, dev, code_bits)
    _check(cache, rc, synth.query(w, device=dev), splits=splits,
           what=f"rope {code_bits}-bit G={G} {q_heads}/{kv_heads} splits={splits}")


@pytest.mark.parametrize("code_bits", [2, 4])
def test_residual_only_and_history_only(code_bits):
    dev = gpu_or_skip()
    for nq, ctx in ((0, 100), (512, 512), (32, 33)):
        w = synth.small(seed=620 + nq + ctx, batch=1, q_heads=4, kv_heads=2, context=ctx, n_quant=nq)
        cache, rc = _setup(w, dev, code_bits)
        _check(cache, rc, synth.query(w, device=dev), what=f"rope {code_bits}-bit n_quant={nq} context={ctx}")


def test_other_base():
    dev = gpu_or_skip()
    w = synth.small(seed=630, batch=1, q_heads=4, kv_heads=4, context=2048 + 50, n_quant=2048)
    cache, rc = _setup(w, dev)
    _check(cache, rc, synth.query(w, device=dev), base=500000.0, what="rope base 5e5")


@pytest.mark.parametrize("code_bits,G,R,flush_all,fused", [
    (2, 32, 128, False, True), (4, 64, 128, False, False), (2, 32, 64, False, False), (2, 32, 64, True, True),
    (4, 32, 128, False, True),
])
def test_decode_loop(code_bits, G, R, flush_all, fused):
    """append then attention each step (kivi_decode_step_rope, or the two separate calls):
    flushes move tokens from the ring (positions n_quant + i) into the history (positions t)
    and the ring head advances; the fused step reads the new token from the caller's buffers."""
    dev = gpu_or_skip()
    kivi = _kivi()
    steps = R + 40
    w = synth.small(seed=640 + G + R, batch=2, q_heads=8, kv_heads=2, context=4 * G + R - 7, n_quant=4 * G,
                    group=G, residual_cap=R, decode_steps=steps + R)
    cache, rc = _setup(w, dev, code_bits, flush_all)
    for s in range(steps):
        kn, vn = synth.step_kv(w, s, device=dev)
        q = synth.query(w, step=s + 1, device=dev)
        f_ref = rc.append(bits(kn).reshape(-1, D), bits(vn).reshape(-1, D))
        if fused:
            out, lse, f = kivi.kivi_decode_step_rope(cache, kn, vn, q, SM, BASE, lse=True)
            assert bool(f) == bool(f_ref), s
            assert cache.state == (rc.n_quant, rc.n_res, rc.res_head), s
            torch.cuda.synchronize()
            ref_out, ref_lse = rc.decode_attn_rope(bits(q), SM, BASE)
            assert_attn_close(out, ref_out, what=f"rope step {code_bits}-bit step {s}")
            assert_lse_close(lse, ref_lse)
            if f or s % 32 == 0:   # the new token reached its ring slot
                torch.cuda.synchronize()
                assert_cache_equal(cache, rc)
        else:
            kivi.kivi_append_flush(cache, kn, vn)
            assert cache.state == (rc.n_quant, rc.n_res, rc.res_head), s
            _check(cache, rc, q, what=f"rope loop {code_bits}-bit step {s}")


@pytest.mark.parametrize("code_bits", [2, 4])
def test_ragged_batch(code_bits):
    """Sequences of different lengths, one empty at first: each sequence's keys turned at its
    own positions, appends with flushes in between."""
    dev = gpu_or_skip()
    kivi = _kivi()
    H, cap = 2, 2048
    lengths = [(0, 0), (1024, 100), (0, 37), (1856, 128), (96, 5)]
    B = len(lengths)
    cache = kivi.Cache(B, H, cap, device=dev, bits=code_bits)
    refs, states = [], []
    for b, (nq, nr) in enumerate(lengths):
        view = cache.sequence(b)
        if nq + nr > 0:
            wb = synth.small(seed=660 + b, batch=1, q_heads=4, kv_heads=H, context=nq + nr, n_quant=nq)
            k, v = synth.prefill_kv(wb, device=dev)
            kivi.kivi_prefill(k, v, nq, view)
            refs.append(ref_cache(1, H, cap, k.cpu(), v.cpu(), nq, bits=code_bits))
        else:
            refs.append(ref.RefCache(1, H, D, 32, 128, token_cap=cap, bits=code_bits))
        states.append(view.state)
    state = kivi.seq_state(states, device=dev)
    sw = synth.small(seed=669, batch=B, q_heads=4, kv_heads=H, context=1, n_quant=0)
    q0 = synth.query(sw, device=dev)
    out, lse = kivi.kivi_decode_attn_rope_ragged(cache, state, q0, SM, BASE, lse=True)
    torch.cuda.synchronize()
    assert not out[0].any() and bool(torch.isinf(lse[0]).all() and (lse[0] < 0).all())   # empty: 0, -inf
    for b in range(1, B):
        ref_out, ref_lse = refs[b].decode_attn_rope(bits(q0[b:b + 1]), SM, BASE)
        assert_attn_close(out[b:b + 1], ref_out, what=f"rope ragged {code_bits}-bit prefill seq {b}")
        assert_lse_close(lse[b:b + 1], ref_lse)
    for s in range(40):
        kn, vn = synth.step_kv(sw, s, device=dev)
        q = synth.query(sw, step=s + 1, device=dev)
        kivi.kivi_append_flush_ragged(cache, state, kn, vn)
        out, lse = kivi.kivi_decode_attn_rope_ragged(cache, state, q, SM, BASE, lse=True)
        torch.cuda.synchronize()
        host = state.cpu().numpy()
        for b, rc in enumerate(refs):
            rc.append(bits(kn[b]).reshape(-1, D), bits(vn[b]).reshape(-1, D))
            assert tuple(host[b, :3]) == (rc.n_quant, rc.n_res, rc.res_head), (s, b)
            ref_out, ref_lse = rc.decode_attn_rope(bits(q[b:b + 1]), SM, BASE)
            assert_attn_close(out[b:b + 1], ref_out, what=f"rope ragged {code_bits}-bit step {s} seq {b}")
            assert_lse_close(lse[b:b + 1], ref_lse)
    assert int(np.count_nonzero(state[:, 3].cpu().numpy())) == 0


def test_long_context_sampled_rows():
    """131,072 tokens, positions up to 131,071 (pair 0 turns 1 radian per position)."""
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.WORKLOADS["long-128k"]
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    q = synth.query(w, device=dev)
    out, lse = kivi.kivi_decode_attn_rope(cache, q, SM, BASE, lse=True)
    torch.cuda.synchronize()
    rows = [0, 13, 31]
    rc = ref_cache(1, len(rows), w.token_cap, k[0, rows].cpu()[None], v[0, rows].cpu()[None], w.n_quant)
    ref_out, ref_lse = rc.decode_attn_rope(bits(q[:, rows].contiguous()), SM, BASE)
    assert_attn_close(out[:, rows], ref_out, what="rope long-128k sampled rows")
    assert_lse_close(lse[:, rows], ref_lse)


@pytest.mark.parametrize("code_bits", [2, 4])
def test_gqa_mistral_sampled_kv_rows(code_bits):
    """The gqa-mistral-7b shape (64 sequences, 32 query / 8 kv heads, 8,064 history + 128
    residual tokens) at the call's own split count (four query heads per workgroup): the four
    query heads of kv rows 0, 261 and 511 against the oracle."""
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.WORKLOADS["gqa-mistral-7b"]
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev, bits=code_bits)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    q = synth.query(w, device=dev)
    out, lse = kivi.kivi_decode_attn_rope(cache, q, SM, BASE, lse=True)
    torch.cuda.synchronize()
    ratio = w.q_heads // w.kv_heads
    for kvrow in (0, 261, 511):
        b, h = divmod(kvrow, w.kv_heads)
        rc = ref_cache(1, 1, w.token_cap, k[b:b + 1, h:h + 1].cpu(), v[b:b + 1, h:h + 1].cpu(), w.n_quant,
                       bits=code_bits)
        qs = q[b:b + 1, ratio * h:ratio * (h + 1)].contiguous()
        ref_out, ref_lse = rc.decode_attn_rope(bits(qs), SM, BASE)
        assert_attn_close(out[b:b + 1, ratio * h:ratio * (h + 1)], ref_out,
                          what=f"rope {code_bits}-bit gqa-mistral-7b kv row {kvrow}")
        assert_lse_close(lse[b:b + 1, ratio * h:ratio * (h + 1)], ref_lse)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("code_bits", [2, 4])
def test_gqa_mistral_all_rows(code_bits):
    """The gqa-mistral-7b cache (64 sequences x 8 kv heads, 8,064 history + 128 residual
    tokens) in one call at its own split count: all 2,048 query rows and their lse against
    the oracle (one oracle cache per slice of the sequences, on host threads)."""
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.WORKLOADS["gqa-mistral-7b"]
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev, bits=code_bits)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    q = synth.query(w, device=dev)
    out, lse = kivi.kivi_decode_attn_rope(cache, q, SM, BASE, lse=True)
    torch.cuda.synchronize()
    rc = SlicedRef(w.batch, w.kv_heads, w.token_cap, k, v, w.n_quant, parts=16, bits=code_bits)
    del k, v
    ref_out, ref_lse = rc.decode_attn_rope(q, SM, BASE)
    assert_attn_close(out, ref_out, what=f"rope {code_bits}-bit gqa-mistral-7b all rows")
    assert_lse_close(lse, ref_lse)
