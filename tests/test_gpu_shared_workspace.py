"""GPU parity when every attention entry point shares one workspace, in turn.

The plain and fused calls of a GQA cache group a KV head's query heads in one workgroup,
the pre-RoPE calls take one query head per workgroup, and the ragged calls plan their own
split counts; all of them keep split partials in the same workspace.  Each call's tag must
exceed every tag an earlier call of any of them left in its rows' partial slots, so the
calls here alternate on one workspace (allocated and cleared once) and every call is checked
against the oracle (2e-3 per row, lse within 2e-3 + 2^-18 |lse|).  The second test forces
the merge's bounded wait to give up (a tag no partial carries, a few polls), from the host,
and checks that the rows come out NaN, the workspace status word says so, and the next
call is exact again."""
import numpy as np
import pytest
import torch

from kivi_testlib import assert_attn_close, assert_cache_equal, assert_lse_close, bits, gpu_or_skip, ref_cache
from kv_cache_bit_quantize_amd import synth

pytestmark = pytest.mark.gpu
SM = synth.SM_SCALE_D128
BASE = 10000.0
D = 128


def _kivi():
    from kv_cache_bit_quantize_amd import kivi
    return kivi


def _setup(w, dev, code_bits):
    kivi = _kivi()
    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, residual_cap=w.residual_cap, device=dev, bits=code_bits)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    torch.cuda.synchronize()
    rc = ref_cache(w.batch, w.kv_heads, w.token_cap, k.cpu(), v.cpu(), w.n_quant, residual_cap=w.residual_cap,
                   bits=code_bits)
    return cache, rc


def _one_workspace(kivi, cache, q_heads, dev):
    """Zeroed once, large enough for every entry point's automatic and explicit split counts."""
    C = kivi.C
    splits = [0, 2, 5, kivi.kivi_decode_attn_ragged_splits(cache, q_heads),
              kivi.kivi_decode_attn_rope_ragged_splits(cache, q_heads)]
    need = max(kivi.lib.kivi_decode_attn_workspace(C.byref(cache.c), q_heads, s) for s in splits)
    need = max(need, 4 * kivi.lib.kivi_decode_attn_workspace(C.byref(cache.c), q_heads, 64))
    return torch.zeros(need, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("code_bits", [2, 4])
def test_entry_points_alternate_on_one_workspace(code_bits):
    dev = gpu_or_skip()
    kivi = _kivi()
    # GQA, 4 query heads per KV head; long enough that every entry point uses several splits
    w = synth.small(seed=900 + code_bits, batch=2, q_heads=32, kv_heads=8, context=4096 + 100, n_quant=4096,
                    decode_steps=80)
    cache, rc = _setup(w, dev, code_bits)
    ws = _one_workspace(kivi, cache, w.q_heads, dev)
    calls = ["attn", "rope", "step", "attn", "rope_ragged", "step_rope", "ragged", "attn_s5", "rope", "attn",
             "ragged", "step", "rope_s2", "attn", "step_rope", "ragged", "rope_ragged", "attn"]
    appended = 0
    for i, kind in enumerate(calls):
        q = synth.query(w, step=100 + i, device=dev)
        splits = int(kind.split("_s")[1]) if "_s" in kind else 0
        if kind.startswith("step"):
            kn, vn = synth.step_kv(w, appended, device=dev)
            appended += 1
            fn = kivi.kivi_decode_step_rope if kind == "step_rope" else kivi.kivi_decode_step
            if kind == "step_rope":
                out, lse, _ = fn(cache, kn, vn, q, SM, BASE, lse=True, workspace=ws)
            else:
                out, lse, _ = fn(cache, kn, vn, q, SM, lse=True, workspace=ws)
            rc.append(bits(kn).reshape(-1, D), bits(vn).reshape(-1, D))
        elif kind in ("ragged", "rope_ragged"):
            st = kivi.seq_state([cache.state] * w.batch, device=dev)
            if kind == "ragged":
                out, lse = kivi.kivi_decode_attn_ragged(cache, st, q, SM, lse=True, workspace=ws)
            else:
                out, lse = kivi.kivi_decode_attn_rope_ragged(cache, st, q, SM, BASE, lse=True, workspace=ws)
        elif kind.startswith("rope"):
            out, lse = kivi.kivi_decode_attn_rope(cache, q, SM, BASE, lse=True, num_splits=splits, workspace=ws)
        else:
            out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        rope = "rope" in kind
        ref_out, ref_lse = (rc.decode_attn_rope(bits(q), SM, BASE) if rope else rc.decode_attn(bits(q), SM))
        assert_attn_close(out, ref_out, what=f"shared workspace {code_bits}-bit call {i} {kind}")
        assert_lse_close(lse, ref_lse)
    assert kivi.workspace_status(ws) == 0
    assert_cache_equal(cache, rc)


def test_merge_gives_up_visibly_then_recovers():
    dev = gpu_or_skip()
    kivi = _kivi()
    w = synth.small(seed=950, batch=1, q_heads=8, kv_heads=2, context=2048 + 40, n_quant=2048)
    cache, rc = _setup(w, dev, 2)
    ws = _one_workspace(kivi, cache, w.q_heads, dev)
    q = synth.query(w, device=dev)
    ref_out, ref_lse = rc.decode_attn(bits(q), SM)
    # a plain call first: its partials and epochs stay in the workspace
    out = kivi.kivi_decode_attn(cache, q, SM, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert_attn_close(out, ref_out, what="before the forced give-up")
    # the merge waits for a tag one above its own, which no partial carries, 4 polls per value
    kivi.kivi_test_next_attention_merge(4, 1)
    out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()
    assert kivi.workspace_status(ws) == kivi.WS_POLL_TIMEOUT
    # the hook was used up; the same workspace serves the next calls exactly
    for s in (4, 3, 0):
        out, lse = kivi.kivi_decode_attn(cache, q, SM, lse=True, num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        assert_attn_close(out, ref_out, what=f"after the forced give-up, splits={s}")
        assert_lse_close(lse, ref_lse)
    assert kivi.workspace_status(ws) == kivi.WS_POLL_TIMEOUT   # never cleared by the library
    # one split: no merge, so the hook changes nothing
    ws.zero_()
    kivi.kivi_test_next_attention_merge(4, 1)
    out = kivi.kivi_decode_attn(cache, q, SM, num_splits=1, workspace=ws)
    torch.cuda.synchronize()
    assert_attn_close(out, ref_out, what="one split with the hook set")
    assert kivi.workspace_status(ws) == 0
