"""GPU parity of ragged batches (sequences of one batch at different lengths, per-sequence
state in device memory) against one oracle cache per sequence.

Each sequence is prefilled through its batch-1 view of the shared buffers; its oracle is an
independent cache of batch 1.  Codes, pairs and rings are compared bit-exactly, attention
to the bar of the other attention tests; the device states must equal the oracle's."""
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


def _ragged(seed, lengths, q_heads, kv_heads, token_cap, dev):
    """lengths: (n_quant, n_res) per sequence.  Returns the GPU cache, its device state, the
    per-sequence oracle caches and a step workload for new tokens and queries."""
    kivi = _kivi()
    B = len(lengths)
    cache = kivi.Cache(B, kv_heads, token_cap, device=dev)
    refs, states = [], []
    for b, (nq, nr) in enumerate(lengths):
        view = cache.sequence(b)
        if nq + nr > 0:
            w = synth.small(seed=seed + 17 * b, batch=1, q_heads=q_heads, kv_heads=kv_heads, context=nq + nr,
                            n_quant=nq)
            k, v = synth.prefill_kv(w, device=dev)
            kivi.kivi_prefill(k, v, nq, view)
            refs.append(ref_cache(1, kv_heads, token_cap, k.cpu(), v.cpu(), nq))
        else:
            refs.append(ref.RefCache(1, kv_heads, D, 32, 128, token_cap=token_cap))
        states.append(view.state)
    torch.cuda.synchronize()
    steps_w = synth.small(seed=seed + 1000, batch=B, q_heads=q_heads, kv_heads=kv_heads, context=1, n_quant=0)
    return cache, kivi.seq_state(states, device=dev), refs, steps_w


def _check_attn(out, lse, q, refs, what, skip=()):
    for b, rc in enumerate(refs):
        if b in skip:
            continue
        if rc.n_quant + rc.n_res == 0:   # empty context: out = 0, lse = -inf
            assert torch.count_nonzero(out[b]).item() == 0, what
            assert torch.isneginf(lse[b]).all().item(), what
            continue
        ref_out, ref_lse = rc.decode_attn(bits(q[b:b + 1]), SM)
        assert_attn_close(out[b:b + 1], ref_out, what=f"{what} seq {b}")
        assert_lse_close(lse[b:b + 1], ref_lse)


def _seq_view(cache, b, state_row):
    view = cache.sequence(b)

    class G:
        pass
    g = G()
    for name in ("k_codes", "v_codes", "k_sz", "v_sz", "k_res", "v_res"):
        setattr(g, name, getattr(view, name))
    g.state = tuple(int(x) for x in state_row[:3])
    return g


LENGTHS = [(0, 0), (0, 37), (320, 128), (1024, 5), (96, 64), (4064, 128)]


@pytest.mark.parametrize("q_heads,kv_heads,splits", [(4, 4, 0), (8, 2, 0), (4, 4, 3), (6, 2, 0)])
def test_ragged_attention(q_heads, kv_heads, splits):
    dev = gpu_or_skip()
    kivi = _kivi()
    cache, state, refs, sw = _ragged(5, LENGTHS, q_heads, kv_heads, 4096, dev)
    q = synth.query(sw, device=dev)
    out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True, num_splits=splits)
    torch.cuda.synchronize()
    _check_attn(out, lse, q, refs, f"ragged {q_heads}/{kv_heads} splits={splits}")
    assert torch.count_nonzero(state[:, 3]).item() == 0


def test_ragged_decode_steps():
    """Appends and attention, step after step, each sequence flushing at its own steps."""
    dev = gpu_or_skip()
    kivi = _kivi()
    lengths = [(64, 127), (0, 128), (32, 3), (0, 0)]
    cache, state, refs, sw = _ragged(9, lengths, 8, 2, 512, dev)
    flushes = {b: [] for b in range(len(lengths))}
    for s in range(70):
        kn, vn = synth.step_kv(sw, s, device=dev)
        q = synth.query(sw, step=s + 1, device=dev)
        kivi.kivi_append_flush_ragged(cache, state, kn, vn)
        out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True)
        torch.cuda.synchronize()
        host_state = state.cpu().numpy()
        for b, rc in enumerate(refs):
            if rc.append(bits(kn[b]).reshape(-1, D), bits(vn[b]).reshape(-1, D)):
                flushes[b].append(s)
            assert tuple(host_state[b, :3]) == (rc.n_quant, rc.n_res, rc.res_head), (s, b)
            if s % 10 == 0 or s in flushes[b] or s == 69:
                assert_cache_equal(_seq_view(cache, b, host_state[b]), rc)
        _check_attn(out, lse, q, refs, f"ragged step {s}")
    assert flushes == {0: [1, 33, 65], 1: [0, 32, 64], 2: [], 3: []}
    assert np.count_nonzero(state[:, 3].cpu().numpy()) == 0


def test_ragged_bad_state_and_capacity():
    """Out-of-range states are flagged and attend over nothing; a sequence whose flush would
    pass token_cap is flagged and left as it was; the others go on normally."""
    dev = gpu_or_skip()
    kivi = _kivi()
    # sequence 3: history at token_cap (256) with a full ring, so its next append cannot flush
    lengths = [(64, 10), (0, 0), (0, 0), (256, 128)]
    cache, state, refs, sw = _ragged(13, lengths, 4, 2, 256, dev)
    state[1, :3] = torch.tensor([33, 0, 0], dtype=torch.int32)    # history not whole groups
    state[2, :3] = torch.tensor([0, 4, 5], dtype=torch.int32)     # ring head off a group boundary
    q = synth.query(sw, device=dev)
    out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True)
    torch.cuda.synchronize()
    _check_attn(out, lse, q, refs, "ragged with bad states", skip=(1, 2))
    for b in (1, 2):
        assert torch.count_nonzero(out[b]).item() == 0 and torch.isneginf(lse[b]).all().item()
    assert state[:, 3].cpu().tolist() == [0, kivi.KIVI_SEQ_BAD_STATE, kivi.KIVI_SEQ_BAD_STATE, 0]

    before = state.cpu().numpy().copy()
    kn, vn = synth.step_kv(sw, 0, device=dev)
    kivi.kivi_append_flush_ragged(cache, state, kn, vn)
    torch.cuda.synchronize()
    after = state.cpu().numpy()
    assert not refs[0].append(bits(kn[0]).reshape(-1, D), bits(vn[0]).reshape(-1, D))
    assert tuple(after[0, :3]) == (refs[0].n_quant, refs[0].n_res, refs[0].res_head)
    assert_cache_equal(_seq_view(cache, 0, after[0]), refs[0])
    assert np.array_equal(after[1:, :3], before[1:, :3])
    assert after[:, 3].tolist() == [0, kivi.KIVI_SEQ_BAD_STATE, kivi.KIVI_SEQ_BAD_STATE, kivi.KIVI_SEQ_CAPACITY]
    assert_cache_equal(_seq_view(cache, 3, after[3]), refs[3])   # untouched


@pytest.mark.parametrize("batch,q_heads,kv_heads", [(130, 8, 2), (300, 1, 1)])
def test_many_sequences(batch, q_heads, kv_heads):
    """Batches past the plan's ranked placement (more than 64 sequences: items in sequence
    order, found chunk by chunk) and past the sequences it keeps in registers (more than 256),
    for query groups and for one query per kv head; short random contexts with empty ones."""
    dev = gpu_or_skip()
    kivi = _kivi()
    rng = np.random.default_rng(batch)
    lengths = [(32 * int(rng.integers(0, 9)), int(rng.integers(0, 129))) for _ in range(batch)]
    lengths[3] = (0, 0)
    lengths[-1] = (256, 128)
    cache, state, refs, sw = _ragged(41, lengths, q_heads, kv_heads, 512, dev)
    q = synth.query(sw, device=dev)
    out, lse = kivi.kivi_decode_attn_ragged(cache, state, q, SM, lse=True)
    torch.cuda.synchronize()
    _check_attn(out, lse, q, refs, f"ragged batch {batch} {q_heads}/{kv_heads}")
    assert torch.count_nonzero(state[:, 3]).item() == 0
