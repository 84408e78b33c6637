"""CPU tests of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments on the host, before any HIP call, leaving the cache state as it
was.  No kernel is launched here (no GPU in this environment)."""
import ctypes as C
import os
import re

import pytest

from kv_cache_bit_quantize_amd import kivi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = kivi.lib
FAKE = 0x7F0000000000          # aligned, never dereferenced (validation fails first)


def _declared():
    text = open(os.path.join(ROOT, "include", "kivi.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\*)\s+(kivi_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 29
    out = os.popen(f"nm -D --defined-only {kivi.LIB_PATH}").read()
    exported = set(re.findall(r" T (kivi_\w+)$", out, re.M))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert hasattr(L, n)


def _cache(**kw):
    f = dict(batch=2, kv_heads=2, head_dim=128, group=32, residual_cap=128, token_cap=256,
             n_quant=64, n_res=10, res_head=0, flags=0)
    f.update({k: v for k, v in kw.items() if k in f})
    c = kivi.kivi_cache(*[f[k] for k in ("batch", "kv_heads", "head_dim", "group", "residual_cap",
                                         "token_cap", "n_quant", "n_res", "res_head", "flags")])
    for name in ("k_codes", "v_codes", "k_sz", "v_sz", "k_res", "v_res"):
        setattr(c, name, kw.get(name, FAKE))
    return c


def _state(c):
    return c.n_quant, c.n_res, c.res_head


def test_time_next_attention_arguments():
    # no device access: the call only stores the two handles for the next attention launch
    assert L.kivi_time_next_attention(None, C.c_void_p(FAKE)) == -1      # KIVI_ERR_NULL
    assert L.kivi_time_next_attention(C.c_void_p(FAKE), None) == -1
    assert L.kivi_time_next_attention(None, None) == kivi.KIVI_OK


def test_fp16_comparator_arguments():
    """kivi_decode_attn_fp16 rejects bad arguments on the host (no kernel is launched)."""
    f = L.kivi_decode_attn_fp16
    P = C.c_void_p(FAKE)
    ws = C.c_void_p(FAKE)
    big = 1 << 30

    def call(k=P, v=P, B=2, Hkv=2, T=100, stride=128, q=P, Hq=4, out=P, lse=None, w=ws, wb=big, splits=0):
        return f(k, v, B, Hkv, T, stride, q, Hq, 0.1, out, lse, w, wb, splits, None)

    assert call(k=None) == -1 and call(q=None) == -1 and call(out=None) == -1
    assert call(T=0) == -2                          # empty context
    assert call(T=200) == -2                        # more tokens than the row stride
    assert call(Hq=3) == -2                         # q_heads not a multiple of kv_heads
    assert call(k=C.c_void_p(FAKE + 8)) == -2       # misaligned
    assert call(splits=-1) == -2
    assert call(w=None) == -5 and call(wb=16) == -5 and call(w=C.c_void_p(FAKE + 16)) == -5
    assert f(P, P, 2, 2, 100, 128, P, 4, float("nan"), P, None, ws, big, 0, None) == -2
    # host-only helpers
    s = L.kivi_decode_attn_fp16_splits(1, 32, 131072, 32)
    assert s == 24                                  # 768 workgroups for 32 single-query rows
    assert L.kivi_decode_attn_fp16_splits(64, 8, 8192, 32) == 1   # 512 query-group rows
    assert L.kivi_decode_attn_fp16_splits(1, 1, 100, 1) == 1      # short context: one split
    assert L.kivi_decode_attn_fp16_splits(1, 1, 0, 1) == -2
    need = L.kivi_decode_attn_fp16_workspace(1, 32, 131072, 32, 0)
    assert need == 256 + 256 + ((24 * 32 * 130 * 8 + 255) // 256) * 256
    assert L.kivi_decode_attn_fp16_workspace(1, 1, 0, 1, 0) == 0


def test_ragged_arguments():
    """The ragged calls check the descriptor and pointers on the host; the per-sequence
    states live on the device and are checked by the kernels (GPU tests)."""
    c = _cache(n_quant=0, n_res=0)             # the descriptor's own state is not used
    st = C.c_void_p(FAKE)
    P = C.c_void_p(FAKE)
    fa = L.kivi_append_flush_ragged
    assert fa(C.byref(c), None, P, P, None) == -1
    assert fa(C.byref(c), st, None, P, None) == -1
    assert fa(C.byref(c), C.c_void_p(FAKE + 4), P, P, None) == -2       # state not 16-byte aligned
    assert fa(C.byref(_cache(head_dim=64)), st, P, P, None) == -3
    assert fa(C.byref(_cache(k_res=0)), st, P, P, None) == -1
    fd = L.kivi_decode_attn_ragged
    ws = C.c_void_p(FAKE)
    assert fd(C.byref(c), None, P, 4, 0.1, P, None, ws, 1 << 30, 0, None) == -1
    assert fd(C.byref(c), C.c_void_p(FAKE + 8), P, 4, 0.1, P, None, ws, 1 << 30, 0, None) == -2
    assert fd(C.byref(c), st, P, 3, 0.1, P, None, ws, 1 << 30, 0, None) == -2   # q_heads % kv_heads
    assert fd(C.byref(c), st, P, 4, 0.1, P, None, ws, 16, 0, None) == -5        # workspace too small
    # split count for the longest context the cache holds: 256 tokens = 8 groups -> 1 split
    assert L.kivi_decode_attn_ragged_splits(C.byref(c), 4) == 1
    big = _cache(batch=1, kv_heads=32, token_cap=131072, n_quant=0, n_res=0)
    assert L.kivi_decode_attn_ragged_splits(C.byref(big), 32) == 32   # four times the uniform count (8)
    assert L.kivi_decode_attn_ragged_splits(C.byref(big), 31) == -2


def test_status_strings():
    for s in range(0, -8, -1):
        assert kivi.status_str(s) and kivi.status_str(s) != "unknown status"
    assert kivi.status_str(-99) == "unknown status"


def test_four_bit_codes_double_the_code_bytes():
    """KIVI_CODES_4BIT: 64 code bytes per token and head for keys and for values, the same
    pairs (160 bytes per quantized token and head at G = 32)."""
    two, four = _cache(token_cap=1024), _cache(token_cap=1024, flags=kivi.KIVI_CODES_4BIT)
    c2, p2, r2 = kivi.kivi_cache_bytes(two)
    c4, p4, r4 = kivi.kivi_cache_bytes(four)
    assert c4 == 2 * c2 and p4 == p2 and r4 == r2
    assert (c4 + p4) // (4 * 1024) == 160
    assert L.kivi_decode_attn_splits(C.byref(four), 2) >= 1


def test_four_bit_rows_hold_at_most_2_26_tokens():
    """4-bit rows are addressed with 32-bit byte offsets: token_cap up to 2^26 is accepted,
    beyond it every call that checks the cache reports KIVI_ERR_UNSUPPORTED (-3)."""
    ok = _cache(token_cap=1 << 26, flags=kivi.KIVI_CODES_4BIT)
    big = _cache(token_cap=(1 << 26) + 32, flags=kivi.KIVI_CODES_4BIT)
    two_bit = _cache(token_cap=(1 << 26) + 32)
    assert L.kivi_decode_attn_splits(C.byref(ok), 2) >= 1
    assert L.kivi_decode_attn_splits(C.byref(two_bit), 2) >= 1
    assert L.kivi_decode_attn_splits(C.byref(big), 2) == -3


def test_cache_bytes_matches_layout():
    c = _cache(batch=3, kv_heads=4, token_cap=4096)
    codes, pairs, res = kivi.kivi_cache_bytes(c)
    rows = 12
    assert codes == 2 * rows * 4096 * 32
    assert pairs == rows * 128 * 128 * 4 + rows * 4096 * 4 * 4
    assert res == 2 * rows * 128 * 128 * 2
    # 96 bytes per quantized token per head: 64 code bytes + 32 pair bytes
    assert (codes + pairs) // (rows * 4096) == 96


@pytest.mark.parametrize("G,per_token", [(32, 96), (64, 80), (128, 72)])
def test_group_sizes_supported_and_sized(G, per_token):
    """Groups of 32, 64 and 128: key pairs per G tokens, value pairs per G channels."""
    c = _cache(group=G, token_cap=1024, residual_cap=128, n_quant=G)
    assert L.kivi_decode_attn_splits(C.byref(c), 2) >= 1
    codes, pairs, _ = kivi.kivi_cache_bytes(c)
    rows = 4
    # bytes per quantized token per head: 64 code bytes + 4*128/G key-pair bytes + 4*128/G value-pair bytes
    assert (codes + pairs) // (rows * 1024) == per_token


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), -3),
    (dict(group=16), -3),
    (dict(group=48), -2),          # channels are not whole groups
    (dict(group=256), -2),
    (dict(head_dim=100), -2),
    (dict(token_cap=100), -2),
    (dict(residual_cap=100), -2),
    (dict(batch=0), -2),
    (dict(flags=4), -2),             # unknown flag bits
])
def test_shape_validation(kw, code):
    c = _cache(**kw)
    assert L.kivi_decode_attn_splits(C.byref(c), 2) == code
    assert L.kivi_quantize_k_per_channel(C.c_void_p(FAKE), 32, 32 * 128, C.byref(c), 0, None) == code


def test_quantize_argument_errors():
    c = _cache()
    st = _state(c)
    q = lambda *a: L.kivi_quantize_k_per_channel(*a)
    assert q(C.c_void_p(FAKE), 33, 33 * 128, C.byref(c), 0, None) == -2          # tokens % G
    assert q(C.c_void_p(FAKE), 32, 32 * 128, C.byref(c), 16, None) == -2         # dst % G
    assert q(C.c_void_p(FAKE), 64, 64 * 128, C.byref(c), 224, None) == -4        # past token_cap
    assert q(None, 32, 32 * 128, C.byref(c), 0, None) == -1
    assert q(C.c_void_p(FAKE), 32, 31 * 128, C.byref(c), 0, None) == -2          # stride too small
    assert q(C.c_void_p(FAKE + 2), 32, 32 * 128, C.byref(c), 0, None) == -2      # misaligned
    assert q(C.c_void_p(FAKE), 0, 0, C.byref(c), 0, None) == 0                   # empty is a no-op
    assert q(C.c_void_p(FAKE), 32, 32 * 128, None, 0, None) == -1
    v = lambda *a: L.kivi_quantize_v_per_token(*a)
    assert v(C.c_void_p(FAKE), 250, 250 * 128, C.byref(c), 10, None) == -4
    assert v(C.c_void_p(FAKE), -1, 0, C.byref(c), 0, None) == -2
    c2 = _cache(v_codes=0)
    assert v(C.c_void_p(FAKE), 1, 128, C.byref(c2), 0, None) == -1
    assert _state(c) == st


def test_prefill_argument_errors_leave_state():
    c = _cache()
    st = _state(c)
    p = lambda *a: L.kivi_prefill(*a)
    assert p(C.c_void_p(FAKE), C.c_void_p(FAKE), 300, 300 * 128, 100, C.byref(c), None) == -2  # n_quant % G
    assert p(C.c_void_p(FAKE), C.c_void_p(FAKE), 300, 300 * 128, 128, C.byref(c), None) == -4  # residual > R
    assert p(C.c_void_p(FAKE), C.c_void_p(FAKE), 600, 600 * 128, 512, C.byref(c), None) == -4  # > token_cap
    assert p(C.c_void_p(FAKE), None, 64, 64 * 128, 32, C.byref(c), None) == -1
    assert p(C.c_void_p(FAKE), C.c_void_p(FAKE), 64, 64 * 128, 96, C.byref(c), None) == -2     # n_quant > tokens
    assert _state(c) == st


def test_append_flush_errors_leave_state():
    flushed = C.c_int32(7)
    full = _cache(n_quant=256, n_res=128, res_head=32)       # flush needed, no room
    st = _state(full)
    assert L.kivi_append_flush(C.byref(full), C.c_void_p(FAKE), C.c_void_p(FAKE), C.byref(flushed), None) == -4
    assert _state(full) == st and flushed.value == 7
    for bad in (dict(n_quant=33), dict(n_res=129), dict(res_head=16), dict(res_head=128), dict(n_quant=288)):
        c = _cache(**bad)
        st = _state(c)
        assert L.kivi_append_flush(C.byref(c), C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -7
        assert _state(c) == st
    c = _cache()
    assert L.kivi_append_flush(C.byref(c), None, C.c_void_p(FAKE), None, None) == -1
    assert L.kivi_append_flush(C.byref(c), C.c_void_p(FAKE + 8), C.c_void_p(FAKE), None, None) == -2
    c = _cache(k_res=0)
    assert L.kivi_append_flush(C.byref(c), C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -1
    # flush of the whole residual (128 tokens): room for one more group is not enough
    whole = _cache(n_quant=160, n_res=128, res_head=0, flags=kivi.KIVI_FLUSH_ALL)
    st = _state(whole)
    assert L.kivi_append_flush(C.byref(whole), C.c_void_p(FAKE), C.c_void_p(FAKE), None, None) == -4
    assert _state(whole) == st
    steps = C.c_int32(7)
    assert L.kivi_decode_step(C.byref(whole), C.c_void_p(FAKE), C.c_void_p(FAKE), C.c_void_p(FAKE), 2, 0.1,
                              C.c_void_p(FAKE), None, C.c_void_p(FAKE), 1 << 30, 0, C.byref(steps), None) == -4
    assert _state(whole) == st and steps.value == 7


def test_decode_attn_argument_errors():
    c = _cache()
    ws_need = L.kivi_decode_attn_workspace(C.byref(c), 4, 0)
    a = lambda cache, q_heads=4, ws=FAKE, wsb=1 << 30, splits=0, q=FAKE, out=FAKE, sm=0.088: L.kivi_decode_attn(
        C.byref(cache), C.c_void_p(q), q_heads, sm, C.c_void_p(out), None, C.c_void_p(ws), wsb, splits, None)
    assert a(c, q_heads=3) == -2                        # not a multiple of kv_heads
    assert a(c, q=0) == -1
    assert a(c, out=0) == -1
    assert a(c, ws=0) == -5
    assert a(c, wsb=ws_need - 1) == -5
    assert a(c, ws=FAKE + 64) == -5                     # workspace alignment
    assert a(c, splits=-1) == -2
    assert a(c, splits=5000) == -2
    assert a(c, sm=float("inf")) == -2
    assert a(_cache(n_quant=0, n_res=0)) == -2          # empty context
    assert a(_cache(n_res=200)) == -7


def test_decode_step_errors_leave_state():
    """The step validates the append and the attention on the post-append state before it
    enqueues anything: every error leaves the cache state as it was."""
    flushed = C.c_int32(7)

    def step(cache, k=FAKE, v=FAKE, q=FAKE, q_heads=4, ws=FAKE, wsb=1 << 30, splits=0):
        return L.kivi_decode_step(C.byref(cache), C.c_void_p(k), C.c_void_p(v), C.c_void_p(q), q_heads, 0.088,
                                  C.c_void_p(FAKE), None, C.c_void_p(ws), wsb, splits, C.byref(flushed), None)
    cases = [(_cache(n_quant=256, n_res=128, res_head=32), {}, -4),     # flush needed, no room
             (_cache(), dict(k=0), -1), (_cache(), dict(v=FAKE + 8), -2),
             (_cache(), dict(q=0), -1), (_cache(), dict(q_heads=3), -2), (_cache(), dict(ws=0), -5),
             (_cache(), dict(splits=-1), -2), (_cache(n_res=129), {}, -7), (_cache(res_head=16), {}, -7)]
    for c, kw, code in cases:
        st = _state(c)
        assert step(c, **kw) == code, (kw, code)
        assert _state(c) == st and flushed.value == 7
    # the workspace check uses the post-append state: a flush adds a group, so the
    # requirement is computed on the cache after the append
    c = _cache(n_quant=64, n_res=128, res_head=0)
    after = _cache(n_quant=96, n_res=97, res_head=32)
    need = L.kivi_decode_attn_workspace(C.byref(after), 4, 0)
    assert step(c, wsb=need - 1) == -5 and _state(c) == (64, 128, 0)


def test_split_selection_and_workspace():
    # one 131,072-token sequence, 32 heads: plenty of splits
    c = _cache(batch=1, kv_heads=32, token_cap=131104, n_quant=131040, n_res=32)
    s = L.kivi_decode_attn_splits(C.byref(c), 32)
    assert 8 <= s <= 1024
    # header: a 256-byte status block, then 8 bytes per query row rounded up to 256
    assert L.kivi_decode_attn_workspace(C.byref(c), 32, 0) == 256 + 256 + ((s * 32 * 130 * 8 + 255) // 256) * 256
    # very short history: one split
    c = _cache(n_quant=32, n_res=0)
    assert L.kivi_decode_attn_splits(C.byref(c), 2) == 1
    assert L.kivi_decode_attn_workspace(C.byref(c), 2, 7) == 256 + 256 + ((7 * 2 * 2 * 130 * 8 + 255) // 256) * 256
    # 40 rows of 16 x 40 heads: the row header takes 16 * 40 * 8 = 5,120 bytes
    c = _cache(batch=16, kv_heads=40, token_cap=4096, n_quant=3968, n_res=128)
    assert L.kivi_decode_attn_workspace(C.byref(c), 40, 1) == 256 + 5120 + ((640 * 130 * 8 + 255) // 256) * 256


def test_decode_step_split_and_workspace_helpers():
    """The step's helpers answer for the state after its append: a full ring flushes first."""
    full = _cache(batch=1, kv_heads=32, token_cap=131104, n_quant=131008, n_res=128, res_head=0)
    after = _cache(batch=1, kv_heads=32, token_cap=131104, n_quant=131040, n_res=97, res_head=32)
    assert L.kivi_decode_step_splits(C.byref(full), 32, 0) == L.kivi_decode_attn_splits(C.byref(after), 32)
    assert L.kivi_decode_step_splits(C.byref(full), 32, 1) == L.kivi_decode_attn_rope_splits(C.byref(after), 32)
    for s in (0, 3):
        assert L.kivi_decode_step_workspace(C.byref(full), 32, s, 0) == L.kivi_decode_attn_workspace(
            C.byref(after), 32, s if s else L.kivi_decode_attn_splits(C.byref(after), 32))
    # room in the ring: the history does not change
    c = _cache(batch=1, kv_heads=32, token_cap=131104, n_quant=131040, n_res=32)
    assert L.kivi_decode_step_splits(C.byref(c), 32, 0) == L.kivi_decode_attn_splits(C.byref(c), 32)
    # flush-all moves R tokens
    fa = _cache(token_cap=512, n_quant=64, n_res=128, flags=kivi.KIVI_FLUSH_ALL)
    fa_after = _cache(token_cap=512, n_quant=192, n_res=1, res_head=0, flags=kivi.KIVI_FLUSH_ALL)
    assert L.kivi_decode_step_workspace(C.byref(fa), 4, 0, 0) == L.kivi_decode_attn_workspace(C.byref(fa_after), 4, 0)
    # errors: a flush past token_cap, a bad state, a bad head count
    assert L.kivi_decode_step_splits(C.byref(_cache(n_quant=256, n_res=128)), 4, 0) == -4
    assert L.kivi_decode_step_workspace(C.byref(_cache(n_quant=256, n_res=128)), 4, 0, 0) == 0
    assert L.kivi_decode_step_splits(C.byref(_cache(n_res=129)), 4, 0) == -7
    assert L.kivi_decode_step_splits(C.byref(_cache()), 3, 0) == -2
    assert L.kivi_decode_step_workspace(C.byref(_cache()), 4, -1, 0) == 0


def test_read_probe_arguments():
    P = C.c_void_p(FAKE)
    assert L.kivi_read_probe(None, 16, P, None) == -1
    assert L.kivi_read_probe(P, 16, None, None) == -1
    assert L.kivi_read_probe(P, 24, P, None) == -2            # not a multiple of 16
    assert L.kivi_read_probe(C.c_void_p(FAKE + 8), 16, P, None) == -2
    assert L.kivi_read_probe(P, 0, P, None) == 0              # nothing to read, nothing enqueued
    assert L.kivi_read_probe_sink_bytes() >= 4
    for fn in (L.kivi_read_probe, L.kivi_read_probe_stream):
        assert fn(None, 16, P, None) == -1
        assert fn(P, 24, P, None) == -2
        assert fn(P, 0, P, None) == 0


def test_merge_test_hook_arguments():
    assert L.kivi_test_next_attention_merge(-1, 0) == -2
    assert L.kivi_test_next_attention_merge(0, 0) == kivi.KIVI_OK   # no device access; clears the setting


def test_rope_attention_arguments():
    """kivi_decode_attn_rope rejects bad arguments on the host (no kernel is launched)."""
    f = L.kivi_decode_attn_rope
    c = _cache()
    P = C.c_void_p(FAKE)
    ws = C.c_void_p(FAKE)
    big = 1 << 30
    for base in (0.0, -1.0, float("nan"), float("inf")):
        assert f(C.byref(c), P, 4, 0.1, base, P, None, ws, big, 0, None) == -2
    assert f(C.byref(c), None, 4, 0.1, 10000.0, P, None, ws, big, 0, None) == -1
    assert f(C.byref(c), P, 3, 0.1, 10000.0, P, None, ws, big, 0, None) == -2      # q_heads % kv_heads
    assert f(C.byref(c), P, 4, 0.1, 10000.0, P, None, ws, 16, 0, None) == -5       # workspace too small
    assert f(C.byref(_cache(head_dim=64)), P, 4, 0.1, 10000.0, P, None, ws, big, 0, None) == -3
    # 2-bit rows beyond 2^27 tokens are not addressed by this kernel
    assert f(C.byref(_cache(token_cap=(1 << 27) + 32)), P, 4, 0.1, 10000.0, P, None, ws, big, 0, None) == -3
    assert f(C.byref(_cache(n_quant=40)), P, 4, 0.1, 10000.0, P, None, ws, big, 0, None) == -7


def test_rope_splits():
    c = _cache(batch=1, kv_heads=32, token_cap=131072, n_quant=131040, n_res=32)
    s = L.kivi_decode_attn_rope_splits(C.byref(c), 32)
    assert s == 768 // 32                              # 4-wave workgroups, three per CU
    small = _cache(token_cap=256, n_quant=64, n_res=10)
    assert L.kivi_decode_attn_rope_splits(C.byref(small), 4) == 1   # two key groups: fewer than the 4 waves
    assert L.kivi_decode_attn_rope_splits(C.byref(c), 33) == -2
    # grouped-query shapes take a kv head's query heads (four, three or two) in one workgroup,
    # two workgroups per CU: one round of 512, whatever the code width
    for flags in (0, kivi.KIVI_CODES_4BIT):
        g = _cache(batch=64, kv_heads=8, token_cap=8192, n_quant=8160, n_res=32, flags=flags)
        assert L.kivi_decode_attn_rope_splits(C.byref(g), 32) == 1      # 512 workgroup rows
        assert L.kivi_decode_attn_rope_splits(C.byref(g), 24) == 1      # ratio 3: 512 rows
        g = _cache(batch=32, kv_heads=8, token_cap=8192, n_quant=8160, n_res=32, flags=flags)
        assert L.kivi_decode_attn_rope_splits(C.byref(g), 24) == 2      # 256 rows
        assert L.kivi_decode_attn_rope_splits(C.byref(g), 16) == 2      # ratio 2: 256 rows
        assert L.kivi_decode_attn_rope_splits(C.byref(g), 8) == 3       # ratio 1: 256 rows of one head, 768 target


def test_rope_ragged_arguments():
    f = L.kivi_decode_attn_rope_ragged
    c = _cache(n_quant=0, n_res=0)
    P = C.c_void_p(FAKE)
    big = 1 << 30
    assert f(C.byref(c), None, P, 4, 0.1, 10000.0, P, None, P, big, 0, None) == -1    # no states
    assert f(C.byref(c), P, P, 4, 0.1, 0.0, P, None, P, big, 0, None) == -2          # base
    assert f(C.byref(c), P, P, 4, 0.1, 10000.0, P, None, P, 16, 0, None) == -5       # workspace
    s = L.kivi_decode_attn_rope_ragged_splits(C.byref(_cache(token_cap=4096)), 4)
    assert 1 <= s <= 4096 // 32 // 4                    # at least a key group for each of 4 waves


def test_rope_step_arguments_leave_the_state():
    """kivi_decode_step_rope validates the append and the attention before enqueueing
    anything and leaves the cache state as it was on an error."""
    f = L.kivi_decode_step_rope
    c = _cache(n_quant=64, n_res=10)
    P = C.c_void_p(FAKE)
    big = 1 << 30
    fl = C.c_int32(7)
    assert f(C.byref(c), P, P, P, 4, 0.1, 0.0, P, None, P, big, 0, C.byref(fl), None) == -2      # base
    assert f(C.byref(c), None, P, P, 4, 0.1, 10000.0, P, None, P, big, 0, C.byref(fl), None) == -1  # k_new
    assert f(C.byref(c), P, P, P, 4, 0.1, 10000.0, P, None, P, 16, 0, C.byref(fl), None) == -5    # workspace
    assert _state(c) == (64, 10, 0) and fl.value == 7
