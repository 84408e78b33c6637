"""Python binding of libkivi (include/kivi.h): argument marshalling only.

PyTorch supplies device memory and streams; every step of the quantize / append /
attention path runs in libkivi's HIP kernels.  There is no fallback: if libkivi.so is
missing, importing this module fails.
"""
import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same sources named by KIVI_LIBRARY (for example
# one with host-side sanitizers)
LIB_PATH = os.environ.get("KIVI_LIBRARY", os.path.join(_PKG, "libkivi.so"))

KIVI_OK = 0
_STATUS_NAMES = {0: "KIVI_OK", -1: "KIVI_ERR_NULL", -2: "KIVI_ERR_SHAPE", -3: "KIVI_ERR_UNSUPPORTED",
                 -4: "KIVI_ERR_CAPACITY", -5: "KIVI_ERR_WORKSPACE", -6: "KIVI_ERR_HIP", -7: "KIVI_ERR_STATE"}

EXPORTS = ["kivi_quantize_k_per_channel", "kivi_quantize_v_per_token", "kivi_prefill", "kivi_append_flush",
           "kivi_decode_attn", "kivi_decode_step", "kivi_decode_attn_splits", "kivi_decode_attn_workspace", "kivi_cache_bytes",
           "kivi_status_str", "kivi_time_next_attention", "kivi_decode_attn_fp16", "kivi_decode_attn_fp16_splits",
           "kivi_decode_attn_fp16_workspace", "kivi_append_flush_ragged", "kivi_decode_attn_ragged",
           "kivi_decode_attn_ragged_splits", "kivi_decode_attn_rope", "kivi_decode_attn_rope_splits",
           "kivi_decode_attn_rope_ragged", "kivi_decode_attn_rope_ragged_splits", "kivi_decode_step_rope",
           "kivi_decode_step_splits", "kivi_decode_step_workspace", "kivi_test_next_attention_merge",
           "kivi_decode_attn_noalloc", "kivi_read_probe", "kivi_read_probe_sink_bytes",
           "kivi_read_probe_stream"]

KIVI_FLUSH_ALL = 1        # kivi_cache.flags: a full residual is flushed whole (else its oldest group)
KIVI_CODES_4BIT = 2       # kivi_cache.flags: 4-bit codes (sixteen levels), token-major nibbles
KIVI_SEQ_CAPACITY = 1     # seq_state flags: an append was skipped (its flush would pass token_cap)
KIVI_SEQ_BAD_STATE = 2    # seq_state flags: the sequence's state was out of range and not used


class KiviError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_STATUS_NAMES.get(status, status)} ({status_str(status)})")


class kivi_cache(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("kv_heads", C.c_int32), ("head_dim", C.c_int32), ("group", C.c_int32),
        ("residual_cap", C.c_int32), ("token_cap", C.c_int32),
        ("n_quant", C.c_int32), ("n_res", C.c_int32), ("res_head", C.c_int32), ("flags", C.c_int32),
        ("k_codes", C.c_void_p), ("v_codes", C.c_void_p), ("k_sz", C.c_void_p), ("v_sz", C.c_void_p),
        ("k_res", C.c_void_p), ("v_res", C.c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libkivi.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    p, i32, i64, cp = C.c_void_p, C.c_int32, C.c_int64, C.POINTER(kivi_cache)
    L.kivi_quantize_k_per_channel.argtypes = [p, i32, i64, cp, i32, p]
    L.kivi_quantize_v_per_token.argtypes = [p, i32, i64, cp, i32, p]
    L.kivi_prefill.argtypes = [p, p, i32, i64, i32, cp, p]
    L.kivi_append_flush.argtypes = [cp, p, p, C.POINTER(i32), p]
    L.kivi_decode_attn.argtypes = [cp, p, i32, C.c_float, p, p, p, C.c_size_t, i32, p]
    L.kivi_decode_step.argtypes = [cp, p, p, p, i32, C.c_float, p, p, p, C.c_size_t, i32, C.POINTER(i32), p]
    L.kivi_decode_attn_splits.argtypes = [cp, i32]
    L.kivi_decode_attn_splits.restype = i32
    L.kivi_decode_attn_workspace.argtypes = [cp, i32, i32]
    L.kivi_decode_attn_workspace.restype = C.c_size_t
    L.kivi_cache_bytes.argtypes = [cp, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]
    L.kivi_status_str.argtypes = [C.c_int]
    L.kivi_time_next_attention.argtypes = [p, p]
    L.kivi_decode_attn_fp16.argtypes = [p, p, i32, i32, i32, i32, p, i32, C.c_float, p, p, p, C.c_size_t, i32, p]
    L.kivi_append_flush_ragged.argtypes = [cp, p, p, p, p]
    L.kivi_decode_attn_ragged.argtypes = [cp, p, p, i32, C.c_float, p, p, p, C.c_size_t, i32, p]
    L.kivi_decode_attn_rope.argtypes = [cp, p, i32, C.c_float, C.c_float, p, p, p, C.c_size_t, i32, p]
    L.kivi_decode_attn_rope_splits.argtypes = [cp, i32]
    L.kivi_decode_step_rope.argtypes = [cp, p, p, p, i32, C.c_float, C.c_float, p, p, p, C.c_size_t, i32,
                                         C.POINTER(i32), p]
    L.kivi_decode_attn_rope_ragged.argtypes = [cp, p, p, i32, C.c_float, C.c_float, p, p, p, C.c_size_t, i32, p]
    L.kivi_decode_attn_rope_ragged_splits.argtypes = [cp, i32]
    L.kivi_decode_attn_rope_ragged_splits.restype = i32
    L.kivi_decode_attn_rope_splits.restype = i32
    L.kivi_decode_attn_ragged_splits.argtypes = [cp, i32]
    L.kivi_decode_attn_ragged_splits.restype = i32
    L.kivi_decode_attn_fp16_splits.argtypes = [i32, i32, i32, i32]
    L.kivi_decode_attn_fp16_splits.restype = i32
    L.kivi_decode_attn_fp16_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.kivi_decode_attn_fp16_workspace.restype = C.c_size_t
    L.kivi_decode_step_splits.argtypes = [cp, i32, i32]
    L.kivi_decode_step_splits.restype = i32
    L.kivi_decode_step_workspace.argtypes = [cp, i32, i32, i32]
    L.kivi_decode_step_workspace.restype = C.c_size_t
    L.kivi_test_next_attention_merge.argtypes = [i32, C.c_uint32]
    L.kivi_decode_attn_noalloc.argtypes = [cp, p, i32, C.c_float, p, p, i32, p]
    L.kivi_read_probe.argtypes = [p, C.c_size_t, p, p]
    L.kivi_read_probe_stream.argtypes = [p, C.c_size_t, p, p]
    L.kivi_read_probe_sink_bytes.argtypes = []
    L.kivi_read_probe_sink_bytes.restype = C.c_size_t
    L.kivi_status_str.restype = C.c_char_p
    for name in EXPORTS:
        L[name].restype = L[name].restype if name in ("kivi_decode_attn_splits", "kivi_decode_attn_workspace",
                                                      "kivi_status_str", "kivi_decode_attn_fp16_splits",
                                                      "kivi_decode_attn_fp16_workspace",
                                                      "kivi_decode_attn_ragged_splits",
                                                      "kivi_decode_step_splits",
                                                      "kivi_decode_step_workspace",
                                                      "kivi_read_probe_sink_bytes") else C.c_int
    return L


lib = _load()


def status_str(status):
    return lib.kivi_status_str(int(status)).decode()


def _check(status, where):
    if status != KIVI_OK:
        raise KiviError(status, where)


def _stream(t):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _zeros(shape, dtype, device):
    """Every cache buffer and workspace is allocated here and every output the wrappers
    allocate in _empty, so that a caller can route them to its own allocator (a pool, or
    buffers with guard bands) by replacing these two functions."""
    return torch.zeros(shape, dtype=dtype, device=device)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class Cache:
    """Device buffers of one KIVI cache (layout of include/kivi.h) and its descriptor."""

    def __init__(self, batch, kv_heads, token_cap, head_dim=128, group=32, residual_cap=128, device="cuda",
                 flush_all=False, bits=2):
        if bits not in (2, 4):
            raise ValueError("bits must be 2 or 4")
        rows = batch * kv_heads
        u8, f16 = torch.uint8, torch.int16
        if bits == 4:                              # token-major, two codes per byte
            self.k_codes = _zeros((rows, token_cap, head_dim // 2), dtype=u8, device=device)
            self.v_codes = _zeros((rows, token_cap, head_dim // 2), dtype=u8, device=device)
        else:                                      # one 1024-byte tile of codes per 32 tokens
            tiles = token_cap // 32
            self.k_codes = _zeros((rows, tiles, 32 * head_dim // 4), dtype=u8, device=device)
            self.v_codes = _zeros((rows, tiles, 32 * head_dim // 4), dtype=u8, device=device)
        self.k_sz = _zeros((rows, token_cap // group, head_dim, 2), dtype=f16, device=device)
        self.v_sz = _zeros((rows, token_cap, head_dim // group, 2), dtype=f16, device=device)
        self.k_res = _zeros((rows, residual_cap, head_dim), dtype=f16, device=device)
        self.v_res = _zeros((rows, residual_cap, head_dim), dtype=f16, device=device)
        flags = (KIVI_FLUSH_ALL if flush_all else 0) | (KIVI_CODES_4BIT if bits == 4 else 0)
        self.c = kivi_cache(batch, kv_heads, head_dim, group, residual_cap, token_cap, 0, 0, 0,
                            flags, self.k_codes.data_ptr(), self.v_codes.data_ptr(), self.k_sz.data_ptr(),
                            self.v_sz.data_ptr(), self.k_res.data_ptr(), self.v_res.data_ptr())
        self.device = torch.device(device)
        self._ws = None

    @property
    def state(self):
        return self.c.n_quant, self.c.n_res, self.c.res_head

    def set_state(self, n_quant, n_res, res_head):
        self.c.n_quant, self.c.n_res, self.c.res_head = n_quant, n_res, res_head

    def sequence(self, b):
        """Batch-1 view of sequence b (its kv_heads rows; the buffers are shared, nothing is
        allocated), for the single-batch calls such as kivi_prefill.  Its state is its own."""
        H = self.c.kv_heads
        v = object.__new__(Cache)
        for name in ("k_codes", "v_codes", "k_sz", "v_sz", "k_res", "v_res"):
            setattr(v, name, getattr(self, name)[b * H:(b + 1) * H])
        v.c = kivi_cache(1, H, self.c.head_dim, self.c.group, self.c.residual_cap, self.c.token_cap, 0, 0, 0,
                         self.c.flags,
                         v.k_codes.data_ptr(), v.v_codes.data_ptr(), v.k_sz.data_ptr(), v.v_sz.data_ptr(),
                         v.k_res.data_ptr(), v.v_res.data_ptr())
        v.device = self.device
        v._ws = None
        return v

    def workspace(self, q_heads, num_splits=0):
        """Attention workspace for this cache, also large enough for a decode step (which
        attends on the state after its append; the library sizes both)."""
        need = max(lib.kivi_decode_attn_workspace(C.byref(self.c), q_heads, num_splits),
                   lib.kivi_decode_step_workspace(C.byref(self.c), q_heads, num_splits, 0))
        if self._ws is None or self._ws.numel() < need:
            # zero-filled: the leading per-row arrival counters must start at zero
            self._ws = _zeros(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws


def _src(t):
    """fp16 [B, H, T, D] (T*D contiguous per row) -> (pointer, tokens, row stride)."""
    if t.dtype != torch.float16:
        raise TypeError("expected float16")
    if t.dim() != 4 or not (t.stride(3) == 1 and t.stride(2) == t.shape[3] and t.stride(0) == t.stride(1) * t.shape[1]):
        raise ValueError("expected [B, H, T, D] with each (b, h) row's T*D contiguous and a common row stride")
    return _ptr(t), t.shape[2], t.stride(1)


def kivi_quantize_k_per_channel(k, cache, dst_token_off=0):
    p, T, stride = _src(k)
    _check(lib.kivi_quantize_k_per_channel(p, T, stride, C.byref(cache.c), dst_token_off, _stream(k)),
           "kivi_quantize_k_per_channel")


def kivi_quantize_v_per_token(v, cache, dst_token_off=0):
    p, T, stride = _src(v)
    _check(lib.kivi_quantize_v_per_token(p, T, stride, C.byref(cache.c), dst_token_off, _stream(v)),
           "kivi_quantize_v_per_token")


def kivi_prefill(k, v, n_quant, cache):
    pk, T, stride = _src(k)
    pv, Tv, stride_v = _src(v)
    if (T, stride) != (Tv, stride_v):
        raise ValueError("k and v must have the same shape and strides")
    _check(lib.kivi_prefill(pk, pv, T, stride, n_quant, C.byref(cache.c), _stream(k)), "kivi_prefill")


def kivi_append_flush(cache, k_new, v_new):
    """k_new, v_new: fp16 [B, Hkv, D] contiguous. Returns True if a group was flushed."""
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.dtype != torch.float16:
        raise ValueError("expected contiguous float16 [B, Hkv, D]")
    flushed = C.c_int32(0)
    _check(lib.kivi_append_flush(C.byref(cache.c), _ptr(k_new), _ptr(v_new), C.byref(flushed), _stream(k_new)),
           "kivi_append_flush")
    return bool(flushed.value)


def kivi_decode_attn(cache, q, sm_scale, out=None, lse=None, num_splits=0, workspace=None):
    """q: fp16 [B, Hq, D] contiguous. Returns out fp16 [B, Hq, D] (and lse fp32 [B, Hq] if
    `lse` is True or a tensor)."""
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else cache.workspace(Hq, num_splits)
    _check(lib.kivi_decode_attn(C.byref(cache.c), _ptr(q), Hq, float(sm_scale), _ptr(out),
                                _ptr(lse) if want_lse else None, _ptr(ws), ws.numel() * ws.element_size(),
                                num_splits, _stream(q)), "kivi_decode_attn")
    return (out, lse) if want_lse else out


NOALLOC_SCRATCH_BYTES = 8 << 20    # KIVI_NOALLOC_SCRATCH_BYTES


def kivi_decode_attn_noalloc(cache, q, sm_scale, out, lse=None, num_splits=0):
    """kivi_decode_attn on the library's per-device scratch (no workspace): q fp16 [B, Hq, D],
    out fp16 [B, Hq, D] and lse fp32 [B, Hq] (or None) supplied by the caller."""
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != torch.float16:
        raise ValueError("expected contiguous float16 out of q's shape")
    Hq = q.shape[1]
    _check(lib.kivi_decode_attn_noalloc(C.byref(cache.c), _ptr(q), Hq, float(sm_scale), _ptr(out), _ptr(lse),
                                        num_splits, _stream(q)), "kivi_decode_attn_noalloc")
    return (out, lse) if lse is not None else out


def kivi_decode_attn_rope_splits(cache, q_heads):
    s = lib.kivi_decode_attn_rope_splits(C.byref(cache.c), q_heads)
    if s < 0:
        raise KiviError(s, "kivi_decode_attn_rope_splits")
    return s


def kivi_decode_attn_rope(cache, q, sm_scale, rope_base=10000.0, out=None, lse=None, num_splits=0, workspace=None):
    """Attention over a cache of pre-RoPE keys: each key is turned by the rotary embedding at
    its sequence position before q.k (q is used as given).  Arguments and results as
    kivi_decode_attn."""
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    splits = num_splits if num_splits > 0 else kivi_decode_attn_rope_splits(cache, Hq)
    ws = workspace if workspace is not None else cache.workspace(Hq, splits)
    _check(lib.kivi_decode_attn_rope(C.byref(cache.c), _ptr(q), Hq, float(sm_scale), float(rope_base), _ptr(out),
                                     _ptr(lse) if want_lse else None, _ptr(ws), ws.numel() * ws.element_size(),
                                     splits, _stream(q)), "kivi_decode_attn_rope")
    return (out, lse) if want_lse else out


def kivi_decode_step(cache, k_new, v_new, q, sm_scale, out=None, lse=None, num_splits=0, workspace=None):
    """kivi_append_flush(cache, k_new, v_new) then kivi_decode_attn(cache, q, ...), one launch
    when no group is flushed.  Returns (out, flushed) or (out, lse, flushed) if `lse`."""
    for t in (k_new, v_new):
        if not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError("expected contiguous float16 [B, Hkv, D]")
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else cache.workspace(Hq, num_splits)
    flushed = C.c_int32(0)
    _check(lib.kivi_decode_step(C.byref(cache.c), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, float(sm_scale),
                                _ptr(out), _ptr(lse) if want_lse else None, _ptr(ws), ws.numel() * ws.element_size(),
                                num_splits, C.byref(flushed), _stream(q)), "kivi_decode_step")
    return (out, lse, bool(flushed.value)) if want_lse else (out, bool(flushed.value))


def kivi_decode_step_rope(cache, k_new, v_new, q, sm_scale, rope_base=10000.0, out=None, lse=None, num_splits=0,
                          workspace=None):
    """kivi_append_flush(cache, k_new, v_new) then kivi_decode_attn_rope(cache, q, ...), one launch
    when no group is flushed.  Returns (out, flushed) or (out, lse, flushed) if `lse`."""
    for t in (k_new, v_new):
        if not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError("expected contiguous float16 [B, Hkv, D]")
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    splits = num_splits
    if splits <= 0:   # the library's choice on the state after the append
        splits = lib.kivi_decode_step_splits(C.byref(cache.c), Hq, 1)
        if splits < 0:
            raise KiviError(splits, "kivi_decode_step_splits")
    ws = workspace if workspace is not None else cache.workspace(Hq, splits)
    flushed = C.c_int32(0)
    _check(lib.kivi_decode_step_rope(C.byref(cache.c), _ptr(k_new), _ptr(v_new), _ptr(q), Hq, float(sm_scale),
                                     float(rope_base), _ptr(out), _ptr(lse) if want_lse else None, _ptr(ws),
                                     ws.numel() * ws.element_size(), splits, C.byref(flushed), _stream(q)),
           "kivi_decode_step_rope")
    return (out, lse, bool(flushed.value)) if want_lse else (out, bool(flushed.value))


def seq_state(states, device="cuda"):
    """Ragged-batch state tensor: int32 [batch, 4] = (n_quant, n_res, res_head, flags) on the
    device, from a list of (n_quant, n_res, res_head) per sequence."""
    return torch.tensor([[int(a), int(b), int(c), 0] for a, b, c in states], dtype=torch.int32, device=device)


def kivi_append_flush_ragged(cache, state, k_new, v_new):
    """One new token per sequence (k_new, v_new fp16 [B, Hkv, D]); per-sequence flush and state
    update on the device (state: int32 [B, 4] from seq_state)."""
    for t in (k_new, v_new):
        if not t.is_contiguous() or t.dtype != torch.float16:
            raise ValueError("expected contiguous float16 [B, Hkv, D]")
    if state.dtype != torch.int32 or not state.is_contiguous():
        raise ValueError("expected contiguous int32 state [B, 4]")
    _check(lib.kivi_append_flush_ragged(C.byref(cache.c), _ptr(state), _ptr(k_new), _ptr(v_new), _stream(k_new)),
           "kivi_append_flush_ragged")


def kivi_decode_attn_ragged(cache, state, q, sm_scale, out=None, lse=None, num_splits=0, workspace=None):
    """kivi_decode_attn with per-sequence states (state: int32 [B, 4] from seq_state)."""
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    if state.dtype != torch.int32 or not state.is_contiguous():
        raise ValueError("expected contiguous int32 state [B, 4]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    splits = num_splits if num_splits > 0 else kivi_decode_attn_ragged_splits(cache, Hq)
    ws = workspace if workspace is not None else cache.workspace(Hq, splits)
    _check(lib.kivi_decode_attn_ragged(C.byref(cache.c), _ptr(state), _ptr(q), Hq, float(sm_scale), _ptr(out),
                                       _ptr(lse) if want_lse else None, _ptr(ws), ws.numel() * ws.element_size(),
                                       num_splits, _stream(q)), "kivi_decode_attn_ragged")
    return (out, lse) if want_lse else out


def kivi_decode_attn_rope_ragged(cache, state, q, sm_scale, rope_base=10000.0, out=None, lse=None, num_splits=0,
                                 workspace=None):
    """kivi_decode_attn_rope with per-sequence states (state: int32 [B, 4] from seq_state):
    each sequence's keys turned at its own positions."""
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    if state.dtype != torch.int32 or not state.is_contiguous():
        raise ValueError("expected contiguous int32 state [B, 4]")
    B, Hq, D = q.shape
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    splits = num_splits if num_splits > 0 else kivi_decode_attn_rope_ragged_splits(cache, Hq)
    ws = workspace if workspace is not None else cache.workspace(Hq, splits)
    _check(lib.kivi_decode_attn_rope_ragged(C.byref(cache.c), _ptr(state), _ptr(q), Hq, float(sm_scale),
                                            float(rope_base), _ptr(out), _ptr(lse) if want_lse else None, _ptr(ws),
                                            ws.numel() * ws.element_size(), splits, _stream(q)),
           "kivi_decode_attn_rope_ragged")
    return (out, lse) if want_lse else out


def kivi_decode_attn_rope_ragged_splits(cache, q_heads):
    s = lib.kivi_decode_attn_rope_ragged_splits(C.byref(cache.c), q_heads)
    if s < 0:
        raise KiviError(s, "kivi_decode_attn_rope_ragged_splits")
    return s


def kivi_decode_attn_ragged_splits(cache, q_heads):
    s = lib.kivi_decode_attn_ragged_splits(C.byref(cache.c), q_heads)
    if s < 0:
        raise KiviError(s, "kivi_decode_attn_ragged_splits")
    return s


def kivi_decode_attn_fp16(k, v, q, sm_scale, tokens=None, out=None, lse=None, num_splits=0, workspace=None):
    """fp16 comparator: decode attention of q (fp16 [B, Hq, D]) over a plain fp16 cache
    k, v (fp16 [B, Hkv, T_cap, D], contiguous), tokens [0, tokens) of each row (default
    T_cap).  Returns out (and lse if `lse`), like kivi_decode_attn."""
    for t in (k, v):
        if not t.is_contiguous() or t.dtype != torch.float16 or t.dim() != 4:
            raise ValueError("expected contiguous float16 k, v [B, Hkv, T, D]")
    if not q.is_contiguous() or q.dtype != torch.float16:
        raise ValueError("expected contiguous float16 q [B, Hq, D]")
    B, Hkv, T_cap, D = k.shape
    tokens = T_cap if tokens is None else tokens
    Hq = q.shape[1]
    if out is None:
        out = _empty(q.shape, dtype=q.dtype, device=q.device)
    want_lse = lse is not None and lse is not False
    if lse is True:
        lse = _empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = lib.kivi_decode_attn_fp16_workspace(B, Hkv, tokens, Hq, num_splits)
        workspace = _zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib.kivi_decode_attn_fp16(_ptr(k), _ptr(v), B, Hkv, tokens, T_cap, _ptr(q), Hq, float(sm_scale), _ptr(out),
                                     _ptr(lse) if want_lse else None, _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), num_splits, _stream(q)),
           "kivi_decode_attn_fp16")
    return (out, lse) if want_lse else out


def kivi_decode_attn_fp16_splits(batch, kv_heads, tokens, q_heads):
    s = lib.kivi_decode_attn_fp16_splits(batch, kv_heads, tokens, q_heads)
    if s < 0:
        raise KiviError(s, "kivi_decode_attn_fp16_splits")
    return s


def kivi_decode_attn_fp16_workspace(batch, kv_heads, tokens, q_heads, num_splits=0):
    return lib.kivi_decode_attn_fp16_workspace(batch, kv_heads, tokens, q_heads, num_splits)


def kivi_decode_step_splits(cache, q_heads, pre_rope=False):
    s = lib.kivi_decode_step_splits(C.byref(cache.c), q_heads, int(bool(pre_rope)))
    if s < 0:
        raise KiviError(s, "kivi_decode_step_splits")
    return s


def kivi_decode_step_workspace(cache, q_heads, num_splits=0, pre_rope=False):
    return lib.kivi_decode_step_workspace(C.byref(cache.c), q_heads, num_splits, int(bool(pre_rope)))


def kivi_test_next_attention_merge(max_polls, tag_skew):
    """Testing hook: the next attention call of this thread polls each split partial at most
    max_polls times and waits for its tag + tag_skew (tag_skew != 0: the give-up path)."""
    _check(lib.kivi_test_next_attention_merge(int(max_polls), int(tag_skew)), "kivi_test_next_attention_merge")


WS_POLL_TIMEOUT = 1   # workspace status word bit (KIVI_WS_POLL_TIMEOUT)


def workspace_status(ws):
    """The workspace's status word (its first 32-bit word; KIVI_WS_POLL_TIMEOUT bits)."""
    return int(ws[:4].view(torch.int32).item())


def kivi_read_probe(buf, sink=None, streaming=False):
    """Measurement helper: one streaming read of the whole (contiguous) device tensor `buf` on
    the current stream, with plain loads (kivi_read_probe) or non-temporal ones
    (kivi_read_probe_stream); returns the sink tensor the kernel wrote to."""
    if not buf.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if sink is None:
        sink = _empty(lib.kivi_read_probe_sink_bytes() // 4, dtype=torch.int32, device=buf.device)
    fn = lib.kivi_read_probe_stream if streaming else lib.kivi_read_probe
    _check(fn(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf)),
           "kivi_read_probe_stream" if streaming else "kivi_read_probe")
    return sink


def kivi_decode_attn_splits(cache, q_heads):
    s = lib.kivi_decode_attn_splits(C.byref(cache.c), q_heads)
    if s < 0:
        raise KiviError(s, "kivi_decode_attn_splits")
    return s


def kivi_time_next_attention(start=None, stop=None):
    """The next attention kernel launched from this thread by kivi_decode_attn or
    kivi_decode_step records its own start and end in two torch.cuda.Event(enable_timing=True)
    objects; start.elapsed_time(stop) is then that kernel's duration in ms.  The events must
    already exist on the device (record each once before); None, None clears the setting."""
    handles = []
    for ev in (start, stop):
        if ev is None:
            handles.append(None)
            continue
        if not ev.cuda_event:
            raise ValueError("record the event once before passing it (it is created on first record)")
        handles.append(C.c_void_p(ev.cuda_event))
    _check(lib.kivi_time_next_attention(*handles), "kivi_time_next_attention")


def kivi_decode_attn_workspace(cache, q_heads, num_splits=0):
    return lib.kivi_decode_attn_workspace(C.byref(cache.c), q_heads, num_splits)


def kivi_cache_bytes(cache_or_struct):
    c = cache_or_struct.c if isinstance(cache_or_struct, Cache) else cache_or_struct
    a, b, d = C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(lib.kivi_cache_bytes(C.byref(c), C.byref(a), C.byref(b), C.byref(d)), "kivi_cache_bytes")
    return a.value, b.value, d.value
