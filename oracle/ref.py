"""ctypes view of the CPU oracle (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
module.  It loads ``libkivi_oracle.so`` (plain C, built by ``oracle/build.py``)
and moves numpy arrays in and out; all arithmetic happens in the C oracle.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        path = os.environ.get("KIVI_ORACLE_LIB")     # an alternative build (mutation tests)
        if path is None:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        L = C.CDLL(path)
        p = C.c_void_p
        i32, i64, f32, f64 = C.c_int32, C.c_int64, C.c_float, C.c_double
        L.kivi_ref_f32_to_f16.argtypes = [f32]
        L.kivi_ref_f32_to_f16.restype = C.c_uint16
        L.kivi_ref_f16_to_f32.argtypes = [C.c_uint16]
        L.kivi_ref_f16_to_f32.restype = f32
        L.kivi_ref_f32_to_f16_array.argtypes = [p, p, C.c_size_t]
        L.kivi_ref_quant_group.argtypes = [p, C.c_ssize_t, i32, p, p, p]
        L.kivi_ref_quant_group_bits.argtypes = [p, C.c_ssize_t, i32, i32, p, p, p]
        L.kivi_ref_quantize_k.argtypes = [p, p, i32, i64, i32]
        L.kivi_ref_quantize_v.argtypes = [p, p, i32, i64, i32]
        L.kivi_ref_prefill.argtypes = [p, p, p, i32, i64, i32]
        L.kivi_ref_append.argtypes = [p, p, p]
        L.kivi_ref_append.restype = i32
        L.kivi_ref_dequant_row.argtypes = [p, i32, p, p]
        L.kivi_ref_attn_dense.argtypes = [p, p, p, i32, i32, f64, p, p]
        L.kivi_ref_decode_attn.argtypes = [p, p, i32, f32, p, p, p, i64]
        L.kivi_ref_rope.argtypes = [p, i32, i64, f64, p]
        L.kivi_ref_decode_attn_rope.argtypes = [p, p, i32, f32, f64, p, p, p, i64]
        L.kivi_ref_attn_partial.argtypes = [p, p, p, i32, i32, i32, f64, p, p, p]
        L.kivi_ref_attn_merge.argtypes = [p, p, p, i32, i32, p, p]
        L.kivi_ref_bytes_per_token.argtypes = [i64, i64, i64, i64, p, p, p]
        _LIB = L
    return _LIB


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- fp16 -------
def f32_to_f16(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().kivi_ref_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f32_scalar(h):
    return lib().kivi_ref_f16_to_f32(int(h))


# ---------------------------------------------------------- quantizer ---------
def quant_group(x_bits, bits=2):
    """One group of fp16 bit patterns -> (scale bits, zero bits, codes[n]); 2^bits levels."""
    x = _c(x_bits, np.uint16).ravel()
    s, z = C.c_uint16(), C.c_uint16()
    codes = np.zeros(x.size, np.uint8)
    if bits == 2:
        lib().kivi_ref_quant_group(_ptr(x), 1, x.size, C.byref(s), C.byref(z), _ptr(codes))
    else:
        lib().kivi_ref_quant_group_bits(_ptr(x), 1, x.size, bits, C.byref(s), C.byref(z), _ptr(codes))
    return s.value, z.value, codes


# -------------------------------------------------------------- cache ---------
class _CacheStruct(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("group", C.c_int32), ("residual_cap", C.c_int32), ("token_cap", C.c_int32),
        ("n_quant", C.c_int32), ("n_res", C.c_int32), ("res_head", C.c_int32), ("flush_all", C.c_int32),
        ("bits", C.c_int32),
        ("k_codes", C.c_void_p), ("v_codes", C.c_void_p),
        ("k_sz", C.c_void_p), ("v_sz", C.c_void_p),
        ("k_res", C.c_void_p), ("v_res", C.c_void_p),
    ]


class RefCache:
    """Host-memory cache in the documented packed layout, driven by the C oracle."""

    def __init__(self, batch, kv_heads, head_dim=128, group=32, residual_cap=128, token_cap=0, flush_all=False,
                 bits=2):
        rows = batch * kv_heads
        self.batch, self.kv_heads, self.head_dim = batch, kv_heads, head_dim
        self.group, self.residual_cap, self.token_cap = group, residual_cap, token_cap
        self.bits = bits
        if bits == 4:                              # token-major, two codes per byte
            self.k_codes = np.zeros((rows, token_cap, head_dim // 2), np.uint8)
            self.v_codes = np.zeros((rows, token_cap, head_dim // 2), np.uint8)
        else:                                      # one 1024-byte tile of codes per 32 tokens
            tiles = token_cap // 32
            self.k_codes = np.zeros((rows, tiles, 32 * head_dim // 4), np.uint8)
            self.v_codes = np.zeros((rows, tiles, 32 * head_dim // 4), np.uint8)
        self.k_sz = np.zeros((rows, token_cap // group, head_dim, 2), np.uint16)
        self.v_sz = np.zeros((rows, token_cap, head_dim // group, 2), np.uint16)
        self.k_res = np.zeros((rows, residual_cap, head_dim), np.uint16)
        self.v_res = np.zeros((rows, residual_cap, head_dim), np.uint16)
        self.s = _CacheStruct(batch, kv_heads, head_dim, group, residual_cap, token_cap, 0, 0, 0, int(flush_all), bits,
                              self.k_codes.ctypes.data, self.v_codes.ctypes.data,
                              self.k_sz.ctypes.data, self.v_sz.ctypes.data,
                              self.k_res.ctypes.data, self.v_res.ctypes.data)

    # state
    @property
    def n_quant(self):
        return self.s.n_quant

    @property
    def n_res(self):
        return self.s.n_res

    @property
    def res_head(self):
        return self.s.res_head

    def set_state(self, n_quant, n_res, res_head):
        self.s.n_quant, self.s.n_res, self.s.res_head = n_quant, n_res, res_head

    # operations
    def quantize_k(self, src, tokens, dst_off=0):
        """src: uint16 fp16 bits [rows, T, D] (T >= tokens); quantizes its first tokens."""
        src = _c(src, np.uint16)
        lib().kivi_ref_quantize_k(C.byref(self.s), _ptr(src), tokens, src.shape[1] * src.shape[2], dst_off)

    def quantize_v(self, src, tokens, dst_off=0):
        src = _c(src, np.uint16)
        lib().kivi_ref_quantize_v(C.byref(self.s), _ptr(src), tokens, src.shape[1] * src.shape[2], dst_off)

    def prefill(self, k, v, n_quant):
        k, v = _c(k, np.uint16), _c(v, np.uint16)
        tokens = k.shape[1]
        lib().kivi_ref_prefill(C.byref(self.s), _ptr(k), _ptr(v), tokens, tokens * k.shape[2], n_quant)

    def append(self, k_new, v_new):
        """k_new, v_new: uint16 [rows, D]. Returns True when a group was flushed."""
        k_new, v_new = _c(k_new, np.uint16), _c(v_new, np.uint16)
        return bool(lib().kivi_ref_append(C.byref(self.s), _ptr(k_new), _ptr(v_new)))

    def dequant_row(self, row):
        n = self.n_quant + self.n_res
        K = np.empty((n, self.head_dim), np.float64)
        V = np.empty((n, self.head_dim), np.float64)
        lib().kivi_ref_dequant_row(C.byref(self.s), row, _ptr(K), _ptr(V))
        return K, V

    def decode_attn(self, q, sm_scale, rows=None):
        """q: uint16 [B, Hq, D]. Returns (out fp64 [B, Hq, D], lse fp64 [B, Hq]).
        With `rows` (flat indices b*Hq+hq) only those rows are computed (others NaN)."""
        q = _c(q, np.uint16)
        B, Hq, D = q.shape
        out = np.full((B, Hq, D), np.nan)
        lse = np.full((B, Hq), np.nan)
        r = None if rows is None else _c(rows, np.int64)
        lib().kivi_ref_decode_attn(C.byref(self.s), _ptr(q), Hq, float(sm_scale), _ptr(out), _ptr(lse),
                                   _ptr(r), 0 if r is None else r.size)
        return out, lse


    def decode_attn_rope(self, q, sm_scale, rope_base, rows=None):
        """decode_attn over pre-RoPE keys, each turned at its sequence position (history
        token t at t, the i-th oldest residual token at n_quant + i)."""
        q = _c(q, np.uint16)
        B, Hq, D = q.shape
        out = np.full((B, Hq, D), np.nan)
        lse = np.full((B, Hq), np.nan)
        r = None if rows is None else _c(rows, np.int64)
        lib().kivi_ref_decode_attn_rope(C.byref(self.s), _ptr(q), Hq, float(sm_scale), float(rope_base),
                                        _ptr(out), _ptr(lse), _ptr(r), 0 if r is None else r.size)
        return out, lse


# ---------------------------------------------------------- attention ---------
def rope(x, pos, base):
    """Rotary embedding of x [d] (float64) at position pos."""
    x = _c(x, np.float64)
    out = np.empty_like(x)
    lib().kivi_ref_rope(_ptr(x), x.size, int(pos), float(base), _ptr(out))
    return out


def attn_dense(q, K, V, sm_scale):
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    out = np.empty(K.shape[1])
    lse = C.c_double()
    lib().kivi_ref_attn_dense(_ptr(q), _ptr(K), _ptr(V), K.shape[0], K.shape[1], float(sm_scale),
                              _ptr(out), C.byref(lse))
    return out, lse.value


def attn_partial(q, K, V, t0, t1, sm_scale):
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    m, l = C.c_double(), C.c_double()
    o = np.empty(K.shape[1])
    lib().kivi_ref_attn_partial(_ptr(q), _ptr(K), _ptr(V), t0, t1, K.shape[1], float(sm_scale),
                                C.byref(m), C.byref(l), _ptr(o))
    return m.value, l.value, o


def attn_merge(ms, ls, os_):
    ms, ls, os_ = _c(ms, np.float64), _c(ls, np.float64), _c(os_, np.float64)
    out = np.empty(os_.shape[1])
    lse = C.c_double()
    lib().kivi_ref_attn_merge(_ptr(ms), _ptr(ls), _ptr(os_), ms.size, os_.shape[1], _ptr(out), C.byref(lse))
    return out, lse.value


def bytes_per_token(layers, kv_heads, head_dim, group):
    a, b, c = C.c_int64(), C.c_int64(), C.c_int64()
    lib().kivi_ref_bytes_per_token(layers, kv_heads, head_dim, group, C.byref(a), C.byref(b), C.byref(c))
    return a.value, b.value, c.value
