"""Helpers shared by the GPU parity tests: move the same fp16 bits to the GPU library
and to the CPU oracle, and compare what comes back."""
import numpy as np
import pytest
import torch

from oracle import ref

# attention outputs: per row, max |o_gpu - o_ref| / max |o_ref| (fp32 accumulation and an
# fp16 output against the fp64 oracle)
ATTN_TOL = 2e-3
# log-sum-exp: 2e-3 absolute plus an fp32 allowance that grows with |lse|.  The kernel forms
# each logit as a binary32 sum of 128 folded products (q.zero + (q*scale).code) whose terms
# can be several times larger than the logit itself; the standard bound for such a sum is
# ~n*2^-24 of the sum of |terms|, its typical size sqrt(n)*2^-24 of it, i.e. a few 1e-6 of
# |lse| once logits reach the thousands (keys with 1e2..7e3 outlier channels do that).
LSE_REL = 2.0 ** -18

REPORT = {}      # test name -> worst relative error seen (written out by conftest)


def record(what, err):
    if what:
        REPORT[what] = max(float(err), REPORT.get(what, 0.0))


def gpu_or_skip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bits(t):
    """fp16 / int16 tensor (any device) -> numpy uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float16:
        t = t.view(torch.int16)
    return t.numpy().view(np.uint16)


_u16 = bits      # for functions whose code-width keyword is also named `bits`


def ref_cache(batch, kv_heads, token_cap, k, v, n_quant, residual_cap=128, group=32, flush_all=False, bits=2):
    """Oracle cache prefilled from fp16 tensors k, v [B, H, T, D]."""
    B, H, T, D = k.shape
    c = ref.RefCache(batch, kv_heads, D, group, residual_cap, token_cap=token_cap, flush_all=flush_all, bits=bits)
    c.prefill(_u16(k).reshape(B * H, T, D), _u16(v).reshape(B * H, T, D), n_quant)
    return c


def assert_cache_equal(gpu, oracle, rows=None, upto=None, ring=True):
    """Bit-exact comparison of the packed history (tokens < upto) and the residual ring."""
    nq = oracle.n_quant if upto is None else upto
    ng = nq if getattr(oracle, "bits", 2) == 4 else nq // 32   # 4-bit: token rows; 2-bit: 32-token tiles
    nk = nq // oracle.group                         # whole key groups (one pair per channel each)
    sel = slice(None) if rows is None else rows
    kc = gpu.k_codes[sel, :ng].cpu().numpy()
    vc = gpu.v_codes[sel, :ng].cpu().numpy()
    ks = bits(gpu.k_sz[sel, :nk])
    vs = bits(gpu.v_sz[sel, :nq])                   # value pairs are per token
    for name, a, b in (("k_codes", kc, oracle.k_codes[sel, :ng]), ("v_codes", vc, oracle.v_codes[sel, :ng]),
                       ("k_sz", ks, oracle.k_sz[sel, :nk]), ("v_sz", vs, oracle.v_sz[sel, :nq])):
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{name}: {bad.shape[0]} mismatches, first at {bad[0].tolist()}: " \
                              f"gpu {a[tuple(bad[0])]} oracle {b[tuple(bad[0])]}"
    assert gpu.state == (oracle.n_quant, oracle.n_res, oracle.res_head)
    if ring:
        assert np.array_equal(bits(gpu.k_res[sel]), oracle.k_res[sel])
        assert np.array_equal(bits(gpu.v_res[sel]), oracle.v_res[sel])


def row_errors(out_gpu, out_ref):
    """[..., D] -> per-row max |diff| / max |ref|."""
    g = out_gpu.detach().float().cpu().numpy().astype(np.float64).reshape(-1, out_ref.shape[-1])
    r = out_ref.reshape(-1, out_ref.shape[-1])
    den = np.abs(r).max(1)
    return np.abs(g - r).max(1) / np.where(den > 0, den, 1.0)


def assert_attn_close(out_gpu, out_ref, rows=None, tol=ATTN_TOL, what=""):
    err = row_errors(out_gpu, out_ref)
    if rows is not None:
        err = err[rows]
    worst = int(np.argmax(err))
    record(what, err.max())
    assert err.max() <= tol, f"{what}: worst row {worst} rel err {err.max():.3e} > {tol}"
    return float(err.max())


def assert_lse_close(lse_gpu, lse_ref, rows=None, tol=ATTN_TOL):
    g = lse_gpu.detach().cpu().numpy().astype(np.float64).reshape(-1)
    r = lse_ref.reshape(-1)
    if rows is not None:
        g, r = g[rows], r[rows]
    bound = tol + LSE_REL * np.abs(r)
    ratio = np.abs(g - r) / bound
    worst = int(np.argmax(ratio))
    assert ratio.max() <= 1.0, f"lse row {worst}: |d| {abs(g[worst] - r[worst]):.3e} > {bound[worst]:.3e} (lse {r[worst]:.1f})"


class Guard:
    """Guard bands around every device buffer the binding allocates (cache buffers,
    workspaces, outputs): each buffer is the middle of a larger allocation whose first and
    last MARGIN bytes hold the CANARY byte, and check() fails if any of them changed, i.e. a
    kernel wrote outside the buffer it was handed.  Outputs start filled with the canary too,
    so an output element the kernel never wrote fails the parity comparison.  Buffers are
    tracked by weak reference and drop out once freed."""
    MARGIN = 4096           # bytes on each side; keeps the buffer 4096-byte aligned
    CANARY = 0xA5

    def __init__(self):
        import weakref
        self._weak = weakref.ref
        self.items = []     # (weakref to the buffer, bytes, description)

    def _alloc(self, shape, dtype, device, zero):
        shape = (shape,) if isinstance(shape, int) else tuple(shape)
        n = int(np.prod(shape, dtype=np.int64)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * self.MARGIN,), self.CANARY, dtype=torch.uint8, device=device)
        t = raw[self.MARGIN:self.MARGIN + n].view(dtype).view(shape)
        if zero:
            t.zero_()
        self.items.append((self._weak(t), n, f"{dtype} {list(shape)}"))
        return t

    def zeros(self, shape, dtype, device):
        return self._alloc(shape, dtype, device, True)

    def empty(self, shape, dtype, device):
        return self._alloc(shape, dtype, device, False)

    def check(self, where=""):
        live = []
        for ref_, n, what in self.items:
            t = ref_()
            if t is not None:
                raw = torch.empty(0, dtype=torch.uint8, device=t.device).set_(t.untyped_storage())
                live.append((raw, n, what))
        self.items = [it for it in self.items if it[0]() is not None]
        if not live:
            return
        if any(raw.is_cuda for raw, _, _ in live):
            torch.cuda.synchronize()
        M, Cb = self.MARGIN, self.CANARY
        bad = torch.stack([torch.stack([(raw[:M] != Cb).any(), (raw[M + n:] != Cb).any()])
                           for raw, n, _ in live]).cpu()
        for (raw, n, what), (lo, hi) in zip(live, bad.tolist()):
            assert not (lo or hi), f"after {where}: a write {'before' if lo else 'past the end of'} the {what} " \
                                   f"buffer ({n} bytes) changed its guard band"


class SlicedRef:
    """One oracle cache per slice of the batch's sequences, driven from host threads (the
    oracle's C calls release the GIL), so that whole full-size caches can be checked in
    seconds.  Sequences are independent in the method, so the slices hold exactly what one
    oracle cache over the whole batch would."""

    def __init__(self, batch, kv_heads, token_cap, k, v, n_quant, parts=16, residual_cap=128, group=32, bits=2):
        import concurrent.futures
        parts = max(1, min(parts, batch))
        self.kv_heads = kv_heads
        self.bounds = [(i * batch // parts, (i + 1) * batch // parts) for i in range(parts)]
        self.pool = concurrent.futures.ThreadPoolExecutor(parts)
        k, v = k.cpu(), v.cpu()
        self.parts = list(self.pool.map(
            lambda b: ref_cache(b[1] - b[0], kv_heads, token_cap, k[b[0]:b[1]], v[b[0]:b[1]], n_quant,
                                residual_cap=residual_cap, group=group, bits=bits), self.bounds))

    @property
    def state(self):
        p = self.parts[0]
        return p.n_quant, p.n_res, p.res_head

    def append(self, k_new, v_new):
        """k_new, v_new: fp16 [B, Hkv, D] (any device).  Returns the flush flag."""
        kn, vn = _u16(k_new), _u16(v_new)
        H = self.kv_heads
        flags = list(self.pool.map(lambda i: self.parts[i].append(
            kn[self.bounds[i][0]:self.bounds[i][1]].reshape(-1, kn.shape[-1]),
            vn[self.bounds[i][0]:self.bounds[i][1]].reshape(-1, vn.shape[-1])), range(len(self.parts))))
        assert all(f == flags[0] for f in flags)
        return flags[0]

    def decode_attn(self, q, sm_scale):
        qb = _u16(q)
        res = list(self.pool.map(lambda i: self.parts[i].decode_attn(qb[self.bounds[i][0]:self.bounds[i][1]], sm_scale),
                                 range(len(self.parts))))
        return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])

    def decode_attn_rope(self, q, sm_scale, rope_base):
        qb = _u16(q)
        res = list(self.pool.map(
            lambda i: self.parts[i].decode_attn_rope(qb[self.bounds[i][0]:self.bounds[i][1]], sm_scale, rope_base),
            range(len(self.parts))))
        return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])

    def assert_cache_equal(self, gpu, ring=True):
        """Bit-exact comparison of the whole packed history and the residual ring, slice by slice."""
        H = self.kv_heads
        for (b0, b1), p in zip(self.bounds, self.parts):
            nq = p.n_quant
            ng = nq // 32
            nk = nq // p.group
            sel = slice(b0 * H, b1 * H)
            for name, a, b in (("k_codes", gpu.k_codes[sel, :ng].cpu().numpy(), p.k_codes[:, :ng]),
                               ("v_codes", gpu.v_codes[sel, :ng].cpu().numpy(), p.v_codes[:, :ng]),
                               ("k_sz", _u16(gpu.k_sz[sel, :nk]), p.k_sz[:, :nk]),
                               ("v_sz", _u16(gpu.v_sz[sel, :nq]), p.v_sz[:, :nq])):
                bad = np.argwhere(a != b)
                assert bad.size == 0, f"{name} rows {b0 * H}..: {bad.shape[0]} mismatches, first at {bad[0].tolist()}"
            if ring:
                assert np.array_equal(_u16(gpu.k_res[sel]), p.k_res)
                assert np.array_equal(_u16(gpu.v_res[sel]), p.v_res)
        assert gpu.state == self.state
