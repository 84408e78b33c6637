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
