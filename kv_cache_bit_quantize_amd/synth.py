"""Seeded synthetic KV-cache workloads.

This module only draws random numbers; it holds none of the quantizer's or the
attention's arithmetic.  The library, the oracle, the tests and the benchmark all
take their inputs from here, and the same fp16 bits go to both sides of every
comparison.

Distributions follow what the KIVI pages report about real caches: keys carry a
few fixed outlier channels whose magnitudes are orders above the rest (up to
~7000 against a median near 0.3; article "Your KV cache doesn't have a bit
problem, it has a geometry problem", paragraph 2), values have none.
  * non-outlier keys, values and queries: N(0, 1), drawn in fp32, cast to fp16 (RNE);
  * per (layer, kv head) a fixed set of outlier channels, the same for every token,
    batch row and decode step, whose elements are N(0, 1) * m_c with a per-channel
    magnitude m_c, log-uniform in [100, 7000] (or a fixed value for the tiny case).
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    q_heads: int
    kv_heads: int
    context: int             # tokens in the cache when attention runs (before any append)
    n_quant: int             # of those, tokens in the quantized history
    layers: int = 1
    head_dim: int = 128
    group: int = 32
    residual_cap: int = 128
    decode_steps: int = 0    # append + attention steps after the prefill
    outliers: int = 4        # outlier key channels per (layer, kv head)
    outlier_mag: tuple = (100.0, 7000.0)   # log-uniform range, or (m, m) for a fixed value
    note: str = field(default="", compare=False)

    @property
    def n_res(self):
        return self.context - self.n_quant

    @property
    def token_cap(self):
        # room for every group that the decode steps can flush
        extra = self.decode_steps + self.group
        return ((self.context + extra) // self.group) * self.group


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, 1, 1, 1, 256, 128, outliers=2, outlier_mag=(50.0, 50.0),
                 note="1x1 head, 4 key groups + 128 residual tokens, one attention step"),
        Workload("llama2-7b-layer", 2, 8, 32, 32, 4096, 3968, decode_steps=64,
                 note="Llama-2-7B-shaped MHA layer, 64 append+attention steps"),
        Workload("llama2-13b-cache", 3, 16, 40, 40, 4096, 3968, layers=40,
                 note="Llama-2-13B-shaped 40-layer cache, attention over every layer per step"),
        Workload("long-128k", 4, 1, 32, 32, 131072, 131040,
                 note="one 131,072-token sequence, 32 heads, split-K attention"),
        Workload("gqa-mistral-7b", 5, 64, 32, 8, 8192, 8064, decode_steps=128,
                 note="Mistral-7B-shaped GQA (4 query heads per kv head), 128 append+attention steps"),
    ]
}

SM_SCALE_D128 = 0.08838834764831845   # 1/sqrt(128); passed to the library as binary32


def _gen(seed, *tags, device="cpu"):
    g = torch.Generator(device=device)
    h = seed
    for t in tags:
        h = (h * 1000003 + int(t) + 12345) % (2 ** 61 - 1)
    g.manual_seed(h)
    return g


def outlier_channels(w: Workload, layer: int, kv_head: int):
    """Fixed outlier channel indices and magnitudes of one (layer, kv head)."""
    g = _gen(w.seed, 1, layer, kv_head)
    idx = torch.randperm(w.head_dim, generator=g)[: w.outliers]
    lo, hi = w.outlier_mag
    u = torch.rand(w.outliers, generator=g, dtype=torch.float64)
    mag = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return idx, mag


def _to_f16(x):
    return x.clamp_(-65504.0, 65504.0).to(torch.float16)


def _key_scale(w: Workload, layer: int, device):
    """[kv_heads, head_dim] multiplier: 1 except on the outlier channels."""
    sc = torch.ones(w.kv_heads, w.head_dim, dtype=torch.float32)
    for h in range(w.kv_heads):
        idx, mag = outlier_channels(w, layer, h)
        sc[h, idx] = mag.to(torch.float32)
    return sc.to(device)


def prefill_kv(w: Workload, layer: int = 0, device="cpu", tokens=None):
    """Keys and values of the prefill context: fp16 [batch, kv_heads, tokens, head_dim]."""
    T = w.context if tokens is None else tokens
    shape = (w.batch, w.kv_heads, T, w.head_dim)
    gk = _gen(w.seed, 2, layer, device=device)
    gv = _gen(w.seed, 3, layer, device=device)
    k = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
    k.mul_(_key_scale(w, layer, device)[None, :, None, :])
    v = torch.randn(shape, generator=gv, device=device, dtype=torch.float32)
    return _to_f16(k), _to_f16(v)


def step_kv(w: Workload, step: int, layer: int = 0, device="cpu"):
    """The token appended at decode step `step`: fp16 [batch, kv_heads, head_dim] each."""
    shape = (w.batch, w.kv_heads, w.head_dim)
    gk = _gen(w.seed, 4, layer, step, device=device)
    gv = _gen(w.seed, 5, layer, step, device=device)
    k = torch.randn(shape, generator=gk, device=device, dtype=torch.float32)
    k.mul_(_key_scale(w, layer, device)[None, :, :])
    v = torch.randn(shape, generator=gv, device=device, dtype=torch.float32)
    return _to_f16(k), _to_f16(v)


def query(w: Workload, step: int = 0, layer: int = 0, device="cpu"):
    """Decode queries: fp16 [batch, q_heads, head_dim]."""
    g = _gen(w.seed, 6, layer, step, device=device)
    q = torch.randn((w.batch, w.q_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)
    return _to_f16(q)


def small(name="small", seed=7, batch=2, q_heads=2, kv_heads=2, context=320, n_quant=256,
          decode_steps=0, outliers=4, outlier_mag=(100.0, 7000.0), **kw):
    """A reduced workload for tests (same distributions, smaller shapes)."""
    return Workload(name, seed, batch, q_heads, kv_heads, context, n_quant,
                    decode_steps=decode_steps, outliers=outliers, outlier_mag=outlier_mag, **kw)
