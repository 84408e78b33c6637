"""The benchmark's algorithmic byte counts agree with the oracle's storage accounting
(codes + (scale, zero) pairs per token, one layer and one kv head) for 2-bit codes, and
with the 4-bit layout's own sizes."""
import importlib.util
import os

import pytest

from oracle import ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("kivi_bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("g", [32, 64, 128])
def test_two_bit_token_bytes_match_the_oracle(g):
    codes, meta, _ = ref.bytes_per_token(1, 1, 128, g)
    assert _bench().quant_token_bytes(g) == codes + meta


@pytest.mark.parametrize("g,expect", [(32, 160), (64, 144), (128, 136)])
def test_four_bit_token_bytes(g, expect):
    # 64 + 64 bytes of nibble codes, 128/g key pairs and 128/g value pairs of 4 bytes
    assert _bench().quant_token_bytes(g, bits=4) == expect == 128 + 2 * (128 // g) * 4


def test_attention_bytes_of_the_long_context():
    b = _bench()
    from kv_cache_bit_quantize_amd import synth
    w = synth.WORKLOADS["long-128k"]
    assert b.attn_bytes(w, w.n_quant, w.n_res) == 32 * (131040 * 96 + 32 * 512) + 2 * 32 * 128 * 2
    assert b.attn_bytes(w, w.n_quant, w.n_res, bits=4) == 32 * (131040 * 160 + 32 * 512) + 2 * 32 * 128 * 2
