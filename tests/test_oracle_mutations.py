"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU, in a
temporary directory), builds it, and runs the oracle pin tests against that build in
a child process: at least one pin must fail.  The real oracle is never modified.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kivi_oracle.c")

# (name, text in the oracle, planted replacement, run the slow exhaustive pins too)
MUTATIONS = [
    ("scale_over_levels", "float s32 = range / top;", "float s32 = range / (top + 1.0f);", False),
    ("ties_away_from_zero", "return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;", "return f + 1.0f;", False),
    ("codes_from_fp32_scale", "float s = kivi_ref_f16_to_f32(s16);", "float s = s32;", False),
    ("reciprocal_multiply", "float t = d / s;", "float t = d * (1.0f / s);", False),
    ("no_clamp", "if (r > top) r = top;", "", False),
    ("zero_is_max", "*zero = kivi_ref_f32_to_f16(mn);", "*zero = kivi_ref_f32_to_f16(mx);", False),
    ("keep_negative_zero", "if (mn == 0.0f) mn = 0.0f;", "", False),
    ("keep_negative_zero_max", "if (mx == 0.0f) mx = 0.0f;", "", False),
    ("value_token_major_packing",
     "return (int64_t)(t / 32) * 1024 + ((tt / 8) * 16 + n) * 16 + (v / 2) * 4 + ((tt % 8) / 4) * 2 + v % 2;",
     "return (int64_t)t * 32 + v * 4 + n / 4;", False),
    ("value_chunk_order",
     "return (int64_t)(t / 32) * 1024 + ((tt / 8) * 16 + n) * 16 + (v / 2) * 4 + ((tt % 8) / 4) * 2 + v % 2;",
     "return (int64_t)(t / 32) * 1024 + (n * 4 + tt / 8) * 16 + (v / 2) * 4 + ((tt % 8) / 4) * 2 + v % 2;", False),
    ("value_byte_pairing",
     "return (int64_t)(t / 32) * 1024 + ((tt / 8) * 16 + n) * 16 + (v / 2) * 4 + ((tt % 8) / 4) * 2 + v % 2;",
     "return (int64_t)(t / 32) * 1024 + ((tt / 8) * 16 + n) * 16 + (v / 2) * 4 + (v % 2) * 2 + (tt % 8) / 4;", False),
    ("value_token_bits_reversed", "static int value_code_shift(int32_t t) { return 2 * (t % 4); }",
     "static int value_code_shift(int32_t t) { return 6 - 2 * (t % 4); }", False),
    ("value_pairs_group_major",
     "return c->v_sz + ((row * c->token_cap + t) * per_tok + k) * 2;",
     "return c->v_sz + ((row * c->token_cap + (int64_t)(t / 32) * 32) * per_tok + k * 32 + t % 32) * 2;", False),
    ("key_token_major_packing",
     "return (int64_t)(t / 32) * 1024 + ((w % 4) * 16 + tt % 16) * 16 + (tt / 16) * 8 + (w / 4) * 4 + (c % 4);",
     "return (int64_t)t * 32 + w * 4 + (c % 4);", False),
    ("key_chunk_order",
     "return (int64_t)(t / 32) * 1024 + ((w % 4) * 16 + tt % 16) * 16 + (tt / 16) * 8 + (w / 4) * 4 + (c % 4);",
     "return (int64_t)(t / 32) * 1024 + ((tt % 16) * 4 + w % 4) * 16 + (tt / 16) * 8 + (w / 4) * 4 + (c % 4);", False),
    ("keys_in_value_order", "return key ? key_code_byte(t, j) : value_code_byte(t, j);",
     "return value_code_byte(t, j);", False),
    ("key_bit_order_packing", "static int key_code_shift(int32_t j) { return 2 * ((j % 16) / 4); }",
     "static int key_code_shift(int32_t j) { return 2 * (j % 4); }", False),
    ("key_pair_per_token", "const uint16_t* kp = k_pair(c, row, t / G, j);",
     "const uint16_t* kp = k_pair(c, row, t % (c->token_cap / G), j);", False),
    ("value_pair_wrong_group", "const uint16_t* vp = v_pair(c, row, t, j / G);",
     "const uint16_t* vp = v_pair(c, row, t, j % (d / G));", False),
    ("no_softmax_scale", "logit[t] = sm_scale * acc;", "logit[t] = acc;", False),
    ("no_normalisation", "for (int32_t j = 0; j < d; ++j) out[j] /= l;", "", False),
    ("lse_without_max", "if (lse) *lse = m + log(l);", "if (lse) *lse = log(l);", False),
    ("gqa_modulo_mapping",
     "int64_t kv_row = b * c->kv_heads + hq / ratio;\n        if (kv_row != last_kv_row) {\n"
     "            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);\n            last_kv_row = kv_row;",
     "int64_t kv_row = b * c->kv_heads + hq % c->kv_heads;\n        if (kv_row != last_kv_row) {\n"
     "            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);\n            last_kv_row = kv_row;", False),
    ("rope_gqa_modulo_mapping",
     "int64_t kv_row = b * c->kv_heads + hq / ratio;\n        if (kv_row != last_kv_row) {\n"
     "            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);\n            for (int32_t t = 0;",
     "int64_t kv_row = b * c->kv_heads + hq % c->kv_heads;\n        if (kv_row != last_kv_row) {\n"
     "            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);\n            for (int32_t t = 0;", False),
    ("flush_newest_tokens", "int32_t slot = (c->res_head + i) % R;",
     "int32_t slot = (c->res_head + R - G + i) % R;", False),
    ("ring_head_not_advanced", "c->res_head = (c->res_head + G) % R;", "", False),
    ("merge_weight_sign", "double w = exp(m[s] - ms);", "double w = exp(ms - m[s]);", False),
    ("f16_ties_away", "return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "return f + 1.0;", True),
    ("f16_subnormals_flushed", "double n = rne_double(a * ldexp(1.0, 24));", "double n = 0.0;", True),
    ("bytes_meta_per_element", "*meta = (elems / group) * 2 * 2;", "*meta = elems * 2;", False),
    ("rope_sin_sign", "out[i] = x0 * cs - x1 * sn;", "out[i] = x0 * cs + x1 * sn;", False),
    ("rope_partner_sign", "out[i + h] = x1 * cs + x0 * sn;", "out[i + h] = x1 * cs - x0 * sn;", False),
    ("rope_frequency_exponent", "double w = pow(base, -2.0 * (double)i / (double)d);",
     "double w = pow(base, -1.0 * (double)i / (double)d);", False),
    ("rope_residual_positions_restart",
     "kivi_ref_rope(K + (int64_t)t * d, d, t, rope_base, Kr + (int64_t)t * d);",
     "kivi_ref_rope(K + (int64_t)t * d, d, t < c->n_quant ? t : t - c->n_quant, rope_base, Kr + (int64_t)t * d);",
     False),
    ("four_bit_high_nibble_first", "if (bits_of(c) == 4) return 4 * (j % 2);",
     "if (bits_of(c) == 4) return 4 * (1 - j % 2);", False),
    ("four_bit_channel_major", "if (bits_of(c) == 4) return (int64_t)t * (c->head_dim / 2) + j / 2;",
     "if (bits_of(c) == 4) return (int64_t)(j / 2) * c->token_cap + t;", False),
    ("four_bit_as_two_bit_levels", "kivi_ref_quant_group_bits(s_row + (int64_t)t * d + k * G, 1, G, bits_of(c),",
     "kivi_ref_quant_group_bits(s_row + (int64_t)t * d + k * G, 1, G, 2,", False),
    ("four_bit_keys_as_two_bit_levels", "kivi_ref_quant_group_bits(s_row + (int64_t)t0 * d + j, d, G, bits_of(c),",
     "kivi_ref_quant_group_bits(s_row + (int64_t)t0 * d + j, d, G, 2,", False),
]


def _build(src_text, out_dir):
    c_path = os.path.join(out_dir, "kivi_oracle.c")
    with open(c_path, "w") as f:
        f.write(src_text)
    with open(os.path.join(ROOT, "oracle", "kivi_oracle.h")) as f:
        hdr = f.read()
    with open(os.path.join(out_dir, "kivi_oracle.h"), "w") as f:
        f.write(hdr)
    lib = os.path.join(out_dir, "libmut.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-w",
                    c_path, "-o", lib, "-lm"], check=True)
    return lib


def _run_pins(lib, slow, workers=0):
    env = dict(os.environ, KIVI_ORACLE_LIB=lib)
    files = [os.path.join(ROOT, "tests", f) for f in
             # cheap pins first: with -x a caught mistake stops at its first failing pin, and
             # the brute-force quantizer pins take most of the time
             ("test_oracle_cache.py", "test_oracle_attn.py", "test_oracle_rope.py", "test_oracle_fp16.py",
              "test_oracle_quant4.py", "test_oracle_quant.py")]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu" if slow else "not gpu and not slow", *files]
    if workers:
        cmd[3:3] = ["-n", str(workers)]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def _caught(mutation):
    name, old, new, slow = mutation
    with open(SRC) as f:
        text = f.read()
    if text.count(old) != 1:
        return name, "mutation site not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        r = _run_pins(_build(text.replace(old, new), d), slow)
    return name, None if r.returncode != 0 else "passed every pin:\n" + r.stdout[-1500:]


@pytest.mark.slow
def test_every_planted_mistake_is_caught():
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_caught, MUTATIONS))
    missed = {name: why for name, why in results if why}
    assert not missed, missed


@pytest.mark.slow
def test_unmutated_copy_passes():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as d:
        r = _run_pins(_build(text, d), False, workers=max(1, min(8, os.cpu_count() or 1)))
    assert r.returncode == 0, r.stdout[-3000:]
