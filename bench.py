"""Decode benchmark of the 2-bit KIVI cache on one MI355X.

One step = one decode step of the whole hot path, kivi_decode_step: the new token enters
the fp16 residual (whenever the residual is already full, the oldest 32 residual tokens
are first quantized into a new key/value group) and fused attention of one query per head
runs over the packed history plus the residual, split-K with the log-sum-exp merge in the
same launch.  A step is one kernel launch, or two when a group is flushed; --separate
times the two separate calls kivi_append_flush + kivi_decode_attn instead.  Inputs are
seeded synthetic tensors already resident in HBM when the timed region starts.

Prints ONE JSON line.  Metric: achieved HBM GB/s (algorithmic bytes / time) and tokens/s.
After the timed steps, the fp16 comparator (kivi_decode_attn_fp16: the same attention over
an uncompressed fp16 cache of the starting context) is timed the same way and reported
beside it ("fp16_comparator"; --no-fp16 skips it), and so is the ragged-batch path on a
serving batch of 64 sequences at different lengths ("ragged_batch"; --no-ragged skips it),
attention alone over the same context quantized at group sizes 64 and 128
("group_sizes"; --sweep-groups sets the list, --group the timed cache's own group size),
attention alone over the same context in 4-bit codes ("four_bit"; --four-bit-groups
sets its group sizes, empty skips it), attention over the same context stored as
pre-RoPE keys, turned at their positions inside the kernel ("pre_rope"; --no-rope skips it),
and the two prefill quantizers over the same context ("prefill_quantize": one
kivi_quantize_k_per_channel and one kivi_quantize_v_per_token call each, one kernel per call).
The other workloads ("workloads"; --no-workloads skips them) are timed by their decode steps,
and the grouped-query one also by its pre-RoPE call ("pre_rope" of its entry).
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn over 2-bit KV: achieved HBM GB/s (% of peak) and tokens/s at 1 GPU"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
D = 128
RES_TOKEN_BYTES = 512          # per kv head: fp16 key + value


def quant_token_bytes(g, bits=2):
    """Bytes of one quantized token per kv head at group size g: D*bits/8 bytes of key codes
    and as many of value codes (32 + 32 B at 2 bits, 64 + 64 B at 4), a 4-byte (scale, zero)
    per channel per g tokens for the keys and per g channels of the token for the values
    (96 B at g = 32 and 2 bits, 160 B at 4 bits)."""
    return 2 * D * bits // 8 + D * 4 // g + (D // g) * 4


QUANT_TOKEN_BYTES = quant_token_bytes(32)
def counters_file(workload):
    return os.path.join(ROOT, "profiles", f"decode_attn_{workload}_counters.json")


def attn_bytes(w, n_quant, n_res, bits=2):
    """Algorithmic HBM bytes of one decode-attention call: the packed history and the
    residual read once per kv head, q read and out written once per query head."""
    rows = w.batch * w.kv_heads
    return (rows * (n_quant * quant_token_bytes(w.group, bits) + n_res * RES_TOKEN_BYTES)
            + 2 * w.batch * w.q_heads * D * 2)


def append_bytes(w, flushed):
    """One append: read k_new, v_new and write them into the ring; a flush also reads G
    ring tokens of keys and values and writes one group of codes and pairs."""
    rows = w.batch * w.kv_heads
    b = rows * 4 * D * 2
    if flushed:
        b += rows * w.group * (RES_TOKEN_BYTES + quant_token_bytes(w.group))
    return b


def cpu_baseline(w, k, v, n_heads, steps_tokens, threads):
    """Time the CPU oracle (as it stands) on a bounded sample: the first n_heads kv heads of
    batch row 0, one decode step (append + attention), the heads split over `threads` host
    threads that each drive their own oracle cache (the oracle's C code releases the GIL)."""
    import concurrent.futures
    from oracle import ref
    from kv_cache_bit_quantize_amd import synth

    def host_bits(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    threads = max(1, min(threads, n_heads))
    bounds = [(i * n_heads // threads, (i + 1) * n_heads // threads) for i in range(threads)]
    kh, vh = host_bits(k[0, :n_heads]), host_bits(v[0, :n_heads])
    kn, vn = steps_tokens
    knh, vnh = host_bits(kn[0, :n_heads]), host_bits(vn[0, :n_heads])
    qh = host_bits(synth.query(w, step=1)[:1, :n_heads])
    caches = [ref.RefCache(1, b1 - b0, D, w.group, w.residual_cap, token_cap=w.token_cap) for b0, b1 in bounds]
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda i: caches[i].prefill(kh[bounds[i][0]:bounds[i][1]], vh[bounds[i][0]:bounds[i][1]],
                                                w.n_quant), range(threads)))
        prefill_s = time.perf_counter() - t0

        def step(i):
            b0, b1 = bounds[i]
            f = caches[i].append(knh[b0:b1], vnh[b0:b1])
            caches[i].decode_attn(qh[:, b0:b1], synth.SM_SCALE_D128)
            return f
        t0 = time.perf_counter()
        flushed = list(ex.map(step, range(threads)))[0]
        step_s = time.perf_counter() - t0
    nq, nr = caches[0].n_quant, caches[0].n_res
    qtb = quant_token_bytes(w.group)
    nbytes = n_heads * (nq * qtb + nr * RES_TOKEN_BYTES) + 2 * n_heads * D * 2 \
        + n_heads * 4 * D * 2 + (n_heads * w.group * (RES_TOKEN_BYTES + qtb) if flushed else 0)
    return {
        "value": nbytes / step_s / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"one decode step (append + fp64 attention over the dequantized cache) of {n_heads} of the "
                  f"{w.batch * w.kv_heads} kv heads of the {w.name} workload on {threads} host threads; "
                  f"{step_s:.2f} s timed (oracle prefill of the sample {prefill_s:.1f} s, untimed)",
        "tokens_per_s": (n_heads / (w.batch * w.kv_heads)) * w.batch / step_s,
        "seconds": step_s,
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_single_thread(synth, names, dev_seed_heads=1):
    """The oracle on one host thread: one decode step (append + fp64 attention) of the first kv
    head of batch row 0 of each named workload (the whole cache for the 1 x 1 tiny one)."""
    from oracle import ref
    res = []
    for name in names:
        w = synth.WORKLOADS[name]
        k, v = synth.prefill_kv(w, tokens=w.context)
        kh = k[0, :1].contiguous().view(torch.int16).numpy().view(np.uint16)
        vh = v[0, :1].contiguous().view(torch.int16).numpy().view(np.uint16)
        kn, vn = synth.step_kv(w, 0)
        knh = kn[0, :1].contiguous().view(torch.int16).numpy().view(np.uint16)
        vnh = vn[0, :1].contiguous().view(torch.int16).numpy().view(np.uint16)
        ratio = w.q_heads // w.kv_heads
        qh = synth.query(w, step=1)[:1, :ratio].contiguous().view(torch.int16).numpy().view(np.uint16)
        c = ref.RefCache(1, 1, D, w.group, w.residual_cap, token_cap=w.token_cap)
        c.prefill(kh, vh, w.n_quant)
        t0 = time.perf_counter()
        f = c.append(knh, vnh)
        c.decode_attn(qh, synth.SM_SCALE_D128)
        sec = time.perf_counter() - t0
        nbytes = c.n_quant * quant_token_bytes(w.group) + c.n_res * RES_TOKEN_BYTES + 2 * ratio * D * 2 + 4 * D * 2 \
            + (w.group * (RES_TOKEN_BYTES + quant_token_bytes(w.group)) if f else 0)
        res.append({"workload": name, "sample": f"1 of {w.batch * w.kv_heads} kv heads ({ratio} query heads), "
                    f"{c.n_quant} + {c.n_res} tokens", "seconds": round(sec, 4),
                    "value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": 1})
        del k, v
    return res


def ragged_measure(kivi, synth, dev, steps, warmup, seed=2402):
    """Ragged batch (sequences at different lengths, per-sequence state on the device): the
    query-group serving shape (batch 64, 32 query heads over 8 kv heads) with context lengths
    drawn uniformly from [512, 8192] tokens; each sequence keeps 64..95 of them in the fp16
    residual.  Times kivi_decode_attn_ragged (kernel-recorded events) against the algorithmic
    bytes of the real lengths."""
    B, Hq, Hkv, lo, hi = 64, 32, 8, 512, 8192
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, size=B)
    cache = kivi.Cache(B, Hkv, hi, device=dev)
    states, byts = [], 2 * B * Hq * D * 2
    for b, L in enumerate(lengths):
        nq = int((L - 64) // 32 * 32)
        w = synth.small(seed=seed + b, batch=1, q_heads=Hq, kv_heads=Hkv, context=int(L), n_quant=nq)
        k, v = synth.prefill_kv(w, device=dev)
        view = cache.sequence(b)
        kivi.kivi_prefill(k, v, nq, view)
        states.append(view.state)
        byts += Hkv * (nq * QUANT_TOKEN_BYTES + (int(L) - nq) * RES_TOKEN_BYTES)
    state = kivi.seq_state(states, device=dev)
    qw = synth.small(seed=seed + 999, batch=B, q_heads=Hq, kv_heads=Hkv, context=1, n_quant=0)
    queries = [synth.query(qw, step=s, device=dev) for s in range(steps + warmup)]
    out = torch.empty_like(queries[0])
    splits = kivi.kivi_decode_attn_ragged_splits(cache, Hq)
    ws = cache.workspace(Hq, splits)
    for s in range(warmup):
        kivi.kivi_decode_attn_ragged(cache, state, queries[s], synth.SM_SCALE_D128, out=out, workspace=ws)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for pair in ev:
        for e in pair:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        kivi.kivi_time_next_attention(*ev[i])
        kivi.kivi_decode_attn_ragged(cache, state, queries[warmup + i], synth.SM_SCALE_D128, out=out, workspace=ws)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    return {
        "workload": "batch 64, 32 q / 8 kv heads, context lengths uniform in [512, 8192] (seeded)",
        "tokens": int(lengths.sum()), "mean_context": round(float(lengths.mean()), 1), "splits": splits,
        "decode_attn_us": round(us, 2), "bytes_per_launch": int(byts), "achieved": round(byts / us / 1e3, 1),
        "unit": "GB/s", "frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4),
        "tokens_per_s": round(B * 1e6 / us, 1),
    }


def time_attention(kivi, cache, queries, sm, steps, warmup, rope_base=None):
    """Mean duration (us) of kivi_decode_attn (or, with rope_base, kivi_decode_attn_rope)
    launches, kernel-recorded events."""
    out = torch.empty_like(queries[0])
    hq = queries[0].shape[1]
    if rope_base is None:
        ws = cache.workspace(hq)
        call = lambda q: kivi.kivi_decode_attn(cache, q, sm, out=out, workspace=ws)
    else:
        splits = kivi.kivi_decode_attn_rope_splits(cache, hq)
        ws = cache.workspace(hq, splits)
        call = lambda q: kivi.kivi_decode_attn_rope(cache, q, sm, rope_base, out=out, num_splits=splits, workspace=ws)
    for s in range(warmup):
        call(queries[s])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for pair in ev:
        for e in pair:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        kivi.kivi_time_next_attention(*ev[i])
        call(queries[warmup + i])
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3


def rope_measure(kivi, synth, w, k, v, queries, steps, warmup, base=10000.0):
    """Attention over the same prefill stored as pre-RoPE keys (2-bit, G = 32), each key
    turned at its position inside the kernel.  Same algorithmic bytes as the plain call; the
    kernel is bound by its vector work, reported against the HBM peak like the others."""
    nq = (w.context - 32) // 32 * 32
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=k.device)
    kivi.kivi_prefill(k, v, nq, cache)
    us = time_attention(kivi, cache, queries, synth.SM_SCALE_D128, steps, warmup, rope_base=base)
    b = attn_bytes(w, nq, w.context - nq)
    ratio = w.q_heads // w.kv_heads
    kernel = "attn_rope_group_kernel" if ratio % 2 == 0 else "attn_rope_kernel"   # 2-bit, uniform batch
    res = {"kernel": kernel, "rope_base": base, "n_quant": nq, "n_res": w.context - nq,
           "splits": kivi.kivi_decode_attn_rope_splits(cache, w.q_heads), "decode_attn_us": round(us, 2),
           "bytes_per_launch": int(b), "achieved": round(b / us / 1e3, 1), "unit": "GB/s",
           "frac": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
    del cache
    return res


def prefill_measure(kivi, w, k, v, steps, warmup):
    """The prefill quantizers over the history of the prefill (n_quant tokens of every row,
    read in place from the [B, H, context, D] tensors), each call one kernel on torch's
    current stream, timed with events around it.  Algorithmic bytes per token and row: 256
    read, 32 of codes and 512/G of pairs written."""
    nq = w.n_quant
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=k.device)
    rows = w.batch * w.kv_heads
    byts = rows * nq * (D * 2 + D // 4 + (D * 4) // w.group)
    res = {}
    for name, fn, src in (("keys", kivi.kivi_quantize_k_per_channel, k), ("values", kivi.kivi_quantize_v_per_token, v)):
        x = src[:, :, :nq]
        for _ in range(warmup):
            fn(x, cache)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            fn(x, cache)
            b.record()
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        res[name] = {"us": round(us, 2), "bytes_per_call": int(byts), "achieved": round(byts / us / 1e3, 1),
                     "unit": "GB/s", "frac": round(byts / us / 1e3 / PEAK_HBM_GBS, 4)}
    res["tokens"] = nq
    del cache
    return res


def group_sweep(kivi, synth, w, k, v, queries, steps, warmup, groups, bits=2):
    """Attention alone (kivi_decode_attn) over the same prefill keys and values quantized at
    other group sizes or code widths: the history is the largest whole number of groups
    that leaves at least 32 tokens in the fp16 residual."""
    import dataclasses
    res = []
    for g in groups:
        nq = (w.context - 32) // g * g
        wg = dataclasses.replace(w, group=g, n_quant=nq)
        cache = kivi.Cache(wg.batch, wg.kv_heads, wg.token_cap, group=g, device=k.device, bits=bits)
        kivi.kivi_prefill(k, v, nq, cache)
        us = time_attention(kivi, cache, queries, synth.SM_SCALE_D128, steps, warmup)
        b = attn_bytes(wg, nq, wg.n_res, bits)
        res.append({"bits": bits, "group": g, "n_quant": nq, "n_res": wg.n_res,
                    "splits": kivi.kivi_decode_attn_splits(cache, w.q_heads),
                    "decode_attn_us": round(us, 2), "bytes_per_launch": int(b), "achieved": round(b / us / 1e3, 1),
                    "unit": "GB/s", "frac": round(b / us / 1e3 / PEAK_HBM_GBS, 4)})
        del cache
    return res


FLUSH_BYTES = 1 << 30          # untimed read between flushed launches: 4x the 256 MB Infinity Cache


def stats_us(ms_list):
    """mean / median / min of launch durations given in ms, in us"""
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return {"mean": round(float(a.mean()), 2), "median": round(float(np.median(a)), 2), "min": round(float(a.min()), 2)}


def event_pairs(n):
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for pair in ev:
        for e in pair:
            e.record()
    return ev


def read_ceiling(kivi, dev, sizes, reps=20):
    """The chip's streaming-read rate: a grid-stride 16-byte read (kivi_read_probe_stream, with the
    non-temporal loads the decode kernels stream the cache with; kivi_read_probe, with plain
    loads, beside it) over buffers of the given sizes, each read's duration from events its
    own dispatch records."""
    res = []
    for nbytes in sizes:
        nbytes = nbytes // 16 * 16
        buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        entry = {"bytes": nbytes}
        for streaming in (True, False):
            sink = kivi.kivi_read_probe(buf, streaming=streaming)
            for _ in range(3):
                kivi.kivi_read_probe(buf, sink, streaming=streaming)
            ev = event_pairs(reps)
            torch.cuda.synchronize()
            for i in range(reps):
                kivi.kivi_time_next_attention(*ev[i])
                kivi.kivi_read_probe(buf, sink, streaming=streaming)
            torch.cuda.synchronize()
            st = stats_us([a.elapsed_time(b) for a, b in ev])
            r = {"us": st, "achieved": round(nbytes / st["median"] / 1e3, 1), "unit": "GB/s",
                 "frac": round(nbytes / st["median"] / 1e3 / PEAK_HBM_GBS, 4)}
            if streaming:
                entry.update(r)
                entry["loads"] = "non-temporal"
            else:
                entry["plain_loads"] = r
        res.append(entry)
        del buf
    return res


def decode_steps_measure(kivi, synth, name, dev, steps, warmup, flush_buf, sink):
    """One single-layer workload's decode steps (kivi_decode_step: append, and attention of one
    query per head over the cache, fused into one launch when nothing is flushed), timed two
    ways: back to back (the wall clock of all steps and the attention kernels' own events; the
    working set may partly stay in the 256 MB Infinity Cache from one step to the next:
    "unflushed"), and with an untimed 1 GiB read between steps, so each attention kernel reads
    the cache from HBM ("flushed", kernel events only)."""
    w = synth.WORKLOADS[name]
    k, v = synth.prefill_kv(w, device=dev)
    res = {"workload": name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
           "context_start": w.context}
    for mode in ("unflushed", "flushed"):
        cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
        kivi.kivi_prefill(k, v, w.n_quant, cache)
        n = min(steps, w.decode_steps - warmup)
        kvs = [synth.step_kv(w, s, device=dev) for s in range(warmup + n)]
        qs = [synth.query(w, step=s + 1, device=dev) for s in range(warmup + n)]
        out = torch.empty_like(qs[0])
        ws = cache.workspace(w.q_heads)
        for s in range(warmup):
            kivi.kivi_decode_step(cache, *kvs[s], qs[s], synth.SM_SCALE_D128, out=out, workspace=ws)
        ev = event_pairs(n)
        flags, byts = [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            if mode == "flushed":
                kivi.kivi_read_probe(flush_buf, sink)
            nq, nr, _ = cache.state
            kivi.kivi_time_next_attention(*ev[i])
            _, f = kivi.kivi_decode_step(cache, *kvs[warmup + i], qs[warmup + i], synth.SM_SCALE_D128, out=out,
                                         workspace=ws)
            flags.append(f)
            nq2, nr2, _ = cache.state
            byts.append(attn_bytes(w, nq2, nr2) + append_bytes(w, f))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        one = [i for i in range(n) if not flags[i]]
        st = stats_us([ev[i][0].elapsed_time(ev[i][1]) for i in one])
        b = float(np.mean([byts[i] for i in one]))
        r = {"steps": n, "flush_steps": int(sum(map(bool, flags))), "decode_attn_us": st,
             "bytes_per_launch": int(b), "achieved": round(b / st["mean"] / 1e3, 1), "unit": "GB/s",
             "frac": round(b / st["mean"] / 1e3 / PEAK_HBM_GBS, 4)}
        if mode == "unflushed":
            r["ms_per_step"] = round(wall / n * 1e3, 5)
            r["wall_GBps"] = round(sum(byts) / wall / 1e9, 1)
            r["tokens_per_s"] = round(w.batch * n / wall, 1)
        res[mode] = r
        del cache, ws
    res["kernel"] = "attn_split_kernel (append fused)" if w.q_heads == w.kv_heads else "attn_gqa_kernel (append fused)"
    if w.q_heads != w.kv_heads:
        # the same prefill as pre-RoPE keys: the query-group form of the pre-RoPE call
        qs = [synth.query(w, step=s + 1, device=dev) for s in range(warmup + steps)]
        res["pre_rope"] = rope_measure(kivi, synth, w, k, v, qs, steps, warmup)
        del qs
    del k, v
    return res


def llama13b_measure(kivi, synth, dev, steps, warmup):
    """The 40-layer Llama-2-13B-shaped cache (16 sequences x 40 kv heads, 3,968 quantized + 128
    fp16 tokens per layer, 11.4 GB): one step is attention of one query per head over all 40
    layers, 40 back-to-back kivi_decode_attn calls on one stream (no append), timed by events
    around the step; then the same 40 calls captured once in a HIP graph and replayed, every
    replay's outputs checked against the eager step's.  The working set is 45x the Infinity
    Cache, so no flush is needed."""
    w = synth.WORKLOADS["llama2-13b-cache"]
    caches, queries, outs = [], [], []
    for layer in range(w.layers):
        k, v = synth.prefill_kv(w, layer=layer, device=dev)
        c = kivi.Cache(w.batch, w.kv_heads, w.token_cap, device=dev)
        kivi.kivi_prefill(k, v, w.n_quant, c)
        del k, v
        caches.append(c)
        queries.append(synth.query(w, layer=layer, device=dev))
        outs.append(torch.empty_like(queries[-1]))
    wss = [c.workspace(w.q_heads) for c in caches]
    per_layer = attn_bytes(w, w.n_quant, w.n_res)
    step_bytes = w.layers * per_layer

    def step():
        for c, q, o, ws in zip(caches, queries, outs, wss):
            kivi.kivi_decode_attn(c, q, synth.SM_SCALE_D128, out=o, workspace=ws)
    for _ in range(warmup):
        step()
    ev = event_pairs(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    eager = stats_us([a.elapsed_time(b) for a, b in ev])
    ref = [o.clone() for o in outs]
    # the same step as one HIP graph
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ev = event_pairs(steps)
    worst = 0.0
    for i in range(steps):
        for o in outs:
            o.zero_()
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
        torch.cuda.synchronize()
        # the kernel's waves take tile pairs from a queue, so the fp32 partition of each sum (and
        # an output's last fp16 bit) can differ between runs: compare at the parity bar
        for o, r in zip(outs, ref):
            d = (o.float() - r.float()).abs().amax(-1) / r.float().abs().amax(-1).clamp_min(1e-30)
            worst = max(worst, float(d.max()))
    graph = stats_us([a.elapsed_time(b) for a, b in ev])
    res = {"workload": "llama2-13b-cache", "layers": w.layers, "batch": w.batch, "q_heads": w.q_heads,
           "kv_heads": w.kv_heads, "n_quant": w.n_quant, "n_res": w.n_res,
           "splits": kivi.kivi_decode_attn_splits(caches[0], w.q_heads),
           "bytes_per_step": int(step_bytes), "steps": steps,
           "eager": {"step_us": eager, "achieved": round(step_bytes / eager["median"] / 1e3, 1),
                     "frac": round(step_bytes / eager["median"] / 1e3 / PEAK_HBM_GBS, 4),
                     "tokens_per_s": round(w.batch * 1e6 / eager["median"], 1)},
           "graph": {"step_us": graph, "achieved": round(step_bytes / graph["median"] / 1e3, 1),
                     "frac": round(step_bytes / graph["median"] / 1e3 / PEAK_HBM_GBS, 4),
                     "tokens_per_s": round(w.batch * 1e6 / graph["median"], 1),
                     "replay_vs_eager_max_row_rel_err": worst, "replays_match_eager": bool(worst <= 2e-3)},
           "unit": "GB/s", "timing": "events around each step (40 launches)"}
    del caches, wss, g
    return res


def read_traffic(workload):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken on the
    current kernel sources; else None."""
    from kv_cache_bit_quantize_amd import traffic
    path = counters_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != traffic.kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long-128k")
    ap.add_argument("--cpu-heads", type=int, default=32, help="kv heads in the CPU oracle sample (0: skip)")
    ap.add_argument("--cpu-threads", type=int, default=16, help="host threads for the CPU oracle sample")
    ap.add_argument("--splits", type=int, default=0, help="split count override (0: library's choice)")
    ap.add_argument("--separate", action="store_true", help="time kivi_append_flush + kivi_decode_attn")
    ap.add_argument("--no-fp16", action="store_true", help="skip the fp16 comparator")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged-batch measurement")
    ap.add_argument("--group", type=int, default=32, help="group size of the timed cache (32, 64 or 128)")
    ap.add_argument("--sweep-groups", default="64,128",
                    help="group sizes of the attention-only sweep (comma list; empty: skip)")
    ap.add_argument("--no-rope", action="store_true", help="skip the pre-RoPE attention measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill quantizer measurement")
    ap.add_argument("--four-bit-groups", default="32",
                    help="group sizes of the 4-bit attention-only measurement (comma list; empty: skip)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads (llama2-7b-layer, gqa-mistral-7b, llama2-13b-cache)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decode hot path shards "
              "by batch or kv head with no communication.", file=sys.stderr)
        sys.exit(2)

    from kv_cache_bit_quantize_amd import kivi, synth
    w = synth.WORKLOADS[args.workload]
    if w.layers != 1:
        raise SystemExit("bench.py times single-layer workloads")
    dev = torch.device("cuda:0")
    total_steps = args.warmup + args.steps
    import dataclasses
    if args.group != w.group:
        w = dataclasses.replace(w, group=args.group, n_quant=(w.context - 32) // args.group * args.group)
    if total_steps > w.token_cap - w.context:
        w = dataclasses.replace(w, decode_steps=total_steps)

    k, v = synth.prefill_kv(w, device=dev)
    cache = kivi.Cache(w.batch, w.kv_heads, w.token_cap, group=w.group, device=dev)
    kivi.kivi_prefill(k, v, w.n_quant, cache)
    steps_kv = [synth.step_kv(w, s, device=dev) for s in range(total_steps)]
    queries = [synth.query(w, step=s + 1, device=dev) for s in range(total_steps)]
    out = torch.empty_like(queries[0])
    ws = cache.workspace(w.q_heads, args.splits)
    torch.cuda.synchronize()

    def step(s, ev=None):
        if args.separate:
            f = kivi.kivi_append_flush(cache, *steps_kv[s])
            if ev is not None:
                kivi.kivi_time_next_attention(*ev)
            kivi.kivi_decode_attn(cache, queries[s], synth.SM_SCALE_D128, out=out, num_splits=args.splits,
                                  workspace=ws)
        else:
            if ev is not None:
                kivi.kivi_time_next_attention(*ev)
            _, f = kivi.kivi_decode_step(cache, *steps_kv[s], queries[s], synth.SM_SCALE_D128, out=out,
                                         num_splits=args.splits, workspace=ws)
        return f, cache.state

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # Every timed step's attention kernel records its own start and end in a pair of HIP
    # events, taken by the kernel's dispatch on the launch stream (kivi_time_next_attention:
    # no marker command enters the stream).  The events are created by one record each,
    # before the timed region.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for pair in evs:
        for e in pair:
            e.record()
    flags, states = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        f, st = step(args.warmup + i, evs[i])
        flags.append(f)
        states.append(st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # the fused kernel (attention with the append) on steps without a flush; every attention
    # launch with --separate
    one_launch = [i for i in range(args.steps) if args.separate or not flags[i]]
    attn_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in one_launch])
    step_bytes = [attn_bytes(w, nq, nr) + append_bytes(w, f) for f, (nq, nr, _) in zip(flags, states)]
    value = sum(step_bytes) / elapsed / 1e9
    launch_b = [attn_bytes(w, *states[i][:2]) + (0 if args.separate else append_bytes(w, False)) for i in one_launch]
    achieved = float(np.mean(launch_b)) / (attn_ms.mean() / 1e3) / 1e9
    splits = kivi.kivi_decode_attn_splits(cache, w.q_heads) if args.splits == 0 else args.splits

    # the same attention with an untimed 1 GiB read before each launch (Infinity Cache evicted)
    flush_buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    sink = kivi.kivi_read_probe(flush_buf)
    evf = event_pairs(args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        kivi.kivi_read_probe(flush_buf, sink)
        kivi.kivi_time_next_attention(*evf[i])
        kivi.kivi_decode_attn(cache, queries[args.warmup + i], synth.SM_SCALE_D128, out=out, num_splits=args.splits,
                              workspace=ws)
    torch.cuda.synchronize()
    nq_end, nr_end, _ = cache.state
    flushed_b = attn_bytes(w, nq_end, nr_end)
    flushed = stats_us([a.elapsed_time(b) for a, b in evf])
    flushed = {"decode_attn_us": flushed, "bytes_per_launch": int(flushed_b),
               "achieved": round(flushed_b / flushed["mean"] / 1e3, 1), "unit": "GB/s",
               "frac": round(flushed_b / flushed["mean"] / 1e3 / PEAK_HBM_GBS, 4),
               "note": "kivi_decode_attn alone, an untimed 1 GiB read before each launch"}

    # fp16 comparator: kivi_decode_attn_fp16 over the prefill's own fp16 keys and values (the
    # context the timed steps start from), the same queries, every launch timed the same way
    fp16 = None
    if not args.no_fp16:
        ws16 = torch.zeros(max(kivi.kivi_decode_attn_fp16_workspace(w.batch, w.kv_heads, w.context, w.q_heads), 256),
                           dtype=torch.uint8, device=dev)
        for s in range(args.warmup):
            kivi.kivi_decode_attn_fp16(k, v, queries[s], synth.SM_SCALE_D128, out=out, workspace=ws16)
        ev16 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for pair in ev16:
            for e in pair:
                e.record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            kivi.kivi_time_next_attention(*ev16[i])
            kivi.kivi_decode_attn_fp16(k, v, queries[args.warmup + i], synth.SM_SCALE_D128, out=out, workspace=ws16)
        torch.cuda.synchronize()
        us16 = float(np.mean([a.elapsed_time(b) for a, b in ev16])) * 1e3
        b16 = w.batch * w.kv_heads * w.context * RES_TOKEN_BYTES + 2 * w.batch * w.q_heads * D * 2
        fp16 = {
            "kernel": "attn_fp16_kernel", "tokens": w.context,
            "splits": kivi.kivi_decode_attn_fp16_splits(w.batch, w.kv_heads, w.context, w.q_heads),
            "decode_attn_us": round(us16, 2), "bytes_per_launch": b16,
            "achieved": round(b16 / us16 / 1e3, 1), "unit": "GB/s", "frac": round(b16 / us16 / 1e3 / PEAK_HBM_GBS, 4),
            "speedup_of_2bit": round(us16 / float(attn_ms.mean() * 1e3), 2),
        }
    kernel = "attn_split_kernel" if w.q_heads == w.kv_heads else "attn_gqa_kernel"

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp16",
        "dtype_detail": "2-bit codes; key logits exact on int8 MFMA (q*scale as 30-bit fixed-point digits, int32 "
                        "sums); P.V on fp16 MFMA with fp16-rounded p*scale weights, fp32 accumulation; softmax, "
                        "residual and merge in fp32; fp16 output",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
            "head_dim": D, "group": w.group, "residual": w.residual_cap, "context_start": w.context,
            "n_quant_start": w.n_quant, "splits": splits,
        },
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.batch * args.steps / elapsed, 1),
        "step_path": "separate append_flush + decode_attn" if args.separate else "fused decode_step",
        "decode_attn_us": round(float(attn_ms.mean()) * 1e3, 2),
        "decode_attn_stats_us": stats_us(attn_ms),
        "event_timed_launches": len(one_launch),
        "cache_state": "unflushed: back-to-back steps; the 403 MB working set exceeds the 256 MB Infinity Cache",
        "decode_attn_flushed": flushed,
        "attn_timing": "kernel start and end recorded by the dispatch (hipExtLaunchKernel events)",
        "flush_steps": int(sum(bool(f) for f in flags)),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel if args.separate else kernel + " (append fused)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(w.name),
            "algorithmic_bytes_per_launch": int(np.mean(launch_b)),
        },
        "cpu_baseline": None,
        "fp16_comparator": fp16,
        "ragged_batch": None,
        "group_sizes": None,
        "four_bit": None,
        "pre_rope": None,
        "prefill_quantize": None,
        "read_ceiling": None,
        "workloads": None,
    }
    del cache, ws
    groups = [int(x) for x in args.sweep_groups.split(",") if x.strip()]
    if groups:
        res["group_sizes"] = group_sweep(kivi, synth, w, k, v, queries, args.steps, args.warmup, groups)
    groups4 = [int(x) for x in args.four_bit_groups.split(",") if x.strip()]
    if groups4:
        res["four_bit"] = group_sweep(kivi, synth, w, k, v, queries, args.steps, args.warmup, groups4, bits=4)
    if not args.no_rope:
        res["pre_rope"] = rope_measure(kivi, synth, w, k, v, queries, args.steps, args.warmup)
    if not args.no_prefill:
        res["prefill_quantize"] = prefill_measure(kivi, w, k, v, min(args.steps, 20), min(args.warmup, 3))
    if not args.no_ragged:
        res["ragged_batch"] = ragged_measure(kivi, synth, dev, args.steps, args.warmup)
    if not args.no_ceiling:
        res["read_ceiling"] = read_ceiling(kivi, dev, [int(np.mean(launch_b)), FLUSH_BYTES])
    if not args.no_workloads:
        del k, v
        torch.cuda.empty_cache()
        res["workloads"] = {
            name: decode_steps_measure(kivi, synth, name, dev, args.steps, args.warmup, flush_buf, sink)
            for name in ("llama2-7b-layer", "gqa-mistral-7b")}
        res["workloads"]["llama2-13b-cache"] = llama13b_measure(kivi, synth, dev, max(20, min(args.steps, 30)),
                                                                min(args.warmup, 5))
        k, v = synth.prefill_kv(w, device=dev)
    if args.cpu_heads > 0:
        kn, vn = steps_kv[0]
        res["cpu_baseline"] = cpu_baseline(w, k, v, min(args.cpu_heads, w.kv_heads), (kn, vn),
                                           min(args.cpu_threads, os.cpu_count() or 1))
        res["cpu_baseline"]["cpu_model"] = cpu_model()
        res["cpu_baseline"]["single_thread"] = cpu_single_thread(synth, ["tiny", "llama2-7b-layer", "long-128k"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
