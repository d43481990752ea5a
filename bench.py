"""Benchmark: packed-KV decode attention on one MI355X.

Workload (one decode step = the decode-attention call over a whole layer):
Qwen2.5-7B-shaped layer, batch 16, 28 query heads over 4 kv heads, head_dim
128, 32768 cached tokens, keys and values packed at 4 bits with binary16
scale/zero, one bfloat16 query token per sequence.  Inputs are seeded
synthetic tensors (see kv_cache_mixed_amd/synth.py); the packed cache is
resident in HBM before timing, and the timed steps rotate over enough
independent copies of it (> 512 MiB together) that no step reads a cache the
256 MB Infinity Cache still holds.

Prints ONE JSON line.  `value` = effective HBM bandwidth of the decode step
(algorithmic bytes: packed codes + scales/zeros + q + out, divided by the step
time), `tokens_per_s` = batch / step time (attention only).  The other rows of
the path (quantize, ERS shrink, mixed-bit decode at 128K) are timed in the same
run and reported under `rows`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0

# HBM bytes of one decode_kernel launch as read by rocprofv3 counters
# (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, profiles/decode_kernel_*.md)
# for the kernel source with the given digest, and the factors that map each
# counter onto true bytes: a plain 512 MiB device copy in the same run reads
# FETCH_SIZE = 262160.5 KiB and WRITE_SIZE = 524288.0 KiB per dispatch, so the
# fetch counter is scaled by 524288/262160.5 and the write counter by 1.  The
# figure is reported only while the kernel source is unchanged.
COUNTER_TRAFFIC = {
    "source_sha256": "00f4b36e8ecfbb924845dc2833802270d4e6366c35fcf5b4ab1e53b4deabe8b8",
    "fetch_kib": 139895.0,
    "write_kib": 3664.0,
    "fetch_factor": 524288.0 / 262160.5,
    "write_factor": 1.0,
}
KERNEL_SOURCES = ("kv_cache_mixed_amd/csrc/decode_attn.hip", "kv_cache_mixed_amd/csrc/kvq_device.h")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed back-to-back steps before the warmup steps (GPU clocks ramp up over "
                         "the first tens of ms of sustained work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="time only the decode step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU work of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy three times (reference "
                         "dispatch for scaling HBM counters)")
    ap.add_argument("--case", choices=sorted(CASES),
                    help="time only the decode call of one workload (cold copies rotated), "
                         "print one line and exit -- for per-kernel profiler runs")
    return ap.parse_args()


def decode_bytes(B, H, Hq, T, k_bits, v_bits, pb):
    """algorithmic bytes of one decode call: codes + S/Z of every stored token,
    plus the bf16 query and the f32 output.  k_bits 0: mixed keys (34 B per
    token); v_bits 0: mixed values (40 B per token, four S/Z pairs)"""
    per_tok = (34 if k_bits == 0 else 16 * k_bits) + (40 if v_bits == 0 else 16 * v_bits)
    params = 2 * pb + 2 * pb * (4 if v_bits == 0 else 1)   # key S,Z (128 per 128-token tile) + value S,Z
    return B * H * T * (per_tok + params) + B * Hq * 128 * 2 + B * Hq * 128 * 4


# single decode workloads for --case: (batch, kv heads, q heads, tokens,
# key bits (0 = mixed), value bits, parameter dtype name)
CASES = {
    "qwen7b_layer_4bit": (16, 4, 28, 32768, 4, 4, "F16"),
    "qwen7b_layer_2bit": (16, 4, 28, 32768, 2, 2, "F16"),
    "qwen7b_b8_layer_2bit": (8, 4, 28, 32768, 2, 2, "F16"),
    "llama8b_layer_2bit": (16, 8, 32, 32768, 2, 2, "F16"),
    "qwen7b_b8_layer_4bit": (8, 4, 28, 32768, 4, 4, "F16"),
    "qwen7b_b8_layer_8bit": (8, 4, 28, 16384, 8, 8, "F16"),
    "qwen32b_layer_4bit": (16, 8, 40, 32768, 4, 4, "F16"),
    "qwen32b_layer_2bit": (16, 8, 40, 32768, 2, 2, "F16"),
    "qwen32b_layer_8bit": (16, 8, 40, 32768, 8, 8, "F16"),
    "llama8b_mixed_128k": (1, 8, 32, 131072, 0, 2, "E4M3"),
    "llama8b_mixed_kv_128k": (1, 8, 32, 131072, 0, 0, "E4M3"),
    "llama8b_mixed_32k_b8": (8, 8, 32, 32768, 0, 2, "E4M3"),
}


def decode_case(name, steps, warmup):
    """decode calls of one workload over rotated cache copies (> 600 MB
    together); prints one JSON line with the event-timed call average"""
    print(json.dumps(decode_case_row(name, steps, warmup)))


def decode_case_row(name, steps, warmup):
    """the timing of decode_case() as a dict"""
    import torch
    from kv_cache_mixed_amd import kvq, synth
    kvq.load()
    dev = torch.device("cuda:0")
    B, H, Hq, T, kb, vb, pname = CASES[name]
    pdt = getattr(kvq, pname)
    scale = 1.0 / math.sqrt(128)
    if kb == 0 and vb == 0:
        inp = synth.mixed_kv_layer_device(B, H, Hq, T, seed=4, device=dev)
        mk = lambda: kvq.PackedCache(B, H, T, kvq.KMIXED, kvq.VMIXED, pdt, slot_chan=inp["slot_chan"],
                                     v_slot_chan=inp["v_slot_chan"], device=dev)
    elif kb == 0:
        inp = synth.mixed_layer_device(B, H, Hq, T, seed=4, device=dev)
        mk = lambda: kvq.PackedCache(B, H, T, kvq.KMIXED, vb, pdt, slot_chan=inp["slot_chan"], device=dev)
    else:
        inp = synth.layer_device(B, H, Hq, T, seed=1234, device=dev)
        mk = lambda: kvq.PackedCache(B, H, T, kb, vb, pdt, device=dev)
    alg = decode_bytes(B, H, Hq, T, kb, vb, kvq.PARAM_BYTES[pdt])
    caches = []
    for _ in range(max(2, math.ceil(600e6 / alg))):
        c = mk()
        c.quantize(inp["k"], inp["v"], 0)
        caches.append(c)
    q = inp["q"]
    del inp
    torch.cuda.empty_cache()
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in caches]
    wss = [c.workspace(Hq) for c in caches]
    nc = len(caches)
    ms = time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc], workspace=wss[i % nc]),
                    steps, warmup)
    del caches, outs, wss
    torch.cuda.empty_cache()
    return {"case": name, "ms": round(ms, 5), "GB/s": round(alg / ms / 1e6, 1),
            "pct_of_peak": round(100 * alg / ms / 1e6 / PEAK_HBM_GBS, 2), "bytes": alg,
            "copies": nc, "steps": steps}


def kernel_source_digest():
    """sha256 of the decode kernel's sources with comments and blank space
    removed (a comment edit does not change the kernel the counters describe)"""
    import hashlib
    import re
    h = hashlib.sha256()
    tok = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/|\s+', re.S)
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            src = f.read()
        code = tok.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per decode launch from the recorded counters, or None when the
    kernel source changed since they were taken"""
    c = COUNTER_TRAFFIC
    if c["source_sha256"] is None or c["source_sha256"] != kernel_source_digest():
        return None
    return round((c["fetch_kib"] * c["fetch_factor"] + c["write_kib"] * c["write_factor"]) * 1024)


def time_events(torch, fn, n, warmup):
    """average duration of fn() over n calls, HIP events on the current stream
    (after ROW_SETTLE_MS of untimed calls and the warmup calls)"""
    settle(torch, fn, ROW_SETTLE_MS)
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(st)
        fn(i)
        evs[i][1].record(st)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(ms) / len(ms), ms[len(ms) // 2]


def settle(torch, fn, ms):
    """fn(i) back to back for about ms milliseconds (untimed): the GPU's
    clocks ramp up over the first tens of milliseconds of sustained work, and
    drop again within milliseconds of idling"""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()


ROW_SETTLE_MS = 200.0   # untimed calls before each row's timing loop (--settle-ms / 5)


def time_block(torch, fn, n, warmup, settle_ms=None):
    """average duration of fn() over n calls issued back to back between one
    pair of HIP events (throughput of a stream of calls), after settle_ms
    (default ROW_SETTLE_MS) of untimed calls and the warmup calls"""
    settle(torch, fn, ROW_SETTLE_MS if settle_ms is None else settle_ms)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def mixed_128k_rows(torch, kvq, synth, dev, scale, vb=2):
    """Llama-3.1-8B-shaped 128K context: mixed 4/3/2/1-bit keys (34 B per token),
    2-bit values (vb = 2) or mixed 4/3/1/2-bit values (vb = 0: 40 B per token,
    four S/Z pairs), e4m3 S/Z.  Quantize of the whole context, then decode
    (cache copies rotated, > 600 MB together)."""
    B, H, Hq, T = 1, 8, 32, 131072
    if vb == 0:
        inp = synth.mixed_kv_layer_device(B, H, Hq, T, seed=4, device=dev)
    else:
        inp = synth.mixed_layer_device(B, H, Hq, T, seed=4, device=dev)
    alg = decode_bytes(B, H, Hq, T, 0, vb, 1)
    caches = [kvq.PackedCache(B, H, T, kvq.KMIXED, vb, kvq.E4M3, slot_chan=inp["slot_chan"],
                              v_slot_chan=inp.get("v_slot_chan"), device=dev)
              for _ in range(max(2, math.ceil(600e6 / alg)))]

    def quant(i):
        c = caches[i % len(caches)]
        c.s.n_tokens = 0
        c.quantize(inp["k"], inp["v"], 0)
    q_ms, _ = time_events(torch, quant, 8, 4)
    q_bytes = 2 * B * H * T * 128 * 4 + decode_bytes(B, H, 0, T, 0, vb, 1)
    for i in range(len(caches)):        # every copy holds the quantized context
        quant(i)
    q = inp["q"]
    del inp
    torch.cuda.empty_cache()
    nc = len(caches)
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in caches]
    wss = [c.workspace(Hq) for c in caches]
    d_ms = time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc], workspace=wss[i % nc]),
                      40, 4)
    tag = "mixed_kv_128k" if vb == 0 else "mixed_128k"
    return {"quantize_" + tag: {"ms": round(q_ms, 4), "GB/s": round(q_bytes / q_ms / 1e6, 1), "bytes": q_bytes,
                                "pct_of_peak": round(100 * q_bytes / q_ms / 1e6 / PEAK_HBM_GBS, 2)},
            "decode_" + tag: {"ms": round(d_ms, 4), "GB/s": round(alg / d_ms / 1e6, 1), "bytes": alg,
                                  "pct_of_peak": round(100 * alg / d_ms / 1e6 / PEAK_HBM_GBS, 2),
                                  "tokens_per_s": round(B / (d_ms * 1e-3), 1),
                                  "note": "%d cache copies rotated (%d MB each), 40 calls back to back"
                                          % (nc, alg // 1000000)}}


def pn_mix_rows(torch, kvq, synth, dev, scale):
    """Pair-granular key widths on the Llama-3.1-8B-shaped 128K layer (pairs
    recipe): RoPE pair norms of the prefill keys (the whole context) and
    queries, the slot map, and decode with that map (mixed keys, 2-bit values,
    e4m3 S/Z; nine cache copies rotated, > 600 MB together)."""
    import numpy as np
    B, H, Hq, T = 1, 8, 32, 131072
    G = Hq // H
    inp = synth.pair_layer_device(B, H, Hq, T, seed=6, device=dev)
    kn = torch.zeros((H, 64), dtype=torch.float32, device=dev)
    n_ms, _ = time_events(torch, lambda i: kvq.pair_norms(inp["k"], 1, out=kn.zero_()), 10, 2)
    n_bytes = B * H * T * 128 * 4
    qn = kvq.pair_norms(inp["q_prefill"], G)
    score = (qn * kvq.pair_norms(inp["k"], 1)).cpu().numpy()
    t0 = time.perf_counter()
    slot_chan = kvq.pair_slot_map(score)
    map_us = (time.perf_counter() - t0) * 1e6
    # the recipe's salient pairs (x8, x4) must hold the 4- and 3-bit slots
    big = np.flatnonzero(inp["pair_scale"][0] >= 4.0)
    assert sorted(slot_chan[0, :8].tolist() + slot_chan[0, 8:24:2].tolist()) == sorted(
        np.concatenate([big, big + 64]).tolist())
    alg = decode_bytes(B, H, Hq, T, 0, 2, 1)
    caches = [kvq.PackedCache(B, H, T, kvq.KMIXED, 2, kvq.E4M3, slot_chan=slot_chan, device=dev)
              for _ in range(max(2, math.ceil(600e6 / alg)))]
    for c in caches:
        c.quantize(inp["k"], inp["v"], 0)
    q = inp["q"]
    del inp
    torch.cuda.empty_cache()
    nc = len(caches)
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in caches]
    wss = [c.workspace(Hq) for c in caches]
    d_ms = time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc], workspace=wss[i % nc]),
                      40, 4)
    return {"pn_mix_pairs_128k": {
        "pair_norms_ms": round(n_ms, 4), "pair_norms_GB/s": round(n_bytes / n_ms / 1e6, 1),
        "slot_map_us": round(map_us, 1),
        "decode_ms": round(d_ms, 4), "decode_GB/s": round(alg / d_ms / 1e6, 1),
        "note": "keys' pair norms over the 128K context (fp32 in); decode with the pair-granular map"}}


def semkv_split_rows(torch, kvq, synth, dev, scale):
    """Per-token split between two adjacent precisions (SemKV page, abstract)
    on the Qwen2.5-7B-shaped layer (B=16, Hkv=4, Hq=28, T=32768): every
    stream's tokens ranked by a model-internal score (the key's L2 norm), the
    top 25% quantized at 4 bits and the rest at 2 bits (2.5 bits on average,
    binary16 S/Z) from the same inputs through the gathered quantize; decode
    over both caches merged by one combine, cache copies rotated past 600 MB."""
    B, H, Hq, T, n_high = 16, 4, 28, 32768, 8192
    inp = synth.layer_device(B, H, Hq, T, seed=77, device=dev)
    t0 = time.perf_counter()
    score = torch.linalg.vector_norm(inp["k"], dim=-1).reshape(B * H, T).cpu().numpy()
    order = kvq.rank_tokens(score, n_high).reshape(B, H, T)
    rank_ms = (time.perf_counter() - t0) * 1e3
    tok_hi = torch.from_numpy(order[:, :, :n_high].copy()).to(dev)
    tok_lo = torch.from_numpy(order[:, :, n_high:].copy()).to(dev)
    alg = decode_bytes(B, H, Hq, n_high, 4, 4, 2) + decode_bytes(B, H, 0, T - n_high, 2, 2, 2)
    pairs = []
    for _ in range(max(2, math.ceil(600e6 / alg))):
        hi = kvq.PackedCache(B, H, n_high, 4, 4, kvq.F16, device=dev)
        lo = kvq.PackedCache(B, H, T - n_high, 2, 2, kvq.F16, device=dev)
        pairs.append((hi, lo))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pairs[0][0].quantize_tokens(inp["k"], inp["v"], tok_hi)
    pairs[0][1].quantize_tokens(inp["k"], inp["v"], tok_lo)
    e1.record()
    torch.cuda.synchronize()
    q_ms = e0.elapsed_time(e1)
    for hi, lo in pairs[1:]:
        hi.quantize_tokens(inp["k"], inp["v"], tok_hi)
        lo.quantize_tokens(inp["k"], inp["v"], tok_lo)
    q = inp["q"]
    del inp, tok_hi, tok_lo
    torch.cuda.empty_cache()
    nc = len(pairs)
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in pairs]
    wss = [kvq.split_workspace(hi, lo, Hq) for hi, lo in pairs]
    d_ms = time_block(torch, lambda i: kvq.decode_attn_split(pairs[i % nc][0], pairs[i % nc][1], q, scale,
                                                             out=outs[i % nc], workspace=wss[i % nc]), 40, 4)
    del pairs, outs, wss
    torch.cuda.empty_cache()
    return {"semkv_split_4_2_bits": {
        "ms": round(d_ms, 4), "GB/s": round(alg / d_ms / 1e6, 1),
        "pct_of_peak": round(100 * alg / d_ms / 1e6 / PEAK_HBM_GBS, 2), "bytes": alg,
        "tokens_per_s": round(B / (d_ms * 1e-3), 1), "mean_bits": 2.5,
        "rank_ms_host": round(rank_ms, 1), "gathered_quantize_ms": round(q_ms, 4),
        "note": "top 25%% of each stream by key norm at 4 bits, the rest at 2 bits; %d copies rotated" % nc}}


def progressive_rows(torch, kvq, synth, dev, scale):
    """Progressive schedule: 128-token groups appended from 16 bits under a
    128 MiB budget (B=8, Hkv=4, Hq=28) up to 32768 tokens.  Times every append
    (the three that halve the cache include the whole-cache ERS), the ERS
    kernel of each halving on its own, and decode at the last token count of
    each width."""
    B, H, Hq, T = 8, 4, 28, 32768
    budget = 128 << 20
    inp = synth.layer_device(B, H, Hq, T, seed=33, device=dev)
    cache = kvq.PackedCache(B, H, T, 16, 16, kvq.F16, layout="pool", pool_bytes=budget, device=dev)
    q = inp["q"]
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    app_ms, events, dec = [], [], {}
    for t0 in range(0, T, 128):
        bits = cache.k_bits
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        n = cache.append(inp["k"][:, :, t0:t0 + 128], inp["v"][:, :, t0:t0 + 128], budget_bytes=budget,
                         floor_bits=2)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        if n:
            events.append({"tokens": t0, "from_bits": bits, "to_bits": cache.k_bits, "append_ms": round(ms, 4),
                           "shrunk_bytes": cache.cache_bytes(t0, bits, bits)})
        else:
            app_ms.append(ms)
        t1 = t0 + 128
        if t1 == T or (t1 < T and cache.cache_bytes(t1 + 128) > budget and cache.k_bits > 2):
            # the last token count of a width: decode over clones of the pool
            # cache (> 600 MB together, so no call finds its cache in the
            # 256 MB Infinity Cache), 40 calls back to back
            alg = decode_bytes(B, H, Hq, t1, cache.k_bits, cache.v_bits, 2)
            clones = [cache.clone() for _ in range(max(2, math.ceil(600e6 / alg)))]
            nc = len(clones)
            wss = [c.workspace(Hq) for c in clones]
            outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in clones]
            dms = time_block(torch, lambda i: clones[i % nc].decode_attn(q, scale, out=outs[i % nc],
                                                                        workspace=wss[i % nc]), 40, 4)
            dec["%d-bit@%d" % (cache.k_bits, t1)] = {
                "ms": round(dms, 4), "GB/s": round(alg / dms / 1e6, 1),
                "pct_of_peak": round(100 * alg / dms / 1e6 / PEAK_HBM_GBS, 2), "bytes": alg,
                "tokens_per_s": round(B / (dms * 1e-3), 1), "cache_copies_rotated": nc}
            del clones, wss, outs
            torch.cuda.empty_cache()
    del cache
    torch.cuda.empty_cache()
    # the ERS kernel of each event on its own: the same (B, Hkv, tokens, width)
    # in the contiguous layout, timed around the one shrink launch (the append
    # above also carries the host-side pool bookkeeping and the group's quantize)
    for ev in events:
        t0, b = ev["tokens"], ev["from_bits"]
        src = kvq.PackedCache(B, H, t0, b, b, kvq.F16, device=dev)
        src.quantize(inp["k"][:, :, :t0], inp["v"][:, :, :t0], 0)
        sh = kvq.PackedCache(B, H, t0, b, b, kvq.F16, device=dev)
        tms = []
        for i in range(4):
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                getattr(sh, name).copy_(getattr(src, name))
            sh.s.n_tokens, sh.s.k_bits, sh.s.v_bits = t0, b, b
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            sh.shrink(b // 2)
            e1.record()
            torch.cuda.synchronize()
            if i:
                tms.append(e0.elapsed_time(e1))
        ms = sum(tms) / len(tms)
        # read both tiles at b bits, write both halves at b/2; read and write S'
        nbytes = B * H * (t0 // 128) * (2 * 2048 * b + 2 * 2048 * (b // 2)) + 2 * 2 * B * H * t0 * 2
        ev["ers_kernel"] = {"ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1), "bytes": nbytes,
                            "pct_of_peak": round(100 * nbytes / ms / 1e6 / PEAK_HBM_GBS, 2)}
        del src, sh
    del inp
    torch.cuda.empty_cache()
    return {"progressive_schedule": {"shrink_events": events,
                                     "append_ms_median": round(sorted(app_ms)[len(app_ms) // 2], 4),
                                     "decode": dec,
                                     "note": "pool layout; decode timed over clones of the pool cache "
                                             "(> 600 MB rotated)"}}


STEP_WIDTHS = (2, 4, 8)
STEP_BUDGET_FRAC = 0.195


def step_width_table(kvq, synth, B=16, H=8, T=32768, L=64):
    """Per-layer widths of the 64-layer step from the block-wise allocation
    (PM-KVQ Key design 2, kvq_allocate_bits): synthetic sensitivities
    (synth.layer_sensitivities), each layer's cache bytes at 2/4/8 bits with
    binary16 scales and zeros, and a budget M of 19.5% of the 64 layers'
    16-bit (binary16) KV size.  Returns (widths, M, objective)."""
    import numpy as np
    sens = synth.layer_sensitivities(L, STEP_WIDTHS, seed=0)
    per = [B * H * T * (128 * b // 8 * 2 + 4 * 2) for b in STEP_WIDTHS]
    nbytes = np.array([per] * L, dtype=np.int64)
    budget = int(STEP_BUDGET_FRAC * L * B * H * T * 128 * 2 * 2)
    choice, obj = kvq.allocate_bits(sens, nbytes, budget)
    return [STEP_WIDTHS[c] for c in choice], budget, obj


def qwen32b_step_rows(torch, kvq, synth, dev, scale, n_steps=5):
    """Qwen2.5-32B-shaped full decode step: 64 layers (B=16, Hkv=8, Hq=40,
    T=32768), each layer's cache packed at the width the block-wise
    allocation gives it under the budget M (step_width_table), generated with
    the layer generator (seed = base + layer) and quantized one layer at a
    time.  One step = the 64 layers' decode calls back to back; the 26 GB of
    packed caches are far larger than the Infinity Cache."""
    B, H, Hq, T, L = 16, 8, 40, 32768, 64
    bits, budget, obj = step_width_table(kvq, synth, B, H, T, L)
    caches, qs, alg = [], [], 0
    for layer, b in enumerate(bits):
        inp = synth.layer_device(B, H, Hq, T, seed=500 + layer, device=dev)
        c = kvq.PackedCache(B, H, T, b, b, kvq.F16, device=dev)
        c.quantize(inp["k"], inp["v"], 0)
        qs.append(inp["q"])
        caches.append(c)
        alg += decode_bytes(B, H, Hq, T, b, b, 2)
        del inp
        torch.cuda.empty_cache()
    ws = caches[0].workspace(Hq)
    for c in caches[1:]:
        assert c.workspace_bytes(Hq) <= ws.numel()
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    def step(i):
        for c, q in zip(caches, qs):
            c.decode_attn(q, scale, out=out, workspace=ws)
    settle(torch, step, 1.5 * ROW_SETTLE_MS)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    counts = {w: bits.count(w) for w in sorted(set(bits))}
    del caches, qs
    torch.cuda.empty_cache()
    return {"qwen32b_64_layer_step": {
        "ms": round(ms, 4), "GB/s": round(alg / ms / 1e6, 1), "pct_of_peak": round(100 * alg / ms / 1e6 / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(B / (ms * 1e-3), 1), "bytes": alg,
        "layers_per_width": {str(k): v for k, v in counts.items()},
        "mean_bits": round(sum(bits) / len(bits), 3),
        "widths_from": "kvq_allocate_bits, synthetic sensitivities, budget M = %d B (%.1f%% of the 16-bit size)"
                       % (budget, 100 * STEP_BUDGET_FRAC),
        "allocation_objective": obj,
        "note": "attention only, 64 back-to-back layer calls per step"}}


def halving_rule_rows(torch, kvq, synth, dev, scale):
    """Ablation of the halving rule (PM-KVQ Key design 1 and its ablation
    table, which reports task accuracy; here the stand-in is the decode
    output): 7B-shaped layer slice (B=4, Hkv=4, Hq=28, T=32768) quantized to
    4 bits, halved to 2 bits by ERS, the direct right shift and the modified
    (rounded) shift.  For each: the shrink kernel's time and the decode
    output's error against binary32 attention over the unquantized K/V (per
    row ||o - o_ref||_inf / ||o_ref||_inf: max and mean over rows); 4-bit
    before the halving and a direct 2-bit quantization for reference."""
    B, H, Hq, T = 4, 4, 28, 32768
    G = Hq // H
    inp = synth.layer_device(B, H, Hq, T, seed=71, device=dev)
    k, v, q = inp["k"], inp["v"], inp["q"]
    # binary32 reference attention over the unquantized keys and values
    qf = q.float().view(B, H, G, 128)
    s_ = torch.matmul(qf, k.transpose(2, 3).contiguous()) * scale          # [B][H][G][T]
    p_ = torch.softmax(s_, dim=-1)
    ref = torch.matmul(p_, v).reshape(B, Hq, 128)
    del s_, p_

    def err(o):
        e = (o - ref).abs().amax(dim=-1) / ref.abs().amax(dim=-1)
        return {"max_row_rel_err": float(e.max()), "mean_row_rel_err": float(e.mean())}
    base = kvq.PackedCache(B, H, T, 4, 4, kvq.F16, device=dev)
    base.quantize(k, v, 0)
    out = {"4-bit": err(base.decode_attn(q, scale))}
    names = {kvq.SHIFT_ERS: "ers", kvq.SHIFT_DIRECT: "direct_shift", kvq.SHIFT_MODIFIED: "modified_shift"}
    nbytes = B * H * (T // 128) * (2 * 8192 + 2 * 4096) + 2 * 2 * B * H * T * 2
    for m, nm in names.items():
        c = kvq.PackedCache(B, H, T, 4, 4, kvq.F16, device=dev)
        tms = []
        for i in range(4):
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                getattr(c, name).copy_(getattr(base, name))
            c.s.n_tokens, c.s.k_bits, c.s.v_bits = T, 4, 4
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            c.shrink(2, method=m)
            e1.record()
            torch.cuda.synchronize()
            if i:
                tms.append(e0.elapsed_time(e1))
        row = err(c.decode_attn(q, scale))
        ms = sum(tms) / len(tms)
        row.update({"shrink_ms": round(ms, 4), "shrink_GB/s": round(nbytes / ms / 1e6, 1)})
        out["4->2 " + nm] = row
        del c
    d2 = kvq.PackedCache(B, H, T, 2, 2, kvq.F16, device=dev)
    d2.quantize(k, v, 0)
    out["2-bit direct quantization"] = err(d2.decode_attn(q, scale))
    for key in out:
        for f in ("max_row_rel_err", "mean_row_rel_err"):
            out[key][f] = round(out[key][f], 5)
    del base, d2, inp, k, v, ref
    torch.cuda.empty_cache()
    return {"halving_rule_ablation": out}


def cpu_baseline(inp, B, H, Hq, k_bits, pdt, seconds):
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    quantize + fp64 decode attention of whole (batch, kv-head) streams, run in
    a thread pool over the host cores; scaled to GB/s of the decode step."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    oracle.build(force=False)
    G = Hq // H
    cores = min(len(os.sched_getaffinity(0)), 16)
    scale = 1.0 / math.sqrt(128)
    streams = [(b, h) for b in range(B) for h in range(H)]
    # calibrate on one stream
    t0 = time.perf_counter()
    st = oracle.quantize_stream(inp["k"][0, 0], inp["v"][0, 0], k_bits, k_bits, pdt)
    t1 = time.perf_counter()
    oracle.decode_attn(st, inp["q_bf16"][0, 0:G], scale)
    t2 = time.perf_counter()
    per_stream = t2 - t1
    n = max(cores, min(len(streams), int(seconds * cores / max(per_stream, 1e-3))))
    n = min(n, len(streams))
    sample = streams[:n]
    packed = {}

    def q_one(bh):
        b, h = bh
        packed[bh] = oracle.quantize_stream(inp["k"][b, h], inp["v"][b, h], k_bits, k_bits, pdt)

    with cf.ThreadPoolExecutor(cores) as ex:
        list(ex.map(q_one, sample))

    def d_one(bh):
        b, h = bh
        return oracle.decode_attn(packed[bh], inp["q_bf16"][b, h * G:(h + 1) * G], scale)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        list(ex.map(d_one, sample))
    dt = time.perf_counter() - t0
    T = inp["k"].shape[2]
    nbytes = decode_bytes(1, n, n * G, T, k_bits, k_bits, 2)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d (batch, kv-head) streams, full 32768 tokens, fp64 decode attention "
                      "over the oracle's own packed cache (%.2f s wall)" % (n, B * H, dt),
            "tokens_per_s": round(n / H / dt, 3) if n >= H else None}


def main():
    global ROW_SETTLE_MS
    args = _parse()
    ROW_SETTLE_MS = args.settle_ms / 5
    if args.case:
        decode_case(args.case, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from kv_cache_mixed_amd import kvq, synth
    kvq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    B, H, Hq, T, BITS = 16, 4, 28, 32768, 4
    pdt = kvq.F16
    scale = 1.0 / math.sqrt(128)
    inp = synth.layer(B, H, Hq, T, seed=1234)
    kd = torch.from_numpy(inp["k"]).to(dev)
    vd = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)

    cache0 = kvq.PackedCache(B, H, T, BITS, BITS, pdt, device=dev)
    rows = {}
    # ---- quantize row: K and V of the whole layer (2 x 1 GiB fp32 read)
    def quant(i):
        cache0.s.n_tokens = 0
        cache0.quantize(kd, vd, 0)
    q_ms, _ = time_events(torch, quant, 5 if not args.no_rows else 1, 1)
    q_bytes = 2 * B * H * T * 128 * 4 + decode_bytes(B, H, 0, T, BITS, BITS, 2)
    rows["quantize_k_v_4bit"] = {"ms": round(q_ms, 4), "GB/s": round(q_bytes / q_ms / 1e6, 1),
                                 "bytes": q_bytes, "pct_of_peak": round(100 * q_bytes / q_ms / 1e6 / PEAK_HBM_GBS, 2)}
    del kd, vd
    torch.cuda.empty_cache()

    # ---- rotate copies of the packed cache (> 512 MiB together)
    alg = decode_bytes(B, H, Hq, T, BITS, BITS, 2)
    n_copies = max(2, math.ceil(600e6 / alg))
    caches = [cache0]
    for _ in range(n_copies - 1):
        c = kvq.PackedCache(B, H, T, BITS, BITS, pdt, device=dev)
        for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
            getattr(c, name).copy_(getattr(cache0, name))
        c.s.n_tokens = T
        caches.append(c)
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in caches]
    wss = [c.workspace(Hq) for c in caches]

    def step(i):
        j = i % len(caches)
        caches[j].decode_attn(q, scale, out=outs[j], workspace=wss[j])

    settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K steps back to back on the launch stream, bracketed by a
    # device synchronisation and a pair of HIP events on that stream
    st = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(st)
    for i in range(args.steps):
        step(i)
    ev1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_avg = ev0.elapsed_time(ev1) / args.steps      # one decode call: main + combine kernel
    ms_per_step = wall * 1e3 / args.steps
    value = alg / (ms_per_step * 1e-3) / 1e9

    # the dominant kernel alone: K calls of the first phase of the C ABI
    # (kvq_decode_attn_partials: the decode kernel only) back to back over the
    # same rotated copies, between one pair of HIP events on the launch
    # stream.  An event pair around every single launch would add the idle
    # launch latency that back-to-back launches hide.
    n_slots = []

    def part(i):
        j = i % len(caches)
        n_slots.append(caches[j].decode_partials(q, scale, workspace=wss[j])[0])

    # median of three rounds, each right after the previous (no idle time)
    kern_avg = sorted(time_block(torch, part, args.steps, args.warmup, 0.0 if r else 50.0) for r in range(3))[1]
    achieved = alg / (kern_avg * 1e-3) / 1e9

    # ---- other rows of the path
    if not args.no_rows:
        # ERS shrink 4 -> 2 of the whole layer (read 4-bit tiles, write 2-bit halves)
        sh = kvq.PackedCache(B, H, T, BITS, BITS, pdt, device=dev)

        def shrink(i):
            for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
                getattr(sh, name).copy_(getattr(cache0, name))
            sh.s.n_tokens, sh.s.k_bits, sh.s.v_bits = T, 4, 4
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            sh.shrink(2)
            ev1.record()
            return ev0, ev1
        tms = []
        for i in range(6):
            e0, e1 = shrink(i)
            torch.cuda.synchronize()
            if i:
                tms.append(e0.elapsed_time(e1))
        s_ms = sum(tms) / len(tms)
        s_bytes = B * H * (T // 128) * (2 * 8192 + 2 * 4096) + 2 * 2 * B * H * T * 2
        rows["ers_shrink_4to2"] = {"ms": round(s_ms, 4), "GB/s": round(s_bytes / s_ms / 1e6, 1),
                                   "bytes": s_bytes, "pct_of_peak": round(100 * s_bytes / s_ms / 1e6 / PEAK_HBM_GBS, 2)}
        a2 = decode_bytes(B, H, Hq, T, 2, 2, 2)
        shs = [sh] + [sh.clone() for _ in range(max(2, math.ceil(600e6 / a2)) - 1)]
        n2 = len(shs)
        out2s = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in shs]
        ws2 = [c.workspace(Hq) for c in shs]
        d2_ms = time_block(torch, lambda i: shs[i % n2].decode_attn(q, scale, out=out2s[i % n2],
                                                                    workspace=ws2[i % n2]), 40, 4)
        rows["decode_2bit_same_layer"] = {"ms": round(d2_ms, 4), "GB/s": round(a2 / d2_ms / 1e6, 1),
                                          "pct_of_peak": round(100 * a2 / d2_ms / 1e6 / PEAK_HBM_GBS, 2),
                                          "note": "%d copies of the shrunk cache rotated" % n2}
        del sh, shs, out2s, ws2
        torch.cuda.empty_cache()
        # decode over the packed layer plus a 128-token bf16 residual segment
        # (the group not yet quantized), against the same call without it
        R = 128
        rk = torch.randn((B, H, R, 128), device=dev).to(torch.bfloat16)
        rv = torch.randn((B, H, R, 128), device=dev).to(torch.bfloat16)
        nc = len(caches)
        # the two variants alternate over 5 rounds (medians): the call time
        # drifts by a few us over a run, as much as the residual costs
        d0s, drs = [], []
        for _ in range(5):
            d0s.append(time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc],
                                                                              workspace=wss[i % nc]), 60, 5))
            drs.append(time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc],
                                                                              workspace=wss[i % nc],
                                                                              res_k=rk, res_v=rv), 60, 5))
        d0_ms, dr_ms = sorted(d0s)[2], sorted(drs)[2]
        ar = alg + 2 * B * H * R * 128 * 2
        rows["decode_4bit_plus_residual_128"] = {
            "ms": round(dr_ms, 4), "GB/s": round(ar / dr_ms / 1e6, 1),
            "ms_without_residual": round(d0_ms, 4),
            "extra_us_per_round": [round((b - a) * 1e3, 1) for a, b in zip(d0s, drs)],
            "extra_us_median": round(sorted(b - a for a, b in zip(d0s, drs))[2] * 1e3, 1),
            "note": "medians of 5 alternating rounds of 60 calls back to back, cache copies rotated as "
                    "in the headline step; residual bf16 [16][4][128][128]"}
        del rk, rv
        # one generation step through the token window: append the new
        # token's key and value (bf16) to the stream windows, then decode over
        # the packed cache and the held tokens (under 128 held: no group packed)
        wins = [kvq.Window(c, torch.bfloat16, keep_first=False) for c in caches]
        nk = torch.randn((65, B, H, 1, 128), device=dev).to(torch.bfloat16)
        nv = torch.randn((65, B, H, 1, 128), device=dev).to(torch.bfloat16)
        # (65 tokens over the 3 cache copies: fewer than 128 per window)

        def window_step(i):
            w = wins[i % nc]
            w.append(nk[i], nv[i])
            wk, wv = w.residual()
            caches[i % nc].decode_attn(q, scale, out=outs[i % nc], workspace=wss[i % nc], res_k=wk, res_v=wv)

        dw_ms = time_block(torch, window_step, 60, 5, settle_ms=0.0)   # 65 tokens: no untimed calls beyond the warmup
        d1_ms = time_block(torch, lambda i: caches[i % nc].decode_attn(q, scale, out=outs[i % nc],
                                                                       workspace=wss[i % nc]), 60, 5)
        rows["decode_step_window_append"] = {
            "ms": round(dw_ms, 4), "ms_decode_only": round(d1_ms, 4),
            "note": "60 steps back to back: kvq_window_append of one bf16 token per stream, then "
                    "decode over the packed layer + the 1..22 held tokens"}
        del wins, nk, nv
        rows.update(mixed_128k_rows(torch, kvq, synth, dev, scale))
        r8 = decode_case_row("llama8b_mixed_32k_b8", 40, 5)
        r8["note"] = ("mixed keys, 2-bit values, e4m3 S/Z, B = 8 x 32768 tokens (two streams per wave); "
                      "cache copies rotated")
        rows["decode_mixed_32k_b8"] = r8
        rows.update(mixed_128k_rows(torch, kvq, synth, dev, scale, vb=0))
        rows.update(pn_mix_rows(torch, kvq, synth, dev, scale))
        rows.update(semkv_split_rows(torch, kvq, synth, dev, scale))
        rows.update(progressive_rows(torch, kvq, synth, dev, scale))
        rows.update(halving_rule_rows(torch, kvq, synth, dev, scale))
        rows.update(qwen32b_step_rows(torch, kvq, synth, dev, scale))

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, B, H, Hq, BITS, pdt, args.cpu_seconds)

    line = {
        "metric": "packed-KV decode attention: effective HBM GB/s (% of peak) and tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "qwen2.5-7b-shaped decode layer", "batch": B, "kv_heads": H,
                   "q_heads": Hq, "head_dim": 128, "cached_tokens": T, "k_bits": BITS,
                   "v_bits": BITS, "param_dtype": "f16", "query": "bf16", "output": "f32",
                   "cache_copies_rotated": len(caches)},
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_step": alg,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": counter_traffic(),
                     "kernel": "decode_kernel<4,4,f16,2>",
                     "kernel_ms_avg": round(kern_avg, 5),
                     "call_ms_avg": round(call_avg, 5),
                     "call_frac": round(alg / (call_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "partial_slots": n_slots[-1],
                     "note": "achieved: algorithmic bytes of one call over the decode kernel's average "
                             "launch time (K kvq_decode_attn_partials calls back to back between HIP events); "
                             "call_frac: over the whole call (decode + combine kernels)"},
        "rows": rows,
        "cpu_baseline": cpu,
        "settle_ms": args.settle_ms,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
