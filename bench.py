"""Decode-step benchmark for the compressed-KV path on one MI355X.

One step = what a decode step does to one attention layer's cache: zf_append_kv (encode one
new K/V token per sequence into the packed paged cache) followed by zf_decode_attention (fused
GQA attention over the packed cache, every value rebuilt in registers).  Steps rotate over
several layer caches (3 by default, 1.35 GB) so that, as in a multi-layer model, a layer's
cache is not still sitting in the 256 MB last-level cache when its next step comes.  Workload: the
Llama-3.1-8B-shaped decode of the ZipFusion video summary ("Run AI Faster With Lossless
Compressed Memory"): batch 32, 32 query / 8 KV heads, head_dim 128, 4096 cached tokens per
sequence, 16-token pages in random order, synthetic bf16 K/V (seeded generator; no model
weights exist here).  Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` = tokens/s of the whole job (sequences x steps / time), one
layer, from the K timed steps, none of which carries a timing stamp.  `roofline` prices the
attention kernel (the dominant one) against HBM: algorithmic bytes per launch (packed planes of
the attended rows, spill slots of their raw blocks, q, out, page table and lengths) / its mean
duration from HIP events on the launch stream, stamped at the kernel's own start and end
(zf_time_next_attention: the interval a kernel trace reports) in a separate pass of at least 60
further decode steps after the timed ones (a stamped launch pays ~8 us more dispatch, so the
timed steps carry no stamps).  Before the warm-up steps, attention calls alone (which change no
state) bring the GPU to its working clock.  `cpu_baseline` times the CPU oracle (plain C) on all
host cores on a bounded sample of the same steps; the one-core rate is in `extra`.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "compressed-KV decode attn: HBM GB/s, % of peak, tokens/s, compression ratio"
WORKLOAD = 1
ATTN_SOURCES = ["decode_attention_encode_amd/csrc/zf_attention.hip",
                "decode_attention_encode_amd/csrc/zf_internal.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_llama8b_b32_ctx4096_hbm_counters.json")


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


STAMPED_STEPS = 60    # decode steps of the stamped pass (kernel start / end) after the timed ones
CLOCK_WARMUP_MS = 30  # attention calls alone before the warm-up steps: an idle MI355X needs
                      # ~10 ms of load to reach its working clock


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--warmup", type=int, default=150, help="untimed decode steps first")
    ap.add_argument("--layers", type=int, default=3,
                    help="layer caches the steps rotate over (1.35 GB at 3, beyond the 256 MB "
                         "last-level cache, as in a multi-layer model)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--extras", action="store_true",
                    help="also time the raw twin, a cache-flushed attention, encode and decode")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("OUT", "FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR",
                                                       "CAL_WRITE_DIR"),
                    help="only summarize rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (of this "
                         "bench and of --calibrate-copy) into OUT (JSON) and exit")
    ap.add_argument("--codec", action="store_true",
                    help="only time full-cache encode and decode (the batch-32 layer and the "
                         "4 x 131072-token cache) and a prefill written as chunked appends, one "
                         "JSON line each, and exit")
    ap.add_argument("--per-config", default="",
                    help="only time the attention call on these workloads (e.g. 1,2,3,4: the "
                         "parity configurations; d1, d2, d8: their diffuse-softmax forms), one "
                         "JSON line each, and exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and is not "
              "sharded across GPUs (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_encode_amd as zf
    import synth

    assert torch.cuda.is_available(), "needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 3}))
        return
    if args.codec:
        for wi in (1, 4):
            print(json.dumps(full_cache_codec(torch, zf, synth, wi, dev)), flush=True)
        print(json.dumps(prefill_chunks(torch, zf, synth, dev)), flush=True)
        return
    if args.per_config:
        for key in args.per_config.split(","):
            print(json.dumps(per_config(torch, zf, synth, key, dev)), flush=True)
        return

    W, K, KS = args.warmup, args.steps, STAMPED_STEPS
    NL = max(1, args.layers)
    NS = W + K + KS  # decode steps in all
    w = synth.WORKLOADS[WORKLOAD].replace(extra_tokens=(NS + NL - 1) // NL + 1)
    t0 = time.time()
    inst = synth.make(w)
    B, H, Hq, D, T = w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, w.page_size
    lens0 = inst.seq_lens.copy()
    to = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    # step s works on layer s % NL; per layer the sequences grow by one token per visit
    visits = [(s // NL) for s in range(NS)]  # appends this layer has seen before step s
    ks, vs, qs = [], [], []
    for s in range(NS):
        k, v = synth.tokens(w, lens0 + visits[s])
        ks.append(k)
        vs.append(v)
        qs.append(synth.query(w, s))
    k_dev = to(np.stack(ks))
    v_dev = to(np.stack(vs))
    q_dev = to(np.stack(qs))
    gen_s = time.time() - t0

    rows_cap = int(lens0.sum()) + B * (w.extra_tokens + 1)
    spill_slots = rows_cap * 2 * H * (D // 64)
    max_len = int(lens0.max()) + w.extra_tokens
    raw = to(inst.raw_pages)
    pt_dev = to(inst.page_table)
    layers = []
    for _ in range(NL):  # one packed cache per layer (same data), own lengths
        cache = zf.PackedCache.empty(inst.num_pages, T, H, D, spill_slots, device=dev)
        seqs = zf.Seqs(pt_dev, to(lens0.copy()), max_len, page_hint(torch, B, H, inst.page_table.shape[1], dev))
        zf.zf_encode_kv(cache, seqs, raw, zf.encode_workspace(seqs))
        layers.append((cache, seqs))
    torch.cuda.synchronize()
    for cache, _ in layers:
        assert zf.zf_get_status(cache.status) == 0
    top0 = int(layers[0][0].spill_top.item())
    rows0 = int(lens0.sum())
    ws = zf.attention_workspace(B, H, Hq, D, max_len, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    scale = fp32_scale(D)
    stream = torch.cuda.current_stream()

    def step(s, ev=None):
        cache, seqs = layers[s % NL]
        zf.zf_append_kv(cache, seqs, k_dev[s], v_dev[s])
        if ev is not None:
            ev[2].record(stream)
            zf.zf_time_next_attention(ev[0], ev[1])  # the kernel's own start / end stamps
        zf.zf_decode_attention(cache, seqs, q_dev[s], scale, out, ws)
        if ev is not None:
            ev[3].record(stream)

    # clock warm-up: attention calls alone (no state changes) for CLOCK_WARMUP_MS
    t0 = time.perf_counter()
    warm_calls = 0
    while time.perf_counter() - t0 < CLOCK_WARMUP_MS / 1e3 or warm_calls < 50:
        for _ in range(10):
            cache, seqs = layers[warm_calls % NL]
            zf.zf_decode_attention(cache, seqs, q_dev[0], scale, out, ws)
            warm_calls += 1
        torch.cuda.synchronize()
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        step(W + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # the stamped pass: KS more decode steps, each with kernel start / end (device timestamps
    # of the dispatch) and call start / end
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(KS)]
    for ev in evs:
        for e in ev:
            e.record(stream)  # creates the events on the device
    torch.cuda.synchronize()
    for i in range(KS):
        step(W + K + i, evs[i])
    torch.cuda.synchronize()
    for cache, _ in layers:
        status = zf.zf_get_status(cache.status)
        assert status == 0, f"device status {status}"
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])   # kernel execution
    call_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])   # call, dispatch included
    stamped = [W + K + i for i in range(KS)]

    # ---- algorithmic bytes of each timed attention launch
    pt = inst.page_table
    row_bytes = 2 * H * (D + D // 2 + D // 64) + 8  # planes + base + row flags + row spill
    flags = [c.row_flags.cpu().numpy().view(np.uint32) for c, _ in layers]
    raw_after = []  # raw blocks in the attended layer right after step s's append
    seen = [top0] * NL
    for s in range(NS):
        lay = s % NL
        pos = lens0 + visits[s]
        pages = pt[np.arange(B), pos // T]
        f = flags[lay][pages, pos % T]
        seen[lay] += sum(bin(int(x)).count("1") for x in f)
        raw_after.append(seen[lay])
    attn_bytes = []
    tokens_attended = []
    for s in stamped:
        L = lens0 + visits[s] + 1
        tokens_attended.append(int(L.sum()))
        nbytes = int(L.sum()) * row_bytes + 32 * int(raw_after[s])
        nbytes += B * Hq * D * (2 + 4) + int(np.ceil(L / T).sum()) * 4 + B * 4
        attn_bytes.append(nbytes)
    attn_bytes = np.array(attn_bytes, np.float64)
    mean_attn_s = attn_ms.mean() / 1e3
    achieved = attn_bytes.mean() / mean_attn_s / 1e9  # bytes of the stamped launches
    uncompressed_eq = np.mean(tokens_attended) * H * 2 * D * 2 / mean_attn_s / 1e9
    packed_valid = rows0 * row_bytes + 32 * top0
    ratio = packed_valid / (rows0 * H * 2 * D * 2)

    traffic = None
    if os.path.exists(PMC_SUMMARY):
        pmc = json.load(open(PMC_SUMMARY))
        if pmc.get("attn_source_hash") == attn_source_hash():
            traffic = pmc.get("hbm_bytes_per_launch")

    extra = {
        "layers_rotated": NL,
        "clock_warmup_attention_calls": warm_calls,
        "attention_kernel_us_mean": round(attn_ms.mean() * 1e3, 2),
        "attention_kernel_us_median": round(float(np.median(attn_ms)) * 1e3, 2),
        "attention_launches_stamped": KS,
        "attention_kernel_us_min": round(attn_ms.min() * 1e3, 2),
        "attention_call_us_mean": round(call_ms.mean() * 1e3, 2),
        "attention_bytes_per_launch": int(attn_bytes.mean()),
        "uncompressed_equivalent_GBps": round(uncompressed_eq, 1),
        "compression_ratio": round(ratio, 4),
        "raw_block_fraction": round(top0 / (rows0 * 2 * H * (D // 64)), 4),
        "generation_s": round(gen_s, 1),
    }

    if args.extras:
        extra.update(extras(torch, zf, inst, layers, raw, q_dev[NS - 1], ws, out, scale,
                            attn_bytes.mean(), row_bytes))
        extra.update(full_cache_codec(torch, zf, synth, 1, dev))
        extra.update(full_cache_codec(torch, zf, synth, 4, dev))
        extra.update(prefill_chunks(torch, zf, synth, dev))
        if not args.no_cpu_baseline:
            extra["oracle_single_thread"] = oracle_ops(w, inst, lens0, ks, vs, qs)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inst, lens0, ks, vs, qs, args.cpu_seconds, host_cores())
        one = cpu_baseline(w, inst, lens0, ks, vs, qs, args.cpu_seconds / 2, 1)
        extra["cpu_baseline_one_core"] = {"value": one["value"], "unit": one["unit"],
                                          "cores": 1, "sample": one["sample"]}

    result = {
        "metric": METRIC,
        "value": round(B * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 K/V: per-channel log-uniform scales, outlier and zero "
                "blocks; no model weights)",
        "config": {"workload": w.name, "batch": B, "context": int(lens0[0]), "q_heads": Hq,
                   "kv_heads": H, "head_dim": D, "page_size": T, "layers_rotated": NL,
                   "step": "one layer: append 1 token/seq + fused compressed attention"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(result))


def extras(torch, zf, inst, layers, raw, q, ws, out, scale, attn_bytes, row_bytes):
    """Twin (uncompressed) attention over the same rotation of layer caches, the unfused
    alternative (decode to bf16, then the twin), a plain streaming read over the same bytes,
    the single-layer warm-cache loop, full-cache encode / decode rates, the single-token append
    in both forms, multi-token append, spill compaction, and the capacity model at a fixed HBM
    budget."""
    res = {}
    stream = torch.cuda.current_stream()
    NL = len(layers)

    def timeit(fn, n=30):
        fn(0)
        torch.cuda.synchronize()
        ts = []
        for i in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i)
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ts])) / 1e3

    status = torch.zeros(1, dtype=torch.int32, device=raw.device)
    # twins: raw pages holding the tokens each packed layer holds now
    twins = []
    for cache, seqs in layers:
        d = torch.zeros_like(raw)
        zf.zf_decode_kv(cache, seqs, d)
        twins.append(d)
    def timeit_pair(fa, fb, n=30, warm=20):
        """fa and fb alternately (a, b, a, b, ...) after `warm` untimed rounds, so that both see
        the same clock and cache state; the mean of each."""
        for i in range(warm):
            fa(i)
            fb(i)
        torch.cuda.synchronize()
        ta, tb = [], []
        for i in range(n):
            for f, acc in ((fa, ta), (fb, tb)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                f(i)
                b.record(stream)
                acc.append((a, b))
        torch.cuda.synchronize()
        mean = lambda ev: float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
        return mean(ta), mean(tb)

    t_pack, t_twin = timeit_pair(
        lambda i: zf.zf_decode_attention(layers[i % NL][0], layers[i % NL][1], q, scale, out, ws),
        lambda i: zf.zf_decode_attention_raw(twins[i % NL], layers[i % NL][1], q, scale, out, ws, status))
    t_warm = timeit(lambda i: zf.zf_decode_attention(layers[0][0], layers[0][1], q, scale, out, ws))
    res["attention_packed_us"] = round(t_pack * 1e6, 2)
    res["attention_twin_uncompressed_us"] = round(t_twin * 1e6, 2)
    res["speedup_vs_uncompressed_twin"] = round(t_twin / t_pack, 3)

    # the same pair by the kernels' own start and end stamps (no dispatch overhead), alternating
    def stamped_pair(fa, fb, n=30):
        ev = []
        for i in range(n):
            for f in (fa, fb):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)  # the events exist on the device before the library stamps them
                b.record(stream)
                zf.zf_time_next_attention(a, b)
                f(i)
                ev.append((a, b))
        torch.cuda.synchronize()
        d = [a.elapsed_time(b) / 1e3 for a, b in ev]
        return float(np.mean(d[0::2])), float(np.mean(d[1::2]))

    k_pack, k_twin = stamped_pair(
        lambda i: zf.zf_decode_attention(layers[i % NL][0], layers[i % NL][1], q, scale, out, ws),
        lambda i: zf.zf_decode_attention_raw(twins[i % NL], layers[i % NL][1], q, scale, out, ws, status))
    res["attention_packed_kernel_us"] = round(k_pack * 1e6, 2)
    res["attention_twin_kernel_us"] = round(k_twin * 1e6, 2)
    res["kernel_speedup_vs_uncompressed_twin"] = round(k_twin / k_pack, 3)
    # the unfused alternative: decode the layer's cache to bf16 pages, then the raw kernel
    scratch = torch.empty_like(raw)

    def unfused(i):
        cache, seqs = layers[i % NL]
        zf.zf_decode_kv(cache, seqs, scratch)
        zf.zf_decode_attention_raw(scratch, seqs, q, scale, out, ws, status)
    t_unf = timeit(unfused)
    res["unfused_decode_then_twin_us"] = round(t_unf * 1e6, 2)
    res["speedup_vs_unfused"] = round(t_unf / t_pack, 3)
    del scratch
    # a plain stream over the same rotation of (uncompressed) buffers: the read rate this GPU
    # achieves at all, context for the attention kernel's
    sink = torch.empty(zf.ZF_PROBE_BLOCKS, dtype=torch.int32, device=raw.device)
    t_rd = timeit(lambda i: zf.zf_stream_read_probe(twins[i % NL], sink))
    rd_bytes = twins[0].numel() * twins[0].element_size()
    res["stream_read_probe_GBps"] = round(rd_bytes / t_rd / 1e9, 1)
    res["stream_read_probe_bytes"] = rd_bytes
    res["attention_single_layer_warm_us"] = round(t_warm * 1e6, 2)
    res["attention_single_layer_warm_GBps"] = round(attn_bytes / t_warm / 1e9, 1)
    # full-cache encode and decode of one layer (the lengths as they are now)
    cache, seqs = layers[0]
    lens = seqs.seq_lens.cpu().numpy()
    rows = int(lens.sum())
    raw_bytes = rows * 2 * inst.w.num_kv_heads * inst.w.head_dim * 2
    top = int(cache.spill_top.item())
    packed_bytes = rows * row_bytes + 32 * top
    c2 = zf.PackedCache.empty(cache.num_pages, cache.page_size, cache.num_kv_heads,
                              cache.head_dim, cache.spill_slots, device=raw.device)
    enc_ws = zf.encode_workspace(seqs)

    def enc(i):
        c2.spill_top.zero_()
        zf.zf_encode_kv(c2, seqs, twins[0], enc_ws)
    t_enc = timeit(enc, n=10)
    t_dec = timeit(lambda i: zf.zf_decode_kv(cache, seqs, twins[0]), n=10)
    res["encode_GBps_read_plus_written"] = round((raw_bytes + packed_bytes) / t_enc / 1e9, 1)
    res["decode_GBps_read_plus_written"] = round((raw_bytes + packed_bytes) / t_dec / 1e9, 1)
    res["encode_us"] = round(t_enc * 1e6, 1)
    # multi-token append: up to 16 new tokens per sequence in one call, written over layer 0's
    # rows at the initial lengths (lengths and spill_top restored after each call); last
    # extra, since it rewrites those rows
    n_new = min(16, inst.w.extra_tokens)
    H, D = inst.w.num_kv_heads, inst.w.head_dim
    gen = torch.Generator(device="cpu").manual_seed(5)
    k16 = torch.randint(0x3C00, 0x4000, (inst.w.batch, n_new, H, D), generator=gen,
                        dtype=torch.int16).to(raw.device)
    v16 = k16.flip(1).contiguous()
    lens_at = torch.from_numpy(inst.seq_lens.copy()).to(raw.device)
    seqs_at = zf.Seqs(seqs.page_table, lens_at.clone(), seqs.max_seq_len)
    top_dev = cache.spill_top.clone()

    # single-token append (the decode step's write) alone, in both forms: HIP events around
    # each call only, lengths and spill_top restored between calls outside the timed interval
    k1, v1 = k16[:, 0].contiguous(), v16[:, 0].contiguous()
    for name, c in (("append_us", cache), ("append_two_launch_us", dataclasses.replace(cache, append_sync=None))):
        if c.append_sync is None and name == "append_us":
            continue
        ts = []
        for i in range(60):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            zf.zf_append_kv(c, seqs_at, k1, v1)
            b.record(stream)
            seqs_at.seq_lens.copy_(lens_at)
            c.spill_top.copy_(top_dev)
            if i >= 10:
                ts.append((a, b))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in ts]
        res[name] = round(float(np.mean(us)), 2)
        res[name.replace("_us", "_us_min")] = round(float(np.min(us)), 2)

    def app(i):
        zf.zf_append_kv_n(cache, seqs_at, k16, v16)
        seqs_at.seq_lens.copy_(lens_at)
        cache.spill_top.copy_(top_dev)
    t_app = timeit(app, n=10)
    assert zf.zf_get_status(cache.status) == 0
    res["append_n_tokens_per_seq"] = n_new
    res["append_n_us"] = round(t_app * 1e6, 1)
    res["append_n_rows_per_s"] = round(inst.w.batch * n_new / t_app, 1)
    res["decode_us"] = round(t_dec * 1e6, 1)
    # spill compaction (sequence free): layer 1 with every sequence live (its slots are
    # interleaved by the appends), then layer 2 with every other sequence freed
    for name, lay, live in (("all_live", 1, slice(None)), ("half_freed", 2, slice(0, None, 2))):
        cache, seqs = layers[lay]
        sub = zf.Seqs(seqs.page_table[live].contiguous(), seqs.seq_lens[live].contiguous(),
                      seqs.max_seq_len)
        cws = zf.compact_workspace(cache, sub)
        top_in = int(cache.spill_top.item())
        t_cmp = timeit(lambda i: zf.zf_compact_spill(cache, sub, cws), n=10)
        assert zf.zf_get_status(cache.status) == 0
        moved = int(cache.spill_top.item())
        res[f"compact_{name}_us"] = round(t_cmp * 1e6, 1)
        res[f"compact_{name}_slots"] = [top_in, moved]
    # capacity at a fixed HBM budget, Llama-3.1-8B-shaped KV (32 layers, 8 kv heads, D 128):
    # 288 GB of HBM less the bf16 weights (8.03e9 parameters x 16 bits / 8) and a 10 % reserve
    w = inst.w
    budget = int(288e9 - 8.03e9 * 16 / 8 - 0.1 * 288e9)
    raw_per_row = top / rows
    ctx = int(inst.seq_lens.max())
    n_bf16 = zf.zf_max_sequences(budget, 32, ctx, w.page_size, w.num_kv_heads, w.head_dim, None)
    n_pack = zf.zf_max_sequences(budget, 32, ctx, w.page_size, w.num_kv_heads, w.head_dim,
                                 raw_per_row)
    res["capacity"] = {"kv_budget_bytes": budget, "layers": 32, "context": ctx,
                       "raw_blocks_per_row": round(raw_per_row, 3),
                       "sequences_bf16": n_bf16, "sequences_packed": n_pack,
                       "gain": round(n_pack / n_bf16, 3)}
    return res


def diffuse_workloads(synth):
    """Diffuse-softmax forms of the batch-32 decode step, the 32k-token split case and the
    8-head groups: the stated value distributions without outlier keys (outlier values kept),
    so that a row's weight spreads over hundreds of tokens instead of one."""
    W = synth.WORKLOADS
    return {"d1": W[1].replace(name="diffuse_b32_ctx4096_v_outliers", outlier_kinds=2, seed=41),
            "d2": W[2].replace(name="diffuse_b16_ctx32768_v_outliers", k_scale=(0.25, 4.0),
                               outlier_kinds=2, seed=43),
            "d8": W[5].replace(name="diffuse_gqa8_b32_ctx4096_v_outliers", outlier_kinds=2, seed=44)}


def per_config(torch, zf, synth, key, dev):
    """Attention alone on one workload (no append): the packed call and its split kernel, and
    the twin, rotating over layer caches well beyond the last-level cache.  `key`: a workload
    index, or d1 / d2 / d8 for a diffuse-softmax form."""
    key = str(key)
    diffuse = diffuse_workloads(synth)
    w = (diffuse[key] if key in diffuse else synth.WORKLOADS[int(key)]).replace(extra_tokens=0)
    wi = int(key) if key.isdigit() else 100 + list(diffuse).index(key)
    inst = synth.make(w)
    to = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    T, H, D, Hq = w.page_size, w.num_kv_heads, w.head_dim, w.num_q_heads
    raw = to(inst.raw_pages)
    NL = max(2, -(-1200_000_000 // (int(inst.seq_lens.sum()) * 3404)))  # >= 1.2 GB of caches
    layers = []
    for _ in range(NL):
        cache = zf.PackedCache.empty(inst.num_pages, T, H, D, int(inst.seq_lens.sum()) * 2 * H * (D // 64),
                                     device=dev)
        seqs = zf.Seqs(to(inst.page_table), to(inst.seq_lens.copy()), int(inst.seq_lens.max()),
                       page_hint(torch, w.batch, H, inst.page_table.shape[1], dev))
        zf.zf_encode_kv(cache, seqs, raw, zf.encode_workspace(seqs))
        layers.append((cache, seqs))
    torch.cuda.synchronize()
    top = int(layers[0][0].spill_top.item())
    rows = int(inst.seq_lens.sum())
    pt_bytes = sum(-(-int(L) // T) for L in inst.seq_lens) * 4
    attn_bytes = rows * 3112 + 32 * top + w.batch * Hq * D * (2 + 4) + pt_bytes + 4 * w.batch
    q = to(synth.query(w, 0))
    out = torch.empty((w.batch, Hq, D), dtype=torch.float32, device=dev)
    ws = zf.attention_workspace(w.batch, H, Hq, D, layers[0][1].max_seq_len, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    scale = fp32_scale(D)
    stream = torch.cuda.current_stream()
    N = 55  # 50 timed calls after the first 5

    def run(fn, stamps):
        for i in range(3 * N):  # untimed: bring the GPU to its working clock
            fn(i)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(N)]
        for e in ev:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        for i in range(N):
            ev[i][0].record(stream)
            if stamps:
                zf.zf_time_next_attention(ev[i][2], ev[i][3])
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        call = np.array([e[0].elapsed_time(e[1]) for e in ev[5:]]) * 1e3
        kern = np.array([e[2].elapsed_time(e[3]) for e in ev[5:]]) * 1e3 if stamps else None
        return call, kern
    packed = lambda i: zf.zf_decode_attention(layers[i % NL][0], layers[i % NL][1], q, scale, out, ws)
    call, _ = run(packed, False)   # plain launches, as the twin's below
    _, kern = run(packed, True)    # stamped launches (slower dispatch) for the kernel's own time
    twins = []
    for cache, seqs in layers[:2]:
        d = torch.zeros_like(raw)
        zf.zf_decode_kv(cache, seqs, d)
        twins.append(d)
    del raw
    twin = lambda i: zf.zf_decode_attention_raw(twins[i % 2], layers[i % 2][1], q, scale, out, ws, status)
    tcall, _ = run(twin, False)
    _, tkern = run(twin, True)
    for cache, _ in layers:
        assert zf.zf_get_status(cache.status) == 0
    # sampled parity against the oracle: 16 (sequence, q head) rows, with their effective token
    # counts (sum w)^2 / sum w^2, so that a row one token dominates is told from a diffuse one
    import oracle
    rng = np.random.default_rng(wi)
    want = np.zeros((w.batch, Hq), np.uint8)
    want.reshape(-1)[rng.choice(w.batch * Hq, size=min(16, w.batch * Hq), replace=False)] = 1
    zf.zf_decode_attention(layers[0][0], layers[0][1], q, scale, out, ws)
    got = out.cpu().numpy().astype(np.float64)
    st, ref, neff = oracle.attention(inst.raw_pages, inst.seq_lens, inst.page_table, synth.query(w, 0),
                                     scale=scale, want=want, threads=host_cores(), with_neff=True)
    assert st == 0
    sel = want.astype(bool)
    err = np.abs(got[sel] - ref[sel])
    big = np.abs(ref[sel]) > 1e-3
    blocks = rows * 2 * H * (D // 64)
    return {"workload": w.name, "batch": w.batch, "tokens": rows, "q_heads": Hq, "kv_heads": H,
            "layers_rotated": NL, "attention_bytes": attn_bytes,
            "call_us_median": round(float(np.median(call)), 2),
            "call_us_mean": round(float(call.mean()), 2),
            "kernel_us_mean": round(float(kern.mean()), 2), "kernel_us_min": round(float(kern.min()), 2),
            "call_GBps": round(attn_bytes / call.mean() / 1e3, 1),
            "call_frac_of_8TBps": round(attn_bytes / call.mean() / 1e3 / 8000, 4),
            "uncompressed_equivalent_GBps": round(rows * H * 2 * D * 2 / call.mean() / 1e3, 1),
            "tokens_per_s": round(w.batch / call.mean() * 1e6, 1),
            "twin_call_us_mean": round(float(tcall.mean()), 2),
            "speedup_vs_twin": round(float(tcall.mean() / call.mean()), 3),
            "twin_kernel_us_mean": round(float(tkern.mean()), 2),
            "kernel_speedup_vs_twin": round(float(tkern.mean() / kern.mean()), 3),
            "compression_ratio": round((rows * 3112 + 32 * top) / (rows * H * 2 * D * 2), 4),
            "raw_block_fraction": round(top / blocks, 4),
            "raw_blocks_by_cause": raw_causes(inst, rng),
            "sampled_max_abs_err": float(err.max()),
            "sampled_max_rel_err": float((err[big] / np.abs(ref[sel][big])).max()) if big.any() else 0.0,
            "sampled_max_abs_ref": float(np.abs(ref[sel]).max()),
            "sampled_effective_tokens_median": round(float(np.median(neff[sel])), 1),
            "note": "call = split kernel + merge when the plan splits sequences; back to back; "
                    "50 timed calls; errors over 16 sampled (sequence, q head) rows against the oracle"}


def raw_causes(inst, rng, sample_rows=20000):
    """Why blocks stay raw, over a sample of token rows (the codec's rule, counted on the host
    from the generated values): an exponent field of 0 (zero or subnormal), one of 255 (Inf,
    NaN), or an exponent window wider than 16.  Fractions of all blocks of the sampled rows."""
    T = inst.w.page_size
    L = inst.seq_lens.astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(L)])
    pick = rng.choice(int(starts[-1]), size=min(sample_rows, int(starts[-1])), replace=False)
    b = np.searchsorted(starts, pick, side="right") - 1
    t = pick - starts[b]
    pages = inst.page_table[b, t // T]
    x = inst.raw_pages[pages, :, :, t % T, :]  # [rows][H][2][D]
    e = (x.reshape(len(pick), -1, 64).astype(np.int32) >> 7) & 0xFF
    zero = (e == 0).any(-1)
    inf_nan = (e == 255).any(-1) & ~zero
    wide = ~zero & ~inf_nan & (e.max(-1) - e.min(-1) > 15)
    n = e.shape[0] * e.shape[1]
    return {"zero_or_subnormal": round(float(zero.sum()) / n, 4), "inf_or_nan": round(float(inf_nan.sum()) / n, 4),
            "window_wider_than_16": round(float(wide.sum()) / n, 4), "sampled_rows": int(len(pick))}


def oracle_ops(w, inst, lens0, ks, vs, qs):
    """The oracle's single-thread rate per operation on the same workload: full-cache encode
    and decode (token rows/s), a one-token append (rows/s) and one step's attention over all
    heads (tokens/s): context for the GPU rates in the same line, not a tuned baseline."""
    import oracle

    T = w.page_size
    c = oracle.Cache(inst.num_pages, T, w.num_kv_heads, w.head_dim,
                     spill_slots=(int(lens0.sum()) + w.batch * 4) * 32)
    rows = int(lens0.sum())
    t0 = time.perf_counter()
    assert c.encode(lens0, inst.page_table, inst.raw_pages) == 0
    t_enc = time.perf_counter() - t0
    t0 = time.perf_counter()
    st, _ = c.decode(lens0, inst.page_table)
    t_dec = time.perf_counter() - t0
    assert st == 0
    lens = lens0.copy()
    t0 = time.perf_counter()
    assert c.append(lens, inst.page_table, ks[0], vs[0]) == 0
    t_app = time.perf_counter() - t0
    t0 = time.perf_counter()
    st, _ = oracle.attention(inst.raw_pages, lens0, inst.page_table, qs[0], scale=fp32_scale(w.head_dim))
    t_att = time.perf_counter() - t0
    assert st == 0
    return {"cores": 1, "encode_rows_per_s": round(rows / t_enc, 1), "decode_rows_per_s": round(rows / t_dec, 1),
            "append_rows_per_s": round(w.batch / t_app, 1), "attention_tokens_per_s": round(w.batch / t_att, 3),
            "rows": rows}


def _pmc_rows(d: str):
    """(kernel name and grid size, counter, value) of every dispatch in the rocprofv3 counter
    CSVs under d."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            rows.append((f'{r["Kernel_Name"]}|{r["Grid_Size"]}', r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def _per_dispatch(rows, counter, match):
    vals = [v for k, c, v in rows if c == counter and match(k)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def pmc_summary(out, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """HBM bytes per dispatch of the path's kernels from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, summed over the chip's channels), each scaled by what the same counter reads for
    a plain device copy of 1 GiB (the --calibrate-copy run)."""
    fetch, write = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    cal_f, _ = _per_dispatch(_pmc_rows(cal_fetch_dir), "FETCH_SIZE", lambda k: "copyBuffer" in k)
    cal_w, _ = _per_dispatch(_pmc_rows(cal_write_dir), "WRITE_SIZE", lambda k: "copyBuffer" in k)
    n = 1 << 30
    ff, wf = n / (cal_f * 1024), n / (cal_w * 1024)
    kernels = {}
    for name in sorted({k for k, _, _ in fetch} | {k for k, _, _ in write}):
        short = name.split("(")[0] + " grid " + name.rsplit("|", 1)[1]
        if short.startswith("void "):
            short = short[5:]
        if not short.startswith("zf::"):
            continue
        f, nf = _per_dispatch(fetch, "FETCH_SIZE", lambda k: k == name)
        w_, nw = _per_dispatch(write, "WRITE_SIZE", lambda k: k == name)
        kernels[short] = {"dispatches": max(nf, nw),
                          "FETCH_SIZE_KiB_per_dispatch": f, "WRITE_SIZE_KiB_per_dispatch": w_,
                          "hbm_read_bytes_per_dispatch": None if f is None else round(f * 1024 * ff),
                          "hbm_write_bytes_per_dispatch": None if w_ is None else round(w_ * 1024 * wf)}
    res = {"attn_source_hash": attn_source_hash(),
           "calibration": {"copy_bytes_read": n, "copy_bytes_written": n, "FETCH_SIZE_KiB": cal_f,
                           "WRITE_SIZE_KiB": cal_w, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": kernels}
    attn = max((v for k, v in kernels.items() if k.startswith("zf::attn_k<zf::PackedLoader")),
               key=lambda v: v["dispatches"], default=None)
    if attn and attn["hbm_read_bytes_per_dispatch"] is not None and attn["hbm_write_bytes_per_dispatch"] is not None:
        res["hbm_bytes_per_launch"] = attn["hbm_read_bytes_per_dispatch"] + attn["hbm_write_bytes_per_dispatch"]
    json.dump(res, open(out, "w"), indent=1)
    print(json.dumps(res, indent=1))


def prefill_chunks(torch, zf, synth, dev, n=512, chunks=4):
    """A prefill written as multi-token appends: 32 sequences take `chunks` chunks of `n`
    tokens each (16 384 rows per call, the chunked form) into an empty cache, each call timed
    with HIP events; rows/s against the full-cache encode of the same rows."""
    w = synth.WORKLOADS[1].replace(name="prefill_b32", ctx_min=n * chunks, ctx_max=n * chunks,
                                   extra_tokens=0, seed=71)
    inst = synth.make(w)
    B, H, D, T = w.batch, w.num_kv_heads, w.head_dim, w.page_size
    to = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    # the tokens of each chunk, [B][n][H][D], from the same pages the encode reads
    pages = inst.raw_pages
    kv = []
    for c in range(chunks):
        t = np.arange(c * n, (c + 1) * n)
        pg = inst.page_table[:, t // T]                       # [B][n]
        x = pages[pg, :, :, (t % T)[None, :], :]              # [B][n][H][2][D]
        kv.append((to(np.ascontiguousarray(x[:, :, :, 0])), to(np.ascontiguousarray(x[:, :, :, 1]))))
    rows = B * n * chunks
    stream = torch.cuda.current_stream()

    def run(timed):
        cache = zf.PackedCache.empty(inst.num_pages, T, H, D, rows * 2 * H * (D // 64), device=dev)
        seqs = zf.Seqs(to(inst.page_table), torch.zeros(B, dtype=torch.int32, device=dev), n * chunks)
        ev = []
        for k, v in kv:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            zf.zf_append_kv_n(cache, seqs, k, v)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        assert zf.zf_get_status(cache.status) == 0
        return cache, seqs, [a.elapsed_time(b) / 1e3 for a, b in ev]
    run(False)
    cache, seqs, ts = run(True)
    # the same rows by one full-cache encode
    raw = to(inst.raw_pages)
    c2 = zf.PackedCache.empty(inst.num_pages, T, H, D, cache.spill_slots, device=dev)
    ws = zf.encode_workspace(seqs)
    zf.zf_encode_kv(c2, seqs, raw, ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c2.spill_top.zero_()
    a.record(stream)
    zf.zf_encode_kv(c2, seqs, raw, ws)
    b.record(stream)
    torch.cuda.synchronize()
    t_enc = a.elapsed_time(b) / 1e3
    same = all(torch.equal(getattr(cache, f), getattr(c2, f)) for f in ("sm", "nib", "base", "row_flags"))
    return {"prefill_chunk_tokens_per_seq": n, "prefill_chunk_rows": B * n,
            "prefill_chunk_us": [round(t * 1e6, 1) for t in ts],
            "prefill_chunked_rows_per_s": round(rows / sum(ts), 1),
            "prefill_encode_rows_per_s": round(rows / t_enc, 1),
            "prefill_chunked_vs_encode_time": round(sum(ts) / t_enc, 3),
            "prefill_chunked_planes_equal_encode": bool(same)}


def page_hint(torch, batch: int, num_kv_heads: int, max_pages: int, dev):
    """Device array for the attention's page-order hint (the encode fills it, appends raise it)."""
    return torch.zeros((batch, num_kv_heads, max_pages), dtype=torch.int32, device=dev)


def fp32_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as the C ABI carries it (an fp32 argument); the oracle gets the same."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def host_cores() -> int:
    """Host cores this process may use (its affinity mask, capped at 16: the host share of one
    GPU on the boxes this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inst, lens0, ks, vs, qs, budget_s, cores):
    """The oracle as it stands (plain C): whole decode steps of the same workload (append one
    token per sequence + fp64 attention for every head, the heads split over `cores` threads
    running the unchanged C routine on disjoint rows), repeated until the budget is spent;
    steps/s -> tokens/s."""
    import oracle

    T = w.page_size
    c = oracle.Cache(inst.num_pages, T, w.num_kv_heads, w.head_dim,
                     spill_slots=(int(lens0.sum()) + w.batch * len(ks)) * 32)
    assert c.encode(lens0, inst.page_table, inst.raw_pages) == 0
    raw = inst.raw_pages.copy()
    lens = lens0.copy()
    scale = fp32_scale(w.head_dim)
    done = 0
    t0 = time.perf_counter()
    cap = inst.page_table.shape[1] * T
    while done < len(ks) and int(lens.max()) < cap:
        k, v = ks[done], vs[done]
        pos = lens.copy()
        assert c.append(lens, inst.page_table, k, v) == 0
        for b in range(w.batch):
            page = inst.page_table[b, pos[b] // T]
            raw[page, :, 0, pos[b] % T] = k[b]
            raw[page, :, 1, pos[b] % T] = v[b]
        st, _ = oracle.attention(raw, lens, inst.page_table, qs[done], scale=scale, threads=cores)
        assert st == 0
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(w.batch * done / el, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{done} full decode steps (batch {w.batch}, append + fp64 attention over "
                      f"{int(lens0[0]) + 1}+ tokens, all {w.num_q_heads} heads), {el:.1f} s on "
                      f"{cores} thread(s) of {cpu_model()}"}


def full_cache_codec(torch, zf, synth, wi, dev):
    """Full-cache encode and decode of one workload (the 4 x 131072-token cache by default),
    each timed alone with HIP events over 10 calls after one untimed call: read + written
    bytes per second (raw bf16 rows read and packed bytes written for encode, the reverse for
    decode), beside the library's plain streaming copy of the raw pages (zf_stream_copy_probe),
    the achievable read-plus-write rate."""
    w = synth.WORKLOADS[wi].replace(extra_tokens=0)
    inst = synth.make(w)
    H, D, T = w.num_kv_heads, w.head_dim, w.page_size
    to = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    raw = to(inst.raw_pages)
    rows = int(inst.seq_lens.sum())
    cache = zf.PackedCache.empty(inst.num_pages, T, H, D, rows * 2 * H * (D // 64), device=dev)
    seqs = zf.Seqs(to(inst.page_table), to(inst.seq_lens.copy()), int(inst.seq_lens.max()))
    ws = zf.encode_workspace(seqs)
    stream = torch.cuda.current_stream()

    def timeit(fn, n=10):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3

    def enc():
        cache.spill_top.zero_()
        zf.zf_encode_kv(cache, seqs, raw, ws)
    t_enc = timeit(enc)
    assert zf.zf_get_status(cache.status) == 0
    top = int(cache.spill_top.item())
    out = torch.empty_like(raw)
    t_dec = timeit(lambda: zf.zf_decode_kv(cache, seqs, out))
    assert zf.zf_get_status(cache.status) == 0
    # the achievable read-plus-write rate on the same buffers: the library's streaming copy of
    # the raw pages into the decode's output
    t_copy = timeit(lambda: zf.zf_stream_copy_probe(raw, out))
    copy_gbps = 2 * raw.numel() * raw.element_size() / t_copy / 1e9
    raw_bytes = rows * 2 * H * D * 2
    packed_bytes = rows * (2 * H * (D + D // 2 + D // 64) + 8) + 32 * top
    enc_gbps = (raw_bytes + packed_bytes) / t_enc / 1e9
    dec_gbps = (raw_bytes + packed_bytes) / t_dec / 1e9
    pref = f"codec_{w.name}"
    return {f"{pref}_encode_us": round(t_enc * 1e6, 1),
            f"{pref}_encode_GBps_read_plus_written": round(enc_gbps, 1),
            f"{pref}_decode_us": round(t_dec * 1e6, 1),
            f"{pref}_decode_GBps_read_plus_written": round(dec_gbps, 1),
            f"{pref}_copy_probe_GBps_read_plus_written": round(copy_gbps, 1),
            f"{pref}_encode_of_copy_probe": round(enc_gbps / copy_gbps, 3),
            f"{pref}_decode_of_copy_probe": round(dec_gbps / copy_gbps, 3),
            f"{pref}_encode_of_8TBps": round(enc_gbps / PEAK_HBM_GBS, 3),
            f"{pref}_decode_of_8TBps": round(dec_gbps / PEAK_HBM_GBS, 3),
            f"{pref}_rows": rows, f"{pref}_raw_blocks": top}


if __name__ == "__main__":
    main()
