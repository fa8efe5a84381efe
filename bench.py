#!/usr/bin/env python
"""KIVI hot path on one MI355X: prefill quantization and decode attention
over the packed 2-bit cache.

One step = one pass of the whole path over one batch of synthetic input:
a one-shot append of the context (K per-channel and V per-token quantization,
packing, residual-ring copy) followed by one decode-attention step (split-K
pass + combine).  The inputs are generated on the device before timing.  Each
phase is timed with HIP events recorded on the stream the kernels run on.  A
1 GiB eviction *read* of an unrelated buffer precedes each phase, so that
neither phase finds its data in the 256 MB Infinity Cache and neither pays for
write-backs of dirty lines left by the previous one (evicting by writing would
leave the cache full of dirty lines and put their write-back inside the timed
phase).

Prints one JSON line; `value` is decode-attention GB/s of algorithmic bytes
(packed codes + fp16 zero/scale + fp16 residual + q + out).

Also measured in the same run: the bandwidth of a plain device copy (512 MiB
read + 512 MiB written by one elementwise kernel), the second yardstick for
"% of peak", and the kernel whose FETCH_SIZE / WRITE_SIZE counter readings
calibrate the HBM-traffic figures.  `roofline.traffic` is taken from the
committed counter summary for this workload only while the kernel sources
still hash to the value recorded with it; otherwise it is null.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COPY_BYTES = 512 << 20          # per direction
KERNEL_SOURCES = ("kv_cache_quantization_amd/csrc/kivi_kernels.hip",
                  "kv_cache_quantization_amd/csrc/kivi_internal.h")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(name, key="traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed counter summary (profiles/name):
    lines 'key: value'.  None unless its kernel_source_sha256 matches."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    return int(kv[key]), name


def decode_bytes(B, H, Hq, n, Q, bits, D=128, G=32):
    per_stream = Q * D * 2 * bits / 8 + (Q // G) * D * 4 + Q * (D // G) * 4 + (n - Q) * D * 2 * 2
    return B * H * per_stream + B * Hq * D * (2 + 4)


def decode_bytes_kv(B, H, Hq, n, qk, qv, bits, D=128, G=32):
    """Decode bytes when keys are quantized up to qk and values up to qv
    (equal under the window policy: then this is decode_bytes)."""
    k = qk * D * bits / 8 + (qk // G) * D * 4 + (n - qk) * D * 2
    v = qv * D * bits / 8 + qv * (D // G) * 4 + (n - qv) * D * 2
    return B * H * (k + v) + B * Hq * D * (2 + 4)


def kcvt_decode_bytes(B, H, Hq, n, Q, bits, segments, D=128):
    """Decode bytes under the segment policy (KCVT): the codes, one fp16 pair
    per token for its 128 value channels, one fp16 pair per key channel and
    segment, the fp16 buffer, q and out."""
    per_stream = Q * D * 2 * bits / 8 + Q * 4 + segments * D * 4 + (n - Q) * D * 2 * 2
    return B * H * per_stream + B * Hq * D * (2 + 4)


def kcvt_append_bytes(B, H, n, Q, bits, segments, D=128, esize=2):
    """A segment-policy append: read K and V, write codes, one value pair per
    token and one key pair per channel and segment, copy the buffer rows."""
    q_el = B * H * Q * D * 2
    return (q_el * (esize + bits / 8) + B * H * (Q * 4 + segments * D * 4)
            + B * H * (n - Q) * D * 2 * 2 * esize)


def append_bytes(B, H, n, Q, bits, D=128, G=32, esize=2):
    """One-shot append of n tokens: read K and V (esize B per element), write
    codes (b/8 B) and zero/scale (4/G B) for the Q quantized tokens, copy the
    n - Q residual rows into the ring (read + write)."""
    q_el = B * H * Q * D * 2
    r_el = B * H * (n - Q) * D * 2
    return q_el * (esize + bits / 8 + 4 / G) + r_el * 2 * esize


def cpu_facts():
    """Host facts for the CPU baseline: usable cores, OMP_NUM_THREADS, CPU model."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(cores, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else cores
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": cores, "OMP_NUM_THREADS": omp, "threads": threads, "cpu_model": model}


def _oracle_stream(k, v, q, bits, R, gq, b, h):
    """The oracle on one (batch, KV-head) stream: build_cache (quantize),
    then dequantize + fp64 attention for its gq query heads.  Returns the
    two durations (the C calls release the GIL, so streams run in parallel)."""
    import oracle
    ks, vs = k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1]
    t0 = time.perf_counter()
    c = oracle.build_cache(ks, vs, bits, 32, R)
    t1 = time.perf_counter()
    kh, vh = oracle.dequant_cache(ks, vs, c)
    oracle.decode_attn(q[b:b + 1, h * gq:(h + 1) * gq], kh, vh)
    t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def _oracle_pass(k, v, q, bits, R, streams, threads):
    """Wall-clock seconds of the oracle over `streams` (list of (b, h)) on
    `threads` threads: quantize of every stream, then decode of every stream
    (two phases, each timed on its own)."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    H, Hq = k.shape[1], q.shape[1]
    gq = Hq // H
    caches = [None] * len(streams)

    def quant(i):
        b, h = streams[i]
        caches[i] = oracle.build_cache(k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], bits, 32, R)

    def dec(i):
        b, h = streams[i]
        ks, vs = k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1]
        kh, vh = oracle.dequant_cache(ks, vs, caches[i])
        oracle.decode_attn(q[b:b + 1, h * gq:(h + 1) * gq], kh, vh)
        caches[i] = None

    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(quant, range(len(streams))))
        t1 = time.perf_counter()
        list(ex.map(dec, range(len(streams))))
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def cpu_baseline(k_dev, v_dev, q_dev, bits, R, H, Hq, c5=None):
    """The CPU oracle as it stands (single-threaded C per call), timed on the
    host's cores with one call per (batch, KV-head) stream spread over a
    thread pool -- the streams are independent -- and on one thread over one
    batch entry.  The whole long-context workload runs on all threads; the
    B32 x 131072 workload (c5 = (k, v, q) of its first 16 streams, host
    arrays) on a fixed sample of 16 of its 256 streams, scaled by its
    bytes.  GB/s are over the same algorithmic bytes as the GPU figures."""
    import oracle
    oracle.lib()
    facts = cpu_facts()
    k = k_dev.cpu().numpy()
    v = v_dev.cpu().numpy()
    q = q_dev.cpu().numpy()
    B, n = k.shape[0], k.shape[2]
    Q = max(0, n - R) // 32 * 32
    streams = [(b, h) for b in range(B) for h in range(H)]
    tq, td = _oracle_pass(k, v, q, bits, R, streams, facts["threads"])
    one = [(0, h) for h in range(H)]
    tq1, td1 = _oracle_pass(k, v, q, bits, R, one, 1)
    res = dict(
        value=decode_bytes(B, H, Hq, n, Q, bits) / td / 1e9,
        unit="GB/s", cores=facts["threads"], kind="oracle",
        quantize_GBps=append_bytes(B, H, n, Q, bits) / tq / 1e9,
        sample="the whole long-context workload (%d streams x %d tokens) on %d threads, one "
               "oracle call per stream; decode = dequantize + fp64 attention, quantize = "
               "build_cache" % (len(streams), n, facts["threads"]),
        seconds=dict(quantize=tq, decode=td),
        one_thread=dict(streams=len(one), decode_GBps=decode_bytes(1, H, Hq, n, Q, bits) / td1 / 1e9,
                        quantize_GBps=append_bytes(1, H, n, Q, bits) / tq1 / 1e9,
                        seconds=dict(quantize=tq1, decode=td1)),
        host=facts)
    if c5 is not None:
        k5, v5, q5, B5, n5 = c5
        Q5 = max(0, n5 - R) // 32 * 32
        sb = k5.shape[0]
        s5 = [(b, h) for b in range(sb) for h in range(H)]
        tq5, td5 = _oracle_pass(k5, v5, q5, bits, R, s5, facts["threads"])
        res["b32_ctx131072"] = dict(
            sample="%d of %d streams (the first %d batch entries), extrapolated: GB/s over the "
                   "sample's bytes" % (len(s5), B5 * H, sb),
            decode_GBps=decode_bytes(sb, H, Hq, n5, Q5, bits) / td5 / 1e9,
            quantize_GBps=append_bytes(sb, H, n5, Q5, bits) / tq5 / 1e9,
            seconds=dict(quantize=tq5, decode=td5), extrapolated=True)
    return res


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak


def attn_measure(cache, B, Hq, n, T, stream, evict, evict_out, do_evict):
    """The attention of T causal queries per head (the last T cached tokens,
    as in a chunked-prefill step) over the cache the decode steps built.
    Useful flops: 2 * 2 * D per (query, visible token, query head)."""
    import torch
    from kv_cache_quantization_amd import synth, kivi
    D = 128
    qm = synth.queries_multi_device(3, B, Hq, T, D)
    out = torch.empty((B, Hq, T, D), dtype=torch.float32, device=qm.device)
    ms = []
    for i in range(6):
        if do_evict:
            torch.amax(evict, dim=0, out=evict_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.attn(qm, causal=True, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 1:
            ms.append(e0.elapsed_time(e1))
    t = sum(ms) / len(ms) / 1e3
    seen = sum(n - T + t_ + 1 for t_ in range(T))
    flops = 4.0 * D * B * Hq * seen
    tf = flops / t / 1e12
    qb, splits, gps = kivi.kivi_attn_plan(cache.handle, T)
    return {
        "workload": "attention of %d causal queries per head (the last %d cached tokens) over "
                    "the same cache, fp16 queries" % (T, T),
        "T": T, "ms": round(t * 1e3, 4), "median_ms": round(sorted(ms)[len(ms) // 2], 4),
        "useful_flops": flops,
        "plan": {"query_blocks": qb, "splits": splits, "groups_per_split": gps},
        "roofline": {"bound": "mfma", "kernel": "attn (one kivi_attn call)",
                     "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None},
    }


def streaming_measure(policy, do_evict, evict, evict_out, steps=512, prefill=8192, B=8, R=128,
                      bits=2, fused=False):
    """The streaming workload: batch 8, 8 KV / 32 query heads, a one-shot
    prefill of 8192 tokens, then `steps` decode steps that each append one
    token (K, V ~ N(0, 1) fp16, outlier key channels) and run decode
    attention with a fresh query (fused: both in one kivi_append_decode call).

    warm: the steps' per-step working set (about 55 MB) stays in the 256 MB
    Infinity Cache, as in a real serving loop.  All steps are captured once
    in a HIP graph (the host cannot issue four launches per step as fast as
    the GPU runs them) and the graph is replayed from the post-prefill
    cache, restored between replays; the time is the replay over `steps`.
    cold: eager steps, each after a 1 GiB eviction read (which also gives
    the host time to enqueue the step), timed with events per step."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth, kivi
    H, Hq, D = 8, 32, 128
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    k0, v0 = synth.kv_device(4, B, H, prefill, chunk=0, device=dev)
    rows = [synth.kv_device(4, B, H, 1, chunk=1 + s, device=dev) for s in range(steps)]
    qs = [synth.queries_device(4, B, Hq, step=s, device=dev) for s in range(steps)]
    outs = torch.empty((steps, B, Hq, D), dtype=torch.float32, device=dev)
    cache = KiviCache(B, H, Hq, prefill + steps, bits=bits, residual=R, device=dev, policy=policy)
    cache.workspace()
    cache.append(k0, v0)
    torch.cuda.synchronize()
    snap = cache.buffer.clone()
    n0 = cache.layout()

    # algorithmic bytes of every step: the appended token (K and V rows into
    # the ring, read + write), the tokens that age out of full precision
    # (read, codes and side data written), and the decode over all n tokens
    total = 0
    flushes = 0
    n, qk, qv = prefill, n0.n_quantized, n0.n_vquantized
    for s in range(steps):
        n += 1
        if policy == kivi.KIVI_FLUSH_PAPER:
            nqk, nqv = n - n % R, max(0, n - R)
        else:
            nqk = nqv = (max(0, n - R) // 32) * 32
        quant = B * H * D * ((nqk - qk) + (nqv - qv)) * (2 + bits / 8 + 4 / 32)
        flushes += nqk > qk
        qk, qv = nqk, nqv
        total += B * H * 2 * D * 2 * 2 + quant + decode_bytes_kv(B, H, Hq, n, qk, qv, bits)
    res = {"policy": "window" if policy == kivi.KIVI_FLUSH_WINDOW else "paper",
           "calls": "kivi_append_decode" if fused else "kivi_append + kivi_decode_attn",
           "steps": steps, "bytes": int(total), "key_flushes": int(flushes)}

    def one_step(s):
        if fused:
            cache.append_decode(*rows[s], qs[s], out=outs[s])
        else:
            cache.append(*rows[s])
            cache.decode(qs[s], out=outs[s])

    def run_steps():
        for s in range(steps):
            one_step(s)

    # warm: capture all steps once, replay from the restored post-prefill cache
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.graph(g, stream=side):
        run_steps()
    torch.cuda.synchronize()
    ms = []
    for i in range(4):
        cache.buffer.copy_(snap)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        if i:
            ms.append(e0.elapsed_time(e1))
    t = sum(ms) / len(ms) / 1e3
    res["warm"] = {"us_per_step": round(t / steps * 1e6, 3), "GBps": round(total / t / 1e9, 1),
                   "timing": "one HIP-graph replay of all steps, mean of 3 replays"}
    del g

    # cold: eager steps, each after an eviction read, timed per step
    if do_evict:
        cache.reset()
        cache.append(k0, v0)
        torch.cuda.synchronize()
        per = []
        for s in range(steps):
            torch.amax(evict, dim=0, out=evict_out)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            one_step(s)
            e1.record(stream)
            per.append((e0, e1))
        torch.cuda.synchronize()
        tc = sum(a.elapsed_time(b) for a, b in per) / 1e3
        res["cold"] = {"us_per_step": round(tc / steps * 1e6, 3),
                       "GBps": round(total / tc / 1e9, 1),
                       "timing": "events around each eager step, 1 GiB eviction read before each"}
    del cache, snap
    torch.cuda.empty_cache()
    return res


def evict_read(evict, evict_out):
    """Read 1 GiB of an unrelated buffer (leaves no dirty lines behind)."""
    import torch
    torch.amax(evict, dim=0, out=evict_out)


def long_context_measure(B, n, R, bits, G, chunk, n_out, steps, warmup, stream, evict, evict_out,
                         do_evict, cfg_id=3, keep=False, policy=0):
    """Prefill + decode on one workload: inputs drawn on the device first;
    each step = a reset cache, the appends of all chunks (quantize + ring),
    then one decode step; each phase timed with HIP events on `stream`,
    after an eviction read.  Returns the record (and with keep=True also
    the cache, inputs and query for later use)."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    H, Hq, D = 8, 32, 128
    dev = stream.device
    chunk = chunk or n
    chunks = []
    for ci in range(0, n, chunk):
        cn = min(chunk, n - ci)
        chunks.append(synth.kv_device(cfg_id, B, H, cn, D, chunk=ci // chunk, device=dev))
    q = synth.queries_device(cfg_id, B, Hq, D, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    cache = KiviCache(B, H, Hq, n, bits=bits, group=G, residual=R, device=dev, key_outliers=n_out,
                      policy=policy)
    cache.workspace()
    torch.cuda.synchronize()

    def step(evs):
        cache.reset()
        if do_evict:
            evict_read(evict, evict_out)
        evs[0].record(stream)
        for k, v in chunks:
            cache.append(k, v)
        evs[1].record(stream)
        if do_evict:
            evict_read(evict, evict_out)
        evs[2].record(stream)
        cache.decode(q, out=out)
        evs[3].record(stream)

    for _ in range(warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(4)])
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s_ in range(steps):
        step(events[s_])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    app_ms = sorted(e[0].elapsed_time(e[1]) for e in events)
    dec_ms = sorted(e[2].elapsed_time(e[3]) for e in events)
    t_app = sum(app_ms) / steps / 1e3
    t_dec = sum(dec_ms) / steps / 1e3
    lo = cache.layout()
    Q = lo.n_quantized
    if policy == 2:
        # KCVT: one segment per flush (every chunk append moves Q here)
        segs = len(chunks)
        dbytes = kcvt_decode_bytes(B, H, Hq, n, Q, bits, segs)
        abytes = kcvt_append_bytes(B, H, n, Q, bits, segs)
    else:
        dbytes = decode_bytes(B, H, Hq, n, Q, bits, G=G)
        abytes = append_bytes(B, H, n, Q, bits, G=G)
    if n_out:
        # the kept channels' fp16 values (2 bytes per token and channel) and
        # their indices (2 bytes per channel and group), read by the decode
        # and written by the append
        extra = B * H * (Q // 32) * n_out * (32 * 2 + 2)
        dbytes += extra
        abytes += extra
    dec_gbps = dbytes / t_dec / 1e9
    app_gbps = abytes / t_app / 1e9
    splits, gps = cache.decode_plan()
    rec = {
        "workload": "%s %d-bit decode over a %s prefill: batch %d, 8 KV heads, 32 query heads, "
                    "head_dim 128, context %d, group %d, residual %d%s"
                    % ("KCVT (one key group per channel and flush segment)" if policy == 2
                       else "KIVI", bits,
                       "one-shot" if chunk == n else "%d-token-chunk" % chunk, B, n, G, R,
                       "" if not n_out else ", %d fp16 key channels per key group" % n_out),
        "batch": B, "context": n, "bits": bits, "group": G, "residual": R, "chunk": chunk,
        "quantized_tokens": Q, "decode_splits_per_stream": splits, "groups_per_split": gps,
        "decode": {"ms": round(t_dec * 1e3, 4), "median_ms": round(dec_ms[len(dec_ms) // 2], 4),
                   "GBps": round(dec_gbps, 1), "bytes": int(dbytes),
                   "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4)},
        "quantize": {"ms": round(t_app * 1e3, 4), "median_ms": round(app_ms[len(app_ms) // 2], 4),
                     "GBps": round(app_gbps, 1), "bytes": int(abytes),
                     "frac_hbm_peak": round(app_gbps / HBM_PEAK_GBPS, 4)},
        "steps": steps, "wall_s": round(t1 - t0, 3),
    }
    if keep:
        return rec, dict(cache=cache, chunks=chunks, q=q, out=out)
    del cache, chunks
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--bits", type=int, default=2, choices=(2, 4, 8))
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--context", type=int, default=32768)
    ap.add_argument("--residual", type=int, default=128)
    ap.add_argument("--group", type=int, default=32, choices=(32, 64, 128))
    ap.add_argument("--key-outliers", type=int, default=0, choices=(0, 1, 2, 3),
                    help="key channels kept in fp16 per 32-token key group (outlier-aware keys)")
    ap.add_argument("--chunk", type=int, default=0, help="prefill chunk (0: one shot)")
    ap.add_argument("--cpu-sample", type=int, default=1,
                    help="time the CPU oracle on the host's cores (0: skip)")
    ap.add_argument("--no-evict", action="store_true")
    ap.add_argument("--stream-steps", type=int, default=512,
                    help="also time the streaming workload (batch 8, prefill 8192, then this many "
                         "single-token append + decode steps) under both flush policies (0: skip)")
    ap.add_argument("--attn-queries", type=int, default=256,
                    help="also time the attention of this many causal queries per head over "
                         "the same cache (a chunked-prefill step; 0: skip)")
    ap.add_argument("--other-configs", type=int, default=1,
                    help="also time the other decode workloads: B32 x 131072 in 8192-token "
                         "chunks at 2 and 4 bits, this workload at 4 bits, and B1 x 4096 with "
                         "residual 32 (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every (batch, "
              "KV-head) stream is independent, so sharding by batch or KV head needs no "
              "communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    B, H, Hq, D = args.batch, 8, 32, 128
    n, R, bits, G = args.context, args.residual, args.bits, args.group
    chunk = args.chunk or n
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    evict = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
    evict_out = torch.empty((), dtype=torch.float32, device=dev)
    do_evict = not args.no_evict
    torch.cuda.synchronize()

    # Copy yardstick: one elementwise kernel reads COPY_BYTES and writes
    # COPY_BYTES (torch.neg; a same-dtype copy_ would become a DMA blit).
    csrc = evict[: COPY_BYTES // 4]
    cdst = torch.empty_like(csrc)
    copy_ms = []
    for _ in range(4):
        torch.amax(evict[COPY_BYTES // 4:], dim=0, out=evict_out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.neg(csrc, out=cdst)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    copy_gbps = 2 * COPY_BYTES / (sorted(copy_ms[1:])[1] / 1e3) / 1e9
    del cdst

    main_rec, kept = long_context_measure(B, n, R, bits, G, chunk, args.key_outliers, args.steps,
                                          args.warmup, stream, evict, evict_out, do_evict, keep=True)
    cache, q = kept["cache"], kept["q"]
    dec_gbps = main_rec["decode"]["GBps"]
    app_gbps = main_rec["quantize"]["GBps"]
    traffic, traffic_src = (None, "workload without a counter summary")
    atraffic = None
    if (B, n, R, bits, chunk, G, args.key_outliers) == (16, 32768, 128, 2, 32768, 32, 0):
        traffic, traffic_src = counter_traffic("decode_b16_ctx32768_2bit_counters.txt")
        atraffic, _ = counter_traffic("decode_b16_ctx32768_2bit_counters.txt",
                                      "append_traffic_bytes_per_launch")

    rec = {
        "metric": "decode-attn GB/s over packed 2-bit KV (% of HBM peak); quantize GB/s",
        "value": dec_gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_rec["wall_s"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u%d codes, f16 side data, f32 accumulate" % bits,
        "data": "synthetic: K,V ~ N(0,1) fp16 with 4 outlier key channels x5 per KV head, "
                "q ~ N(0,1) fp16, seeded torch generator on the device",
        "config": dict({k_: main_rec[k_] for k_ in ("workload", "batch", "context", "group",
                                                   "residual", "bits", "quantized_tokens",
                                                   "decode_splits_per_stream", "groups_per_split")},
                       kv_heads=H, q_heads=Hq, head_dim=D),
        "decode": dict(main_rec["decode"], pct_hbm_peak=round(100 * dec_gbps / HBM_PEAK_GBPS, 2),
                       pct_copy=round(100 * dec_gbps / copy_gbps, 2)),
        "quantize": dict(main_rec["quantize"], pct_hbm_peak=round(100 * app_gbps / HBM_PEAK_GBPS, 2),
                         pct_copy=round(100 * app_gbps / copy_gbps, 2)),
        "copy": {"GBps": round(copy_gbps, 1), "bytes": 2 * COPY_BYTES,
                 "what": "torch.neg over 512 MiB fp32 (read 512 MiB + write 512 MiB), median of 3"},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode (split-K pass + combine, one kivi_decode_attn call)",
            "achieved": dec_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
        },
        "roofline_quantize": {
            "bound": "hbm", "kernel": "append (quantize + ring copy, one kivi_append call)",
            "achieved": app_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(app_gbps / HBM_PEAK_GBPS, 4), "traffic": atraffic,
        },
        "timing": "HIP events on the launch stream around each phase; mean over the timed steps;"
                  " 1 GiB eviction read before each phase (outside the phase events)"
                  if do_evict else "HIP events, no eviction (warm)",
    }
    if args.attn_queries > 0:
        rec["attn"] = attn_measure(cache, B, Hq, n, args.attn_queries, stream, evict, evict_out,
                                   do_evict)
    host_inputs = None
    if args.cpu_sample > 0 and chunk == n and G == 32 and args.key_outliers == 0:
        k0, v0 = kept["chunks"][0]
        host_inputs = (k0.cpu(), v0.cpu(), q.cpu())
    del cache, kept
    torch.cuda.empty_cache()
    c5_host = None
    if args.other_configs > 0:
        others = {}
        # the largest workload: B32 x 131072 tokens appended in 8192-token
        # chunks, decode over the full packed cache, at 2 and 4 bits
        for b5 in (2, 4):
            others["b32_ctx131072_%dbit" % b5] = long_context_measure(
                32, 131072, 128, b5, 32, 8192, 0, 10, 2, stream, evict, evict_out, do_evict,
                cfg_id=5)
        if bits != 4 or (B, n) != (16, 32768):
            others["b16_ctx32768_4bit"] = long_context_measure(
                16, 32768, 128, 4, 32, 0, 0, 10, 2, stream, evict, evict_out, do_evict)
        # KCVT at 4 bits (the GEAR review's backbone at that width): one key
        # segment over the whole prompt, values grouped over all 128 channels
        others["b16_ctx32768_kcvt_4bit"] = long_context_measure(
            16, 32768, 128, 4, 128, 0, 0, 10, 2, stream, evict, evict_out, do_evict, policy=2)
        # one layer of a single sequence: launch-bound, reported only
        others["b1_ctx4096_2bit"] = long_context_measure(
            1, 4096, 32, 2, 32, 0, 0, 20, 5, stream, evict, evict_out, do_evict, cfg_id=2)
        # HBM traffic from the committed counter summary (while the kernel
        # sources still match it)
        t5, src5 = counter_traffic("decode_b32_ctx131072_2bit_counters.txt")
        others["b32_ctx131072_2bit"]["decode"]["traffic"] = t5
        others["b32_ctx131072_2bit"]["decode"]["traffic_source"] = src5
        rec["other_configs"] = others
        if args.cpu_sample > 0:
            from kv_cache_quantization_amd import synth
            k5, v5 = synth.kv_device(5, 32, H, 8192, D, chunk=0, device=dev)
            # the sample's streams over their whole 131072-token context
            ks = [k5[:2]]
            vs = [v5[:2]]
            del k5, v5
            for ci in range(1, 16):
                kc, vc = synth.kv_device(5, 32, H, 8192, D, chunk=ci, device=dev)
                ks.append(kc[:2].clone())
                vs.append(vc[:2].clone())
                del kc, vc
            q5 = synth.queries_device(5, 32, Hq, D, device=dev)[:2]
            c5_host = (torch.cat(ks, 2).cpu().numpy(), torch.cat(vs, 2).cpu().numpy(),
                       q5.cpu().numpy(), 32, 131072)
            del ks, vs
            torch.cuda.empty_cache()
    if args.stream_steps > 0:
        from kv_cache_quantization_amd import kivi
        rec["streaming"] = {
            "workload": "batch 8, 8 KV heads, 32 query heads, head_dim 128, 2-bit, group 32, "
                        "residual 128: prefill 8192 tokens, then %d steps of (append one token, "
                        "decode attention)" % args.stream_steps,
            "policies": [streaming_measure(pol, do_evict, evict, evict_out,
                                           steps=args.stream_steps, fused=fu)
                         for pol, fu in ((kivi.KIVI_FLUSH_WINDOW, False),
                                         (kivi.KIVI_FLUSH_WINDOW, True),
                                         (kivi.KIVI_FLUSH_PAPER, False))],
        }
    if host_inputs is not None:
        rec["cpu_baseline"] = cpu_baseline(*host_inputs, bits, R, H, Hq, c5=c5_host)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
