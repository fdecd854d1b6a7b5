#!/usr/bin/env python3
"""Benchmark of the TurboQuant key path on one MI355X.

One step = the whole hot path over one batch: encode a full key cache
(1,048,576 bf16 keys of the Llama-3.1-8B-shaped decode workload: batch 16,
8 KV heads x 8192 positions, d = 128, b = 3) and score one decode step of
queries (32 heads, GQA 4) against a packed cache.  Inputs are resident in
HBM before timing starts; buffers rotate over more than the 256 MB
Infinity Cache so that every launch streams from HBM.

Prints one JSON line (driver contract) with the end-to-end keys/s, per
kernel throughput, the roofline of the dominant kernel (HIP events on the
launch stream), and the oracle timed on the host cores on a bounded sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed keys scored/s + HBM GB/s (d=128, b=3); keys encoded/s"
PEAK_HBM_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload (1 = the headline decode config)")
    ap.add_argument("--bits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--preroll", type=float, default=1.0,
                    help="seconds of untimed back-to-back steps before the counted warm-up "
                         "(brings the GPU clock to its loaded steady state)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for p in ("kv_cache_vector_rotate_amd/csrc/tq_kernels.hip", "kv_cache_vector_rotate_amd/csrc/tq_host.cpp"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole groups, encode + score, until ~budget_s of work."""
    import oracle as O
    from kv_cache_vector_rotate_amd import workloads as W
    avail = len(os.sched_getaffinity(0))
    blas = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(avail)
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        pass
    cbo = O.make_codebook(wl.d, wl.bits, wl.m, 42)
    keys_done, t_work, groups = 0, 0.0, 0
    for g in range(wl.G):
        k = W.group_keys(wl, g)
        q = W.group_queries(wl, g)
        t0 = time.perf_counter()
        e = O.encode(cbo, k)
        buf = O.pack(cbo, e.codes[None], e.signs[None], e.nu16[None], e.rho16[None])
        O.score(cbo, buf, 1, wl.N, q[None])
        t_work += time.perf_counter() - t0
        keys_done += wl.N
        groups += 1
        if t_work >= budget_s:
            break
    return {"value": keys_done / t_work, "unit": "keys/s", "cores": int(blas or 1), "kind": "oracle",
            "sample": f"{groups} of {wl.G} groups ({keys_done} keys): fp64 encode + pack + score of "
                      f"{wl.Qg} queries per group, {t_work:.1f} s",
            "blas_threads": blas, "affinity_cores": avail, "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "note": "numpy fp64 oracle; its matrix products use the BLAS threads, the rest runs "
                    "on one Python thread"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def clock_mhz(K, torch):
    """Core clock seen by one wave over 40 us (constant 100 MHz reference)."""
    t = K.clock_probe(4000)
    torch.cuda.synchronize()
    cyc, ticks = (int(v) for v in t.cpu().tolist())
    return round(100.0 * cyc / max(ticks, 1), 1)


def preroll(step, seconds, torch):
    """Untimed back-to-back steps for `seconds` of wall time (GPU kept busy:
    one synchronisation per 50 steps)."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "steps": n}


def run_decode(args):
    """Workloads 0, 1, 3 (and 2 through run_long_context): one step = encode + score."""
    import torch
    import kv_cache_vector_rotate_amd as K
    from kv_cache_vector_rotate_amd import workloads as W

    wl = W.workload(args.config, bits=args.bits)
    G, N, Qg, d, bits = wl.G, wl.N, wl.Qg, wl.d, wl.bits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    keys_np = W.all_keys(wl)
    q_np = W.all_queries(wl)
    if wl.key_dtype == "bf16":
        keys0 = torch.from_numpy(keys_np.view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(q_np.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        keys0 = torch.from_numpy(keys_np).to(dev)
        q = torch.from_numpy(q_np).to(dev)
    del keys_np
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    cb = K.Codebook(d, bits, d, 42)
    key_bytes = keys0.numel() * keys0.element_size()
    pbytes = K.packed_nbytes(cb, G, N)
    logit_bytes = G * Qg * N * 4
    mall = 256 << 20
    nk = max(2, -(-3 * mall // key_bytes))          # key copies
    npk = max(4, -(-3 * mall // pbytes))            # packed copies
    nl = max(2, -(-mall // logit_bytes))
    keys = [keys0] + [keys0.clone() for _ in range(nk - 1)]
    packed = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(npk)]
    logits = [torch.empty((G, Qg, N), dtype=torch.float32, device=dev) for _ in range(nl)]
    ws = torch.empty(max(16, K.score_workspace_nbytes(cb, G, Qg)), dtype=torch.uint8, device=dev)
    for i in range(npk):
        K.encode_keys(cb, keys[i % nk], out=packed[i])
    torch.cuda.synchronize()

    def step(i, evs=None):
        if evs is not None:
            evs[0].record()
        K.encode_keys(cb, keys[i % nk], out=packed[i % npk])
        if evs is not None:
            evs[1].record()
        # score a cache encoded earlier (not the one just written, which may still
        # sit in the Infinity Cache)
        K.score_logits(cb, q, packed[(i + npk // 2) % npk], N, out=logits[i % nl], ws=ws)
        if evs is not None:
            evs[2].record()

    clk_idle = clock_mhz(K, torch)
    pre = preroll(step, args.preroll, torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    clk_before = clock_mhz(K, torch)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    clk_after = clock_mhz(K, torch)
    # the clock while the encoder runs: eight encodes back to back on the
    # library's stream, the probe's single wave on a second stream beside them
    # (the second stream is used once first: its first launch starts late);
    # reported only when the probe's events fall inside the encodes' window
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        K.clock_probe(4000)
    torch.cuda.synchronize()
    clk_enc = None
    for _ in range(3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for i in range(8):
            K.encode_keys(cb, keys[i % nk], out=packed[i % npk])
        ev[1].record()
        with torch.cuda.stream(side):
            ev[2].record()
            tprobe = K.clock_probe(4000)
            ev[3].record()
        torch.cuda.synchronize()
        if ev[0].elapsed_time(ev[3]) < ev[0].elapsed_time(ev[1]):
            cyc, ticks = (int(v) for v in tprobe.cpu().tolist())
            clk_enc = round(100.0 * cyc / max(ticks, 1), 1)
            break
    enc_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    sc_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    keys_per_step = G * N
    ms_per_step = wall * 1e3 / args.steps
    enc_alg = key_bytes + pbytes                               # read keys, write records
    q_bytes = q.numel() * q.element_size()
    sc_alg = pbytes + logit_bytes + q_bytes                    # read records + queries, write logits
    # rates from the median launch time (the mean is reported beside it)
    enc_avg_s = float(np.median(enc_ms)) * 1e-3
    sc_avg_s = float(np.median(sc_ms)) * 1e-3
    enc_gbps = enc_alg / enc_avg_s / 1e9
    sc_gbps = sc_alg / sc_avg_s / 1e9
    dominant = "encode" if enc_avg_s >= sc_avg_s else "score"
    traffic = read_traffic(f"encode128_{wl.key_dtype}_b{bits}_workload{args.config}.txt" if dominant == "encode"
                           else f"score128_b{bits}_workload{args.config}.txt")
    enc_kernel = (f"encode128_bf16_t16_kernel<{bits - 1}>" if wl.key_dtype == "bf16"
                  else f"encode128_f32_kernel<{bits - 1}>")
    sc_kernel = f"score128_kernel<{bits - 1}, {'true' if wl.key_dtype == 'bf16' else 'false'}>"
    roof = {"bound": "hbm", "kernel": enc_kernel if dominant == "encode" else sc_kernel,
            "achieved": round(enc_gbps if dominant == "encode" else sc_gbps, 1),
            "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round((enc_gbps if dominant == "encode" else sc_gbps) / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(enc_alg if dominant == "encode" else sc_alg),
            "time": "median HIP-event duration of the kernel's launches on the library's stream"}
    ceil = ceilings(K, cb, keys, packed, logits, G, Qg, N, nk, npk, nl)
    out = {
        "metric": METRIC,
        "value": round(keys_per_step / (ms_per_step * 1e-3), 1),
        "unit": "keys/s (encode full cache + score one decode step, per step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "groups": G, "keys_per_group": N, "queries_per_group": Qg,
                   "d": d, "bits": bits, "m": wl.m, "key_dtype": wl.key_dtype},
        "score": {"keys_per_s": round(keys_per_step / sc_avg_s, 1),
                  "logits_per_s": round(G * Qg * N / sc_avg_s, 1),
                  "hbm_GBps": round(sc_gbps, 1), "frac_of_peak": round(sc_gbps / PEAK_HBM_GBPS, 4),
                  "packed_kv_GBps": round(pbytes / sc_avg_s / 1e9, 1),
                  "us_median": round(float(np.median(sc_ms)) * 1e3, 2),
                  "us_mean": round(float(sc_ms.mean()) * 1e3, 2),
                  "us_p10": round(float(np.percentile(sc_ms, 10)) * 1e3, 2),
                  "us_p90": round(float(np.percentile(sc_ms, 90)) * 1e3, 2),
                  "algorithmic_bytes": int(sc_alg),
                  "frac_of_score_pattern_ceiling": round(sc_gbps / ceil["score_pattern_GBps"], 4)},
        "encode": {"keys_per_s": round(keys_per_step / enc_avg_s, 1),
                   "hbm_GBps": round(enc_gbps, 1), "frac_of_peak": round(enc_gbps / PEAK_HBM_GBPS, 4),
                   "packed_kv_GBps": round(pbytes / enc_avg_s / 1e9, 1),
                   "us_median": round(float(np.median(enc_ms)) * 1e3, 2),
                   "us_mean": round(float(enc_ms.mean()) * 1e3, 2),
                   "us_p10": round(float(np.percentile(enc_ms, 10)) * 1e3, 2),
                   "us_p90": round(float(np.percentile(enc_ms, 90)) * 1e3, 2),
                   "algorithmic_bytes": int(enc_alg),
                   "frac_of_encode_mix_ceiling": round(enc_gbps / ceil["encode_mix_GBps"], 4)},
        "roofline": roof,
        "ceilings": ceil,
        "clock_MHz": {"idle": clk_idle, "before_timed": clk_before, "after_timed": clk_after,
                      "during_encode": clk_enc,
                      "how": "one wave counts core-clock cycles over 40 us of the 100 MHz reference "
                             "(during_encode: on a second stream while encodes run back to back)"},
        "preroll": dict(pre, note="untimed back-to-back steps before the counted warm-up"),
        "rotation": {"key_copies": nk, "packed_copies": npk, "logit_copies": nl},
    }
    out["append"] = run_append(K, cb, keys0, q, G, N, Qg)
    out["decode_attention"] = run_attention(K, cb, keys0, q, G, N, Qg, packed, npk, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def ceilings(K, cb, keys, packed, logits, G, Qg, N, nk, npk, nl, reps=40):
    """Measured streaming ceilings on the same buffers (rotating past the
    Infinity Cache), median of `reps` launches each:
      read_only:     the key cache read with 16-byte loads, nothing written;
      copy:          key cache to key cache (equal read and write bytes);
      encode_mix:    the encoder's bytes (bf16 keys read, records written);
      score_mix:     the scorer's bytes (records read, logits written) by the
                     generic stream kernel, four workgroups per CU;
      score_pattern: the scorer's own grid, record loads and logit stores
                     without its set-up and arithmetic."""
    kb = keys[0].numel() * keys[0].element_size()
    pb = K.packed_nbytes(cb, G, N)
    lb = G * Qg * N * 4
    flat = lambda t: t.view(-1).view(torch_u8())
    out = {}
    t = _event_times(lambda i: K.stream_probe(flat(keys[i % nk])), reps)
    out["read_only_GBps"] = round(kb / (np.median(t) * 1e-3) / 1e9, 1)
    t = _event_times(lambda i: K.stream_probe(flat(keys[i % nk]), flat(keys[(i + 1) % nk])), reps)
    out["copy_GBps"] = round(2 * kb / (np.median(t) * 1e-3) / 1e9, 1)
    t = _event_times(lambda i: K.stream_probe(flat(keys[i % nk]), packed[i % npk]), reps)
    out["encode_mix_GBps"] = round((kb + pb) / (np.median(t) * 1e-3) / 1e9, 1)
    t = _event_times(lambda i: K.stream_probe(packed[i % npk], flat(logits[i % nl])), reps)
    out["score_mix_GBps"] = round((pb + lb) / (np.median(t) * 1e-3) / 1e9, 1)
    t = _event_times(lambda i: K.score_stream_probe(cb, G, Qg, packed[i % npk], N, logits[i % nl]), reps)
    out["score_pattern_GBps"] = round((pb + lb) / (np.median(t) * 1e-3) / 1e9, 1)
    out["score_pattern_us_median"] = round(float(np.median(t)) * 1e3, 2)
    return out


def torch_u8():
    import torch
    return torch.uint8


def run_append(K, cb, keys0, q, G, N, Qg, steps=64):
    """Decode loop on the same shapes: a cache of N + steps records per group,
    prefilled with the N keys, then per step one new key per group appended
    (tq_append_keys, T = 1) and the filled prefix scored (tq_score_cache).
    Event times of each call; the append is launch-latency bound."""
    import torch
    Ncap = N + steps
    cache = torch.empty(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device=keys0.device)
    K.append_keys(cb, keys0, cache, Ncap, 0)
    new = [keys0[:, i:i + 1].contiguous() for i in range(steps)]   # stand-in new tokens
    lg = torch.empty(G * Qg * Ncap, dtype=torch.float32, device=keys0.device)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        L = N + i + 1
        ev[i][0].record()
        K.append_keys(cb, new[i], cache, Ncap, L - 1)
        ev[i][1].record()
        K.score_cache(cb, q, cache, Ncap, L, out=lg[:G * Qg * L].view(G, Qg, L))
        ev[i][2].record()
    torch.cuda.synchronize()
    ap = np.array([e[0].elapsed_time(e[1]) for e in ev[4:]])
    sc = np.array([e[1].elapsed_time(e[2]) for e in ev[4:]])
    filler = lambda: K.stream_probe(keys0.view(-1).view(torch.uint8))
    app_us, app_ok = burst_us(K, torch, [(lambda i=i: K.append_keys(cb, new[i], cache, Ncap, N + i))
                                         for i in range(steps)], filler)
    out = {"note": "one decode step: append 1 key per group into a cache of N + 64 records, "
                   "then score the filled prefix; the cache fits the Infinity Cache here",
           "append_gpu_us": round(app_us, 2), "back_to_back": bool(app_ok),
           "keys_per_append": G,
           "append_us_median": round(float(np.median(ap)) * 1e3, 2),
           "append_us_p90": round(float(np.percentile(ap, 90)) * 1e3, 2),
           "score_cache_us_median": round(float(np.median(sc)) * 1e3, 2),
           "score_cache_us_p90": round(float(np.percentile(sc, 90)) * 1e3, 2)}
    out["paged"] = run_paged(K, cb, keys0, q, G, N, Qg, steps)
    return out


def burst_us(K, torch, calls, filler, n_fill=40):
    """GPU time per call of short launches: `n_fill` long streaming launches
    are queued first, so the host has enqueued every call before the GPU
    reaches them and they run back to back; the events bracket the calls
    only.  Returns (us per call, whether the host kept ahead)."""
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(n_fill):
        filler()
    e1.record()
    t0 = time.perf_counter()
    for c in calls:
        c()
    host_s = time.perf_counter() - t0
    e2.record()
    torch.cuda.synchronize()
    ahead = host_s * 1e3 < e0.elapsed_time(e1)
    return e1.elapsed_time(e2) * 1e3 / len(calls), ahead


def run_paged(K, cb, keys0, q, G, N, Qg, steps, ps=256):
    """The same decode loop on a paged cache: pages of 256 records assigned to
    the groups in a shuffled order, the N keys appended as one batch, then per
    step one new key per group (the G single rows take the latency kernel,
    one key per workgroup)
    and the paged score of every group's records."""
    import torch
    dev = keys0.device
    ppg = -(-(N + steps) // ps)
    num_pages = G * ppg
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(0)).to(torch.int32)
    table = perm.view(G, ppg).to(dev)
    pool = torch.empty(K.paged_pool_nbytes(cb, num_pages, ps), dtype=torch.uint8, device=dev)
    K.paged_append_keys(cb, keys0, pool, ps, table, torch.zeros(G, dtype=torch.int32, device=dev))
    new = [keys0[:, i:i + 1].contiguous() for i in range(steps)]
    lens = [torch.full((G,), N + i, dtype=torch.int32, device=dev) for i in range(steps + 1)]
    lg = torch.empty(G * Qg * (N + steps), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        L = N + i + 1
        ev[i][0].record()
        K.paged_append_keys(cb, new[i], pool, ps, table, lens[i])
        ev[i][1].record()
        K.paged_score(cb, q, pool, ps, table, lens[i + 1], L, out=lg[:G * Qg * L].view(G, Qg, L))
        ev[i][2].record()
    torch.cuda.synchronize()
    ap = np.array([e[0].elapsed_time(e[1]) for e in ev[4:]])
    sc = np.array([e[1].elapsed_time(e[2]) for e in ev[4:]])
    # back-to-back GPU times: the same appends alone, then the whole steps
    filler = lambda: K.stream_probe(keys0.view(-1).view(torch.uint8))
    app = [(lambda i=i: K.paged_append_keys(cb, new[i], pool, ps, table, lens[i])) for i in range(steps)]
    step_calls = []
    for i in range(steps):
        L = N + i + 1
        step_calls.append(app[i])
        step_calls.append(lambda i=i, L=L: K.paged_score(cb, q, pool, ps, table, lens[i + 1], L,
                                                         out=lg[:G * Qg * L].view(G, Qg, L)))
    app_us, app_ok = burst_us(K, torch, app, filler)
    step_us, step_ok = burst_us(K, torch, step_calls, filler)
    # the same measure for a minimal launch (one workgroup reading 4 KB)
    tiny = torch.zeros(4096, dtype=torch.uint8, device=dev)
    floor_us, _ = burst_us(K, torch, [lambda: K.stream_probe(tiny, grid=1)] * steps, filler)
    return {"page_size": ps, "pages": num_pages, "keys_per_append": G,
            "append_gpu_us": round(app_us, 2), "decode_step_gpu_us": round(2 * step_us, 2),
            "launch_floor_gpu_us": round(floor_us, 2),
            "back_to_back": bool(app_ok and step_ok),
            "append_us_median": round(float(np.median(ap)) * 1e3, 2),
            "append_us_p90": round(float(np.percentile(ap, 90)) * 1e3, 2),
            "score_us_median": round(float(np.median(sc)) * 1e3, 2),
            "score_us_p90": round(float(np.percentile(sc, 90)) * 1e3, 2),
            "note": "*_gpu_us: launches queued behind long streaming kernels run back to back "
                    "(GPU time per call); *_us_median: one event pair per call, which also holds "
                    "the host's launch gap when the GPU waits for it"}


def run_attention(K, cb, keys0, q, G, N, Qg, packed, npk, steps):
    """Value path on the same shapes: value records for the cache (values drawn
    like the keys: the key rows in reverse order), then decode attention of the
    step's queries over packed keys and values, with both caches rotating past
    the Infinity Cache.  Reports the value encoder and the attention call (the
    scorer with its value phase, then the combine) by HIP events."""
    import torch
    vals = keys0.flip(1).contiguous()
    vbytes = K.value_packed_nbytes(cb, G, N)
    nv = max(3, -(-3 * (256 << 20) // vbytes))
    vpk = [K.encode_values(cb, vals) for _ in range(nv)]
    ws = torch.empty(max(16, K.attention_workspace_nbytes(cb, G, Qg, N)), dtype=torch.uint8,
                     device=keys0.device)
    out = torch.empty((G, Qg, cb.d), dtype=torch.float32, device=keys0.device)
    enc = _event_times(lambda i: K.encode_values(cb, vals, out=vpk[i % nv]), steps)
    att = _event_times(lambda i: K.attention_decode(cb, q, packed[i % npk], vpk[i % nv], N, out=out,
                                                    ws=ws), steps)
    key_bytes = keys0.numel() * keys0.element_size()
    kbytes = K.packed_nbytes(cb, G, N)
    # attention, the method's own bytes: read key and value records and the
    # queries, write the outputs (anything the kernels stage in between is
    # not counted)
    att_alg = kbytes + vbytes + q.numel() * q.element_size() + G * Qg * cb.d * 4
    return {"values_encode": _stats(enc, key_bytes + vbytes, G * N, "values"),
            "attention": _stats(att, att_alg, G * N, "keys"),
            "value_record_bytes": int(vbytes // (G * N)),
            "note": "attention = scorer with its value phase (logits through the caches, "
                    "per-range softmax state) + combine (ranges merged, rotated back)",
            "cache_step": run_cache_step(K, cb, keys0, vals, q, G, N, Qg)}


def run_cache_step(K, cb, keys0, vals, q, G, N, Qg, steps=64):
    """The decode step of a serving loop on the same shapes: key and value
    caches of N + steps records per group, prefilled with the N keys and
    values; per step one new key and one new value per group appended
    (tq_append_keys, tq_append_values, T = 1) and attention over the filled
    prefix (tq_attention_cache).  Back-to-back GPU times per call and per
    step; the caches fit the Infinity Cache here."""
    import torch
    Ncap = N + steps
    kc = torch.empty(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device=keys0.device)
    vc = torch.empty(K.value_packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device=keys0.device)
    K.append_keys(cb, keys0, kc, Ncap, 0)
    K.append_values(cb, vals, vc, Ncap, 0)
    newk = [keys0[:, i:i + 1].contiguous() for i in range(steps)]   # stand-in new tokens
    newv = [vals[:, i:i + 1].contiguous() for i in range(steps)]
    ws = torch.empty(max(16, K.attention_workspace_nbytes(cb, G, Qg, Ncap)), dtype=torch.uint8,
                     device=keys0.device)
    out = torch.empty((G, Qg, cb.d), dtype=torch.float32, device=keys0.device)
    torch.cuda.synchronize()
    filler = lambda: K.stream_probe(keys0.view(-1).view(torch.uint8))
    app_us, app_ok = burst_us(K, torch, [(lambda i=i: K.append_values(cb, newv[i], vc, Ncap, N + i))
                                         for i in range(steps)], filler)
    att = _event_times(lambda i: K.attention_cache(cb, q, kc, vc, Ncap, N + steps, out=out, ws=ws), 20)
    calls = []
    for i in range(steps):
        L = N + i + 1
        calls.append(lambda i=i, L=L: K.append_keys(cb, newk[i], kc, Ncap, L - 1))
        calls.append(lambda i=i, L=L: K.append_values(cb, newv[i], vc, Ncap, L - 1))
        calls.append(lambda L=L: K.attention_cache(cb, q, kc, vc, Ncap, L, out=out, ws=ws))
    step_us, step_ok = burst_us(K, torch, calls, filler, n_fill=150)
    return {"values_per_append": G,
            "append_values_gpu_us": round(app_us, 2),
            "attention_cache_us_median": round(float(np.median(att)) * 1e3, 2),
            "decode_step_gpu_us": round(3 * step_us, 2),
            "back_to_back": bool(app_ok and step_ok),
            "note": "decode step = append key + append value + attention over the prefix, "
                    "GPU time back to back"}


def _event_times(fn, reps, warm=2, preroll_s=0.0):
    """Per-launch HIP-event times (ms) of `reps` calls of fn, after `warm`
    untimed calls and `preroll_s` seconds of untimed back-to-back calls (the
    core clock ramps up under load on a fresh box)."""
    import torch
    for _ in range(warm):
        fn(-1)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < preroll_s:
        for _ in range(10):
            fn(-1)
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])   # ms


def _stats(ms, alg_bytes=None, units=None, unit_name="keys"):
    """Rates from the median launch time (the mean is reported beside it)."""
    out = {"us_median": round(float(np.median(ms)) * 1e3, 2),
           "us_mean": round(float(ms.mean()) * 1e3, 2),
           "us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
           "us_p90": round(float(np.percentile(ms, 90)) * 1e3, 2)}
    med_s = float(np.median(ms)) * 1e-3
    if units is not None:
        out[f"{unit_name}_per_s"] = round(units / med_s, 1)
    if alg_bytes is not None:
        gbps = alg_bytes / med_s / 1e9
        out.update({"algorithmic_bytes": int(alg_bytes), "hbm_GBps": round(gbps, 1),
                    "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)})
    return out


def run_long_context(args):
    """Workload 2 (G=32 x N=131072, b=4): score against the packed cache and the
    in-library bf16 q.K GEMV on the same shapes, both against the HBM roofline."""
    import torch
    import kv_cache_vector_rotate_amd as K
    from kv_cache_vector_rotate_amd import workloads as W
    wl = W.workload(2, bits=args.bits)
    G, N, Qg, d, bits = wl.G, wl.N, wl.Qg, wl.d, wl.bits
    dev = torch.device("cuda:0")
    keys0 = torch.from_numpy(W.all_keys(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(W.all_queries(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    cb = K.Codebook(d, bits, d, 42)
    key_bytes = keys0.numel() * 2
    pbytes = K.packed_nbytes(cb, G, N)
    mall = 256 << 20
    keys = [keys0, keys0.clone()]
    npk = max(3, -(-3 * mall // pbytes))
    packed = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(npk)]
    for p_ in packed:
        K.encode_keys(cb, keys0, out=p_)
    logits = torch.empty((G, Qg, N), dtype=torch.float32, device=dev)
    enc = _event_times(lambda i: K.encode_keys(cb, keys[i % 2], out=packed[i % npk]), max(10, args.steps // 2),
                       preroll_s=args.preroll)
    sc = _event_times(lambda i: K.score_logits(cb, q, packed[i % npk], N, out=logits), args.steps,
                      preroll_s=args.preroll)
    dn = _event_times(lambda i: K.dense_logits_bf16(q, keys[i % 2], out=logits), args.steps)
    logit_bytes = G * Qg * N * 4
    q_bytes = q.numel() * 2
    out = {"metric": "packed keys scored/s + HBM GB/s; bf16 q.K GEMV on the same shapes",
           "config": {"workload": wl.name, "groups": G, "keys_per_group": N, "queries_per_group": Qg,
                      "d": d, "bits": bits},
           "encode": _stats(enc, key_bytes + pbytes, G * N),
           "score": _stats(sc, pbytes + logit_bytes + q_bytes, G * N),
           "dense_bf16_gemv": _stats(dn, key_bytes + logit_bytes + q_bytes, G * N),
           "score_speedup_vs_dense": round(float(dn.mean() / sc.mean()), 3),
           "bytes_ratio_dense_over_score": round((key_bytes + logit_bytes) / (pbytes + logit_bytes), 3)}
    print(json.dumps(out), flush=True)


def run_cache_sweep(args):
    """Workload 3 (Qwen2.5-3B-shaped cache, 72 groups x 8192 keys, Qg=8) at
    b = 2, 3, 4: encode/score throughput, packed bytes against the fp16 K+V
    cache, and the cosine between estimated and exact logits per query head."""
    import torch
    import kv_cache_vector_rotate_amd as K
    from kv_cache_vector_rotate_amd import workloads as W
    wl = W.workload(3)
    G, N, Qg, d = wl.G, wl.N, wl.Qg, wl.d
    dev = torch.device("cuda:0")
    keys = torch.from_numpy(W.all_keys(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(W.all_queries(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    exact = torch.matmul(q.float(), keys.float().transpose(1, 2).contiguous())   # [G, Qg, N]
    fp16_kv = G * N * d * 2 * 2
    rows = []
    for bits in (2, 3, 4):
        cb = K.Codebook(d, bits, d, 42)
        pbytes = K.packed_nbytes(cb, G, N)
        packed = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
        enc = _event_times(lambda i: K.encode_keys(cb, keys, out=packed[i % 2]), max(10, args.steps // 2),
                           preroll_s=args.preroll)
        lg = torch.empty((G, Qg, N), dtype=torch.float32, device=dev)
        sc = _event_times(lambda i: K.score_logits(cb, q, packed[i % 2], N, out=lg), args.steps,
                          preroll_s=args.preroll)
        est = K.score_logits(cb, q, packed[0], N).double()
        ex = exact.double()
        cos = (est * ex).sum(-1) / (est.norm(dim=-1) * ex.norm(dim=-1))
        v_bytes = G * N * (bits * d // 8 + 2)          # values: bits-bit MSE codes + one half norm
        rows.append({"bits": bits, "packed_key_bytes": int(pbytes), "value_bytes_mse": int(v_bytes),
                     "kv_bytes": int(pbytes + v_bytes), "fp16_kv_bytes": int(fp16_kv),
                     "compression_vs_fp16": round(fp16_kv / (pbytes + v_bytes), 3),
                     "logit_cosine_mean": round(float(cos.mean()), 6),
                     "logit_cosine_min": round(float(cos.min()), 6),
                     "query_heads": int(cos.numel()),
                     "encode": _stats(enc, keys.numel() * 2 + pbytes, G * N),
                     "score": _stats(sc, pbytes + G * Qg * N * 4 + q.numel() * 2, G * N)})
    print(json.dumps({"metric": "bytes vs fp16 K+V, logit cosine, keys/s per bit width",
                      "config": {"workload": wl.name, "groups": G, "keys_per_group": N,
                                 "queries_per_group": Qg, "d": d}, "sweep": rows}), flush=True)


def run_search(args):
    """Workload 4 (1,048,576 unit vectors, d = m = 1024, b = 4, 256 queries):
    encode all vectors, then the top-10 per query by the estimated inner
    product.  The encoder's projection is matrix-core bound; with 256 queries
    the top-10 is a dense contraction on the matrix cores as well (five fp16
    products per output: levels hi*hi + hi*lo + lo*hi, signs hi + lo)."""
    import torch
    import kv_cache_vector_rotate_amd as K
    from kv_cache_vector_rotate_amd import workloads as W
    wl = W.workload(4)
    N, d, bits, Qn = wl.N, wl.d, wl.bits, wl.Qg
    dev = torch.device("cuda:0")
    t0 = time.time()
    keys = torch.empty((1, N, d), dtype=torch.float32, device=dev)
    step = 1 << 16
    for s0 in range(0, N, step):
        keys[0, s0:s0 + step] = torch.from_numpy(W.group_keys(wl, 0, s0, min(step, N - s0))).to(dev)
        if (s0 // step) % 4 == 3:
            print(f"[bench] {s0 + step} vectors generated", file=sys.stderr, flush=True)
    q = torch.from_numpy(W.group_queries(wl, 0)).to(dev)[None]
    print(f"[bench] search inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    cb = K.Codebook(d, bits, d, 42)
    pbytes = K.packed_nbytes(cb, 1, N)
    packed = torch.empty(pbytes, dtype=torch.uint8, device=dev)
    enc = _event_times(lambda i: K.encode_keys(cb, keys, out=packed), max(10, args.steps // 2), warm=1,
                       preroll_s=args.preroll)
    ws = torch.empty(K.score_topk_workspace_nbytes(cb, 1, Qn, N, 10), dtype=torch.uint8, device=dev)
    tk = _event_times(lambda i: K.score_topk(cb, q, packed, N, 10, ws=ws), 5, warm=1, preroll_s=args.preroll)
    # recall@10 against the exact top-10 by true inner product (fp32 products
    # in chunks of 64K vectors; a quality report outside the timed launches)
    idx, _ = K.score_topk(cb, q, packed, N, 10, ws=ws)
    best_s = torch.full((Qn, 10), -float("inf"), device=dev)
    best_i = torch.zeros((Qn, 10), dtype=torch.int64, device=dev)
    for s0 in range(0, N, step):
        sc = torch.mm(q[0], keys[0, s0:s0 + step].t().contiguous())
        cat_s = torch.cat([best_s, sc], dim=1)
        cat_i = torch.cat([best_i, torch.arange(s0, s0 + sc.shape[1], device=dev).expand(Qn, -1)], dim=1)
        best_s, pos = torch.topk(cat_s, 10, dim=1)
        best_i = torch.gather(cat_i, 1, pos)
    est_i = idx[0].long().cpu().numpy()
    ex_i = best_i.cpu().numpy()
    recall = float(np.mean([len(set(est_i[j]) & set(ex_i[j])) / 10.0 for j in range(Qn)]))
    enc_flops = 2.0 * d * d * N * 2        # two fp16 products per output: S R^T (r_hi + r_lo)
    enc_s = float(np.median(enc)) * 1e-3
    tk_flops = 2.0 * d * N * Qn * 5        # 32 query rows per block: Qn = 256 fills them
    tk_s = float(np.median(tk)) * 1e-3
    out = {"metric": "vectors encoded/s; (vector, query) pairs scored/s with top-10",
           "config": {"workload": wl.name, "vectors": N, "d": d, "bits": bits, "queries": Qn, "k": 10},
           "encode": dict(_stats(enc, keys.numel() * 4 + pbytes, N, "vectors"),
                          mfma_TFLOPs=round(enc_flops / enc_s / 1e12, 1),
                          mfma_frac_of_fp16_dense_peak=round(enc_flops / enc_s / 2.5e15, 4)),
           "topk": dict(_stats(tk, None, N * Qn, "pairs"),
                        mfma_TFLOPs=round(tk_flops / tk_s / 1e12, 1),
                        mfma_frac_of_fp16_dense_peak=round(tk_flops / tk_s / 2.5e15, 4),
                        recall_at_10_vs_exact=round(recall, 4))}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    if args.config == 2:
        run_long_context(args)
    elif args.config == 3 and args.bits is None:
        run_cache_sweep(args)
    elif args.config == 4:
        run_search(args)
    else:
        run_decode(args)


if __name__ == "__main__":
    main()
