"""Benchmark of the TurboQuant packed-key attention hot path on one MI355X.

Default workload (one decode step at 32K context): batch 32 x 8 KV heads x
32768 tokens x d=128 bf16 keys with 4 outlier channels per head (x10), 32 query
heads (GQA group 4), 3-bit TurboQuant (2-bit Lloyd-Max codes + 1-bit QJL).
The packed cache for tokens 0..T-2 is built before timing; one step then
  1. quantizes the new token's key of every (batch, KV head) stream straight
     into cache slot T-1 and prepares the queries (tq_decode_prep: both jobs
     in one launch),
  2. scores all T packed keys against the prepared queries (tq_scores_prepared),
  3. takes the fp32 softmax of logits / sqrt(d) over the T tokens (tq_softmax),
all on one stream.  The metric is logits per second over the whole step; for
the roofline figure the scores kernel of every 5th timed step is bracketed by
HIP events on the launch stream.

Also reported (separate timed loops, not part of `value`): streaming quantize
throughput on 2^20 anisotropic bf16 vectors at b = 2, 3, 4; fused decode
attention at 128K (keys 3-bit TurboQuant, values 3-bit MSE-only); top-10 vector
search over 10^6 packed d=200 vectors for 10^4 queries with recall 1@k.

Usage: python bench.py [--steps K] [--warmup W] [--bits 3] [--no-cpu] [--no-extra]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
FP32_VALU_TFLOPS = 78.6        # non-packed fp32 FMA: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz x 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM bytes per tq_scores call of the default decode workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE counters scaled by a plain copy's counters.  The
# record holds the SHA-256 of the sources of the counted kernels; once those
# change the figure is stale and reported as null.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "scores_decode32k_b{}_hbm_traffic.txt")
TRAFFIC_SOURCES = ("tq_scores.hip", "tq_score_core.h")


def scores_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "oblivious_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(bits, alg_bytes):
    path = TRAFFIC_RECORD.format(bits)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            k, sep, v = line.partition(":")
            if sep and k.strip() in ("sources_sha256", "hbm_bytes_per_call"):
                rec[k.strip()] = v.strip()
    if rec.get("sources_sha256") != scores_sources_sha256() or "hbm_bytes_per_call" not in rec:
        return None
    return float(rec["hbm_bytes_per_call"])


def cpu_baseline(bits, budget_s=12.0):
    """Time the oracle's estimator on a bounded sample of the same workload."""
    import oracle as O
    from oblivious_kv_cache_amd import workloads as wl
    d, T, qpg = 128, 32768, 4
    p = O.make_params(d, bits, 0)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    cores = len(os.sched_getaffinity(0))
    # one (batch, KV head) stream of the workload, quantized by the oracle (untimed)
    K, _ = wl.outlier_keys_np(1, 1, T, d, seed=2)
    X = wl.bf16_round(K.reshape(T, d))
    rec = O.quantize(p, X)
    Q = wl.gaussian((qpg, d), 7, np.float64)
    n_groups, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while elapsed < budget_s:
        O.scores(p, Q, rec["codes"], rec["signs"], rec["norms"], rec["rnorms"])
        n_groups += 1
        elapsed = time.perf_counter() - t0
    logits = n_groups * qpg * T
    return {"value": logits / elapsed, "unit": "logits/s", "cores": min(cores, blas_threads) or 1,
            "kind": "oracle",
            "sample": f"{n_groups} (batch, KV-head) streams x {T} tokens x {qpg} query heads "
                      f"(fp64 NumPy oracle, {elapsed:.1f} s; host cores {cores}, BLAS threads {blas_threads})"}


def cpu_quantize_baseline(bits, n=1 << 20):
    import oracle as O
    from oblivious_kv_cache_amd import workloads as wl
    p = O.make_params(128, bits, 0)
    X = wl.bf16_round(wl.power_law(n, 128, seed=3))
    t0 = time.perf_counter()
    O.quantize(p, X)
    return n / (time.perf_counter() - t0)


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return min(len(os.sched_getaffinity(0)), blas) or 1


def cpu_attend_baseline():
    """Oracle decode attention on one (batch, KV head) group of the 128K workload
    (random packed records of the same geometry; 4 query heads)."""
    import oracle as O
    from oblivious_kv_cache_amd import workloads as wl
    d, T = 128, 131072
    pk, pv = O.make_params(d, 3, 0), O.make_params(d, 3, 1, "mse")
    kc, ks, kn, kr = wl.random_records(T, 32, 16, seed=50)
    vc, _, vn, _ = wl.random_records(T, 48, 16, seed=51)
    Q = wl.gaussian((4, d), 52, np.float64)
    t0 = time.perf_counter()
    O.attend(pk, pv, Q, kc, ks, kn, kr, vc, vn, 1.0 / math.sqrt(d))
    el = time.perf_counter() - t0
    return {"value": T / el, "unit": "tokens/s (one group, 4 heads)", "cores": _host_threads(),
            "kind": "oracle", "sample": f"1 group x {T} tokens, {el:.1f} s"}


def cpu_topk_baseline(n=100000, nq=4):
    """Oracle estimator scores + top-10 for 4 queries over 10^5 random d=200
    records (b=2 geometry), scaled to pairs/s."""
    import oracle as O
    from oblivious_kv_cache_amd import workloads as wl
    d = 200
    p = O.make_params(d, 2, 0)
    c, sg, nu, ga = wl.random_records(n, 32, 32, seed=53)
    Q = wl.gaussian((nq, d), 54, np.float64)
    t0 = time.perf_counter()
    O.topk(O.scores(p, Q, c, sg, nu, ga), 10)
    el = time.perf_counter() - t0
    return {"value": nq * n / el, "unit": "pairs/s", "cores": _host_threads(), "kind": "oracle",
            "sample": f"{nq} queries x {n} vectors, {el:.1f} s"}


def cpu_softmax_baseline(rows=1024, T=32768):
    import oracle as O
    L = np.random.default_rng(55).standard_normal((rows, T))
    t0 = time.perf_counter()
    O.softmax(L, 0.088)
    el = time.perf_counter() - t0
    return {"value": rows * T / el, "unit": "values/s", "cores": _host_threads(), "kind": "oracle",
            "sample": f"{rows} rows x {T}, {el:.2f} s"}


def _time(torch, fn, reps, warmup=2):
    for _ in range(warmup):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def bench_attend(tq, wl, dev):
    """Long-context decode at 128K: 4 x 8 KV heads x 131072 tokens, d=128, keys
    3-bit TurboQuant, values 3-bit MSE-only, 32 query heads, fused logits +
    softmax + value sum."""
    import torch
    B, Hkv, T, d, Hq = 4, 8, 131072, 128, 32
    G, qpg = B * Hkv, Hq // Hkv
    log("attend 128K: setup")
    kctx, vctx = tq.Context(d, 3, 0), tq.Context(d, 3, 1, tq.TQ_MODE_MSE)
    K, _ = wl.outlier_keys_torch(B, Hkv, T, d, seed=4, device=dev)
    krec = tq.tq_quantize(kctx, K.view(G * T, d))
    del K
    V = wl.gaussian_torch((G * T, d), 44, dev, torch.bfloat16)
    vrec = tq.tq_quantize(vctx, V)
    del V
    q = wl.gaussian_torch((B, Hq, d), 45, dev).view(G, qpg, d).contiguous()
    ws = kctx.workspace(tq.TQ_OP_ATTEND, G, qpg, T, device=dev)
    scale = 1.0 / math.sqrt(d)
    # steady state: the first calls after setup run measurably slower
    ms = _time(torch, lambda: tq.tq_attend(kctx, vctx, q, krec, vrec, scale, ws=ws), 50, warmup=20)
    kv_bytes = G * T * (kctx.code_bytes + kctx.sign_bytes + 8 + vctx.code_bytes + 4)
    # the value sum is 4 heads x d fp32 FMAs per token and group; non-packed
    # fp32 VALU peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz FMAs
    fmas = G * T * 4 * d
    r = {"ms": ms, "tokens_per_s": G * T / (ms / 1e3), "logits_per_s": G * qpg * T / (ms / 1e3),
         "kv_bytes": kv_bytes, "alg_gbs": kv_bytes / (ms / 1e3) / 1e9,
         "hbm_frac": kv_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
         "value_fma_tflops": 2 * fmas / (ms / 1e3) / 1e12,
         "value_fma_frac_of_fp32_valu": 2 * fmas / (ms / 1e3) / 1e12 / FP32_VALU_TFLOPS}
    log(f"  attend: {ms:.3f} ms, {r['alg_gbs']:.0f} GB/s of packed K+V, value FMAs "
        f"{r['value_fma_tflops']:.1f} TF/s")
    # the whole online step: append the new key and value of every group at
    # token T-1, then attend over the T tokens (tq_decode_step, one call)
    nk = wl.gaussian_torch((G, d), 46, dev, torch.bfloat16)
    nv = wl.gaussian_torch((G, d), 47, dev, torch.bfloat16)
    ms_step = _time(torch, lambda: tq.tq_decode_step(kctx, vctx, q, nk, nv, krec, vrec, T - 1, scale,
                                                     ldk=T, ws=ws), 50, warmup=20)
    r["decode_step_ms"] = ms_step
    r["decode_step_tokens_per_s"] = G * T / (ms_step / 1e3)
    log(f"  decode step (append K and V + attend): {ms_step:.3f} ms")
    return r


def bench_decode_bits(tq, wl, dev, bits, steps=50, frac=False):
    """The default decode step (32 x 8 KV heads x 32768 tokens, d=128, GQA 4)
    at another bit width: step time and the scores kernel's duration.  With
    frac, bits is twice the fractional width (5: 2.5 bits, 7: 3.5 bits); the
    new key is then appended by tq_quantize and the queries prepared by
    tq_prep_queries (two launches instead of the fused one)."""
    import torch
    B, Hkv, T, d, Hq = 32, 8, 32768, 128, 32
    qpg, G = Hq // Hkv, B * Hkv
    name = f"{bits / 2:g}" if frac else f"{bits}"
    log(f"decode 32K at b={name}: setup")
    ctx = tq.Context(d, bits, 0, tq.TQ_MODE_FRAC) if frac else tq.Context(d, bits, seed=0)
    K, _ = wl.outlier_keys_torch(B, Hkv, T, d, seed=2, device=dev)
    cache = ctx.empty_records(G * T, dev)
    tq.tq_quantize(ctx, K.view(G * T, d), out=cache)
    del K
    new_k, _ = wl.outlier_keys_torch(B, Hkv, 1, d, seed=102, device=dev)
    new_k = new_k.view(G, d)
    q = wl.gaussian_torch((B, Hq, d), 7, dev).view(G, qpg, d).contiguous()
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev)
    probs = torch.empty_like(logits)
    ws = ctx.workspace(tq.TQ_OP_SCORES, G, qpg, device=dev)
    scale = 1.0 / math.sqrt(d)
    ev_every = 5                    # the scores kernel of every 5th timed step carries the events
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((steps + ev_every - 1) // ev_every)]

    slot = {k: v[T - 1:] for k, v in cache.items()}       # record T-1 of group g at (T-1) + g T

    def step(e=None):
        if frac:
            tq.tq_quantize(ctx, new_k, out=slot, ldr=T)
            tq.tq_prep_queries(ctx, q, ws=ws)
        else:
            tq.tq_decode_prep(ctx, q, new_k, cache, T - 1, ldk=T, ws=ws)
        tq.tq_scores_prepared(ctx, ws, G, qpg, cache, T=T, ldk=T, logits=logits, events=e)
        tq.tq_softmax(logits, scale, probs=probs)

    for e in ev:                    # creates the events (first record) before timing
        e[0].record()
        e[1].record()
    for _ in range(10):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(None if i % ev_every else ev[i // ev_every])
    torch.cuda.synchronize()
    ms = 1000.0 * (time.perf_counter() - t0) / steps
    sms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    sbytes = G * T * (ctx.code_bytes + ctx.sign_bytes + 8) + G * qpg * T * 4 + ws.numel()
    r = {"ms_per_step": ms, "logits_per_s": G * qpg * T / (ms / 1e3), "scores_ms": sms,
         "key_bytes_per_token": ctx.code_bytes + ctx.sign_bytes + 8,
         "scores_traffic": None if frac else recorded_traffic(bits, sbytes),
         "scores_bytes": sbytes, "scores_gbs": sbytes / (sms / 1e3) / 1e9,
         "scores_hbm_frac": sbytes / (sms / 1e3) / 1e9 / HBM_PEAK_GBS}
    log(f"  b={name}: step {ms:.3f} ms, scores kernel {sms * 1e3:.1f} us = {r['scores_gbs']:.0f} GB/s")
    ctx.close()
    return r


def bench_many_queries(tq, wl, dev, G=8, heads=4, npos=2048, T=2048, d=128, bits=3):
    """Scores with many queries per key group: every position of a 2048-token
    prefill (4 query heads each) against the group's 2048 keys, 8 KV groups,
    b=3: 134M logits per call.  Bound by the bit-plane VALU work and the logits
    writes, not by key bytes (the keys are re-read from cache)."""
    import torch
    qpg = heads * npos
    log(f"many queries per group: {G} groups x {qpg} queries x {T} keys, b={bits}")
    ctx = tq.Context(d, bits, 0)
    K, _ = wl.outlier_keys_torch(1, G, T, d, seed=8, device=dev)
    rec = tq.tq_quantize(ctx, K.view(G * T, d))
    del K
    q = wl.gaussian_torch((G, qpg, d), 9, dev)
    ws = tq.tq_prep_queries(ctx, q)
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev)
    for _ in range(3):
        tq.tq_scores_prepared(ctx, ws, G, qpg, rec, T=T, ldk=T, logits=logits)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e in ev:
        e[0].record()
        e[1].record()
    for e in ev:
        tq.tq_scores_prepared(ctx, ws, G, qpg, rec, T=T, ldk=T, logits=logits, events=e)
    prep_ms = _time(torch, lambda: tq.tq_prep_queries(ctx, q, ws), 5)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    n = G * qpg * T
    cb16, sb16, w = ctx.code_bytes // 16, ctx.sign_bytes // 16, ctx.w
    nm = 2 * cb16 + (2 * ((cb16 + 2) // 3) if w == 3 else 0) + 2 * sb16
    mfma_ops = n / 64 * nm * 2 * 16 * 16 * 64          # NM int8 MFMAs per 16 keys x 4 queries
    out = {"scores_ms": ms, "prep_ms": prep_ms, "logits_per_s": n / (ms / 1e3),
           "logits_write_gbs": 4 * n / (ms / 1e3) / 1e9,
           "int8_mfma_tops": mfma_ops / (ms / 1e3) / 1e12,
           "int8_mfma_frac": mfma_ops / (ms / 1e3) / 1e12 / INT8_PEAK_TOPS}
    log(f"  scores {ms * 1e3:.1f} us ({n / (ms / 1e3):.3e} logits/s, int8 MFMA "
        f"{100 * out['int8_mfma_frac']:.0f} % of peak), query prep {prep_ms * 1e3:.1f} us")
    del logits, ws, q, rec
    return out


def bench_practical_bandwidth(torch, dev, scores_gbs, extra):
    """What a plain streaming kernel reaches on this GPU: torch's elementwise
    1 GiB -> 1 GiB copy (torch.neg), timed like the library's kernels, with
    the HBM-bound kernels' algorithmic rates as fractions of it."""
    log("practical bandwidth: 1 GiB -> 1 GiB copy (torch.neg)")
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = _time(torch, lambda: torch.neg(src, out=dst), 10)
    del src, dst
    copy_gbs = 2 * (1 << 30) / (copy_ms / 1e3) / 1e9
    out = {"copy_gbs": copy_gbs, "copy_frac_of_peak": copy_gbs / HBM_PEAK_GBS,
           "scores_frac_of_copy": scores_gbs / copy_gbs}
    if "softmax_32k" in extra:
        out["softmax_frac_of_copy"] = extra["softmax_32k"]["gbs"] / copy_gbs
    log(f"  copy {copy_gbs:.0f} GB/s; scores kernel = {100 * scores_gbs / copy_gbs:.0f} % of it")
    return out


def bench_topk(tq, wl, dev, nq=10000, n=1000000, d=200, k=10):
    """Vector search: 10^6 unit-norm d=200 power-law database vectors, 10^4
    queries, top-10 by the estimator, recall of the exact fp32 top-1."""
    import torch
    log("topk 10^6 x 10^4: setup")
    DB = wl.power_law_torch(n, d, seed=5, device=dev, dtype=torch.float32, unit=True)
    Q = wl.power_law_torch(nq, d, seed=6, device=dev, dtype=torch.float32, unit=True)
    top1 = torch.empty(nq, dtype=torch.int64, device=dev)
    DB64 = DB.double()
    for s0 in range(0, nq, 256):                      # exact brute force, fp64 dot products
        top1[s0:s0 + 256] = (Q[s0:s0 + 256].double() @ DB64.T).argmax(dim=1)
    del DB64
    out = {}
    for bits in (2, 4):
        ctx = tq.Context(d, bits, 0)
        rec = tq.tq_quantize(ctx, DB)
        ws = ctx.workspace(tq.TQ_OP_TOPK, nq, n, k, device=dev)
        ms_q = _time(torch, lambda: tq.tq_quantize(ctx, DB, out=rec), 3)
        res = {}
        ms = _time(torch, lambda: res.__setitem__("r", tq.tq_topk(ctx, Q, rec, k, ws=ws)), 3)
        ids = res["r"][0]
        rec_k = {str(kk): float((ids[:, :kk] == top1[:, None]).any(dim=1).float().mean()) for kk in (1, 2, 4, 8, 10)}
        db_bytes = n * (ctx.code_bytes + ctx.sign_bytes + 8)
        # int8 MFMA work: per 16 vectors x 4 queries, NM v_mfma_i32_16x16x64_i8
        # (2 per 32-bit word and lane group: code words, merged parity words of
        # 3-bit codes (one per three code words), sign words)
        cb16, sb16, w = ctx.code_bytes // 16, ctx.sign_bytes // 16, ctx.w
        nm = 2 * cb16 + (2 * ((cb16 + 2) // 3) if w == 3 else 0) + 2 * sb16
        mfma_ops = nq * n / 64 * nm * 2 * 16 * 16 * 64
        out[f"b{bits}"] = {"ms": ms, "pairs_per_s": nq * n / (ms / 1e3), "queries_per_s": nq / (ms / 1e3),
                           "db_bytes": db_bytes, "db_quantize_ms": ms_q, "recall_1_at_k": rec_k,
                           "int8_mfma_tops": mfma_ops / (ms / 1e3) / 1e12,
                           "int8_mfma_frac": mfma_ops / (ms / 1e3) / 1e12 / INT8_PEAK_TOPS}
        log(f"  b={bits}: topk {ms:.2f} ms ({nq * n / (ms / 1e3):.3e} pairs/s), "
            f"db quantize {ms_q:.3f} ms, recall1@k {rec_k}")
        del rec, ws
    return out


def bench_tiny(tq, wl, dev, reps=50):
    """The small oracle case: 4096 fp32 N(0,1) keys, d=128, b=3, 16 fp32
    queries: quantize the keys, score them, softmax (one call each, on one
    stream).  Latency-bound at this size: reported, not judged."""
    import torch
    K, Q = wl.tiny_case(seed=0)
    ctx = tq.Context(128, 3, 0)
    k = torch.from_numpy(K).to(dev)
    q = torch.from_numpy(Q).to(dev).view(1, 16, 128)
    rec = ctx.empty_records(4096, dev)
    ws = ctx.workspace(tq.TQ_OP_SCORES, 1, 16, device=dev)
    logits = torch.empty((1, 16, 4096), dtype=torch.float32, device=dev)
    probs = torch.empty_like(logits)

    def run():
        tq.tq_quantize(ctx, k, out=rec)
        tq.tq_scores(ctx, q, rec, T=4096, ldk=4096, logits=logits, ws=ws)
        tq.tq_softmax(logits, 1.0 / math.sqrt(128), probs=probs)

    ms = _time(torch, run, reps)
    qms = _time(torch, lambda: tq.tq_quantize(ctx, k, out=rec), reps)
    sms = _time(torch, lambda: tq.tq_scores(ctx, q, rec, T=4096, ldk=4096, logits=logits, ws=ws), reps)
    r = {"ms_per_call": ms, "quantize_ms": qms, "scores_ms": sms,
         "logits_per_s": 16 * 4096 / (ms / 1e3), "vec_per_s": 4096 / (qms / 1e3)}
    log(f"  tiny case: quantize+scores+softmax {ms * 1e3:.1f} us (quantize {qms * 1e3:.1f} us, "
        f"scores {sms * 1e3:.1f} us)")
    ctx.close()
    return r


def bench_softmax_cold(tq, dev, rows=1024, T=32768, nbuf=4, reps=20):
    """Softmax over logits that are not cache-resident: the rows come from
    nbuf rotating buffers (537 MB in all, twice the 256 MB Infinity Cache),
    so every call reads its logits from HBM."""
    import torch
    bufs = [torch.randn((rows, T), device=dev) for _ in range(nbuf)]
    outs = [torch.empty_like(b) for b in bufs]
    i = [0]

    def run():
        j = i[0] % nbuf
        tq.tq_softmax(bufs[j], 0.088, probs=outs[j])
        i[0] += 1

    ms = _time(torch, run, reps)
    by = 2 * rows * T * 4
    del bufs, outs
    return {"ms": ms, "bytes": by, "gbs": by / (ms / 1e3) / 1e9, "hbm_frac": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}


def run_config(args):
    """One of the five workloads on its own (--config 1, 3, 4 or 5), one JSON
    line.  Config 2 (decode 32K) is the default run in main()."""
    import torch
    from oblivious_kv_cache_amd import binding as tq
    from oblivious_kv_cache_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    line = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    if args.config == 1:
        r = bench_tiny(tq, wl, dev, reps=max(args.steps, 10))
        line.update({"metric": "tiny case: logits/s of quantize + scores + softmax", "value": r["logits_per_s"],
                     "unit": "logits/s", "ms_per_step": r["ms_per_call"], "dtype": "int8-mfma/f32",
                     "config": {"workload": "4096 fp32 keys d=128 b=3, 16 queries"}, "extra": r})
    elif args.config == 3:
        d, b = 128, args.bits
        Xs = [wl.power_law_torch(1 << 20, d, seed=3 + i, device=dev) for i in range(2)]
        c2 = tq.Context(d, b, seed=0)
        out = c2.empty_records(1 << 20, dev)
        it = [0]

        def run():
            tq.tq_quantize(c2, Xs[it[0] % 2], out=out)
            it[0] += 1

        ms = _time(torch, run, max(args.steps, 10))
        vps = (1 << 20) / (ms / 1e3)
        hw = vps * (2 + 3) * 2 * d * d / 1e12
        line.update({"metric": "quantize vec/s (2^20 bf16 d=128)", "value": vps, "unit": "vec/s",
                     "ms_per_step": ms, "dtype": "bf16-mfma/f32",
                     "config": {"workload": f"2^20 x 128 bf16 power-law vectors, b={b}"},
                     "roofline": {"bound": "mfma", "achieved": hw, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": hw / BF16_PEAK_TFLOPS, "traffic": None}})
        if not args.no_cpu:
            v = cpu_quantize_baseline(b)
            line["cpu_baseline"] = {"value": v, "unit": "vec/s", "cores": _host_threads(), "kind": "oracle",
                                    "sample": "2^20 power-law vectors, d=128"}
    elif args.config == 4:
        r = bench_attend(tq, wl, dev)
        line.update({"metric": "attention 128K: tokens/s (logits + softmax + value sum)",
                     "value": r["tokens_per_s"], "unit": "tokens/s", "ms_per_step": r["ms"], "dtype": "int8-mfma/f32",
                     "config": {"workload": "4 x 8 KV heads x 131072 tokens, d=128, K b=3 prod, V b=3 mse, GQA 4"},
                     "roofline": {"bound": "hbm", "achieved": r["alg_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": r["hbm_frac"], "traffic": None}, "extra": r})
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_attend_baseline()
    elif args.config == 5:
        r = bench_topk(tq, wl, dev)
        key = f"b{args.bits if args.bits in (2, 4) else 2}"
        line.update({"metric": "vector search: query-vector pairs/s (top-10 over 10^6 d=200)",
                     "value": r[key]["pairs_per_s"], "unit": "pairs/s", "ms_per_step": r[key]["ms"],
                     "dtype": "int8-mfma/f32", "config": {"workload": f"10^4 queries x 10^6 d=200, {key}, top-10"},
                     "extra": r})
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_topk_baseline()
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--bits", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=(1, 2, 3, 4, 5),
                    help="workload: 1 tiny oracle case, 2 decode 32K (default, the headline metric), "
                         "3 streaming quantize, 4 attention 128K, 5 vector search")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with 3 launches of a plain 1 GiB -> 1 GiB elementwise copy (torch.neg), "
                         "the known-size reference for the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs "
              "on a single GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.config != 2:
        run_config(args)
        return

    import torch
    from oblivious_kv_cache_amd import binding as tq
    from oblivious_kv_cache_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hkv, T, d, Hq = 32, 8, 32768, 128, 32
    qpg, G = Hq // Hkv, B * Hkv
    bits = args.bits

    log(f"setup: keys [{B},{Hkv},{T},{d}] bf16, b={bits}")
    ctx = tq.Context(d, bits, seed=0)
    K, _ = wl.outlier_keys_torch(B, Hkv, T, d, seed=2, device=dev)
    cache = ctx.empty_records(G * T, dev)
    tq.tq_quantize(ctx, K.view(G * T, d), out=cache)          # prefill (untimed)
    del K
    new_k, _ = wl.outlier_keys_torch(B, Hkv, 1, d, seed=102, device=dev)
    new_k = new_k.view(G, d)
    q = wl.gaussian_torch((B, Hq, d), 7, dev).view(G, qpg, d).contiguous()
    logits = torch.empty((G, qpg, T), dtype=torch.float32, device=dev)
    probs = torch.empty_like(logits)
    ws = ctx.workspace(tq.TQ_OP_SCORES, G, qpg, device=dev)
    scale = 1.0 / math.sqrt(d)
    torch.cuda.synchronize()

    # HIP events time the scores kernel of every 5th timed step.  They are
    # recorded by the kernel's own dispatch (tq_scores_prepared_timed, i.e.
    # hipExtLaunchKernel with start/stop events), so they bracket exactly the
    # kernel; a step whose kernel carries them still runs ~4 us longer (0.152
    # against 0.148 ms when every step has them), so they are on one step in
    # five.
    EV_EVERY = 5
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((args.steps + EV_EVERY - 1) // EV_EVERY)]
    for e in ev:                    # creates the events (first record) before timing
        e[0].record()
        e[1].record()

    # One stream: the append of the new keys and the query prep run in one
    # launch (tq_decode_prep), then the scores kernel, then the softmax.
    def step(i=None):
        tq.tq_decode_prep(ctx, q, new_k, cache, T - 1, ldk=T, ws=ws)
        tq.tq_scores_prepared(ctx, ws, G, qpg, cache, T=T, ldk=T, logits=logits,
                              events=None if i is None or i % EV_EVERY else ev[i // EV_EVERY])
        tq.tq_softmax(logits, scale, probs=probs)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1000.0 * wall / args.steps
    score_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    n_logits = G * qpg * T
    value = n_logits / (ms_step / 1000.0)

    cb, sb = ctx.code_bytes, ctx.sign_bytes
    key_bytes = G * T * (cb + sb + 8)
    ws_bytes = ws.numel()                      # prepared queries, read once per block
    scores_bytes = key_bytes + n_logits * 4 + ws_bytes
    achieved = scores_bytes / (score_ms / 1000.0) / 1e9
    log(f"step {ms_step:.3f} ms; scores kernel {score_ms:.4f} ms = {achieved:.0f} GB/s algorithmic")

    extra = {"scores_ms": score_ms, "scores_event_samples": len(ev), "scores_bytes_per_launch": scores_bytes,
             "key_bytes_per_token": cb + sb + 8, "logits_per_step": n_logits}

    if not args.no_extra:
        log("softmax: 1024 rows x 32768")
        sm_ms = _time(torch, lambda: tq.tq_softmax(logits, scale, probs=probs), 20)
        sm_bytes = 2 * n_logits * 4
        extra["softmax_32k"] = {"ms": sm_ms, "bytes": sm_bytes, "gbs": sm_bytes / (sm_ms / 1e3) / 1e9,
                                "hbm_frac": sm_bytes / (sm_ms / 1e3) / 1e9 / HBM_PEAK_GBS}
        log(f"  softmax: {sm_ms * 1e3:.1f} us, {extra['softmax_32k']['gbs']:.0f} GB/s (logits just written: "
            "partly cache-resident)")
        extra["softmax_32k_cold"] = bench_softmax_cold(tq, dev)
        log(f"  softmax cold: {extra['softmax_32k_cold']['ms'] * 1e3:.1f} us, "
            f"{extra['softmax_32k_cold']['gbs']:.0f} GB/s")
        log("tiny case (4096 keys, 16 queries)")
        extra["tiny_4096"] = bench_tiny(tq, wl, dev)
        for b in (2, 4):
            if b != bits:
                extra[f"decode_32k_b{b}"] = bench_decode_bits(tq, wl, dev, b)
        for hb in (5, 7):               # fractional widths 2.5 and 3.5 bits
            extra[f"decode_32k_b{hb / 2:g}"] = bench_decode_bits(tq, wl, dev, hb, frac=True)
        log("quantize throughput: 2^20 x 128 bf16, power-law spectrum (two input sets, alternated)")
        Xs = [wl.power_law_torch(1 << 20, d, seed=3 + i, device=dev) for i in range(2)]
        qz = {}
        for b in (2, 3, 4):
            c2 = tq.Context(d, b, seed=0)
            out = c2.empty_records(1 << 20, dev)
            for i in range(10):
                tq.tq_quantize(c2, Xs[i % 2], out=out)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            reps = 30
            for i in range(reps):
                tq.tq_quantize(c2, Xs[i % 2], out=out)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e) / reps
            vps = (1 << 20) / (ms / 1000.0)
            alg_tflops = vps * 4 * d * d / 1e12
            hw_tflops = vps * (2 + 3) * 2 * d * d / 1e12
            io_gbs = (1 << 20) * (2 * d + c2.code_bytes + c2.sign_bytes + 8) / (ms / 1000.0) / 1e9
            qz[f"b{b}"] = {"ms": ms, "vec_per_s": vps, "alg_tflops": alg_tflops,
                           "alg_frac_bf16_peak": alg_tflops / BF16_PEAK_TFLOPS,
                           "mfma_tflops_split": hw_tflops,
                           "mfma_frac_bf16_peak": hw_tflops / BF16_PEAK_TFLOPS,
                           "io_gbs": io_gbs, "io_hbm_frac": io_gbs / HBM_PEAK_GBS}
            log(f"  b={b}: {ms:.3f} ms, {vps:.3e} vec/s, alg {alg_tflops:.0f} TF/s, "
                f"MFMA {hw_tflops:.0f} TF/s, io {io_gbs:.0f} GB/s")
            c2.close()
            del out
        # the other encoders on the same 2^20 vectors: PolarQuant (NEXT-4, MSE stage,
        # b bits per angle) and the fractional widths (NEXT-3, 2.5 / 3.5 bits)
        other = {}
        for name, mode, b in (("polar_b2", tq.TQ_MODE_POLAR, 2), ("polar_b4", tq.TQ_MODE_POLAR, 4),
                              ("frac_2.5", tq.TQ_MODE_FRAC, 5), ("frac_3.5", tq.TQ_MODE_FRAC, 7)):
            c2 = tq.Context(d, b, 0, mode)
            out = c2.empty_records(1 << 20, dev)
            ms = _time(torch, lambda: tq.tq_quantize(c2, Xs[0], out=out), 10, warmup=5)
            vps = (1 << 20) / (ms / 1000.0)
            rec_b = c2.code_bytes + c2.sign_bytes + (8 if c2.sign_bytes else 4)
            io_gbs = (1 << 20) * (2 * d + rec_b) / (ms / 1000.0) / 1e9
            other[name] = {"ms": ms, "vec_per_s": vps, "record_bytes": rec_b, "io_gbs": io_gbs,
                           "io_hbm_frac": io_gbs / HBM_PEAK_GBS}
            log(f"  {name}: {ms:.3f} ms, {vps:.3e} vec/s, {rec_b} B records")
            c2.close()
            del out
        del Xs
        extra["quantize_2p20"] = qz
        extra["quantize_2p20_other_modes"] = other
        extra["attend_128k"] = bench_attend(tq, wl, dev)
        extra["topk_1e6"] = bench_topk(tq, wl, dev)
        extra["many_queries_2k"] = bench_many_queries(tq, wl, dev)
        extra["practical_bandwidth"] = bench_practical_bandwidth(torch, dev, achieved, extra)

    if args.calib_copy:
        log("calibration copy: torch.neg, 2^30 bytes read + 2^30 bytes written per launch")
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu:
        log("cpu baseline: oracle estimator on a bounded sample")
        cpu = cpu_baseline(bits)
        extra["cpu_oracle_quantize_vec_per_s"] = cpu_quantize_baseline(bits)
        if not args.no_extra:
            log("cpu oracle: softmax, attention (one 128K group), top-k sample")
            extra["cpu_oracle_softmax"] = cpu_softmax_baseline()
            extra["cpu_oracle_attend_128k"] = cpu_attend_baseline()
            extra["cpu_oracle_topk"] = cpu_topk_baseline()

    line = {
        "metric": "packed-key attention logits/s (d=128, 3-bit, decode 32K)",
        "value": value,
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma/f32",
        "data": "synthetic",
        "config": {"workload": f"decode step: batch {B} x {Hkv} KV heads x {T} tokens x d={d} bf16 "
                               f"keys (4 outlier channels/head x10), {Hq} query heads (GQA 4), "
                               f"b={bits}; append 1 token/stream + scores + softmax",
                   "global_batch": B, "seq_len": T, "bits": bits, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(bits, scores_bytes),
                     "kernel": "tq_scores_prepared (scores_kernel)"},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
