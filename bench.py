#!/usr/bin/env python3
"""Benchmark of the decode hot path on one MI355X.

One step = one replay of the captured hipGraph of the whole decode step (indexer scores,
exact top-k, residency lookup / eviction / allocation, recall gather from pinned host memory,
priorities) over the default workload: 8 requests x 65536 cached tokens, H=64, d=128 FP8
integer-grid q/k, top-2048, 90% of the selected tokens resident in a full GPU pool of
65536 slots, misses recalled from a pinned host pool of 524288 rows.  All inputs are seeded
and synthetic and resident in HBM / pinned host memory before timing starts.

Before every replay the pool is restored from a pristine device copy on the same stream;
the restore is outside the per-step HIP-event timing (it is inside the wall-clock bracket,
which is reported separately).

Prints ONE JSON line.  --gpus N > 1 is refused: this path runs on one GPU.

Every measurement (the headline step, the prefill indexer, the chunked prefill with offload, the
decode loop, the prefetch modes) runs in a child process of its own (`--section NAME`); the
main process only starts them and prints the one JSON line, so a failure in one of them is
recorded in its place and the line is still printed.
"""

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "indexed tokens/sec (score+top-k+recall) and % of HBM peak at L=64K-128K, 1 GPU"
WORKLOADS = {
    "b8_64k": "decode step: 8 requests x 65536 tokens, H=64 d=128 FP8 (integer grid) q/k, "
              "top-2048, 90% pool hit rate, N_G=65536, N_H=524288",
    "b32_ragged": "decode step: 32 requests x U[16384,131072] tokens, general FP8 q/k with "
                  "per-token scale, top-2048, 70% pool hit rate, host pool 8x GPU pool",
    "b64_128k": "decode step: 64 requests x 131072 tokens, general FP8 q/k with per-token "
                "scale, top-2048, 50% pool hit rate, threshold prefetch from a 4096-score "
                "sample (ranged; fused with --prefetch fused), 131072 free slots, "
                "N_G=1048576, N_H=8388608",
    "tiny": "decode step: 1 request x 4096 tokens, integer grid, top-256, half of all tokens resident",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(root, summary="profiles/score_decode_hist_b8_64k_hbm_traffic.md"):
    """HBM bytes per scoring launch from the committed hardware-counter summary, or None when
    the summary is missing or the kernel sources changed since the counters were taken."""
    import hashlib
    try:
        fields = {}
        for line in open(os.path.join(root, summary)):
            if ":" in line:
                key, _, val = line.strip().partition(":")
                fields[key.strip()] = val.strip()
        h = hashlib.sha256()
        for f in fields["kernel_sources"].split():
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest()[:16] != fields["kernel_sources_sha256_16"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def kernel_time_us(torch, stream, fn, reps):
    """Average duration of fn()'s launches on `stream`, from HIP events on that stream."""
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1000.0 / reps


def measure_link_gbs(torch, nbytes=256 << 20, reps=5):
    """Best-of-5 pinned host -> device copy rate (the host-link reference for recall)."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        dst.copy_(src, non_blocking=True)
        e.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (s.elapsed_time(e) / 1e3) / 1e9)
    return best


FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published


def prefill_measure(torch, B, gen, reps=5):
    """Causal prefill indexer on 32768 x 32768 (integer grid): achieved fp8 MFMA TFLOP/s on the
    algorithmic flops (16384 per causal pair), plus the per-row top-2048 time."""
    cfg = gen.PREFILL["prefill_32k"]
    n = cfg["n"]
    q, w, k = gen.make_prefill_inputs(n, seed=cfg["seed"])
    dq, dw, dk = (torch.from_numpy(a).cuda() for a in (q, w, k))
    sc = torch.empty((n, n), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    t_score = kernel_time_us(torch, st, lambda: B.index_scores_prefill(dq, dw, dk, sc, ld=n, stream=st), reps)
    lens = torch.arange(1, n + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty((n, cfg["topk"]), dtype=torch.int32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    t_topk = kernel_time_us(torch, st, lambda: B.topk(sc, lens, n, cfg["topk"], idx, ws, ld=n, stream=st), reps)
    flops = 16384.0 * n * (n + 1) / 2
    tfs = flops / (t_score / 1e6) / 1e12
    del sc
    return {"bound": "mfma", "kernel": "score_prefill_kernel", "workload": "prefill_32k: causal "
            "32768 x 32768, H=64 d=128 fp8 integer grid", "achieved": round(tfs, 1),
            "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tfs / FP8_PEAK_TFLOPS, 4),
            "flops_per_launch": flops, "us_per_launch": round(t_score, 1),
            "topk_rows_us": round(t_topk, 1)}


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        return 1


def run_loop(torch, LoopRunner, m, host_kv, topk, batch, reserve, mode):
    """The captured loop step replayed for every step of m; per-step timings and counters."""
    rn = LoopRunner(m, host_kv, topk, prefetch=mode, pf=dict(n_chunks=4, cap=2048, cap_div=32),
                    device_step=True, reserve=reserve)
    steps = []
    try:
        rn.capture()
        for st in m.steps:
            theta_used = rn.theta.cpu().numpy().astype(np.float64)
            rn.load_step(st)
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(rn.main)
            rn.graph.launch(rn.main)
            e.record(rn.main)
            torch.cuda.synchronize()
            c = rn.counters.cpu().numpy()
            kth = rn.kth.cpu().numpy().astype(np.float64)
            assert int(rn.status.cpu()[0]) == 0, "pool status after a loop step"
            err = (np.abs(theta_used - kth) / np.maximum(np.abs(kth), 1e-30)
                   if not np.isnan(theta_used).any() else None)
            steps.append({"us": round(s.elapsed_time(e) * 1000.0, 1),
                          "hit_rate": round(1.0 - int(c[0]) / float(batch * topk), 4),
                          "misses": int(c[0]), "prefetch_demand": int(c[1]),
                          "prefetched": int(c[2]),
                          "ema_rel_err_median": None if err is None else round(float(np.median(err)), 4)})
    finally:
        rn.close()
    return steps


def loop_measure(torch, B, gen, batch=8, length=65536, n_steps=16, topk=2048, drift=0.05,
                 cpu=True):
    """Decode steps in a row: every step appends one token per request (key, host row written
    through, GPU slot) and runs the decode step with prefetch against the EMA estimate of the
    k-th score (alpha = 0.5).  8 requests x 65536 tokens, integer grid, top-2048, a full pool of
    N_G = 65536 slots whose guaranteed recall leaves 8 x 2048 slots free for the next step's
    prefetch, consecutive queries alike (5% of q's bytes redrawn per step).  The whole step (stamp advance, append, decode step) is one captured graph replayed
    every step; timed per step with HIP events around the replay on its stream (the upload of
    the step's query and new tokens precedes the start event).  Reports the pool hit rate of
    the guaranteed recall, the rows prefetched and the EMA's prediction error per step, with the
    ranged prefetch (scoring in 4 launches) and again, on the same inputs, with the fused one
    (one scoring launch with a host-gather wave per workgroup) and with prefetch off."""
    from dsa_indexer_top_amd.runner import LoopRunner
    n_gpu = batch * length // 8
    reserve = batch * topk                     # room for a full step of prefetch
    m, host_kv = gen.make_multistep_inputs(batch, length, n_steps, n_gpu, seed=51, drift=drift)
    steps = run_loop(torch, LoopRunner, m, host_kv, topk, batch, reserve, "ranged")
    fused = run_loop(torch, LoopRunner, m, host_kv, topk, batch, reserve, "fused")
    off = run_loop(torch, LoopRunner, m, host_kv, topk, batch, reserve, False)
    later = steps[1:]
    out = {}
    if cpu:
        # the oracle's loop on the first step of the same workload (append, scores, top-k, pool
        # step, EMA), as it is, on the host cores
        import oracle
        from oracle import multistep as ms
        cache = ms.KeyCache(m.k, m.k_scale, m.key_begin, m.key_len, m.req_to_host, m.capacity)
        p = m.pool
        st = oracle.PoolState(p.free, p.priority, p.to_host, p.host_to_gpu, p.indices_buf, p.gpu_kv)
        t0 = time.perf_counter()
        ms.decode_loop(cache, st, host_kv, m.steps[:1], topk, reserve=reserve)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(batch * (length + 1) / dt, 1), "unit": "indexed tokens/s",
                               "cores": int(oracle_threads()), "kind": "oracle",
                               "seconds": round(dt, 3),
                               "sample": "the oracle's loop on the first step of this workload"}
    out.update({"workload": "%d requests x %d tokens, %d steps, top-%d, integer grid, q drift %.2f, "
                        "full pool N_G=%d with %d slots kept free for prefetch, prefetch against "
                        "the EMA estimate" % (batch, length, n_steps, topk, drift, n_gpu, reserve),
            "timing": "one captured graph (echo_step_advance + echo_decode_append + "
                      "echo_decode_select, step stamp on the device) replayed per step; HIP "
                      "events around each replay",
            "us_per_step_median": round(float(np.median([x["us"] for x in later])), 1),
            "hit_rate_median": round(float(np.median([x["hit_rate"] for x in later])), 4),
            "indexed_tokens_per_s": round(batch * (length + n_steps / 2) /
                                          (float(np.median([x["us"] for x in later])) / 1e6), 1),
            "steps": steps,
            "fused": {"us_per_step_median": round(float(np.median([x["us"] for x in fused[1:]])), 1),
                      "hit_rate_median": round(float(np.median([x["hit_rate"] for x in fused[1:]])), 4),
                      "prefetched_median": int(np.median([x["prefetched"] for x in fused[1:]])),
                      "steps": fused},
            "off": {"us_per_step_median": round(float(np.median([x["us"] for x in off[1:]])), 1),
                    "hit_rate_median": round(float(np.median([x["hit_rate"] for x in off[1:]])), 4),
                    "steps": off}})
    return out


def prefill_offload_measure(torch, B, gen, n=32768, chunk=2048, topk=2048, seed=4, cpu=True):
    """Chunked prefill of one request with its KV offloaded and the inter-query prefetch
    (§6.2): per 2048-row chunk, the causal scores, the approximate subsets under the EMA shift,
    the prefetch of their union, the exact top-k and the guaranteed residency of its union.
    32768 tokens, integer grid, top-2048, a GPU pool of 32768 slots, empty at the start.
    Reports per chunk the time of the chunk's enqueues (HIP events on their stream), the
    median threshold-bin size with the shift and, from one extra launch on the same scores,
    without it, the subset's median share of k, the rows prefetched and the misses left for
    the guaranteed recall."""
    from dsa_indexer_top_amd.runner import PrefillChunkRunner
    q, w, k = gen.make_prefill_inputs(n, seed=seed)
    req_to_host = np.random.default_rng(seed).permutation(n).astype(np.int32)
    host_kv = gen.fill_latent_rows(seed, np.empty((n, 576), np.uint16))
    INF = 2**31 - 1
    pool = gen.PoolArrays(np.ones(n, np.uint8), np.full(n, -1, np.int32), np.full(n, INF, np.int32),
                          np.full(n, INF, np.int32), np.full(n, -1, np.int32),
                          np.full((n, 576), 0xFFFF, np.uint16), step_id=1)
    rn = PrefillChunkRunner(q, w, k, req_to_host, pool, host_kv, chunk, topk, prefetch=True)
    plain_thr = torch.empty(chunk, dtype=torch.int32, device="cuda")
    plain_sub = torch.empty((chunk, topk), dtype=torch.int32, device="cuda")
    plain_cnt = torch.empty(chunk, dtype=torch.int32, device="cuda")
    chunks = []
    try:
        for c in range(-(-n // chunk)):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            shift = float(rn.theta.cpu()[0])
            s.record(rn.main)
            rows = rn.run_chunk(c, 1 + c)
            e.record(rn.main)
            torch.cuda.synchronize()
            t1 = min(n, (c + 1) * chunk)
            B.topk_subset(rn.scores[:rows], rn.lens[:rows], t1, topk, None, plain_sub[:rows],
                          plain_cnt[:rows], plain_thr[:rows], ld=n, stream=rn.main)
            got = rn.results(rows)
            assert got["status"] == 0, "pool status in the chunked prefill"
            full = np.minimum(np.arange(c * chunk + 1, t1 + 1), topk)
            chunks.append({"us": round(s.elapsed_time(e) * 1000.0, 1),
                           "thr_bin_median_shifted": int(np.median(got["thr_cnt"])),
                           "thr_bin_median_unshifted": int(np.median(plain_thr[:rows].cpu().numpy())),
                           "subset_share_median": round(float(np.median(got["subset_cnt"] / full)), 4),
                           "union": int(got["uni_cnt"].sum()), "prefetched": got["n_prefetched"],
                           "misses_after_prefetch": got["n_miss"],
                           "shift": None if np.isnan(shift) else round(shift, 4)})
        # the approximate top-k alone on the last chunk's scores: HBM-bound, 4 B per score read
        # by its histogram pass (the ordered pass re-reads them: overhead, not algorithmic)
        rows = n - (len(chunks) - 1) * chunk
        t_sub = kernel_time_us(torch, rn.main, lambda: B.topk_subset(
            rn.scores[:rows], rn.lens[:rows], n, topk, rn.theta, rn.subset[:rows],
            rn.subset_cnt[:rows], None, ld=n, stream=rn.main), 20)
        n_scores = int(rn.lens[:rows].sum().item())
        sub_gbs = 4.0 * n_scores / (t_sub / 1e6) / 1e9
    finally:
        rn.close()
    later = chunks[2:]
    pairs = n * (n + 1) // 2
    total_us = sum(x["us"] for x in chunks)
    extra = {"pairs_per_s": round(pairs / (total_us / 1e6), 1), "unit": "causal (query, key) pairs/s",
             "us_total": round(total_us, 1)}
    if cpu:
        # the oracle's chunk loop, as it is, on the first chunk of the same request
        import oracle
        from oracle import interquery as iq
        st = oracle.PoolState.empty(n, n)
        t0 = time.perf_counter()
        iq.prefill_chunk_loop(q[:chunk], w[:chunk], k[:chunk], req_to_host, st, host_kv, chunk,
                              topk, step0=1)
        dt = time.perf_counter() - t0
        extra["cpu_baseline"] = {"value": round(chunk * (chunk + 1) / 2 / dt, 1),
                                 "unit": "causal (query, key) pairs/s", "cores": int(oracle_threads()),
                                 "kind": "oracle", "seconds": round(dt, 3),
                                 "sample": "the oracle's chunk loop on the first %d rows" % chunk}
    return {**extra, "subset_kernel": {"kernel": "topk_subset_kernel", "bound": "hbm",
                              "us_per_launch": round(t_sub, 1), "scores": n_scores,
                              "achieved": round(sub_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(sub_gbs / HBM_PEAK_GBS, 4)},
            "workload": "chunked prefill with offload: %d tokens, chunks of %d rows, top-%d, "
                        "integer grid, GPU pool %d slots (empty at the start)" % (n, chunk, topk, n),
            "timing": "HIP events around each chunk's enqueues on their stream",
            "thr_bin_median_shifted": int(np.median([x["thr_bin_median_shifted"] for x in later])),
            "thr_bin_median_unshifted": int(np.median([x["thr_bin_median_unshifted"] for x in later])),
            "chunks": chunks}


def prefetch_modes_measure(torch, B, gen, inp, hb, sel, reserve, steps=20, warmup=3,
                           kernel_reps=10):
    """The captured decode step on one starting pool (the workload's inputs, `reserve` slots
    free) with prefetch off, ranged (scoring in n_chunks launches, each gathering the range
    before it) and fused (one scoring launch whose workgroups each carry a host-gather wave).
    Per mode: the step's mean and median replay time, the guaranteed-recall misses, the
    prefetch demand and the rows prefetched.  Also the fused scoring launch alone
    (echo_index_scores_fused, the pool restored before every launch, outside its events)
    against the plain scoring launch on the same inputs."""
    from dsa_indexer_top_amd.runner import DecodeRunner, DEFAULT_PREFETCH
    host_kv = hb.array.view(np.uint16).reshape(inp.n_host, 576)
    pool = gen.make_pool_state(inp, sel, host_kv, reserve=reserve)
    tokens = int(inp.key_len.astype(np.int64).sum())
    out = {"reserve": reserve, "free_slots_at_start": int(pool.free.sum()),
           "cap": DEFAULT_PREFETCH["cap"], "cap_div": DEFAULT_PREFETCH["cap_div"]}
    for mode in ("off", "ranged", "fused"):
        rn = DecodeRunner(inp, pool, host_buf=hb, prefetch=mode)
        try:
            rn.capture()
            for _ in range(warmup):
                rn.restore()
                rn.replay()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            torch.cuda.synchronize()
            for s_, e_ in ev:
                rn.restore()
                s_.record(rn.main)
                rn.replay()
                e_.record(rn.main)
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
            res = rn.results()
            out[mode] = {"us_per_step": round(float(t.mean()), 2),
                         "us_per_step_median": round(float(np.median(t)), 2),
                         "indexed_tokens_per_s": round(tokens / (float(t.mean()) / 1e6), 1),
                         "status": res["status"], "n_miss": int(res["counters"][0]),
                         "prefetch_demand": int(res["counters"][1]),
                         "prefetched": int(res["counters"][2])}
            if mode == "fused":
                # the fused scoring launch alone, from the same starting pool every time
                theta = torch.empty(rn.n_rows, dtype=torch.float32, device="cuda")
                B.prefetch_threshold(rn.q, rn.w, rn.k, rn.k_scale, rn.key_begin, rn.key_len,
                                     rn.max_len, DEFAULT_PREFETCH["n_sample"],
                                     DEFAULT_PREFETCH["percentile"], theta, stream=rn.main)
                npf = torch.zeros(1, dtype=torch.int32, device="cuda")
                ws = torch.empty(B.fused_workspace_bytes(rn.n_rows, rn.n_gpu), dtype=torch.uint8,
                                 device="cuda")
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(kernel_reps)]
                for s_, e_ in ev:
                    rn.restore()
                    s_.record(rn.main)
                    B.index_scores_fused(rn.q, rn.w, rn.k, rn.k_scale, rn.key_begin, rn.key_len,
                                         rn.max_len, rn.scores, theta, rn.req_to_host, rn.pool,
                                         DEFAULT_PREFETCH["cap"], DEFAULT_PREFETCH["cap_div"], 0,
                                         npf, None, ws, stream=rn.main)
                    e_.record(rn.main)
                torch.cuda.synchronize()
                tf = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
                t_plain = kernel_time_us(torch, rn.main, lambda: B.index_scores(
                    rn.q, rn.w, rn.k, rn.k_scale, rn.key_begin, rn.key_len, rn.max_len,
                    rn.scores, stream=rn.main), kernel_reps)
                moved = int(npf.cpu()[0])
                out["fused_launches_alone"] = {
                    "us_median": round(float(np.median(tf)), 2),
                    "plain_scoring_us": round(t_plain, 2), "rows_moved": moved,
                    "host_bytes_moved": moved * 576 * 2,
                    "note": "free-slot count and list, the fused kernel and the totals; the "
                            "threshold (sample percentile) computed once beforehand"}
        finally:
            rn.close()
    return out


def cpu_baseline(inp, host_kv, pool_arrays, min_s=10.0, budget_s=30.0):
    """The oracle, as it is, timed on the host cores on a bounded sample of the same workload:
    the whole oracle decode step (float64 scores, exact top-k, canonical pool step with the
    recall copy) repeated from the same pool state until at least min_s seconds have passed.
    A workload whose single step would exceed the budget is sampled by whole requests instead
    (scores and top-k request by request until the budget is spent, then the pool step for the
    sampled requests)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = 1

    def state():
        return oracle.PoolState(pool_arrays.free.copy(), pool_arrays.priority.copy(),
                                pool_arrays.to_host.copy(), pool_arrays.host_to_gpu.copy(),
                                pool_arrays.indices_buf.copy(), pool_arrays.gpu_kv.copy())

    t0 = time.perf_counter()
    reps, tokens, n = 0, 0, len(inp.key_len)
    while True:
        sel, tok = [], 0
        for r in range(len(inp.key_len)):
            sl = slice(r, r + 1)
            s = oracle.index_scores(inp.q[sl], inp.w[sl], inp.k, inp.k_scale, inp.key_begin[sl],
                                    inp.key_len[sl])
            sel.append(oracle.topk_rows(s, inp.cfg.topk)[0])
            tok += int(inp.key_len[r])
            if reps == 0 and time.perf_counter() - t0 > budget_s:
                n = r + 1
                break
        oracle.pool_step(state(), host_kv, np.stack(sel), inp.key_begin[:n], inp.req_to_host,
                         pool_arrays.step_id)
        reps += 1
        tokens += tok
        if n < len(inp.key_len) or time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    if n < len(inp.key_len):
        sample = ("oracle decode step on requests 0..%d of the workload (%d tokens): scores in "
                  "float64, exact top-k, canonical pool step incl. recall copy" % (n - 1, tokens))
    else:
        sample = ("%d x the whole oracle decode step, %d tokens each (fp64 scores, exact top-k, "
                  "pool step, recall copy)" % (reps, tokens // reps))
    return {"value": round(tokens / dt, 1), "unit": "indexed tokens/s", "cores": int(cores),
            "cpu_model": cpu_model(), "kind": "oracle", "seconds": round(dt, 3), "sample": sample}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo) and its online core count."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return "%s (%d cores online)" % (name, os.cpu_count() or 0)


SECTIONS = ("headline", "prefill", "prefill_offload", "loop", "prefetch_modes", "c3", "c5",
            "layers")
# the other decode workloads of the metric's range, each reported by a section of its own
SIDE_WORKLOADS = {"c3": "b32_ragged", "c5": "b64_128k"}


def summarize_extra(extra):
    """The secondary measurements as they go into the one JSON line: summaries only."""
    out = {}
    for name, val in extra.items():
        if not isinstance(val, dict) or "error" in val:
            out[name] = val
        elif name == "loop":
            out[name] = {k: val.get(k) for k in ("us_per_step_median", "hit_rate_median",
                                                  "indexed_tokens_per_s")}
            if "fused" in val:
                out[name]["fused"] = {k: val["fused"].get(k) for k in
                                      ("us_per_step_median", "hit_rate_median", "prefetched_median")}
            if "off" in val:
                out[name]["off"] = {k: val["off"].get(k) for k in ("us_per_step_median", "hit_rate_median")}
        elif name == "prefill_offload":
            out[name] = {k: val.get(k) for k in ("pairs_per_s", "us_total", "thr_bin_median_shifted",
                                                  "thr_bin_median_unshifted")}
            if "subset_kernel" in val:
                out[name]["subset_kernel_frac"] = val["subset_kernel"]["frac"]
        elif name == "prefetch_modes":
            out[name] = compact_modes(val)
            if "fused_launches_alone" in val:
                out[name]["fused_launches_alone_us"] = val["fused_launches_alone"]["us_median"]
        else:
            out[name] = val
    return out


# the keys of the headline measurement the one JSON line keeps (the rest goes to stderr)
LINE_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
             "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "error")


def one_line(out, extra):
    """The one JSON line: the contract's keys, the roofline, the step's link and HBM figures,
    the CPU baseline and one short entry per secondary measurement, kept under 2000 characters
    so that a reader of the output's tail gets it whole."""
    line = {k: out[k] for k in LINE_KEYS if k in out}
    cfg = out.get("config", {})
    line["config"] = {k: cfg[k] for k in ("workload", "batch", "tokens", "topk", "prefetch",
                                          "n_gpu_slots", "n_host_slots", "free_slots_at_start")
                      if k in cfg}
    if "roofline" in out:
        rl = out["roofline"]
        line["roofline"] = {k: rl[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                               "us_per_launch") if k in rl}
        line["roofline"]["kernel"] = "score_decode_kernel (the step's scoring launch)"
    if "step" in out:
        line["step"] = {k: out["step"][k] for k in ("hbm_frac", "link_floor_us") if k in out["step"]}
    if "recall" in out:
        rc = out["recall"]
        line["recall"] = {"achieved_gbs": rc.get("achieved"), "link_gbs": rc.get("peak_measured_h2d"),
                          "frac": rc.get("frac"), "rows": rc.get("rows"),
                          "memcpy_baseline_us": rc.get("memcpy_baseline_us_median")}
    if "cpu_baseline" in out:
        line["cpu_baseline"] = {k: v for k, v in out["cpu_baseline"].items() if k != "seconds"}
        if isinstance(line["cpu_baseline"].get("cpu_model"), str):
            line["cpu_baseline"]["cpu_model"] = line["cpu_baseline"]["cpu_model"][:60]
    short = {}
    for name, val in extra.items():
        if not isinstance(val, dict) or "error" in val:
            short[name] = val
        elif name in SIDE_WORKLOADS:
            short[name] = {k: val.get(k) for k in ("us_per_step", "scoring_frac", "recall_frac_of_link")}
            if name == "c5":
                short[name]["memcpy_recall_us"] = val.get("memcpy_recall_us")
            if "prefetch_modes" in val:
                short[name]["modes_us"] = {m: v.get("us") for m, v in val["prefetch_modes"].items()}
        elif name == "layers":
            short[name] = {k: val.get(k) for k in ("us_per_model_step", "us_per_layer")}
        elif name == "prefill":
            short[name] = {k: val.get(k) for k in ("frac", "us_per_launch", "topk_rows_us")}
        elif name == "prefill_offload":
            short[name] = {k: val.get(k) for k in ("pairs_per_s", "thr_bin_median_shifted",
                                                    "thr_bin_median_unshifted")}
        elif name == "loop":
            short[name] = {"ranged_us": val.get("us_per_step_median"), "hit_rate": val.get("hit_rate_median")}
            for m in ("fused", "off"):
                if isinstance(val.get(m), dict):
                    short[name][m + "_us"] = val[m].get("us_per_step_median")
            if isinstance(val.get("off"), dict):
                short[name]["off_hit_rate"] = val["off"].get("hit_rate_median")
        elif name == "prefetch_modes":
            short[name] = {m: v["us"] for m, v in val.items() if isinstance(v, dict) and "us" in v}
        else:
            short[name] = val
    line.update(short)
    return line


def compact_decode(res):
    """The figures of one decode-step measurement that the one JSON line carries."""
    rl, rc, st = res["roofline"], res["recall"], res["step"]
    return {"workload": res["config"]["workload"], "prefetch": res["config"]["prefetch"],
            "us_per_step": res["breakdown_us"]["step"], "indexed_tokens_per_s": res["value"],
            "step_hbm_frac": st["hbm_frac"], "scoring_us": rl["us_per_launch"],
            "scoring_frac": rl["frac"], "scoring_floor_us": st["scoring_floor_us"],
            "n_miss": res["counters"]["n_miss"], "prefetched": res["counters"]["prefetched"],
            "recall_us": rc["us_per_launch"], "recall_gbs": rc["achieved"],
            "link_gbs": rc["peak_measured_h2d"], "recall_frac_of_link": rc["frac"],
            "link_floor_us": st["link_floor_us"], "memcpy_recall_us": rc["memcpy_baseline_us_median"]}


def compact_modes(pm):
    """Step time per prefetch mode (one starting pool), with the rows each moved."""
    return {m: {"us": pm[m]["us_per_step"], "n_miss": pm[m]["n_miss"],
                "prefetched": pm[m]["prefetched"]} for m in ("off", "ranged", "fused") if m in pm}


def modes_for(workload, args, torch, B, gen):
    """prefetch_modes_measure on the inputs of `workload`, its resident set drawn around the
    selection."""
    cfg = gen.CONFIGS[workload]
    inp = gen.make_decode_inputs(cfg)
    hb = B.HostBuffer(inp.n_host * 576 * 2)
    try:
        gen.fill_latent_rows(cfg.seed, hb.array.view(np.uint16).reshape(inp.n_host, 576))
        n_rows, max_len = len(inp.key_len), int(inp.key_len.max())
        dq, dw, dk = (torch.from_numpy(a).cuda() for a in (inp.q, inp.w, inp.k))
        dks = None if inp.k_scale is None else torch.from_numpy(inp.k_scale).cuda()
        dkb, dkl = torch.from_numpy(inp.key_begin).cuda(), torch.from_numpy(inp.key_len).cuda()
        sc = torch.empty((n_rows, max_len), dtype=torch.float32, device="cuda")
        sel = torch.empty((n_rows, cfg.topk), dtype=torch.int32, device="cuda")
        tws = torch.empty(B.topk_workspace_bytes(n_rows, max_len), dtype=torch.uint8, device="cuda")
        B.index_scores(dq, dw, dk, dks, dkb, dkl, max_len, sc)
        B.topk(sc, dkl, max_len, cfg.topk, sel, tws)
        sel_idx = sel.cpu().numpy()
        del dq, dw, dk, dks, dkb, dkl, sc, sel, tws
        reserve = args.reserve if args.reserve is not None else max(cfg.reserve, n_rows * cfg.topk)
        return prefetch_modes_measure(torch, B, gen, inp, hb, sel_idx, reserve,
                                      steps=min(args.steps, 20), warmup=min(args.warmup, 3))
    finally:
        hb.close()


def run_section(name, args, timeout_s=900):
    """One measurement in a child process; its JSON (or the failure) as a dict."""
    cmd = [sys.executable, os.path.abspath(__file__), "--section", name, "--workload", args.workload,
           "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--kernel-reps", str(args.kernel_reps), "--prefetch", args.prefetch]
    if args.reserve is not None:
        cmd += ["--reserve", str(args.reserve)]
    if args.percentile is not None:
        cmd += ["--percentile", str(args.percentile)]
    if args.cap_div is not None:
        cmd += ["--cap-div", str(args.cap_div)]
    if args.no_cpu_baseline:
        cmd.append("--no-cpu-baseline")
    try:
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=None, text=True, timeout=timeout_s)
    except subprocess.TimeoutExpired:
        return {"error": "section process timed out after %d s" % timeout_s}
    lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
    if p.returncode != 0 or not lines:
        return {"error": "section process exited with status %d" % p.returncode}
    return json.loads(lines[-1])


def layers_measure(torch, B, gen, n_layers=61, batch=4, length=16384, topk=2048, page=64,
                   steps=10, warmup=2):
    """The decode step of every layer of a 61-layer model in one captured graph (ECHO page §5.1:
    a GPU pool per layer, one host pool per model): per layer its own indexer inputs, its
    indexer-K cache in 64-token pages scattered in a random order, its own pool (N_G = N_H / 8,
    90% of the selection resident), its slice of one pinned host allocation.  Timed with HIP
    events around each replay of the whole graph; every layer's pool restored before each
    replay, outside the events."""
    from dsa_indexer_top_amd.runner import DecodeRunner
    row_bytes = 576 * 2
    cfgs = [gen.DecodeConfig("layer%d" % ell, batch, length, topk, "int", False, 0.9, 8,
                             seed=700 + ell) for ell in range(n_layers)]
    inps = [gen.make_decode_inputs(c) for c in cfgs]
    for inp in inps[1:]:
        inp.req_to_host[:] = inps[0].req_to_host          # one token, one host row, every layer
    n_host = inps[0].n_host
    hb = B.HostBuffer(n_layers * n_host * row_bytes)
    runners = []
    try:
        host_all = hb.array.view(np.uint16).reshape(n_layers, n_host, 576)
        for ell, inp in enumerate(inps):
            gen.fill_latent_rows(800 + ell, host_all[ell])
            dq, dw, dk = (torch.from_numpy(a).cuda() for a in (inp.q, inp.w, inp.k))
            dkb, dkl = torch.from_numpy(inp.key_begin).cuda(), torch.from_numpy(inp.key_len).cuda()
            sc = torch.empty((batch, length), dtype=torch.float32, device="cuda")
            sel = torch.empty((batch, topk), dtype=torch.int32, device="cuda")
            tws = torch.empty(B.topk_workspace_bytes(batch, length), dtype=torch.uint8, device="cuda")
            B.index_scores(dq, dw, dk, None, dkb, dkl, length, sc)
            B.topk(sc, dkl, length, topk, sel, tws)
            pool = gen.make_pool_state(inp, sel.cpu().numpy(), host_all[ell])
            del dq, dw, dk, dkb, dkl, sc, sel, tws
            pk = gen.page_key_cache(inp.k, None, inp.key_begin, inp.key_len, page, seed=ell)
            rn = DecodeRunner(inp, pool, host_buf=hb, pages=pk)
            rn.pool.host_kv = hb.dev_ptr + ell * n_host * row_bytes
            runners.append(rn)
        stream = runners[0].main
        torch.cuda.synchronize()

        def enqueue(st):
            for rn in runners:
                B.decode_select(rn.args, rn.pool, rn.out, rn.ws, st)

        g = B.CapturedGraph(enqueue, stream)
        try:
            times = []
            for it in range(warmup + steps):
                for rn in runners:
                    rn.restore()
                torch.cuda.synchronize()
                s_ = torch.cuda.Event(enable_timing=True)
                e_ = torch.cuda.Event(enable_timing=True)
                s_.record(stream)
                g.launch(stream)
                e_.record(stream)
                torch.cuda.synchronize()
                if it >= warmup:
                    times.append(s_.elapsed_time(e_) * 1000.0)
            for rn in runners:
                assert int(rn.status.cpu()[0]) == 0, "pool status of a layer"
            n_miss = sum(int(rn.counters.cpu()[0]) for rn in runners)
        finally:
            g.close()
    finally:
        for rn in runners:
            rn.close()
        hb.close()
    t = float(np.median(times))
    tokens = n_layers * batch * length
    return {"workload": "%d layers x %d requests x %d tokens, top-%d, integer grid, indexer keys "
                        "in %d-token pages, N_G = N_H/8 per layer, 90%% of the selection resident"
                        % (n_layers, batch, length, topk, page, ),
            "us_per_model_step": round(t, 1), "us_per_layer": round(t / n_layers, 2),
            "indexed_tokens_per_s": round(tokens / (t / 1e6), 1), "misses_all_layers": n_miss,
            "host_pool_bytes": n_layers * n_host * row_bytes,
            "timing": "HIP events around each replay of the one graph of all layers' steps"}


def child_section(name, args, torch, B, gen):
    """--section NAME: the measurement alone, printed as one JSON object."""
    import copy
    cpu = not args.no_cpu_baseline
    if name == "prefill":
        return prefill_measure(torch, B, gen)
    if name == "prefill_offload":
        return prefill_offload_measure(torch, B, gen, cpu=cpu)
    if name == "loop":
        return loop_measure(torch, B, gen, cpu=cpu)
    if name == "layers":
        return layers_measure(torch, B, gen)
    if name in SIDE_WORKLOADS:
        from dsa_indexer_top_amd.runner import DecodeRunner
        wl = SIDE_WORKLOADS[name]
        a2 = copy.copy(args)
        a2.workload, a2.no_cpu_baseline = wl, True
        a2.steps, a2.warmup, a2.kernel_reps = min(args.steps, 10), min(args.warmup, 3), min(args.kernel_reps, 10)
        cfg = gen.CONFIGS[wl]
        out = compact_decode(headline(a2, torch, B, gen, DecodeRunner, cfg, cfg.prefetch))
        if name == "c5":
            out["prefetch_modes"] = compact_modes(modes_for(wl, a2, torch, B, gen))
        return out
    return modes_for(args.workload, args, torch, B, gen)


def headline(args, torch, B, gen, DecodeRunner, cfg, prefetch):
    """The headline measurement (the captured decode step of the workload) with its roofline,
    live kernel timings and, unless disabled, the oracle's CPU baseline, as one dict."""
    log("workload", args.workload, "prefetch", prefetch)
    t_setup = time.perf_counter()
    inp = gen.make_decode_inputs(cfg)
    hb = B.HostBuffer(inp.n_host * 576 * 2)
    host_kv = hb.array.view(np.uint16).reshape(inp.n_host, 576)
    gen.fill_latent_rows(cfg.seed, host_kv)
    log("inputs drawn in %.1fs" % (time.perf_counter() - t_setup))

    # the resident set is drawn around the step's own selection (computed once, untimed)
    n_rows, max_len = len(inp.key_len), int(inp.key_len.max())
    dq, dw, dk = (torch.from_numpy(a).cuda() for a in (inp.q, inp.w, inp.k))
    dks = None if inp.k_scale is None else torch.from_numpy(inp.k_scale).cuda()
    dkb, dkl = torch.from_numpy(inp.key_begin).cuda(), torch.from_numpy(inp.key_len).cuda()
    sc = torch.empty((n_rows, max_len), dtype=torch.float32, device="cuda")
    sel = torch.empty((n_rows, cfg.topk), dtype=torch.int32, device="cuda")
    tws = torch.empty(B.topk_workspace_bytes(n_rows, max_len), dtype=torch.uint8, device="cuda")
    B.index_scores(dq, dw, dk, dks, dkb, dkl, max_len, sc)
    B.topk(sc, dkl, max_len, cfg.topk, sel, tws)
    pool = gen.make_pool_state(inp, sel.cpu().numpy(), host_kv, reserve=args.reserve)
    del sc, sel, tws
    pf = {}
    if args.percentile is not None:
        pf["percentile"] = args.percentile
    if args.cap_div is not None:
        pf["cap_div"] = args.cap_div
    pf = pf or None
    rn = DecodeRunner(inp, pool, host_buf=hb, prefetch=prefetch, pf=pf)
    rn.capture()
    log("setup done in %.1fs" % (time.perf_counter() - t_setup))

    main_s = rn.main
    for _ in range(args.warmup):
        rn.restore()
        rn.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for s, e in ev:
        rn.restore()
        s.record(main_s)
        rn.replay()
        e.record(main_s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = np.array([s.elapsed_time(e) for s, e in ev])
    res = rn.results()
    assert res["status"] == 0, "pool status %d" % res["status"]
    n_miss = int(res["counters"][0])
    tokens = int(inp.key_len.astype(np.int64).sum())
    ms = float(step_ms.mean())
    value = tokens / (ms / 1e3)
    log("step %.1f us (median %.1f, min %.1f), wall incl. restores %.1f us/step" % (
        ms * 1e3, np.median(step_ms) * 1e3, step_ms.min() * 1e3, wall / args.steps * 1e6))

    # ---- live kernel timings on the main stream (same launch configuration as the step)
    reps = args.kernel_reps
    score_bytes = tokens * 128 + (tokens * 4 if inp.k_scale is not None else 0)
    # the step's own scoring launch: scores plus the top-k histogram (echo_index_scores_hist),
    # the kernel the captured step runs for prefetch off
    hist = torch.zeros((n_rows, 2048), dtype=torch.int32, device="cuda")
    t_step_score = kernel_time_us(torch, main_s, lambda: B.index_scores_hist(
        rn.q, rn.w, rn.k, rn.k_scale, rn.key_begin, rn.key_len, rn.max_len, rn.scores, hist,
        stream=main_s), reps)
    del hist
    t_score = kernel_time_us(torch, main_s, lambda: B.index_scores(
        rn.q, rn.w, rn.k, rn.k_scale, rn.key_begin, rn.key_len, rn.max_len, rn.scores,
        stream=main_s), reps)
    tws = torch.empty(B.topk_workspace_bytes(n_rows, rn.max_len), dtype=torch.uint8, device="cuda")
    t_topk = kernel_time_us(torch, main_s, lambda: B.topk(
        rn.scores, rn.key_len, rn.max_len, rn.topk, rn.topk_idx, tws, stream=main_s), reps)
    # recall gather alone, re-copying the step's miss list
    rn.restore()
    rn.replay()
    torch.cuda.synchronize()
    t_recall = kernel_time_us(torch, main_s, lambda: B.recall(
        rn.pool, rn.miss_host, rn.miss_slot, rn.counters[0:1], n_rows * rn.topk, stream=main_s), reps)
    recall_bytes = n_miss * 576 * 2
    # the same rows by the host-driven baseline: the host reads the list and issues one
    # hipMemcpyAsync per row (wall clock from the call to the copies' end, 5 repetitions)
    t_memcpy = []
    for _ in range(5):
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        B.recall(rn.pool, rn.miss_host, rn.miss_slot, rn.counters[0:1], n_rows * rn.topk,
                 mode=B.RECALL_MEMCPY, stream=main_s)
        torch.cuda.synchronize()
        t_memcpy.append((time.perf_counter() - w0) * 1e6)
    link = measure_link_gbs(torch)
    score_gbs = score_bytes / (t_step_score / 1e6) / 1e9
    plain_gbs = score_bytes / (t_score / 1e6) / 1e9
    recall_gbs = recall_bytes / (t_recall / 1e6) / 1e9 if t_recall > 0 else 0.0
    log("step scoring launch %.1f us (%.0f GB/s), plain scoring %.1f us (%.0f GB/s), top-k %.1f us, "
        "recall %.1f us (%.1f GB/s of %.1f link)" % (t_step_score, score_gbs, t_score, plain_gbs,
                                                     t_topk, t_recall, recall_gbs, link))

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "indexed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded)",
        "config": {"workload": args.workload, "description": WORKLOADS[args.workload],
                   "batch": n_rows, "tokens": tokens, "topk": rn.topk, "n_gpu_slots": rn.n_gpu,
                   "n_host_slots": rn.n_host,
                   "prefetch": ("off", "ranged", "fused")[B.prefetch_mode(prefetch)],
                   "free_slots_at_start": int(pool.free.sum()),
                   "timing": "HIP events around each graph replay; pool restored between "
                             "replays outside the events"},
        "roofline": {"bound": "hbm",
                     "kernel": "score_decode_kernel<%s, false, true, false, false> (the step's scoring "
                               "launch, echo_index_scores_hist)" % str(inp.k_scale is not None).lower(),
                     "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__)))
                     if args.workload == "b8_64k" else None,
                     "bytes_per_launch": score_bytes, "us_per_launch": round(t_step_score, 2),
                     "plain_scoring_us": round(t_score, 2)},
        # hbm_frac: the step's key bytes / step time / 8 TB/s; link floor: the missed rows over
        # the measured pinned H2D rate
        "step": {"hbm_frac": round(score_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "link_floor_us": round(recall_bytes / (link * 1e3), 1) if link else None,
                 "scoring_floor_us": round(score_bytes / (HBM_PEAK_GBS * 1e3), 1)},
        "recall": {"bound": "host link", "kernel": "recall_gather_kernel",
                   "achieved": round(recall_gbs, 2), "peak_measured_h2d": round(link, 2),
                   "unit": "GB/s", "frac": round(recall_gbs / link, 4) if link else None,
                   "rows": n_miss, "bytes_per_launch": recall_bytes,
                   "us_per_launch": round(t_recall, 2),
                   # the host reads the miss list and issues one hipMemcpyAsync per row (wall
                   # clock incl. the host sync)
                   "memcpy_baseline_us_median": round(float(np.median(t_memcpy)), 1)},
        "breakdown_us": {"step": round(ms * 1e3, 2), "step_median": round(float(np.median(step_ms)) * 1e3, 2),
                         "score_step_launch": round(t_step_score, 2), "score": round(t_score, 2),
                         "topk": round(t_topk, 2), "recall": round(t_recall, 2),
                         "wall_per_step_incl_restore": round(wall / args.steps * 1e6, 2)},
        "counters": {"n_miss": n_miss, "prefetch_demand": int(res["counters"][1]),
                     "prefetched": int(res["counters"][2]),
                     # prefetched rows keep priority 0 unless the step selects them; the starting
                     # pool's priorities are a permutation, so at most one other slot holds 0
                     "prefetched_unselected_approx": int((res["pool"]["priority"] == 0).sum())},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        try:
            out["cpu_baseline"] = cpu_baseline(inp, host_kv, pool)
            log("cpu baseline %.3g %s on %d threads" % (out["cpu_baseline"]["value"],
                                                         out["cpu_baseline"]["unit"],
                                                         out["cpu_baseline"]["cores"]))
        except Exception as e:                       # noqa: BLE001
            out["cpu_baseline"] = {"error": "%s: %s" % (type(e).__name__, e)}
    rn.close()
    hb.close()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b8_64k", choices=sorted(WORKLOADS))
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-loop", action="store_true", help="skip the decode-loop measurement")
    ap.add_argument("--prefetch", choices=("auto", "on", "off", "ranged", "fused"), default="auto",
                    help="prefetch of the headline step (on = ranged)")
    ap.add_argument("--no-prefetch-modes", action="store_true",
                    help="skip the off / ranged / fused prefetch comparison")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the 61-layer decode step in one graph")
    ap.add_argument("--no-side-workloads", action="store_true",
                    help="skip the ragged 32-request and the 64 x 128K decode steps")
    ap.add_argument("--section", choices=SECTIONS, default=None,
                    help="run one secondary measurement alone and print its JSON (the main run "
                         "starts each of them this way, in a child process)")
    ap.add_argument("--reserve", type=int, default=None,
                    help="free GPU slots in the starting pool (default: the workload's own)")
    ap.add_argument("--cap-div", type=int, default=None,
                    help="prefetch cap divisor: a request prefetches at most ceil(L / cap_div) rows")
    ap.add_argument("--percentile", type=float, default=None,
                    help="prefetch threshold percentile of the score sample (default 95)")
    ap.add_argument("--probe", choices=("score", "copy", "prefill"), default=None,
                    help="short program for hardware-counter runs, then exit: 20 launches of the "
                         "step's scoring launch on the workload, 20 device copies of 256 MiB, or 3 "
                         "causal prefill launches on 32768^2")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this decode path runs on one GPU; --gpus %d is not supported "
              "(the batch shards across GPUs with no exchange, see the design notes)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.section is None and args.probe is None:
        # this process only starts the measurements, each in a child process of its own, and
        # never touches the GPU: a failure in one of them (a Python error, a crash, a time-out)
        # is recorded in its place, and the one JSON line is always printed
        log("headline: workload", args.workload)
        out = run_section("headline", args, timeout_s=1500)
        if "error" in out:
            log("headline failed:", out["error"])
            out = {"metric": METRIC, "value": None, "unit": "indexed tokens/s", "n_gpus": 1,
                   "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                   "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded)",
                   "config": {"workload": args.workload}, "error": out["error"]}
        extra = {}

        def section(name, fn, summary):
            try:
                extra[name] = fn()
            except Exception as e:                       # noqa: BLE001
                extra[name] = {"error": "%s: %s" % (type(e).__name__, e)}
            if "error" in extra[name]:
                log("%s failed: %s" % (name, extra[name]["error"]))
                return
            try:
                log(summary(extra[name]))
            except Exception:                            # noqa: BLE001
                log("%s done" % name)

        if not args.no_side_workloads:
            for name, wl in SIDE_WORKLOADS.items():
                log("decode step %s (%s) ..." % (wl, name))
                section(name, lambda name=name: run_section(name, args),
                        lambda p: "%s: %.1f us/step, scoring %.1f%% of HBM, recall %.1f%% of the link"
                        % (p["workload"], p["us_per_step"], 100 * p["scoring_frac"],
                           100 * p["recall_frac_of_link"]))
        if not args.no_layers:
            log("61 layers in one graph, paged indexer keys ...")
            section("layers", lambda: run_section("layers", args),
                    lambda p: "layers: %.1f us per model step, %.2f us per layer"
                    % (p["us_per_model_step"], p["us_per_layer"]))
        if not args.no_prefill:
            log("prefill indexer (32768^2) ...")
            section("prefill", lambda: run_section("prefill", args),
                    lambda p: "prefill %.1f us = %.0f TFLOP/s (%.1f%% of fp8 peak), top-k rows %.1f us"
                    % (p["us_per_launch"], p["achieved"], 100 * p["frac"], p["topk_rows_us"]))
            log("chunked prefill with offload and inter-query prefetch ...")
            section("prefill_offload", lambda: run_section("prefill_offload", args),
                    lambda p: "chunked prefill: threshold bin median %d shifted vs %d unshifted"
                    % (p["thr_bin_median_shifted"], p["thr_bin_median_unshifted"]))
        if not args.no_loop:
            log("decode loop (EMA threshold, new tokens every step) ...")
            section("loop", lambda: run_section("loop", args),
                    lambda p: "loop: ranged %.1f us/step (hit rate %.3f), fused %.1f, prefetch off "
                    "%.1f (hit rate %.3f)" % (p["us_per_step_median"], p["hit_rate_median"],
                                              p["fused"]["us_per_step_median"], p["off"]["us_per_step_median"],
                                              p["off"]["hit_rate_median"]))
        if not args.no_prefetch_modes:
            log("prefetch off / ranged / fused on one starting pool ...")
            section("prefetch_modes", lambda: run_section("prefetch_modes", args),
                    lambda p: "prefetch modes: off %.1f, ranged %.1f, fused %.1f us/step; fused "
                    "launches alone %.1f us vs plain scoring %.1f us" % (
                        p["off"]["us_per_step"], p["ranged"]["us_per_step"], p["fused"]["us_per_step"],
                        p["fused_launches_alone"]["us_median"], p["fused_launches_alone"]["plain_scoring_us"]))
        # full details on stderr; the one line keeps the summaries (per-step and per-chunk
        # arrays stay out of it), the headline's own keys first
        log("details headline: %s" % json.dumps(out))
        for name, val in extra.items():
            log("details %s: %s" % (name, json.dumps(val)))
        print(json.dumps(one_line(out, summarize_extra(extra))), flush=True)
        return

    import torch
    from dsa_indexer_top_amd import binding as B, inputs as gen
    from dsa_indexer_top_amd.runner import DecodeRunner

    if args.probe == "copy":
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(20):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 20 x 256 MiB device copies")
        return
    cfg = gen.CONFIGS[args.workload]
    prefetch = (cfg.prefetch if args.prefetch == "auto" else
                {"on": "ranged", "off": False}.get(args.prefetch, args.prefetch))
    if args.section:
        try:
            if args.section == "headline":
                res = headline(args, torch, B, gen, DecodeRunner, cfg, prefetch)
            else:
                res = child_section(args.section, args, torch, B, gen)
            torch.cuda.synchronize()
        except Exception as e:                       # noqa: BLE001
            res = {"error": "%s: %s" % (type(e).__name__, e)}
        print(json.dumps(res), flush=True)
        return
    if args.probe == "prefill":
        pc = gen.PREFILL["prefill_32k"]
        n = pc["n"]
        q, w, k = gen.make_prefill_inputs(n, seed=pc["seed"])
        dq, dw, dk = (torch.from_numpy(x).cuda() for x in (q, w, k))
        sc = torch.empty((n, n), dtype=torch.float32, device="cuda")
        for _ in range(3):
            B.index_scores_prefill(dq, dw, dk, sc, ld=n)
        torch.cuda.synchronize()
        log("prefill probe: 3 launches of echo_index_scores_prefill on 32768 x 32768")
        return
    if args.probe == "score":
        inp = gen.make_decode_inputs(cfg)
        dq, dw, dk = (torch.from_numpy(x).cuda() for x in (inp.q, inp.w, inp.k))
        dks = None if inp.k_scale is None else torch.from_numpy(inp.k_scale).cuda()
        dkb, dkl = torch.from_numpy(inp.key_begin).cuda(), torch.from_numpy(inp.key_len).cuda()
        max_len = int(inp.key_len.max())
        sc = torch.empty((len(inp.key_len), max_len), dtype=torch.float32, device="cuda")
        hist = torch.zeros((len(inp.key_len), 2048), dtype=torch.int32, device="cuda")
        for _ in range(20):
            B.index_scores_hist(dq, dw, dk, dks, dkb, dkl, max_len, sc, hist)
        torch.cuda.synchronize()
        log("score probe: 20 launches of echo_index_scores_hist (the step's scoring launch) on",
            args.workload)
        return
    raise SystemExit("bench.py: unknown --probe")

if __name__ == "__main__":
    main()
