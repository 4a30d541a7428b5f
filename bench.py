"""Benchmark: unified-max split-KV decode attention on one MI355X.

A step is one fd_attn_decode call -- the chunk kernel (partials, in-place
recompute of out-of-band chunks) and the merge, which for grids beyond one
round of workgroups is a second small launch -- over the 32K-context
grouped-query workload (batch 32, 64 query / 8 KV heads, head_dim 128, ragged
lengths U{1024..32768}, bf16 cache, chunk 1024), inputs resident in HBM.
Prints one JSON line: KV GB/s (valid K and V bytes / time per call over K
uninstrumented calls), calls/s, the chunk kernel's roofline (algorithmic
bytes / its average duration in a second pass of K calls, from start/stop
events stamped by its own dispatch on its stream), the read ceiling of the
same call's loads (its units streamed through the kernel's DMA ring with
nothing computed, include/fd_probe.h) beside it, and the float64 CPU oracle
timed on a bounded sample as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--config N]

With --stats N a step is one fd_attn_score_stats call (per-row score extremes
and a 4096-bin histogram, the calibration pass for phi) on decode workload N;
the line reports K bytes read per second against HBM peak.

With --prefill N a step is one fd_attn_prefill call on prefill workload N
(2: batch 2, 32 query / 8 KV heads, a causal 8192-token prompt, bf16); the
line then reports attention TFLOP/s (4 * head_dim flops per visible
query-key pair: the score and the weighted value) against the dense bf16
matrix-core peak.

With --gemm N a step is one pass of fd_flat_gemm over the linear layers of
GEMM workload N (2: the Q/K/V, O, gate/up and down projections of a 7B-class
decoder block at M = 16 decode tokens, bf16 weights); the line reports weight
GB/s (the bytes of the four weight matrices / time per step) against HBM
peak.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s and % of HBM peak; calls/sec at GQA 32K ctx"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
DEFAULT_CONFIG = 3
PREFILL_METRIC = "prefill-attn TFLOP/s (causal, unified max) and % of bf16 matrix peak"


def source_hash(entry: str = "fd_attn.hip") -> str:
    """Hash of one entry source and every library file it includes, so a
    counter record stays valid until the kernels it measured change."""
    dirs = [os.path.join(ROOT, "split_kv_asynchronous_amd", "csrc"), os.path.join(ROOT, "include")]
    seen, todo = set(), [entry]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        for d in dirs:
            path = os.path.join(d, name)
            if os.path.exists(path):
                seen.add(name)
                text = open(path).read()
                todo += re.findall(r'#include "([^"]+)"', text)
                break
    h = hashlib.sha256()
    for name in sorted(seen):
        for d in dirs:
            path = os.path.join(d, name)
            if os.path.exists(path):
                with open(path, "rb") as f:
                    h.update(name.encode() + f.read())
                break
    return h.hexdigest()[:16]


def kernel_bytes(prob, fused) -> int:
    """Algorithmic bytes the chunk kernel must move: every valid K and V
    element once, the queries, the lengths and the used block-table entries,
    plus the output rows and flags when it also merges.  Chunk partials are
    overhead, not counted."""
    qb = prob.q.nbytes
    lens = np.clip(prob.seq_lens, 0, prob.max_seq_len).astype(np.int64)
    extra = prob.seq_lens.nbytes
    if prob.page_size:
        extra += int((-(-lens // prob.page_size)).sum()) * 4
    if fused:
        rows = prob.batch * prob.num_q_heads
        extra += rows * prob.head_dim * 4 + rows
    return prob.kv_bytes() + qb + extra


def cpu_baseline(prob, min_seconds=10.0, max_passes=20):
    """The float64 oracle, as it stands, on the host cores: whole calls of the
    same workload repeated until about min_seconds of CPU time have passed
    (or, for a workload too slow for one pass in that time, the first batch
    entries only)."""
    import oracle
    B, Hq = prob.batch, prob.num_q_heads
    # one batch entry first, to size the sample
    t = time.perf_counter()
    oracle.decode_exact(**prob.args(), rows=np.arange(Hq, dtype=np.int32))
    per_entry = time.perf_counter() - t
    lens = np.clip(prob.seq_lens, 0, prob.max_seq_len).astype(np.int64)
    est_full = per_entry * B * max(1.0, lens.mean() / max(1, lens[0]))
    if est_full <= 2 * min_seconds:
        nb, rows = B, None
    else:
        nb = max(1, min(B, int(min_seconds / max(per_entry, 1e-9))))
        rows = np.arange(nb * Hq, dtype=np.int32)
    passes, spent, threads = 0, 0.0, 1
    while passes < max_passes and (passes == 0 or spent < min_seconds):
        t = time.perf_counter()
        _, _, _, threads = oracle.decode_exact(**prob.args(), rows=rows, with_threads=True)
        spent += time.perf_counter() - t
        passes += 1
    elt = {"f32": 4, "bf16": 2, "e4m3fn": 1}[prob.kv_dtype]
    sample_bytes = int(lens[:nb].sum()) * prob.num_kv_heads * prob.head_dim * 2 * elt
    gbs = sample_bytes * passes / spent / 1e9
    what = ("the whole call" if nb == B else "batch entries 0..%d (all %d query heads)" % (nb - 1, Hq))
    # the same oracle on one core, over the first batch entry's rows (or a
    # share of them) for about a third of the time
    oracle.set_threads(1)
    try:
        n1 = max(1, min(Hq, int(Hq * (min_seconds / 3) / max(per_entry * threads, 1e-9))))
        rows1 = np.arange(n1, dtype=np.int32)
        t = time.perf_counter()
        _, _, _, th1 = oracle.decode_exact(**prob.args(), rows=rows1, with_threads=True)
        spent1 = time.perf_counter() - t
    finally:
        oracle.set_threads(0)
    bytes1 = int(lens[0]) * n1 * prob.head_dim * 2 * elt   # K and V of row (0, h) each read once per row
    one = {"value": round(bytes1 / spent1 / 1e9, 4), "unit": "GB/s", "cores": int(th1),
           "sample": "query heads 0..%d of batch entry 0, %.1f s (K/V bytes counted once per query head)"
                     % (n1 - 1, spent1)}
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%s, %d pass(es), %.1f s, float64 exact softmax + band test; "
                      "calls/s equivalent %.4f" % (what, passes, spent, gbs * 1e9 / prob.kv_bytes()),
            "one_thread": one}


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def copy_calibration():
    """Five plain device copies of 1 GiB: the reference against which the HBM
    counters of a profiled run are scaled."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()


def prefill_cpu_baseline(prob, min_seconds=10.0):
    """The float64 prefill oracle on the host cores: query rows drawn evenly
    over every (sequence, head, position) until about min_seconds of CPU time
    have passed; flops counted per visible query-key pair as on the GPU."""
    import oracle
    B, Hq, Lq = prob.batch, prob.num_q_heads, prob.q_len
    kv = np.clip(prob.kv_lens.astype(np.int64), 0, prob.max_seq_len)
    n = 64
    spent, flops, rows_done, threads = 0.0, 0, 0, 1
    while spent < min_seconds and rows_done < B * Hq * Lq:
        rows = np.linspace(rows_done * 7919 % (B * Hq * Lq), B * Hq * Lq - 1, n).astype(np.int32)
        rows = np.unique(rows % (B * Hq * Lq))
        t = time.perf_counter()
        _, _, _, threads = oracle.prefill_exact(**prob.args(), rows=rows, with_threads=True)
        spent += time.perf_counter() - t
        j = rows % Lq
        b = rows // (Hq * Lq)
        flops += int(np.clip(kv[b] - Lq + j + 1, 0, None).sum()) * 4 * prob.head_dim
        rows_done += len(rows)
        n = min(4096, n * 2)
    tf = flops / spent / 1e12
    return {"value": round(tf, 7), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d query rows spread over all (sequence, head, position), %.1f s, "
                      "float64 exact causal softmax + band test" % (rows_done, spent)}


def main_prefill(args):
    import torch

    import synthetic
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_device import DevicePrefill

    t_gen = time.perf_counter()
    prob = synthetic.make_prefill_config(args.prefill)
    print("generated %s in %.1f s" % (prob.workload, time.perf_counter() - t_gen),
          file=sys.stderr, flush=True)
    dp = DevicePrefill(prob)
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    for _ in range(W):
        dp.run()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        dp.run()
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / K
    # second pass with the kernel's dispatch-stamped events (its durations)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        dp.run(stage_events=evs[i])
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in range(K)]))

    if args.copy_calibration:
        copy_calibration()

    pairs = prob.visible_pairs()
    flops = pairs * 4 * prob.head_dim
    value = flops / per_call / 1e12
    achieved = flops / (kernel_ms / 1e3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(per_call * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": prob.workload, "batch": prob.batch,
                   "num_q_heads": prob.num_q_heads, "num_kv_heads": prob.num_kv_heads,
                   "head_dim": prob.head_dim, "q_len": prob.q_len,
                   "kv_lens": prob.kv_lens.tolist(), "visible_pairs": pairs,
                   "flops_per_call": flops, "phi": prob.phi,
                   "band": [prob.phi - prob.a, prob.phi + prob.b]},
        "tokens_per_s": round(prob.batch * prob.q_len / per_call, 1),
        "kernel_ms": round(kernel_ms, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(prob.workload, "fd_prefill.hip"), "kernel": "prefill kernel",
                     "flops_per_launch": flops},
        "source_hash": source_hash("fd_prefill.hip"),
    }
    res["cpu_baseline"] = None if args.no_cpu_baseline else prefill_cpu_baseline(prob)
    print(json.dumps(res), flush=True)


def stats_cpu_baseline(prob, min_seconds=10.0):
    """The float64 calibration oracle (extremes + histogram) on the host cores,
    on whole batch entries until about min_seconds have passed."""
    import oracle
    B, Hq = prob.batch, prob.num_q_heads
    lens = np.clip(prob.seq_lens, 0, prob.max_seq_len).astype(np.int64)
    elt = {"f32": 4, "bf16": 2, "e4m3fn": 1}[prob.kv_dtype]
    spent, nbytes, done, threads = 0.0, 0, 0, 1
    while spent < min_seconds and done < B:
        sub = dict(prob.args())
        sl = slice(done, done + 1)
        sub["q"] = prob.q[sl]
        sub["seq_lens"] = prob.seq_lens[sl]
        if prob.page_size:
            sub["block_table"] = prob.block_table[sl]
        else:
            sub["k_cache"] = prob.k_cache[sl]
            sub["v_cache"] = prob.v_cache[sl]
        t = time.perf_counter()
        _, _, _, threads = oracle.score_stats(**sub, hist_lo=-8.0, hist_hi=8.0, nbins=4096,
                                              with_threads=True)
        spent += time.perf_counter() - t
        nbytes += int(lens[done]) * prob.num_kv_heads * prob.head_dim * elt
        done += 1
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(), "sample": "batch entries 0..%d (all %d query heads), %.1f s, float64 "
                                        "scores, extremes and 4096-bin histogram" % (done - 1, Hq, spent)}


def main_stats(args):
    import torch

    import split_kv_asynchronous_amd as fd
    import synthetic
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_device import DeviceProblem

    prob = synthetic.make_config(args.stats)
    print("generated %s" % prob.workload, file=sys.stderr, flush=True)
    dp = DeviceProblem(prob)

    def run():
        return fd.fd_attn_score_stats(dp.q, dp.k, dp.seq_lens, dp.block_table,
                                      max_seq_len=prob.max_seq_len, chunk_size=prob.chunk_size,
                                      num_kv_heads=prob.num_kv_heads, page_size=prob.page_size,
                                      scale=prob.scale, k_scale=dp.k_scale, hist_lo=-8.0,
                                      hist_hi=8.0, nbins=4096, q_dtype=prob.q_dtype,
                                      kv_dtype=prob.kv_dtype)
    K, W = args.steps, args.warmup
    for _ in range(W):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        run()
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / K
    elt = {"f32": 4, "bf16": 2, "e4m3fn": 1}[prob.kv_dtype]
    lens = np.clip(prob.seq_lens, 0, prob.max_seq_len).astype(np.int64)
    kbytes = int(lens.sum()) * prob.num_kv_heads * prob.head_dim * elt
    value = kbytes / per_call / 1e9
    if args.copy_calibration:
        copy_calibration()
    res = {
        "metric": "score-statistics pass (phi calibration): K GB/s and % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(per_call * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"f32": "f32", "bf16": "bf16", "e4m3fn": "fp8e4m3"}[prob.kv_dtype],
        "data": "synthetic",
        "config": {"workload": prob.workload, "k_bytes_per_call": kbytes, "nbins": 4096,
                   "hist_range": [-8.0, 8.0]},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("stats:" + prob.workload, "fd_calib.hip"),
                     "kernel": "score-statistics kernel (whole call: init + pass)",
                     "bytes_per_launch": kbytes},
        "source_hash": source_hash("fd_calib.hip"),
    }
    res["cpu_baseline"] = None if args.no_cpu_baseline else stats_cpu_baseline(prob)
    print(json.dumps(res), flush=True)


def gemm_cpu_baseline(cfg, inputs, min_seconds=10.0):
    """The float64 flat-GEMM oracle on the host cores, layer after layer until
    about min_seconds have passed; weight bytes per second."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    spent, nbytes, done = 0.0, 0, []
    while spent < min_seconds:
        for (name, n, k), (a, w) in zip(cfg["layers"], inputs):
            t = time.perf_counter()
            oracle.flat_gemm(a, w)
            spent += time.perf_counter() - t
            nbytes += w.nbytes
            done.append(name)
            if spent >= min_seconds:
                break
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(), "sample": "%d layer products (%s), %.1f s, float64 matrix multiply"
                                        % (len(done), ",".join(done[:8]), spent)}


def main_gemm(args):
    import torch

    import split_kv_asynchronous_amd as fd
    import synthetic
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_device import to_device

    cfg = synthetic.GEMM_CONFIGS[args.gemm]
    m = cfg["m"]
    inputs = [synthetic.make_gemm(m, n, k, seed=synthetic.SEED_BASE + 200 + i)
              for i, (_, n, k) in enumerate(cfg["layers"])]
    print("generated %s" % cfg["workload"], file=sys.stderr, flush=True)
    # consecutive steps use different copies of the weights (as consecutive
    # decoder blocks would), so no step finds its weights in the chip's
    # last-level cache: > 1 GB of weights in the rotation
    wbytes = sum(w.nbytes for _, w in inputs)
    copies = max(1, -(-(1 << 30) // wbytes))
    dev = [[(to_device(a, "bf16"), to_device(w, "bf16")) for a, w in inputs]]
    for _ in range(copies - 1):
        dev.append([(a.clone(), w.clone()) for a, w in dev[0]])
    # weights are packed once, as a model would at load time, into the
    # fragment-major layout (fd_flat_gemm_pack_weights); not timed
    dev = [[(a, fd.fd_flat_gemm_pack_weights(w)) for a, w in blk] for blk in dev]
    torch.cuda.synchronize()
    plans = [fd.fd_flat_gemm_plan(m, n, k, w_layout="packed") for _, n, k in cfg["layers"]]
    outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _, n, _ in cfg["layers"]]
    wss = [torch.empty(max(fd.fd_flat_gemm_workspace_size(m, n, k, w_layout="packed"), 256),
                       dtype=torch.uint8, device="cuda") for _, n, k in cfg["layers"]]
    ns = [n for _, n, _ in cfg["layers"]]
    stream = torch.cuda.current_stream()
    L = len(cfg["layers"])

    def step(j, evs=None):
        for i in range(L):
            a, w = dev[j % copies][i]
            fd.fd_flat_gemm(a, w, outs[i], out_dtype="bf16", workspace=wss[i], n=ns[i],
                            stage_events=None if evs is None else evs[i])

    K, W = args.steps, args.warmup
    for j in range(W):
        step(j)
    torch.cuda.synchronize()
    # one graph per weight copy: a decode step's linear layers are replayed
    # from a captured graph, so the host's launch cost does not gate the GPU
    cap = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(cap):
        for j in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(j)
            graphs.append(g)
    torch.cuda.synchronize()
    for j in range(copies):
        graphs[j].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        graphs[(W + i) % copies].replay()
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / K
    # per-kernel durations: the same K steps launched directly, each
    # partial-sum kernel stamping start/stop events from its own dispatch
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)]
           for _ in range(K)]
    for row in evs:
        for pair in row:
            for e in pair:
                e.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        step(W + i, evs[i])
    torch.cuda.synchronize()
    value = wbytes / per_step / 1e9
    layers = {}
    for li, (name, n, k) in enumerate(cfg["layers"]):
        ms = float(np.mean([evs[i][li][0].elapsed_time(evs[i][li][1]) for i in range(K)]))
        algo = n * k * 2 + m * k * 2 + m * n * 2      # W, A and C once; split partials are overhead
        layers[name] = {"n": n, "k": k, "kernel_ms": round(ms, 5),
                        "kernel_GBps": round(algo / (ms / 1e3) / 1e9, 2), "plan": plans[li],
                        "bytes_per_launch": algo}
    # each layer's weights read alone (include/fd_probe.h): one unit per
    # 16-row block of the packed weights, its halves from the two halves of
    # the buffer, through the 4 x 2 DMA ring with nothing computed, the
    # copies rotated as in the step: what one launch reading that many bytes
    # reaches on this device
    sink = torch.empty(1, dtype=torch.int32, device="cuda")
    for li, (name, n, k) in enumerate(cfg["layers"]):
        nblk = -(-n // 16)
        if nblk % 2:
            layers[name]["read_ceiling_GBps"] = None
            continue
        ub = nblk // 2 * 32 * k // nblk          # bytes of a block in each half
        units = np.zeros(nblk, dtype=fd.PROBE_UNIT)
        units["offset"] = np.arange(nblk, dtype=np.uint64) * ub
        units["bytes"] = ub
        ud = torch.from_numpy(units.view(np.uint8).copy()).cuda()
        half = nblk * ub

        def probe(j):
            raw = dev[j % copies][li][1].view(torch.uint8)
            fd.fd_probe_read(raw[:half], raw[half:2 * half], ud, 0, None, 0, sink)
        for j in range(copies):
            probe(j)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(K):
            probe(W + i)
        e1.record()
        e1.synchronize()
        ceil = 2 * half / (e0.elapsed_time(e1) / K / 1e3) / 1e9
        layers[name]["read_ceiling_GBps"] = round(ceil, 2)
        layers[name]["kernel_frac_of_ceiling"] = round(layers[name]["kernel_GBps"] / ceil, 4)
    # the dominant kernel: the partial-sum kernel of the largest layer
    big = max(layers, key=lambda x: layers[x]["n"] * layers[x]["k"])
    achieved = layers[big]["kernel_GBps"]
    if args.copy_calibration:
        copy_calibration()
    res = {
        "metric": "flat GEMM of the decode linear layers: weight GB/s and % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(per_step * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["workload"], "m": m,
                   "layers": [[name, n, k] for name, n, k in cfg["layers"]],
                   "weight_bytes_per_step": wbytes, "out_dtype": "bf16",
                   "weight_copies_rotated": copies, "weight_layout": "packed at load",
                   "timing": "graph replay per step"},
        "tflops": round(2.0 * m * sum(n * k for _, n, k in cfg["layers"]) / per_step / 1e12, 3),
        "layers": layers,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("gemm:%s:%s" % (cfg["workload"], big), "fd_gemm.hip"),
                     "kernel": "flat GEMM partial-sum kernel (%s layer)" % big,
                     "bytes_per_launch": layers[big]["bytes_per_launch"]},
        "source_hash": source_hash("fd_gemm.hip"),
    }
    res["cpu_baseline"] = None if args.no_cpu_baseline else gemm_cpu_baseline(cfg, inputs)
    print(json.dumps(res), flush=True)


def load_traffic(workload: str, entry: str = "fd_attn.hip"):
    """HBM bytes per kernel launch from committed rocprofv3 counter runs,
    if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_hash") != source_hash(entry):
        return None
    return rec.get("bytes_per_launch")


# Serving-sized batches of ragged decode calls (sequences x query heads / KV
# heads, length range, cache format, page size, chunk size): the unit search
# of the grouped kernels at batches of hundreds to thousands of sequences.
SERVING_CASES = [
    ("gqa64/8-bf16-B32-1K..32K", 32, 64, 8, 1024, 32768, "bf16", 0, 1024),
    ("gqa64/8-bf16-B512-512..4K", 512, 64, 8, 512, 4096, "bf16", 0, 1024),
    ("gqa64/8-bf16-B2048-128..1K", 2048, 64, 8, 128, 1024, "bf16", 0, 1024),
    ("gqa32/8-fp8-paged16-B512-512..4K", 512, 32, 8, 512, 4096, "e4m3fn", 16, 512),
    ("gqa32/8-fp8-paged16-B2048-256..2K", 2048, 32, 8, 256, 2048, "e4m3fn", 16, 512),
]


def library_plan_line(fd, dp, prob, K, torch):
    """K back-to-back calls of the bench workload with chunk_size 0 (the
    library's table picks the chunks, or balanced shares), on the inputs
    already resident: {plan, ms per call, GB/s of K/V}."""
    import dataclasses
    lp = dataclasses.replace(prob, chunk_size=0)
    ws = torch.empty(max(fd.fd_attn_workspace_size(fd.make_desc(
        batch=lp.batch, num_q_heads=lp.num_q_heads, num_kv_heads=lp.num_kv_heads, max_seq_len=lp.max_seq_len,
        chunk_size=0, page_size=lp.page_size,
        max_blocks_per_seq=0 if lp.block_table is None else lp.block_table.shape[1],
        num_pages=lp.k_cache.shape[0] if lp.page_size else 0, scale=lp.scale, q_dtype=lp.q_dtype,
        kv_dtype=lp.kv_dtype)), 256), device="cuda", dtype=torch.uint8)
    call = fd.prepare_decode(dp.q, dp.k, dp.v, dp.seq_lens, dp.block_table, lp.phi, lp.a, lp.b, dp.out, dp.flags,
                             chunk_size=0, max_seq_len=lp.max_seq_len, num_kv_heads=lp.num_kv_heads,
                             page_size=lp.page_size, scale=lp.scale, k_scale=dp.k_scale, v_scale=dp.v_scale,
                             workspace=ws, q_dtype=lp.q_dtype, kv_dtype=lp.kv_dtype, out_dtype=dp.out_dtype)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        call()
    torch.cuda.synchronize()
    per_call = (time.perf_counter() - t0) / K
    plan = fd.fd_attn_plan(call.desc) if hasattr(call, "desc") else None
    out = {"chunk_size": 0, "ms_per_call": round(per_call * 1e3, 5),
           "gbs": round(prob.kv_bytes() / per_call / 1e9, 2), "plan": plan}
    # the bench's own call runs after this one on dp's workspace: restore its outputs
    dp.run()
    torch.cuda.synchronize()
    return out


def heads_per_block(g: int) -> int:
    """Query heads per head block of the grouped-query kernels: the largest
    divisor of the group size up to 16."""
    return next((k for k in range(min(g, 16), 1, -1) if g % k == 0), 1)


def probe_units(prob, chunk: int):
    """The chunk kernel's units of a grouped-query call, in the kernel's
    order: every sequence's full chunks (sequence-major, chunks outer, head
    blocks inner), then the partial last chunks.  A unit of head block hb
    reads its KV head's tokens of the chunk.  Contiguous cache: (units as
    byte ranges, None, 0).  Paged: (units indexing a page list, the page list
    -- byte offsets of (page, KV head) pieces, as the block table gives them
    --, page bytes)."""
    import split_kv_asynchronous_amd as fd
    row = prob.head_dim * {"bf16": 2, "e4m3fn": 1, "f32": 4}[prob.kv_dtype]
    G = prob.num_q_heads // prob.num_kv_heads
    GB = heads_per_block(G)
    nhb = prob.num_q_heads // GB
    kvh = np.arange(nhb) * GB // G
    P = prob.page_size
    order = []   # (b, chunk, tokens)
    for b, L in enumerate(prob.seq_lens.tolist()):
        order += [(b, c, chunk) for c in range(L // chunk)]
    for b, L in enumerate(prob.seq_lens.tolist()):
        if L % chunk or L == 0:
            order.append((b, L // chunk, L - L // chunk * chunk))
    units = np.zeros(len(order) * nhb, dtype=fd.PROBE_UNIT)
    if not P:
        S = prob.max_seq_len
        for n, (b, c, t) in enumerate(order):
            units["offset"][n * nhb:(n + 1) * nhb] = ((b * prob.num_kv_heads + kvh) * S + c * chunk) * row
            units["bytes"][n * nhb:(n + 1) * nhb] = t * row
        return units, None, 0
    assert chunk % P == 0
    pages = []
    for n, (b, c, t) in enumerate(order):
        blocks = prob.block_table[b, c * chunk // P:c * chunk // P + -(-t // P)].astype(np.int64)
        for i, h in enumerate(kvh.tolist()):
            units["offset"][n * nhb + i] = len(pages)
            units["bytes"][n * nhb + i] = t * row
            pages += ((blocks * prob.num_kv_heads + h) * P * row).tolist()
    return units, np.array(pages, dtype=np.int64), P * row


# probe ring shape per (kernel family, kernel shape) of the plan: the grouped
# bf16 kernel's 4 x 2 and 4 x 3 rings, the cooperative E4M3FN kernel's 2 x 3
PROBE_SHAPES = {(0, 0): 0, (0, 1): 1, (1, 0): 2}


def read_ceiling(fd, dp, prob, plan, K, torch):
    """The decode call's loads alone (include/fd_probe.h): the chunk kernel's
    units, in its order, streamed through its DMA ring shape with nothing
    computed, K back-to-back launches timed by events.  For the grouped
    kernels' fixed-chunk plans whose ring the probe has; None otherwise."""
    shape = PROBE_SHAPES.get((plan["family"], plan["shape"]))
    if shape is None or plan["shares"] or plan["chunk_size"] % max(prob.page_size, 1):
        return None
    units, pages, page_bytes = probe_units(prob, plan["chunk_size"])
    if pages is not None and int(units["bytes"].max()) > 64 * page_bytes:
        return None
    nbytes = 2 * int(units["bytes"].sum())
    dev = torch.from_numpy(units.view(np.uint8).copy()).cuda()
    pg = None if pages is None else torch.from_numpy(pages).cuda()
    sink = torch.empty(1, dtype=torch.int32, device="cuda")

    def run():
        fd.fd_probe_read(dp.k, dp.v, dev, shape, pg, page_bytes, sink)
    for _ in range(5):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        run()
    e1.record()
    e1.synchronize()
    per = e0.elapsed_time(e1) / K / 1e3
    ring = {0: "4 wavefronts x 2 stages of 8 KiB", 1: "4 wavefronts x 3 stages of 8 KiB",
            2: "2 wavefronts x 3 stages of 4 KiB"}[shape]
    return {"value": round(nbytes / per / 1e9, 2), "unit": "GB/s", "ms_per_launch": round(per * 1e3, 5),
            "bytes_per_launch": nbytes, "units": len(units),
            "ring": ring + ", non-temporal 1 KiB DMA" + (", whole pages" if pages is not None else "")}


def main_serving(args):
    """One JSON line per serving-batch case: whole-call and chunk-kernel TB/s
    of K/V over K back-to-back calls at the case's chunk size, and the same
    batch under the library's own plan (a side measurement, not the bench
    line)."""
    import torch

    import split_kv_asynchronous_amd as fd
    import synthetic
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_device import DeviceProblem

    for name, B, hq, hkv, lo, hi, kv, page, chunk in SERVING_CASES:
        lens = np.random.default_rng(3).integers(lo, hi + 1, size=B).astype(np.int32)
        prob = synthetic.make_problem(batch=B, num_q_heads=hq, num_kv_heads=hkv, seq_lens=lens, kv_dtype=kv,
                                      page_size=page, chunk_size=chunk, seed=77, workload=name)
        dp = DeviceProblem(prob)
        for _ in range(args.warmup):
            dp.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dp.run()
        torch.cuda.synchronize()
        per_call = (time.perf_counter() - t0) / args.steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for row in evs:
            for e in row:
                e.record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            dp.run(stage_events=evs[i])
        torch.cuda.synchronize()
        kms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        kvb = prob.kv_bytes()
        line = {"workload": name, "batch": B, "kv_bytes_per_call": kvb,
                "ms_per_call": round(per_call * 1e3, 5), "call_tbs": round(kvb / per_call / 1e12, 3),
                "kernel_ms": round(kms, 5), "kernel_tbs": round(kvb / kms / 1e9, 3),
                "plan": fd.fd_attn_plan(dp.desc())}
        # the same batch under the library's own plan (chunk_size 0)
        line["library_plan"] = library_plan_line(fd, dp, prob, args.steps, torch)
        print(json.dumps(line), flush=True)
        del dp
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--stats", type=int, default=0,
                    help="time fd_attn_score_stats (phi calibration pass) on this decode workload")
    ap.add_argument("--prefill", type=int, default=0,
                    help="time fd_attn_prefill on this prefill workload instead of decode")
    ap.add_argument("--gemm", type=int, default=0,
                    help="time fd_flat_gemm over the linear layers of this GEMM workload")
    ap.add_argument("--serving", action="store_true",
                    help="side measurement: ragged decode at serving batch sizes, one line per case")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode-attention path is built and timed on a "
              "single MI355X; multi-GPU runs are not part of this library", file=sys.stderr)
        sys.exit(2)
    if args.serving:
        main_serving(args)
        return
    if args.prefill:
        main_prefill(args)
        return
    if args.stats:
        main_stats(args)
        return
    if args.gemm:
        main_gemm(args)
        return

    import torch

    import split_kv_asynchronous_amd as fd
    import synthetic
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_device import DeviceProblem

    t_gen = time.perf_counter()
    prob = synthetic.make_config(args.config)
    print("generated %s in %.1f s" % (prob.workload, time.perf_counter() - t_gen),
          file=sys.stderr, flush=True)
    dp = DeviceProblem(prob)
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup

    for _ in range(W):
        dp.run()
    torch.cuda.synchronize()

    # timed region: K back-to-back calls, uninstrumented
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        dp.run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call = elapsed / K

    # a second pass of K calls in which the chunk kernel of every call stamps
    # its start/stop into that call's events (events 0/1, recorded by the
    # kernel's own dispatch): the kernel durations for the roofline
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for row in evs:            # create the HIP events before the pass
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(K):
        dp.run(stage_events=evs[i])
    torch.cuda.synchronize()
    kernel_ms = [evs[i][0].elapsed_time(evs[i][1]) for i in range(K)]

    # the same call captured once into a graph and replayed K times (the
    # per-token graph execute of a serving loop): reported beside the value
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.graph(graph, stream=side):
        dp.run()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        graph.replay()
    torch.cuda.synchronize()
    graph_per_call = (time.perf_counter() - t0) / K
    del graph

    kv = prob.kv_bytes()
    value = kv / per_call / 1e9
    rows_flagged = int(dp.results()[1].sum())
    chunks_recomputed = dp.recomputed()
    kernel_s = float(np.mean(kernel_ms)) / 1e3
    plan = fd.fd_attn_plan(dp.desc())
    fused = bool(plan["fused"])
    nbytes = kernel_bytes(prob, fused)
    achieved = nbytes / kernel_s / 1e9

    # the same workload under the library's own pick of chunks and plan
    # (chunk_size 0), K calls on the same inputs: reported beside the value,
    # which keeps the workload's stated chunk size
    lib = library_plan_line(fd, dp, prob, K, torch)
    # the same call's loads with nothing computed: what its load pattern can
    # reach on this device, beside the roofline's published peak
    ceil = read_ceiling(fd, dp, prob, plan, K, torch)

    if args.copy_calibration:
        copy_calibration()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(per_call * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3fn": "fp8e4m3"}[prob.kv_dtype],
        "data": "synthetic",
        "config": {"workload": prob.workload, "batch": prob.batch,
                   "num_q_heads": prob.num_q_heads, "num_kv_heads": prob.num_kv_heads,
                   "head_dim": prob.head_dim, "sum_seq_len": int(prob.seq_lens.sum()),
                   "max_seq_len": prob.max_seq_len, "chunk_size": prob.chunk_size,
                   "page_size": prob.page_size, "kv_bytes_per_call": kv,
                   "phi": prob.phi, "band": [prob.phi - prob.a, prob.phi + prob.b]},
        "calls_per_s": round(1.0 / per_call, 2),
        "graph_ms_per_call": round(graph_per_call * 1e3, 5),
        "plan": plan,
        # a cache under twice the 256 MB last-level cache is re-read from it, in
        # part or whole, call after call: such a line is not an HBM figure
        "cache_resident": kv < (512 << 20),
        # fallback activity of the last call: rows flagged, (row, chunk) pairs recomputed
        "rows_flagged": rows_flagged,
        "chunks_recomputed": chunks_recomputed,
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": round(float(np.mean(kernel_ms)), 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(prob.workload),
                     "kernel": "chunk kernel" + (" (with the merge)" if fused else ""),
                     "bytes_per_launch": nbytes},
        "read_ceiling": None if ceil is None else dict(ceil, kernel_frac=round(achieved / ceil["value"], 4)),
        "source_hash": source_hash(),
        "library_plan": lib,
    }
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(prob)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
