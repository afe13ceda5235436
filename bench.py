"""Benchmark of the NVFP4 paged-KV hot path on one MI355X.

One step = one attention layer of a 2048x2048 causal prefill with
Qwen3-8B-shaped attention (1 request, q_len = kv_len = 2048, 32 query heads,
8 KV heads, head_dim 128, page size 16): append the 2048 new K/V rows to the
NVFP4 paged cache through the slot mapping, then run the causal paged
prefill over those pages.  The plan step runs once per batch (as in a
serving engine, where one plan serves every layer) and its host time is
reported separately.

Prints one JSON line.  `value` is causal-prefill TFLOP/s over the whole step
(algorithmic flops 4 * head_dim * allowed (query, key) pairs per query head,
divided by the step time).  Also reported: per-kernel launch durations
(HIP events on the launch stream around replays of a graph of back-to-back
launches of that kernel), the roofline of the dominant kernel, the append's
achieved GB/s on this workload and on the 65,536-token append stress
workload, and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill TFLOP/s + append GB/s on NVFP4 paged KV (% of MI355X roofline)"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("prefill.hip", "append.hip", "decode.hip", "nvfp4kv_codec.hpp"):
        h.update(open(os.path.join(ROOT, "nvfp4_paged_kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def attention_flops(q_lens, kv_lens, num_q_heads, head_dim):
    """4 * D * sum over requests, query heads and query rows of the allowed keys."""
    tot = 0
    for lq, lk in zip(q_lens, kv_lens):
        lq, lk = int(lq), int(lk)
        tot += lq * (lk - lq) + lq * (lq + 1) // 2
    return 4 * head_dim * num_q_heads * tot


def append_bytes(tokens, heads, d):
    """bf16 K and V read + packed NVFP4 and scale bytes written + int64 slots."""
    return tokens * heads * (2 * d + d // 2 + d // 16) * 2 + 8 * tokens


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the clocks settle after ~30-40 ms of sustained launches; 1000 warm-up
    # steps (~60 ms) reach the steady state the timed steps measure
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append-stress", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured achievable peaks (copy, MFMA-only loop)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the dequant-placement ablation of the prefill")
    ap.add_argument("--ablation-only", action="store_true",
                    help="only launch the prefill under the three dequant placements (for counters)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each step's work is one GPU's share; see the design notes on sharding).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_paged_kv_amd as K
    import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE read for it give
        # the scale between those counters and bytes actually moved
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel(), "launches": 5}))
        return
    w = W.prefill_2k(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    qo_h, kvl_h = torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens)
    kvp_h = torch.from_numpy(w.kv_indptr)
    qo_d, kvl_d = qo_h.to(dev), kvl_h.to(dev)
    kvp_d, pt_d = kvp_h.to(dev), torch.from_numpy(w.page_table).to(dev)
    out = torch.empty_like(w.q)

    if args.ablation_only:
        cache.append(w.k, w.v, w.slot_mapping)
        print(json.dumps({"dequant_ablation": bench_dequant_ablation(
            K, w, cache, (qo_d, kvp_d, pt_d, kvl_d), out, torch, per_graph=10, replays=2)}), flush=True)
        return
    t0 = time.perf_counter()
    nplan = 200
    for _ in range(nplan):
        plan = K.plan(qo_h, kvl_h, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                      kv_indptr=kvp_h)
    plan_us = (time.perf_counter() - t0) / nplan * 1e6

    def step():
        cache.append(w.k, w.v, w.slot_mapping)
        K.paged_prefill_causal(w.q, qo_d, kvp_d, pt_d, kvl_d, cache, out, w.sm_scale, plan=plan)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps, bracketed by device synchronization
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3
    bits = K.read_device_error(dev)
    if bits:
        raise SystemExit(f"device error bits {bits}")

    # per-kernel launch durations: each kernel's launches captured back to back
    # into a graph and replayed between two HIP events on the launch stream
    # (torch's current stream), so that host-side launch cost does not pace
    # the short append kernel
    app_ms = graph_launch_ms(torch, lambda: cache.append(w.k, w.v, w.slot_mapping))
    pre_ms = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, qo_d, kvp_d, pt_d, kvl_d, cache,
                                                                   out, w.sm_scale, plan=plan))

    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    abytes = append_bytes(int(w.kv_lens.sum()), w.num_kv_heads, w.head_dim)
    value = flops / (ms_per_step * 1e-3) / 1e12
    pre_tflops = flops / (pre_ms * 1e-3) / 1e12
    G = w.num_q_heads // w.num_kv_heads
    kernel_name = f"prefill_kernel<{w.head_dim},{G},{plan.block_q * G // 32},{'true' if 64 % w.page_size == 0 else 'false'},0>"
    traffic = _traffic("prefill_2k")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": 1, "q_len": 2048, "kv_len": 2048,
                   "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
                   "kv_format": "nvfp4 (e2m1 + e4m3 per 16, fp32 global scale)",
                   "step": "append 2048 K/V rows + causal paged prefill",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": kernel_name,
                     "achieved": round(pre_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic, "flops_per_launch": flops,
                     "avg_launch_us": round(pre_ms * 1e3, 2)},
        "append": {"bound": "hbm", "bytes_per_launch": abytes, "avg_launch_us": round(app_ms * 1e3, 2),
                   "achieved_GBps": round(abytes / (app_ms * 1e-3) / 1e9, 1), "peak_GBps": HBM_PEAK_GBS,
                   "frac": round(abytes / (app_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "plan_host_us": round(plan_us, 2),
        "plan_bench": bench_plan(K, torch, np),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_append_stress:
        result["append_stress"] = bench_append_stress(K, W, dev, torch, np)
    if not args.no_decode:
        result["decode"] = bench_decode(K, W, dev, torch, np)
    if not args.no_ablation:
        result["dequant_ablation"] = bench_dequant_ablation(K, w, cache, (qo_d, kvp_d, pt_d, kvl_d), out,
                                                            torch)
    if not args.no_achievable:
        ach = bench_achievable(W, dev, torch, np)
        ach["prefill_frac_of_mfma_loop"] = round(pre_tflops / ach["mfma_bf16_TFLOPs"], 4)
        if "append_stress" in result:
            got = result["append_stress"]["achieved_GBps"]
            ach["append_stress_frac_of_copy"] = round(got / ach["copy_GBps"], 4)
            ach["append_stress_frac_of_traffic_probe"] = round(got / ach["append_traffic_GBps"], 4)
        result["achievable"] = ach
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, flops)
    print(json.dumps(result), flush=True)


def graph_launch_ms(torch, fn, per_graph=50, replays=20):
    """Average duration (ms) of one launch of `fn`: `per_graph` launches
    captured into one graph, replayed `replays` times between two events."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / (per_graph * replays)


def bench_dequant_ablation(K, w, cache, dev_args, out, torch, per_graph=50, replays=20):
    """The 2048x2048 prefill under the three dequant placements of the PR #4769
    page's comparison (graph-timed launches; 4-wave tiles, as the plan picks):
    tiles decoded once per workgroup into f16 LDS (the kernel's own design), K
    decoded in registers inside the matrix loop, a byte-table decode, and the
    f16 design with bf16 staging and bf16 matrix instructions instead."""
    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    res = {}
    for mode, name in ((0, "lds_once_per_tile"), (1, "k_in_loop_registers"), (2, "lds_byte_table"),
                       (3, "lds_once_per_tile_bf16")):
        plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                      tile_waves=4, dequant_mode=mode)
        ms = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *dev_args, cache, out, w.sm_scale,
                                                                   plan=plan), per_graph, replays)
        res[name] = {"dequant_mode": mode, "avg_launch_us": round(ms * 1e3, 2),
                     "TFLOP_s": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return res


def bench_plan(K, torch, np, batches=(64, 256, 1024), reps=50):
    """Host time of the plan step on ragged batches of B requests (q_len
    U{1..512}, kv_len = q_len + U{0..3584}, seeded): the library's plan call
    (length checks, maxima, totals, tile counts, chunk split) through the
    binding, against two ways of taking only its first part (max q/kv length,
    totals, the q_len <= kv_len check) in Python: a loop over the requests
    reading one tensor element at a time, and whole-tensor reductions."""
    res = {}
    for B in batches:
        rng = np.random.default_rng(1000 + B)
        ql = rng.integers(1, 513, B).astype(np.int32)
        kvl = (ql + rng.integers(0, 3585, B)).astype(np.int32)
        qo = torch.from_numpy(np.concatenate([[0], np.cumsum(ql)]).astype(np.int32))
        kv = torch.from_numpy(kvl)

        def native():
            return K.plan(qo, kv, 32, 8, 128, 16)

        def loop():
            mq = mk = tq = tk = 0
            for i in range(B):
                a, b = int(qo[i + 1]) - int(qo[i]), int(kv[i])
                if a > b:
                    raise ValueError("q_len > kv_len")
                mq, mk, tq, tk = max(mq, a), max(mk, b), tq + a, tk + b
            return mq, mk, tq, tk

        def vectorised():
            d = qo[1:] - qo[:-1]
            if bool((d > kv).any()):
                raise ValueError("q_len > kv_len")
            return int(d.max()), int(kv.max()), int(qo[-1]), int(kv.sum())

        p = native()
        assert (p.max_q_len, p.max_kv_len, p.total_q, p.total_kv) == loop() == vectorised()
        row = {}
        for name, fn, n in (("native_us", native, reps), ("python_loop_us", loop, max(3, reps // 10)),
                            ("torch_vectorised_us", vectorised, reps)):
            fn()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            row[name] = round((time.perf_counter() - t0) / n * 1e6, 2)
        res[str(B)] = row
    return res


def _traffic(key):
    """HBM bytes per launch of one profiled kernel (profiles/traffic.json),
    or None when the kernel sources changed since the counters were taken."""
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_source_hash") == kernel_source_hash():
            return t.get(key, {}).get("bytes_per_launch")
    return None


def bench_decode(K, W, dev, torch, np, iters=12):
    """One decode step of 32 requests x 8192 cached keys (paged_decode, the
    plan's automatic chunking), cold like the append stress: median of 12
    launches, each after the untimed cache-flush read.  Bytes = the NVFP4 K
    and V codes and scales of every cached key (plus q and out)."""
    w = W.decode_batch(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    cache.append(w.k, w.v, w.slot_mapping)
    args = [torch.from_numpy(x).to(dev) for x in (w.kv_indptr, w.page_table, w.kv_lens)]
    out = torch.empty_like(w.q)
    plan = K.decode_plan(torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads, w.head_dim,
                         w.page_size)
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(3):
        K.paged_decode(w.q, *args, cache, out, w.sm_scale, plan)
    times = []
    for _ in range(iters):
        torch.amax(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        K.paged_decode(w.q, *args, cache, out, w.sm_scale, plan)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    bits = K.read_device_error(dev)
    if bits:
        raise SystemExit(f"device error bits {bits} in the decode")
    ms = float(np.median(times))
    nbytes = (int(w.kv_lens.sum()) * w.num_kv_heads * (w.head_dim // 2 + w.head_dim // 16) * 2
              + 2 * w.q.numel() * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "bound": "hbm", "bytes_per_launch": nbytes,
            "median_launch_us": round(ms * 1e3, 2), "achieved_GBps": round(gbs, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "chunk_len": plan.chunk_len, "cache": "cold (flushed)", "traffic": _traffic("decode")}


def bench_achievable(W, dev, torch, np):
    """Measured achievable rates on this device.  Cold, like the append and
    decode figures (the 256 MB Infinity Cache flushed by an untimed 512 MiB
    read before every launch; median of 12 launches, HIP events on the launch
    stream): a 16-byte-per-lane copy of 128 MiB (read + write bytes / time),
    and the 65,536-token append's own data movement without its arithmetic
    (peak.hip append_traffic: the same bf16 loads and the same code and
    scale stores through the same scattered slots; the append's algorithmic
    bytes / time).  Warm: the MFMA-only loop of peak.hip (dense
    v_mfma_f32_32x32x16_bf16, two waves per SIMD; median of 10)."""
    import ctypes
    from nvfp4_paged_kv_amd.build import PEAK_LIB
    if not os.path.exists(PEAK_LIB):
        raise SystemExit(f"{PEAK_LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PEAK_LIB)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    vp = ctypes.c_void_p
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)

    def timed(fn, n=10, cold=False):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(n):
            if cold:
                torch.amax(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    def check(rc, what):
        if rc != 0:
            raise SystemExit(f"{what} probe launch failed")

    src = torch.ones(128 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    L.nvfp4kv_copy_probe.argtypes = [vp, vp, ctypes.c_int64, vp]
    copy_s = timed(lambda: check(L.nvfp4kv_copy_probe(vp(src.data_ptr()), vp(dst.data_ptr()),
                                                      src.numel() // 16, stream), "copy"), n=12, cold=True)
    out = {"copy_GBps": round(2 * src.numel() / copy_s / 1e9, 1)}
    del src, dst

    a = W.append_stress(dev)
    cache = [torch.empty((a.num_pages, a.page_size, a.num_kv_heads, a.head_dim // d), dtype=torch.uint8,
                         device=dev) for d in (2, 2, 16, 16)]
    L.nvfp4kv_append_traffic_probe.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int64, vp, vp, vp, vp, vp]
    traffic_s = timed(lambda: check(L.nvfp4kv_append_traffic_probe(
        vp(a.k.data_ptr()), vp(a.v.data_ptr()), vp(a.slot_mapping.data_ptr()), a.k.shape[0],
        a.num_kv_heads, a.head_dim, a.num_pages * a.page_size, *(vp(c.data_ptr()) for c in cache),
        stream), "append traffic"), n=12, cold=True)
    out["append_traffic_GBps"] = round(append_bytes(a.k.shape[0], a.num_kv_heads, a.head_dim)
                                       / traffic_s / 1e9, 1)
    del a, cache, flush

    L.nvfp4kv_mfma_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.nvfp4kv_mfma_peak_probe_flops.restype = ctypes.c_double
    L.nvfp4kv_mfma_peak_probe_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    blocks, iters = 256 * 4, 2000
    buf = torch.empty(blocks * 512, dtype=torch.float32, device=dev)

    def mfma():
        if L.nvfp4kv_mfma_peak_probe(blocks, iters, ctypes.c_void_p(buf.data_ptr()), stream) != 0:
            raise SystemExit("MFMA peak probe launch failed")

    mfma_s = timed(mfma)
    out["mfma_bf16_TFLOPs"] = round(L.nvfp4kv_mfma_peak_probe_flops(blocks, iters) / mfma_s / 1e12, 1)
    return out


def bench_append_stress(K, W, dev, torch, np, iters=12):
    """65,536-token append (Student-t(3) values, scattered slots).  The 256 MB
    Infinity Cache is flushed before every timed launch by reading a 512 MiB
    buffer (untimed; a read leaves no dirty lines to write back during the
    timed launch); median of 12 launches, HIP events on the launch stream."""
    a = W.append_stress(dev)
    cache = K.PagedCache.empty(a.num_pages, a.page_size, a.num_kv_heads, a.head_dim, dev,
                               a.k_scale, a.v_scale)
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(3):
        cache.append(a.k, a.v, a.slot_mapping)
    times = []
    for _ in range(iters):
        torch.amax(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.append(a.k, a.v, a.slot_mapping)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    nbytes = append_bytes(a.k.shape[0], a.num_kv_heads, a.head_dim)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": a.name, "bound": "hbm", "bytes_per_launch": nbytes,
            "median_launch_us": round(ms * 1e3, 2), "achieved_GBps": round(gbs, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "cache": "cold (flushed)",
            "traffic": _traffic("append_stress")}


def cpu_baseline(w, flops_full, hk_s=8):
    """The oracle (plain C, fp64 attention) on the step's workload: append of
    all 2048 K/V rows and the prefill of hk_s of the 8 KV heads (all of them
    by default: the whole step is a few seconds of CPU work); TFLOP/s over
    the sample's algorithmic flops."""
    import numpy as np
    import torch

    import oracle as O
    import workloads as W
    G = w.num_q_heads // w.num_kv_heads
    q = W.bf16_bits(w.q[:, : hk_s * G])
    k, v = W.bf16_bits(w.k), W.bf16_bits(w.v)
    slots = w.slot_mapping.cpu().numpy()
    P, ps, H, D = w.num_pages, w.page_size, w.num_kv_heads, w.head_dim
    threads = O._threads()
    t0 = time.perf_counter()
    c = [np.zeros((P, ps, H, D // 2), np.uint8), np.zeros((P, ps, H, D // 2), np.uint8),
         np.zeros((P, ps, H, D // 16), np.uint8), np.zeros((P, ps, H, D // 16), np.uint8)]
    O.append(k, v, slots, w.k_scale, w.v_scale, *c, ps, nthreads=threads)
    c = [np.ascontiguousarray(x[:, :, :hk_s]) for x in c]
    O.prefill(q, w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens, *c, w.k_scale, w.v_scale,
              hk_s * G, w.sm_scale, nthreads=threads)
    sec = time.perf_counter() - t0
    flops = flops_full * hk_s // w.num_kv_heads
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "seconds": round(sec, 3),
            "sample": f"append of all 2048 K/V rows + causal prefill of {hk_s} of 8 KV heads "
                      f"({hk_s * G} of 32 query heads), fp64 oracle"}


if __name__ == "__main__":
    main()
