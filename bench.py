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
divided by the step time).  Also reported:
  * roofline: the prefill kernel on that workload (the dominant kernel),
    launch duration from HIP events on the launch stream around replays of a
    graph of back-to-back launches, against the 0.40 target;
  * configs: every workload (the 2x128 small batch, the 2048x2048 prefill,
    the 1024x1024 uniform batch, the ragged chunked-prefill batch, the
    65,536-token append) with its prefill TFLOP/s and append GB/s and their
    fractions of the MI355X roofline, and the prefill kernel on equal-cost
    tiles (64 x 32 queries over 8192 keys: no causal imbalance);
  * schedule: the prefill of the two large batches under the three issue
    orders (heaviest first, stream order, request order), and of the
    2048x2048 batch heaviest first and paired (the plan's choice);
  * the decode step, the dequant-placement ablation, the measured achievable
    peaks, board power and shader clocks under the prefill and the MFMA-only
    loop (amd-smi), the plan's host time, and the CPU oracle timed on bounded
    samples.

Before the W warm-up steps the step runs untimed until the clocks have
settled (at least SETTLE_MS of back-to-back steps; reported as settle_steps):
the GPU needs ~30-40 ms of sustained work to leave its idle clocks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill TFLOP/s + append GB/s on NVFP4 paged KV (% of MI355X roofline)"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 (= f16) MFMA, TFLOP/s
SCHEDULE_NAMES = {1: "heaviest_first", 2: "stream_order", 3: "request_order", 4: "paired"}
PREFILL_TARGET_FRAC = 0.40  # of the MFMA peak, on the 2048x2048 prefill
APPEND_TARGET_FRAC = 0.70   # of HBM bandwidth, on the 65,536-token append
SETTLE_MS = 60.0
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


def tflops_row(flops, ms):
    t = flops / (ms * 1e-3) / 1e12
    return {"avg_launch_us": round(ms * 1e3, 2), "TFLOP_s": round(t, 1), "frac": round(t / BF16_PEAK_TFLOPS, 4)}


def gbs_row(nbytes, ms, key="avg_launch_us"):
    g = nbytes / (ms * 1e-3) / 1e9
    return {key: round(ms * 1e3, 2), "GB_s": round(g, 1), "frac": round(g / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload rows and the schedule comparison")
    ap.add_argument("--no-append-stress", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured achievable peaks (copy, MFMA-only loop)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the dequant-placement ablation of the prefill")
    ap.add_argument("--ablation-only", action="store_true",
                    help="only launch the prefill under the dequant placements (for counters)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (HBM-counter calibration)")
    ap.add_argument("--steady-only", action="store_true",
                    help="only launch the 2048x2048 prefill and the steady-state batch (for counters)")
    ap.add_argument("--steady-dequant-mode", type=int, default=None,
                    help="with --steady-only: the staging form of both prefills (default: the plan's, "
                         "3 = bf16; 0 = f16)")
    ap.add_argument("--power", action="store_true",
                    help="only sample board power and shader clocks (amd-smi) while the 2048x2048 "
                         "prefill and the MFMA-only loop with random operands run back to back")
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
    if args.power:
        print(json.dumps(power_telemetry(K, W, dev, torch, np)))
        return
    w = W.prefill_2k(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    qo_h, kvl_h = torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens)
    kvp_h = torch.from_numpy(w.kv_indptr)
    qo_d, kvl_d = qo_h.to(dev), kvl_h.to(dev)
    kvp_d, pt_d = kvp_h.to(dev), torch.from_numpy(w.page_table).to(dev)
    out = torch.empty_like(w.q)

    if args.steady_only:
        cache.append(w.k, w.v, w.slot_mapping)
        plan = K.plan(qo_h, kvl_h, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=kvp_h,
                      dequant_mode=args.steady_dequant_mode)
        for _ in range(60):
            K.paged_prefill_causal(w.q, qo_d, kvp_d, pt_d, kvl_d, cache, out, w.sm_scale, plan=plan)
        torch.cuda.synchronize()
        print(json.dumps({"steady_state": bench_steady(K, W, dev, torch, launches=12,
                                                       dequant_mode=args.steady_dequant_mode)}), flush=True)
        return
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

    # clock settling (untimed), then the W warm-up steps, then exactly K timed steps
    settle = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        for _ in range(50):
            step()
        settle += 50
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
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
    paired = plan.schedule == K.SCHEDULE_PAIRED
    kernel_name = (f"prefill_kernel<{w.head_dim},{G},{plan.block_q * G // 32},"
                   f"{'true' if 64 % w.page_size == 0 else 'false'},{plan.dequant_mode},"
                   f"{'true' if paired else 'false'}>")
    traffic = _traffic("prefill_2k")
    frac = pre_tflops / BF16_PEAK_TFLOPS
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": 1, "q_len": 2048, "kv_len": 2048,
                   "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "page_size": 16,
                   "kv_format": "nvfp4 (e2m1 + e4m3 per 16, fp32 global scale)",
                   "staging": "bf16 LDS tile, bf16 MFMA (dequant_mode 3; the f16 form, f16 staging + f16 "
                              "MFMA, is dequant_mode 0: configs.*.prefill_f16)",
                   "step": "append 2048 K/V rows + causal paged prefill",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": kernel_name, "schedule": SCHEDULE_NAMES[plan.schedule],
                     "achieved": round(pre_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(frac, 4),
                     "traffic": traffic, "flops_per_launch": flops,
                     "avg_launch_us": round(pre_ms * 1e3, 2),
                     "target_frac": PREFILL_TARGET_FRAC, "meets_target": bool(frac >= PREFILL_TARGET_FRAC)},
        "append": {"bound": "hbm", "bytes_per_launch": abytes, **gbs_row(abytes, app_ms)},
        "plan_host_us": round(plan_us, 2),
        "plan_bench": bench_plan(K, torch, np),
        "kernel_source_hash": kernel_source_hash(),
    }
    configs = {}
    if not args.no_configs:
        configs["small_2x128"] = bench_config_small(K, W, dev, torch)
    configs["prefill_2k"] = {"workload": w.name, "prefill": {"flops_per_launch": flops, **tflops_row(flops, pre_ms)},
                             "append": {"bytes_per_launch": abytes, **gbs_row(abytes, app_ms)}}
    if not args.no_configs:
        # the same prefill under heaviest-first and paired issue (bitwise the
        # same outputs), interleaved
        sched = {}
        for rep in range(2):
            for name, s in (("heaviest_first", K.SCHEDULE_HEAVIEST), ("paired", K.SCHEDULE_PAIRED)):
                p = K.plan(qo_h, kvl_h, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                           kv_indptr=kvp_h, schedule=s)
                ms = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, qo_d, kvp_d, pt_d, kvl_d, cache,
                                                                           out, w.sm_scale, plan=p))
                if rep == 1:
                    sched[name] = tflops_row(flops, ms)
        sched["paired_speedup"] = round(sched["heaviest_first"]["avg_launch_us"] / sched["paired"]["avg_launch_us"], 3)
        sched["plan_choice"] = SCHEDULE_NAMES[plan.schedule]
        configs["prefill_2k"]["schedule"] = sched
    del cache, out
    if not args.no_configs:
        configs["uniform_1024x1024"], result["schedule_uniform_1024x1024"] = bench_config_large(
            K, W.uniform_batch_1k(dev), torch)
        torch.cuda.empty_cache()
        configs["ragged_chunked_256"], result["schedule_ragged_chunked_256"] = bench_config_large(
            K, W.ragged_chunked(dev), torch, chunk_append=True)
        torch.cuda.empty_cache()
    if not args.no_append_stress:
        st = bench_append_stress(K, W, dev, torch, np)
        result["append_stress"] = st
        configs["append_stress_65536"] = {"workload": st["workload"], "append": {
            "bytes_per_launch": st["bytes_per_launch"], "cold_median_us": st["median_launch_us"],
            "cold_back_to_back_us": st["back_to_back_avg_us"], "frac": st["frac"],
            "frac_back_to_back": st["frac_back_to_back"]}}
    if not args.no_configs:
        configs["steady_state_64x32x8192"] = bench_steady(K, W, dev, torch)
    result["configs"] = configs
    if not args.no_decode:
        result["decode"] = bench_decode(K, W, dev, torch, np)
    if not args.no_ablation:
        w2 = W.prefill_2k(dev)
        c2 = K.PagedCache.empty(w2.num_pages, w2.page_size, w2.num_kv_heads, w2.head_dim, dev,
                                w2.k_scale, w2.v_scale)
        c2.append(w2.k, w2.v, w2.slot_mapping)
        result["dequant_ablation"] = bench_dequant_ablation(K, w2, c2, (qo_d, kvp_d, pt_d, kvl_d),
                                                            torch.empty_like(w2.q), torch)
        # the f16 form on this batch (paired 4-wave tiles, as the plan picks for it)
        configs["prefill_2k"]["prefill_f16"] = result["dequant_ablation"]["lds_once_per_tile"]
        del w2, c2
    if not args.no_achievable:
        ach = bench_achievable(K, W, dev, torch, np)
        ach["prefill_frac_of_mfma_loop"] = round(pre_tflops / ach["mfma_bf16_TFLOPs"], 4)
        ach["prefill_frac_of_mfma_loop_random_operands"] = round(
            pre_tflops / ach["mfma_bf16_random_operands_TFLOPs"], 4)
        if "append_stress" in result:
            got = result["append_stress"]["achieved_GBps"]
            ach["append_stress_frac_of_copy"] = round(got / ach["copy_GBps"], 4)
            ach["append_stress_frac_of_traffic_probe"] = round(got / ach["append_traffic_GBps"], 4)
        if "decode" in result and "decode_traffic_1_ahead_GBps" in ach:
            got = result["decode"]["achieved_GBps"]
            ach["decode_frac_of_traffic_probe"] = round(got / ach["decode_traffic_1_ahead_GBps"], 4)
        result["achievable"] = ach
        # board power and clocks under the prefill and the MFMA-only loop
        # (amd-smi; context for the roofline fraction, see --power)
        try:
            result["power"] = power_telemetry(K, W, dev, torch, np, secs=4.0)
        except Exception as e:  # amd-smi missing or unreadable: report, do not fail
            result["power"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, flops, W, dev, torch, np)
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


def _dev_arrays(w, dev, torch):
    return [torch.from_numpy(x).to(dev) for x in (w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens)]


def bench_config_small(K, W, dev, torch):
    """The 2 x 128 small batch (head_dim 64, 4/2 heads): launch-latency bound."""
    w = W.tiny(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    cache.append(w.k, w.v, w.slot_mapping)
    args = _dev_arrays(w, dev, torch)
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                  w.num_kv_heads, w.head_dim, w.page_size)
    out = torch.empty_like(w.q)
    pre = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=plan))
    plan0 = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                   w.num_kv_heads, w.head_dim, w.page_size, dequant_mode=0)
    pre0 = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=plan0))
    app = graph_launch_ms(torch, lambda: cache.append(w.k, w.v, w.slot_mapping))
    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    nbytes = append_bytes(int(w.kv_lens.sum()), w.num_kv_heads, w.head_dim)
    return {"workload": w.name, "prefill": {"flops_per_launch": flops, **tflops_row(flops, pre)},
            "prefill_f16": {"dequant_mode": 0, **tflops_row(flops, pre0)},
            "append": {"bytes_per_launch": nbytes, **gbs_row(nbytes, app)},
            "note": "a few microseconds of work: bound by launch latency, not by the roofline"}


def bench_steady(K, W, dev, torch, launches=0, dequant_mode=None):
    """The prefill kernel of the 2048x2048 batch (4-wave tiles, no KV split)
    on equal-cost tiles: 64 requests x 32 queries over 8192 keys, 512 tiles
    of 128 KV tiles each, two per CU, so neither causal imbalance nor the
    prologue weighs.  launches > 0: just that many launches (for counters)."""
    w = W.steady_state(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    cache.append(w.k, w.v, w.slot_mapping)
    args = _dev_arrays(w, dev, torch)
    out = torch.empty_like(w.q)
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr), tile_waves=4, split_len=-1,
                  dequant_mode=dequant_mode)
    fn = lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=plan)
    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    if launches:
        for _ in range(launches):
            fn()
        torch.cuda.synchronize()
        return {"workload": w.name, "launches": launches}
    ms = graph_launch_ms(torch, fn, per_graph=10, replays=5)
    return {"workload": w.name, "prefill": {"flops_per_launch": flops, "tiles": plan.num_tiles,
                                            "block_q": plan.block_q, **tflops_row(flops, ms)}}


def bench_config_large(K, w, torch, chunk_append=False):
    """A large batch: the append of its new rows and the prefill under the
    plan's own choices, then the prefill under each issue order (heaviest
    first over every stream, stream order, request order; bitwise the same
    results).  chunk_append: only the trailing q_len rows of each request
    are the step's new rows (the prefix is appended once, untimed)."""
    dev = w.q.device
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                               w.k_scale, w.v_scale)
    cache.append(w.k, w.v, w.slot_mapping)
    args = _dev_arrays(w, dev, torch)
    out = torch.empty_like(w.q)
    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    if chunk_append:
        import numpy as np
        rows = np.concatenate([np.arange(w.kv_token_indptr[r + 1] - w.q_lens[r], w.kv_token_indptr[r + 1])
                               for r in range(w.batch)])
        ri = torch.from_numpy(rows).to(dev)
        k, v, slots = w.k.index_select(0, ri), w.v.index_select(0, ri), w.slot_mapping.index_select(0, ri)
    else:
        k, v, slots = w.k, w.v, w.slot_mapping
    app = graph_launch_ms(torch, lambda: cache.append(k, v, slots), per_graph=5, replays=4)
    nbytes = append_bytes(k.shape[0], w.num_kv_heads, w.head_dim)

    def mk(schedule=0):
        return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size, schedule=schedule)

    plan = mk()
    pre = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=plan),
                          per_graph=4, replays=3)
    plan0 = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                   w.num_kv_heads, w.head_dim, w.page_size, dequant_mode=0)
    pre0 = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=plan0),
                           per_graph=4, replays=3)
    row = {"workload": w.name, "prefill": {"flops_per_launch": flops, "schedule": plan.schedule,
                                           "block_q": plan.block_q, "split_len": plan.split_len,
                                           **tflops_row(flops, pre)},
           "prefill_f16": {"dequant_mode": 0, **tflops_row(flops, pre0)},
           "append": {"bytes_per_launch": nbytes, "rows": int(k.shape[0]), **gbs_row(nbytes, app)}}
    sched = {}
    for name, s in (("heaviest_first", K.SCHEDULE_HEAVIEST), ("stream_order", K.SCHEDULE_STREAM),
                    ("request_order", K.SCHEDULE_REQUEST)):
        p = mk(s)
        ms = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale, plan=p),
                             per_graph=4, replays=3)
        sched[name] = tflops_row(flops, ms)
    base = sched["request_order"]["avg_launch_us"]
    for name in ("heaviest_first", "stream_order"):
        sched[name]["speedup_vs_request_order"] = round(base / sched[name]["avg_launch_us"], 3)
    sched["plan_choice"] = SCHEDULE_NAMES[plan.schedule]
    bits = K.read_device_error(dev)
    if bits:
        raise SystemExit(f"device error bits {bits} on {w.name}")
    return row, sched


def bench_dequant_ablation(K, w, cache, dev_args, out, torch, per_graph=50, replays=20):
    """The 2048x2048 prefill under the dequant placements of the PR #4769
    page's comparison (graph-timed launches; paired 4-wave tiles, as the plan
    picks): tiles decoded once per workgroup into f16 LDS, K decoded in
    registers inside the matrix loop, a byte-table decode (the three in f16,
    bitwise the same outputs), tiles decoded once into bf16 LDS with bf16
    matrix instructions (the kernel's own design, the plan's choice), and the
    native low-precision scores (K requantized to MXFP4, or MXFP8, while
    staged, Q in MXFP8, the scaled matrix instruction; looser accuracy
    contracts of their own)."""
    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    res = {}
    for mode, name in ((0, "lds_once_per_tile"), (1, "k_in_loop_registers"), (2, "lds_byte_table"),
                       (3, "lds_once_per_tile_bf16"), (4, "native_mx_scores_fp4_keys"),
                       (5, "native_mx_scores_fp8_keys")):
        plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                      tile_waves=4, dequant_mode=mode)
        ms = graph_launch_ms(torch, lambda: K.paged_prefill_causal(w.q, *dev_args, cache, out, w.sm_scale,
                                                                   plan=plan), per_graph, replays)
        res[name] = {"dequant_mode": mode, **tflops_row(flops, ms)}
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


def bench_decode(K, W, dev, torch, np, iters=12, per_graph=20, replays=3):
    """One decode step of 32 requests x 8192 cached keys (paged_decode, the
    plan's automatic chunking: both of its kernels), two ways like the append
    stress.  (1) Cold: median of 12 launches, each after the untimed
    cache-flush read and between its own pair of events.  (2) Back to back:
    `per_graph` steps captured into one graph, replayed between two events;
    each step reads the whole 302 MB cache, more than the Infinity Cache
    holds.  Bytes = the NVFP4 K and V codes and scales of every cached key
    (plus q and out)."""
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
    del flush
    b2b = graph_launch_ms(torch, lambda: K.paged_decode(w.q, *args, cache, out, w.sm_scale, plan),
                          per_graph=per_graph, replays=replays)
    bits = K.read_device_error(dev)
    if bits:
        raise SystemExit(f"device error bits {bits} in the decode")
    ms = float(np.median(times))
    nbytes = (int(w.kv_lens.sum()) * w.num_kv_heads * (w.head_dim // 2 + w.head_dim // 16) * 2
              + 2 * w.q.numel() * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    gbs2 = nbytes / (b2b * 1e-3) / 1e9
    return {"workload": w.name, "bound": "hbm", "bytes_per_launch": nbytes,
            "median_launch_us": round(ms * 1e3, 2), "achieved_GBps": round(gbs, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "back_to_back_avg_us": round(b2b * 1e3, 2), "back_to_back_GBps": round(gbs2, 1),
            "frac_back_to_back": round(gbs2 / HBM_PEAK_GBS, 4),
            "chunk_len": plan.chunk_len, "heads_per_wave": plan.heads_per_wave,
            "cache": "cold (flushed)", "traffic": _traffic("decode")}


def bench_achievable(K, W, dev, torch, np):
    """Measured achievable rates on this device.  Cold, like the append and
    decode figures (the 256 MB Infinity Cache flushed by an untimed 512 MiB
    read before every launch; median of 12 launches, HIP events on the launch
    stream): a 16-byte-per-lane copy of 128 MiB (read + write bytes / time),
    the 65,536-token append's own data movement without its arithmetic
    (peak.hip append_traffic: the same bf16 loads and the same code and
    scale stores through the same scattered slots; the append's algorithmic
    bytes / time), and the 32 x 8192 decode's reads without its arithmetic
    (peak.hip decode_traffic: the same waves, page lookups and per-lane
    loads, with one tile in flight as the decode has, and with two; the
    decode's algorithmic bytes / time).  Warm: the MFMA-only loop of peak.hip
    (dense v_mfma_f32_32x32x16_bf16, two waves per SIMD; median of 10), with
    smooth operands and with random operand bits (the part's clock depends
    on them)."""
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
    del a, cache

    w = W.decode_batch(dev)
    dcache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev,
                                w.k_scale, w.v_scale)
    dcache.append(w.k, w.v, w.slot_mapping)
    dplan = K.decode_plan(torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads, w.head_dim,
                          w.page_size)
    if w.head_dim == 128 and dplan.heads_per_wave == 2:
        kvp, pt, kvl = (torch.from_numpy(x).to(dev) for x in (w.kv_indptr, w.page_table, w.kv_lens))
        words = torch.empty(dplan.num_items * 64, dtype=torch.int32, device=dev)
        L.nvfp4kv_decode_traffic_probe.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                                   vp, ctypes.c_int, vp]
        dbytes = (int(w.kv_lens.sum()) * w.num_kv_heads * (w.head_dim // 2 + w.head_dim // 16) * 2
                  + 2 * w.q.numel() * 2)
        for ahead in (1, 2):
            t = timed(lambda: check(L.nvfp4kv_decode_traffic_probe(
                vp(kvp.data_ptr()), vp(pt.data_ptr()), vp(kvl.data_ptr()), dplan.num_items, w.num_kv_heads,
                w.page_size, w.num_pages, dplan.chunk_len, dplan.max_chunks,
                *(vp(c.data_ptr()) for c in (dcache.k_cache, dcache.v_cache, dcache.k_sf, dcache.v_sf)),
                vp(words.data_ptr()), ahead, stream), "decode traffic"), n=12, cold=True)
            out[f"decode_traffic_{ahead}_ahead_GBps"] = round(dbytes / t / 1e9, 1)
        del kvp, pt, kvl, words
    del w, dcache, flush

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
    L.nvfp4kv_mfma_random_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def mfma_random():
        if L.nvfp4kv_mfma_random_peak_probe(blocks, iters, ctypes.c_void_p(buf.data_ptr()), stream) != 0:
            raise SystemExit("MFMA peak probe launch failed")

    out["mfma_bf16_random_operands_TFLOPs"] = round(
        L.nvfp4kv_mfma_peak_probe_flops(blocks, iters) / timed(mfma_random) / 1e12, 1)
    return out


def power_telemetry(K, W, dev, torch, np, secs=6.0, period=0.3):
    """Board power and shader clocks while the 2048x2048 prefill (the plan's
    kernel, back to back) and then the MFMA-only loop of peak.hip with random
    operand bits run for `secs` seconds each: `amd-smi metric -p -c` sampled
    every `period` seconds from a thread; per phase the median socket power
    and the median over samples of the lowest and highest of the reported
    gfx clocks, the first second of each phase dropped (the readings lag)."""
    import ctypes
    import re
    import subprocess
    import threading
    from nvfp4_paged_kv_amd.build import PEAK_LIB
    samples, phase, done = [], ["idle"], threading.Event()

    def poll():
        while not done.is_set():
            t = time.time()
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
            except (OSError, subprocess.SubprocessError):
                done.wait(period)
                continue
            p = re.search(r'"socket_power":\s*\{\s*"value":\s*(\d+)', r.stdout)
            clk = [int(x) for x in re.findall(r'"gfx_\d+":\s*\{\s*"clk":\s*\{\s*"value":\s*(\d+)', r.stdout)]
            if p and clk:
                samples.append((phase[0], t, int(p.group(1)), min(clk), max(clk)))
            done.wait(period)

    w = W.prefill_2k(dev)
    cache = K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, dev, w.k_scale, w.v_scale)
    cache.append(w.k, w.v, w.slot_mapping)
    args = _dev_arrays(w, dev, torch)
    out = torch.empty_like(w.q)
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size)
    L = ctypes.CDLL(PEAK_LIB)
    L.nvfp4kv_mfma_random_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = 256 * 4, 2000
    buf = torch.empty(blocks * 512, dtype=torch.float32, device=dev)

    def mfma():
        if L.nvfp4kv_mfma_random_peak_probe(blocks, iters, ctypes.c_void_p(buf.data_ptr()), stream) != 0:
            raise SystemExit("MFMA peak probe launch failed")

    flops = attention_flops(w.q_lens, w.kv_lens, w.num_q_heads, w.head_dim)
    th = threading.Thread(target=poll, daemon=True)
    th.start()
    time.sleep(1.5)
    res = {"sampler": "amd-smi metric -p -c --json", "period_s": period}
    for name, fn in (("prefill_2048x2048", lambda: K.paged_prefill_causal(w.q, *args, cache, out, w.sm_scale,
                                                                            plan=plan)),
                     ("mfma_loop_random_operands", mfma)):
        phase[0] = name
        t0, n = time.time(), 0
        while time.time() - t0 < secs:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            n += 20
        res[name] = {"launches": n, "avg_launch_us": round((time.time() - t0) / n * 1e6, 2), "t0": t0}
        phase[0] = "idle"
        time.sleep(1.5)
    done.set()
    th.join()
    res["prefill_2048x2048"]["TFLOP_s"] = round(flops / (res["prefill_2048x2048"]["avg_launch_us"] * 1e-6) / 1e12, 1)
    for name in ("prefill_2048x2048", "mfma_loop_random_operands"):
        r = res[name]
        t_start = r.pop("t0")
        sel = [s for s in samples if s[0] == name and s[1] > t_start + 1.0]
        r["samples"] = len(sel)
        if sel:
            r["socket_power_W"] = float(np.median([s[2] for s in sel]))
            r["gfx_clk_MHz_low"] = float(np.median([s[3] for s in sel]))
            r["gfx_clk_MHz_high"] = float(np.median([s[4] for s in sel]))
    idle = [s[2] for s in samples if s[0] == "idle"]
    res["idle_socket_power_W"] = float(np.min(idle)) if idle else None
    return res


def bench_append_stress(K, W, dev, torch, np, iters=12, sets=4, rounds=3, replays=2):
    """65,536-token append (Student-t(3) values, scattered slots), cold, two
    ways.  (1) The 256 MB Infinity Cache is flushed before every timed launch
    by reading a 512 MiB buffer (untimed; a read leaves no dirty lines to
    write back during the timed launch); median of 12 launches, each between
    its own pair of HIP events (the pair adds a few microseconds).  (2) Back
    to back without per-launch events: `sets` copies of the K/V input (256 MB
    each) appended in rotation, `sets` x `rounds` launches captured into one
    graph and replayed between two events, so that every launch reads inputs
    untouched for the last sets-1 launches (768 MB of other traffic, more
    than the Infinity Cache holds)."""
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
    del flush
    ms = float(np.median(times))
    inputs = [(a.k, a.v)] + [(a.k.clone(), a.v.clone()) for _ in range(sets - 1)]
    rot = [0]

    def one():
        k, v = inputs[rot[0] % sets]
        rot[0] += 1
        cache.append(k, v, a.slot_mapping)

    b2b = graph_launch_ms(torch, one, per_graph=sets * rounds, replays=replays)
    bits = K.read_device_error(dev)
    if bits:
        raise SystemExit(f"device error bits {bits} in the append")
    nbytes = append_bytes(a.k.shape[0], a.num_kv_heads, a.head_dim)
    gbs = nbytes / (ms * 1e-3) / 1e9
    gbs2 = nbytes / (b2b * 1e-3) / 1e9
    return {"workload": a.name, "bound": "hbm", "bytes_per_launch": nbytes,
            "median_launch_us": round(ms * 1e3, 2), "achieved_GBps": round(gbs, 1),
            "peak_GBps": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4), "cache": "cold (flushed)",
            "back_to_back_avg_us": round(b2b * 1e3, 2), "back_to_back_GBps": round(gbs2, 1),
            "frac_back_to_back": round(gbs2 / HBM_PEAK_GBS, 4),
            "target_frac": APPEND_TARGET_FRAC, "meets_target": bool(gbs / HBM_PEAK_GBS >= APPEND_TARGET_FRAC),
            "traffic": _traffic("append_stress")}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _host_requests(w, reqs, W, np):
    """Host copies of the requests `reqs` of workload w as a compact batch
    (own page pool, pages in order), for the oracle."""
    import torch
    reqs = list(reqs)
    ps = w.page_size
    q_lens, kv_lens = w.q_lens[reqs], w.kv_lens[reqs]
    npg = (kv_lens + ps - 1) // ps
    kvp = np.zeros(len(reqs) + 1, np.int32)
    kvp[1:] = np.cumsum(npg)
    pt = np.arange(kvp[-1], dtype=np.int32)
    qo = np.zeros(len(reqs) + 1, np.int32)
    qo[1:] = np.cumsum(q_lens)
    qr = np.concatenate([np.arange(w.qo_indptr[r], w.qo_indptr[r + 1]) for r in reqs])
    kr = np.concatenate([np.arange(w.kv_token_indptr[r], w.kv_token_indptr[r + 1]) for r in reqs])
    slots = np.concatenate([pt[kvp[i] + np.arange(kv_lens[i]) // ps] * ps + np.arange(kv_lens[i]) % ps
                            for i in range(len(reqs))]).astype(np.int64)
    qi, ki = torch.from_numpy(qr).to(w.q.device), torch.from_numpy(kr).to(w.k.device)
    return dict(q=W.bf16_bits(w.q.index_select(0, qi)), k=W.bf16_bits(w.k.index_select(0, ki)),
                v=W.bf16_bits(w.v.index_select(0, ki)), qo=qo, kvp=kvp, pt=pt,
                kvl=kv_lens.astype(np.int32), slots=slots, P=int(kvp[-1]))


def _oracle_sample(O, w, reqs, W, np, threads, hk_s=None):
    """Oracle append + prefill of the requests `reqs` (KV heads [0, hk_s));
    returns (seconds, sampled flops, sampled (request, query head) pairs)."""
    s = _host_requests(w, reqs, W, np)
    H, D, ps = w.num_kv_heads, w.head_dim, w.page_size
    G = w.num_q_heads // H
    hk_s = hk_s or H
    t0 = time.perf_counter()
    c = [np.zeros((s["P"], ps, H, D // 2), np.uint8), np.zeros((s["P"], ps, H, D // 2), np.uint8),
         np.zeros((s["P"], ps, H, D // 16), np.uint8), np.zeros((s["P"], ps, H, D // 16), np.uint8)]
    O.append(s["k"], s["v"], s["slots"], w.k_scale, w.v_scale, *c, ps, nthreads=threads)
    c = [np.ascontiguousarray(x[:, :, :hk_s]) for x in c]
    q = np.ascontiguousarray(s["q"][:, : hk_s * G])
    O.prefill(q, s["qo"], s["kvp"], s["pt"], s["kvl"], *c, w.k_scale, w.v_scale, hk_s * G, w.sm_scale,
              nthreads=threads)
    sec = time.perf_counter() - t0
    flops = attention_flops(w.q_lens[list(reqs)], w.kv_lens[list(reqs)], hk_s * G, D)
    return sec, flops, len(list(reqs)) * hk_s * G


def cpu_baseline(w, flops_full, W, dev, torch, np, hk_s=8):
    """The oracle (plain C, fp64 attention), timed on this host's cores with
    the oracle's own thread count (capped at 16, this GPU's share of the
    host):
      value: the 2048x2048 step (append of all 2048 K/V rows + the prefill
        of hk_s of the 8 KV heads), TFLOP/s over the sample's flops;
      append_stress: the full 65,536-token append, GB/s over its bytes;
      uniform_1024x1024 / ragged_chunked_256: sampled requests, all heads and
        rows (16 seeded requests; the 8 longest, 8 shortest and 16 random
        requests), reported as a measured rate per (request, query head) pair
        and per flop, and an extrapolation of that flop rate to the whole
        batch (labelled as such)."""
    import oracle as O
    threads = O._threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    G = w.num_q_heads // w.num_kv_heads
    sec, flops, _ = _oracle_sample(O, w, [0], W, np, threads, hk_s)
    res = {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle", "seconds": round(sec, 3),
           "sample": f"append of all 2048 K/V rows + causal prefill of {hk_s} of 8 KV heads "
                     f"({hk_s * G} of 32 query heads), fp64 oracle",
           "host": {"cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
                    "threads_used": threads,
                    "thread_cap": "min(os.cpu_count(), 16): 16 host threads per GPU"}}
    a = W.append_stress(dev)
    P, ps, H, D = a.num_pages, a.page_size, a.num_kv_heads, a.head_dim
    k, v, slots = W.bf16_bits(a.k), W.bf16_bits(a.v), a.slot_mapping.cpu().numpy()
    c = [np.zeros((P, ps, H, D // 2), np.uint8), np.zeros((P, ps, H, D // 2), np.uint8),
         np.zeros((P, ps, H, D // 16), np.uint8), np.zeros((P, ps, H, D // 16), np.uint8)]
    t0 = time.perf_counter()
    O.append(k, v, slots, a.k_scale, a.v_scale, *c, ps, nthreads=threads)
    asec = time.perf_counter() - t0
    nbytes = append_bytes(a.k.shape[0], H, D)
    res["append_stress"] = {"seconds": round(asec, 3), "GB_s": round(nbytes / asec / 1e9, 3),
                            "sample": "the whole 65,536-token append"}
    del a, k, v, c
    for name, mkw, pick in (
            ("uniform_1024x1024", W.uniform_batch_1k,
             lambda wl: np.random.default_rng(7).choice(wl.batch, 16, replace=False)),
            ("ragged_chunked_256", W.ragged_chunked,
             lambda wl: _ragged_pick(wl, np))):
        wl = mkw(dev)
        reqs = [int(r) for r in pick(wl)]
        sec, flops, pairs = _oracle_sample(O, wl, reqs, W, np, threads)
        full = attention_flops(wl.q_lens, wl.kv_lens, wl.num_q_heads, wl.head_dim)
        rate = flops / sec
        res[name] = {"seconds": round(sec, 3), "sampled_requests": len(reqs),
                     "sampled_request_head_pairs": pairs, "sampled_flops": flops,
                     "TFLOP_s": round(rate / 1e12, 6),
                     "seconds_per_request_head_pair": round(sec / pairs, 5),
                     "extrapolated_full_batch_seconds": round(full / rate, 1),
                     "extrapolation": "the sample's measured flop rate applied to the whole batch's "
                                      f"{full} flops (not measured)"}
        del wl
        torch.cuda.empty_cache()
    return res


def _ragged_pick(w, np):
    order = np.argsort(w.kv_lens, kind="stable")
    rest = np.setdiff1d(np.arange(w.batch), np.concatenate([order[:8], order[-8:]]))
    return np.concatenate([order[-8:], order[:8], np.random.default_rng(3).choice(rest, 16, replace=False)])


if __name__ == "__main__":
    main()
