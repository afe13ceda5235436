"""GPU parity of the causal paged prefill against the fp64 oracle, within
|err| <= 1e-2 + 1e-2 |ref| per element: full outputs on the small and the
2048x2048 workloads and on ragged batches covering every (head_dim, GQA
group) kernel; sampled requests on the 1024x1024 batch and the ragged
chunked-prefill batch at full size; scheduling-order independence (bitwise);
page-id range errors; no host synchronization."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, banner, force_tile_waves, oracle_outputs, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _check(K, O, w, reqs=None, **kw):
    out, cache, plan = run_gpu(K, w, **kw)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(O, w, reqs)
    got = out.index_select(0, torch.from_numpy(rows).cuda())
    return assert_close(got, ref, w.name), out, plan


def test_prefill_tiny_full(K, oracle):
    banner("prefill tiny")
    e, _, _ = _check(K, oracle, W.tiny("cuda"))
    print(f"max err {e:.3g}")


@pytest.mark.parametrize("hq,hk,d", [(32, 8, 128), (16, 8, 128), (8, 8, 128), (64, 8, 128),
                                     (8, 4, 64), (4, 2, 64), (2, 2, 64), (16, 2, 64)])
def test_prefill_ragged_small_all_kernels(K, oracle, hq, hk, d):
    banner(f"prefill ragged small hq={hq} hk={hk} d={d}")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    w = W.make_attention(f"ragged_small_{hq}_{hk}_{d}", q, kv, hq, hk, d, 16, 120, seed=11,
                         device="cuda", scales="lognormal", lognormal=(-3.0, 0.5))
    _check(K, oracle, w)


@pytest.mark.parametrize("ps,d,waves", [(1, 128, 4), (8, 64, 4), (32, 128, 8), (64, 128, 4),
                                         (5, 128, 4), (48, 64, 4), (128, 128, 8), (100, 128, 4)])
def test_prefill_page_sizes(K, oracle, ps, d, waves):
    """Page sizes that divide the 64-key tile (a key keeps its page slot and
    row in every tile) and page sizes that do not (a tile spans part of a
    page, or crosses page boundaries at varying rows), both tile widths."""
    banner(f"prefill page size {ps}, head_dim {d}, {waves}-wave tiles")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    pool = sum((k + ps - 1) // ps for k in kv) + 9
    w = W.make_attention(f"page_size_{ps}_{d}", q, kv, 16, 4, d, ps, pool, seed=18, device="cuda",
                         scales="amax")
    _check(K, oracle, w, plan=force_tile_waves(K, w, waves if d == 128 else 4))


@pytest.mark.parametrize("hq,hk", [(32, 8), (16, 8), (8, 8), (64, 8)])
def test_prefill_ragged_small_wide_tiles(K, oracle, hq, hk):
    """The 8-wave (256-row) head_dim-128 kernels on the small ragged batch
    (the plan picks 4-wave tiles for small batches)."""
    banner(f"prefill ragged small, 8-wave tiles, hq={hq} hk={hk}")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    w = W.make_attention(f"ragged_small_wide_{hq}_{hk}", q, kv, hq, hk, 128, 16, 120, seed=14,
                         device="cuda", scales="amax")
    _check(K, oracle, w, plan=force_tile_waves(K, w, 8))


@pytest.mark.parametrize("split_len,waves", [(1, 4), (2, 4), (3, 8), (7, 4), (1, 8), (5, 8)])
def test_prefill_split_kv_chunks(K, oracle, split_len, waves):
    """Q tiles whose KV range is cut into chunks merged by the last one to
    finish (forced chunk lengths, including 1-tile chunks where some rows see
    no key of a chunk), for both tile widths."""
    banner(f"prefill split KV, chunk length {split_len}, {waves}-wave tiles")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    w = W.make_attention(f"split_{split_len}_{waves}", q, kv, 32, 8, 128, 16, 120, seed=15,
                         device="cuda", scales="amax")
    plan = force_tile_waves(K, w, waves, split_len=split_len)
    assert plan.num_split_tiles > 0
    _check(K, oracle, w, plan=plan)
    _check(K, oracle, w, plan=plan)  # the counters were left at zero


def test_prefill_split_kv_head_dim_64(K, oracle):
    banner("prefill split KV, head_dim 64")
    w = W.make_attention("split_d64", [200, 64, 129], [333, 700, 130], 16, 2, 64, 16, 120, seed=16,
                         device="cuda", scales="amax")
    plan = force_tile_waves(K, w, 4, split_len=2)
    assert plan.num_split_tiles > 0
    _check(K, oracle, w, plan=plan)


def test_prefill_auto_split_short_chunk_long_cache(K, oracle):
    """A 512-token chunk over an 8192-token cache: too few Q tiles for the
    GPU, so the plan splits their KV ranges by itself."""
    banner("prefill 512 over 8192 (automatic split)")
    w = W.make_attention("chunk_512_8192", [512], [8192], 32, 8, 128, 16, 520, seed=17, device="cuda",
                         scales="amax")
    e, out, plan = _check(K, oracle, w)
    assert plan.split_len > 0 and plan.max_chunks > 1
    print(f"max err {e:.3g}")


def test_prefill_uniform_small_batch(K, oracle):
    banner("prefill uniform small batch")
    w = W.make_attention("uniform_small", [96] * 5, [160] * 5, 32, 8, 128, 16, 64, seed=12,
                         device="cuda", scales="amax")
    e, out, plan = _check(K, oracle, w)
    assert plan.uniform_q == 1
    e8, out8, plan8 = _check(K, oracle, w, plan=force_tile_waves(K, w, 8))


def test_prefill_2k_full(K, oracle):
    banner("prefill 1x2048 full")
    w = W.prefill_2k("cuda")
    e, out, plan = _check(K, oracle, w)
    assert plan.block_q == 32 and plan.split_len == 0  # 512 4-wave tiles fill the GPU
    assert plan.schedule == K.SCHEDULE_PAIRED and plan.dequant_mode == 3
    print(f"max err {e:.3g}")
    # heaviest first (one 4-wave tile per workgroup): the same bits
    heavy = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                   kv_indptr=torch.from_numpy(w.kv_indptr), schedule=K.SCHEDULE_HEAVIEST)
    o2, _, _ = run_gpu(K, w, plan=heavy)
    torch.cuda.synchronize()
    assert torch.equal(o2, out)


def test_prefill_uniform_1k_sampled(K, oracle):
    banner("prefill 1024x1024 uniform, 16 sampled requests")
    w = W.uniform_batch_1k("cuda")
    reqs = np.random.default_rng(2).choice(w.batch, 16, replace=False)
    e, out, plan = _check(K, oracle, w, reqs=reqs)
    assert plan.uniform_q == 1 and plan.head_first == 0
    print(f"max err {e:.3g}")


def test_prefill_ragged_chunked_sampled(K, oracle):
    banner("prefill ragged chunked 256 requests, 32 sampled")
    w = W.ragged_chunked("cuda")
    order = np.argsort(w.kv_lens, kind="stable")
    rest = np.setdiff1d(np.arange(w.batch), np.concatenate([order[:8], order[-8:]]))
    reqs = np.concatenate([order[-8:], order[:8], np.random.default_rng(3).choice(rest, 16, replace=False)])
    e, out, plan = _check(K, oracle, w, reqs=reqs)
    assert plan.uniform_q == 0
    print(f"max err {e:.3g}")


@pytest.mark.parametrize("seed", range(24))
def test_prefill_random_shapes(K, oracle, seed):
    """Seeded random batches against the oracle: 1-6 requests of 1-600 keys
    with 0..kv_len queries each, 1/2/3/4/8 KV heads, GQA group 1/2/4/8,
    head_dim 64/128, page sizes that do and do not divide a tile, 4- or
    8-wave tiles (head_dim 128), no / automatic / forced KV splits, f16 or
    bf16 staging."""
    r = np.random.default_rng(2000 + seed)
    B = int(r.integers(1, 7))
    hk = int(r.choice([1, 2, 3, 4, 8]))
    g = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    ps = int(r.choice([1, 5, 16, 32, 64]))
    waves = int(r.choice([4, 8])) if d == 128 else 4
    split = int(r.choice([-1, 0, 2, 3]))
    mode = int(r.choice([0, 3]))
    kv = [int(x) for x in r.integers(1, 601, B)]
    q = [int(r.integers(0, k + 1)) if r.random() < 0.8 else k for k in kv]
    if sum(q) == 0:
        q[0] = kv[0]
    pool = sum((k + ps - 1) // ps for k in kv) + 3
    banner(f"prefill random shape {seed}: hk={hk} G={g} d={d} page={ps} waves={waves} split={split} "
           f"mode={mode} q={q} kv={kv}")
    w = W.make_attention(f"prefill_rand_{seed}", q, kv, hk * g, hk, d, ps, pool, seed=80 + seed,
                         device="cuda", scales="amax")
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr), split_len=split,
                  tile_waves=waves, dequant_mode=mode)
    e, _, plan = _check(K, oracle, w, plan=plan)
    print(f"max err {e:.3g}; tiles {plan.num_tiles}, split {plan.split_len}, chunks {plan.max_chunks}")


@pytest.mark.parametrize("mode,split,waves", [(3, -1, 4), (3, 2, 4), (0, 0, 8), (3, -1, 8)])
def test_prefill_empty_requests(K, oracle, mode, split, waves):
    """Requests without queries, with and without cached keys, between
    ordinary ones (a non-uniform batch: the device work list), with no,
    forced and automatic KV splits, both staging forms and both tile widths:
    the empty requests own no output rows and every other row matches the
    oracle."""
    q = [0, 37, 0, 100, 0, 1, 0]
    kv = [0, 200, 50, 100, 0, 64, 0]
    banner(f"prefill empty requests mode={mode} split={split} waves={waves}")
    w = W.make_attention(f"prefill_empty_{mode}_{split}_{waves}", q, kv, 32, 8, 128, 16, 40, seed=51,
                         device="cuda", scales="amax")
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr), split_len=split,
                  tile_waves=waves, dequant_mode=mode)
    assert plan.uniform_q == 0 and plan.total_q == sum(q)
    e, _, plan = _check(K, oracle, w, plan=plan)
    print(f"max err {e:.3g}; split {plan.split_len}")


def test_prefill_without_queries_launches_nothing(K):
    """A batch with no query rows -- every request empty (one of them with
    cached keys), or no request at all -- plans no tile, launches nothing and
    leaves the device error word clear."""
    for q, kv in (([0, 0, 0], [0, 30, 0]), ([], [])):
        banner(f"prefill without queries q={q} kv={kv}")
        w = W.make_attention("prefill_noq", q, kv, 8, 2, 64, 16, 4, seed=52, device="cuda")
        out, _, plan = run_gpu(K, w)
        torch.cuda.synchronize()
        assert plan.num_tiles == 0 and out.numel() == 0
        assert K.read_device_error("cuda") == 0


def test_schedule_orders_give_identical_bits(K):
    """Uniform O(1) decode and the device work list, each in the three issue
    orders (heaviest first, stream order, request order), and split Q tiles
    in heaviest-first and request order, compute every tile the same way:
    outputs are bitwise identical."""
    banner("schedule order independence")
    w = W.make_attention("order", [256] * 6, [300] * 6, 32, 8, 128, 16, 200, seed=13, device="cuda",
                         scales="amax")

    def mk(**kw):
        return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16, **kw)

    base, cache, plan = run_gpu(K, w, plan=mk(split_len=-1))
    runs = 0
    for uq in (1, 0):
        for order in (K.SCHEDULE_HEAVIEST, K.SCHEDULE_STREAM, K.SCHEDULE_REQUEST):
            p2 = mk(split_len=-1, schedule=order)
            if not uq:
                p2.struct.uniform_q = 0
                p2.struct.workspace_bytes = ((p2.struct.num_items * 16 + 255) // 256) * 256
            o, _, _ = run_gpu(K, w, cache=cache, plan=p2)
            assert torch.equal(o, base), (uq, order)
            runs += 1
    split = [run_gpu(K, w, cache=cache, plan=mk(split_len=2, schedule=order))[0]
             for order in (K.SCHEDULE_HEAVIEST, K.SCHEDULE_REQUEST)]
    assert torch.equal(split[0], split[1])
    with pytest.raises(K.NVFP4KVError, match="unsupported"):
        run_gpu(K, w, cache=cache, plan=mk(split_len=2, schedule=K.SCHEDULE_STREAM))
    assert runs == 6


def test_stream_ordered_work_list_layout(K):
    """The work list of a ragged batch whose KV is taken not to fit in L2:
    every (request, Q tile, KV head) item exactly once; position p holds a
    stream of head h only when p % 8 == h % 8 (workgroup p runs on XCD p % 8);
    a stream's items are consecutive in its XCD's sequence, heaviest tile
    first; requests appear in non-increasing total cost."""
    banner("stream-ordered work list layout")
    q_lens = [37, 512, 1, 200, 64, 300, 129, 5]
    kv_lens = [900, 3000, 40, 200, 2500, 1700, 129, 4000]
    w = W.make_attention("wl", q_lens, kv_lens, 32, 8, 128, 16, 800, seed=17, device="cuda",
                         scales="amax")
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                  split_len=-1, tile_waves=8, schedule=K.SCHEDULE_STREAM)
    out, cache, plan = run_gpu(K, w, plan=plan)
    torch.cuda.synchronize()
    n = plan.num_items
    lst = plan.workspace("cuda")[: n * 16].view(torch.int32).view(n, 4).cpu().numpy()
    bq, hk = plan.block_q, 8

    def cost(r, t):
        lq, off = int(w.q_lens[r]), int(w.kv_lens[r] - w.q_lens[r])
        return (off + min((t + 1) * bq, lq) - 1) // 64 + 1

    seen = set()
    for p, (r, y, z, sp) in enumerate(lst):
        t, h = divmod(int(y), hk)
        assert sp == -1 and z == cost(r, t)
        assert p % 8 == h % 8
        seen.add((int(r), t, h))
    expect = {(r, t, h) for r in range(w.batch) for t in range(-(-int(w.q_lens[r]) // bq)) for h in range(hk)}
    assert seen == expect and len(seen) == n
    totals = []
    for x in range(8):
        seq = lst[x::8]
        run = []
        for r, y, _, _ in seq:
            t, h = divmod(int(y), hk)
            if run and run[-1][0] == (r, h):
                assert t == run[-1][1] - 1  # consecutive, heaviest first
                run[-1][1] = t
            else:
                assert not any(k == (r, h) for k, _ in run)  # a stream appears once
                assert t == -(-int(w.q_lens[r]) // bq) - 1
                run.append([(r, h), t])
        if x == 0:
            totals = [sum(cost(r, t) for t in range(-(-int(w.q_lens[r]) // bq))) for (r, h), _ in run]
    assert all(a >= b for a, b in zip(totals, totals[1:]))


def test_page_id_out_of_range_sets_flag(K):
    w = W.tiny("cuda")
    out, cache, plan = run_gpu(K, w)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    pt = torch.from_numpy(w.page_table).cuda()
    pt[3] = w.num_pages + 5
    K.paged_prefill_causal(w.q, torch.from_numpy(w.qo_indptr).cuda(), torch.from_numpy(w.kv_indptr).cuda(),
                           pt, torch.from_numpy(w.kv_lens).cuda(), cache, out, w.sm_scale, plan=plan)
    assert K.read_device_error("cuda") == K.DEV_PAGE_OOB


def test_prefill_does_not_synchronize(K):
    w = W.tiny("cuda")
    out, cache, plan = run_gpu(K, w)
    args = (torch.from_numpy(w.qo_indptr).cuda(), torch.from_numpy(w.kv_indptr).cuda(),
            torch.from_numpy(w.page_table).cuda(), torch.from_numpy(w.kv_lens).cuda())
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    K.paged_prefill_causal(w.q, *args[:3], args[3], cache, out, w.sm_scale, plan=plan)
    assert not torch.cuda.current_stream().query()
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [1, 2])
def test_prefill_dequant_ablation_modes(K, oracle, mode):
    """The dequant-placement ablation kernels (K decoded in registers inside
    the matrix loop; byte-table decode) stage the same f16 values, so their
    outputs equal the f16 form's (mode 0) bit for bit; and the oracle parity."""
    banner(f"prefill dequant ablation mode {mode}")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    w = W.make_attention(f"dequant_mode_{mode}", q, kv, 32, 8, 128, 16, 120, seed=19, device="cuda",
                         scales="amax")
    f16 = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                 kv_indptr=torch.from_numpy(w.kv_indptr), split_len=-1, tile_waves=4, dequant_mode=0)
    base, cache, _ = run_gpu(K, w, plan=f16)
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                  kv_indptr=torch.from_numpy(w.kv_indptr), split_len=-1, tile_waves=4,
                  dequant_mode=mode)
    out, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))
    ref, rows = oracle_outputs(oracle, w)
    assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)


def test_prefill_bf16_staging_mode(K, oracle):
    """The bf16 variant of the kernel (bf16 staging tile, queries and
    probabilities, bf16 matrix instructions) against the oracle."""
    banner("prefill bf16 staging (dequant mode 3)")
    q = [1, 37, 200, 64, 3, 129]
    kv = [1, 37, 333, 700, 3, 130]
    w = W.make_attention("dequant_mode_3", q, kv, 32, 8, 128, 16, 120, seed=19, device="cuda",
                         scales="amax")
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16,
                  kv_indptr=torch.from_numpy(w.kv_indptr), split_len=2, tile_waves=4,
                  dequant_mode=3)
    assert plan.num_split_tiles > 0
    out, _, _ = run_gpu(K, w, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(oracle, w)
    assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)


@pytest.mark.parametrize("mode", [1, 2, 4, 5, 6])
def test_prefill_dequant_ablation_unsupported_shape(K, mode):
    """The in-loop and byte-table ablation kernels and the MX score kernels
    exist for head_dim 128, GQA group 4, 4-wave tiles only (the bf16 form,
    mode 3, for every shape), and modes above 5 not at all: other requests
    are refused before any launch."""
    w = W.make_attention("dequant_mode_d64", [64], [64], 8, 2, 64, 16, 8, seed=20, device="cuda")
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 8, 2, 64, 16,
                  dequant_mode=mode)
    with pytest.raises(K.NVFP4KVError, match="unsupported"):
        run_gpu(K, w, plan=plan)
    if mode == 6:  # not a mode even on the supported shape
        w2 = W.make_attention("dequant_mode_6", [64], [64], 32, 8, 128, 16, 8, seed=20, device="cuda")
        plan2 = K.plan(torch.from_numpy(w2.qo_indptr), torch.from_numpy(w2.kv_lens), 32, 8, 128, 16,
                       tile_waves=4, dequant_mode=mode)
        with pytest.raises(K.NVFP4KVError, match="unsupported"):
            run_gpu(K, w2, plan=plan2)


# Paired issue order: uniform batches whose Q tiles t and QT - 1 - t share one
# 8-wave workgroup (the light tile's waves stage every KV tile).  Shapes: both
# head dims, every GQA group, an odd Q tile count (the middle tile alone), a
# single Q tile (no light tile), page sizes dividing the KV tile and not,
# the bf16 form, and the ablation and MX score modes.
PAIRED_CASES = [
    ("g4_d128", [256] * 3, [300] * 3, 32, 8, 128, 16, 0),
    ("g4_d128_odd_tiles", [160] * 2, [400] * 2, 32, 8, 128, 16, 0),
    ("g4_d128_one_tile", [20] * 3, [90] * 3, 32, 8, 128, 16, 0),
    ("g1_d128_ps5", [200] * 2, [333] * 2, 8, 8, 128, 5, 0),
    ("g2_d128_bf16", [100] * 3, [100, 300, 700], 16, 8, 128, 16, 3),
    ("g8_d128_ps32", [64] * 2, [64, 1000], 64, 8, 128, 32, 0),
    ("g4_d64", [300] * 2, [300, 450], 16, 4, 64, 16, 0),
    ("g8_d64_ps48_bf16", [77] * 3, [77, 500, 1200], 16, 2, 64, 48, 3),
    ("g4_d128_mode1", [200] * 2, [260] * 2, 32, 8, 128, 16, 1),
    ("g4_d128_mode2", [200] * 2, [260] * 2, 32, 8, 128, 16, 2),
    ("g4_d128_mode4", [200] * 2, [260] * 2, 32, 8, 128, 16, 4),
    ("g4_d128_mode5", [200] * 2, [260] * 2, 32, 8, 128, 16, 5),
]


@pytest.mark.parametrize("case", PAIRED_CASES, ids=[c[0] for c in PAIRED_CASES])
def test_paired_order(K, oracle, case):
    """Paired issue computes every row as heaviest-first issue does: bitwise
    the same outputs; and (modes 0-3) the oracle parity."""
    name, q, kv, hq, hk, d, ps, mode = case
    banner(f"paired order {name}")
    pool = sum((k + ps - 1) // ps for k in kv) + 5
    w = W.make_attention(f"paired_{name}", q, kv, hq, hk, d, ps, pool, seed=33, device="cuda",
                         scales="amax")

    def mk(schedule):
        return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), hq, hk, d, ps,
                      kv_indptr=torch.from_numpy(w.kv_indptr), split_len=-1, tile_waves=4,
                      dequant_mode=mode, schedule=schedule)

    base, cache, _ = run_gpu(K, w, plan=mk(K.SCHEDULE_HEAVIEST))
    out, _, plan = run_gpu(K, w, cache=cache, plan=mk(K.SCHEDULE_PAIRED))
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    assert torch.equal(out, base)
    print(f"Q tiles per head {plan.q_tiles_per_head}: bitwise equal to heaviest first")
    if mode <= 3:
        ref, rows = oracle_outputs(oracle, w)
        e = assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)
        print(f"max err {e:.3g}")


def test_paired_order_unavailable(K):
    """Paired issue needs a uniform batch (no work list), 4-wave tiles and no
    split: other requests are refused before any launch."""
    banner("paired order where it is not available")
    w = W.make_attention("paired_no", [64, 100], [64, 100], 32, 8, 128, 16, 20, seed=34, device="cuda")
    u = W.make_attention("paired_no_u", [128] * 2, [128] * 2, 32, 8, 128, 16, 20, seed=34, device="cuda")

    def mk(x, **kw):
        return K.plan(torch.from_numpy(x.qo_indptr), torch.from_numpy(x.kv_lens), 32, 8, 128, 16,
                      kv_indptr=torch.from_numpy(x.kv_indptr), schedule=K.SCHEDULE_PAIRED, **kw)

    for x, kw in ((w, dict(split_len=-1)), (u, dict(split_len=1)), (u, dict(split_len=-1, tile_waves=8))):
        with pytest.raises(K.NVFP4KVError, match="unsupported"):
            run_gpu(K, x, plan=mk(x, **kw))
    out, _, plan = run_gpu(K, u, plan=mk(u, split_len=-1, tile_waves=4))
    torch.cuda.synchronize()
    assert plan.schedule == K.SCHEDULE_PAIRED and K.read_device_error("cuda") == 0
