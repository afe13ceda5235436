"""GPU parity of the paged decode step (one query token per request over the
NVFP4 cache) against the fp64 oracle (the prefill definition with q_len = 1),
within |err| <= 1e-2 + 1e-2 |ref| per element: every (head_dim, GQA group)
kernel on a ragged batch (lengths 1 .. 2049, tile and chunk edges), forced
chunk lengths down to one 64-key tile per chunk, the automatic plan, and the
32 x 8192 decode workload on sampled requests; page-id range errors and no
host synchronization."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, banner, gpu_cache, oracle_outputs

pytestmark = pytest.mark.gpu

RAGGED_KV = [1, 17, 63, 64, 65, 300, 1000, 2049]


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _run(K, w, plan=None, cache=None, chunk_len=0):
    if cache is None:
        cache = gpu_cache(K, w)
        cache.append(w.k, w.v, w.slot_mapping)
    if plan is None:
        plan = K.decode_plan(torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads, w.head_dim,
                             w.page_size, chunk_len=chunk_len)
    out = torch.empty_like(w.q)
    args = [torch.from_numpy(x).cuda() for x in (w.kv_indptr, w.page_table, w.kv_lens)]
    K.paged_decode(w.q, *args, cache, out, w.sm_scale, plan)
    return out, cache, plan


def _check(K, O, w, reqs=None, **kw):
    out, cache, plan = _run(K, w, **kw)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(O, w, reqs)
    got = out.index_select(0, torch.from_numpy(rows).cuda())
    return assert_close(got, ref, w.name), plan


def _ragged(hq, hk, d, seed, kv=RAGGED_KV):
    pool = int(sum((k + 15) // 16 for k in kv)) + 7
    return W.make_attention(f"decode_ragged_{hq}_{hk}_{d}", [1] * len(kv), kv, hq, hk, d, 16, pool,
                            seed=seed, device="cuda", scales="amax")


@pytest.mark.parametrize("hq,hk,d", [(32, 8, 128), (16, 8, 128), (8, 8, 128), (64, 8, 128),
                                     (8, 4, 64), (4, 2, 64), (2, 2, 64), (16, 2, 64)])
def test_decode_ragged_all_kernels(K, oracle, hq, hk, d):
    banner(f"decode ragged hq={hq} hk={hk} d={d}")
    e, plan = _check(K, oracle, _ragged(hq, hk, d, seed=21))
    print(f"max err {e:.3g}; chunk_len {plan.chunk_len}, chunks {plan.max_chunks}")


# every (head_dim, GQA group, heads per wave) kernel: odd KV head counts take
# one head per wave, head_dim 128 two, head_dim 64 four when the KV heads and
# the 16 score columns allow
EVERY_HP = [(1, 1, 128, 1), (6, 3, 128, 1), (12, 3, 128, 1), (24, 3, 128, 1),
            (2, 2, 128, 2), (4, 2, 128, 2), (8, 2, 128, 2), (16, 2, 128, 2),
            (3, 3, 64, 1), (6, 3, 64, 1), (12, 3, 64, 1), (24, 3, 64, 1),
            (2, 2, 64, 2), (4, 2, 64, 2), (8, 2, 64, 2), (16, 2, 64, 2),
            (4, 4, 64, 4), (8, 4, 64, 4), (16, 4, 64, 4)]


@pytest.mark.parametrize("hq,hk,d,hp", EVERY_HP)
def test_decode_every_heads_per_wave_kernel(K, oracle, hq, hk, d, hp):
    """Each kernel instance against the oracle, with several chunks per
    request (forced 128-key chunks) and lengths ending inside a tile."""
    banner(f"decode hq={hq} hk={hk} d={d}: {hp} KV heads per wave")
    kv = [1, 31, 33, 129, 300, 517]
    e, plan = _check(K, oracle, _ragged(hq, hk, d, seed=29, kv=kv), chunk_len=128)
    assert plan.heads_per_wave == hp and plan.max_chunks == 5
    print(f"max err {e:.3g}")


@pytest.mark.parametrize("seed", range(24))
def test_decode_random_shapes(K, oracle, seed):
    """Seeded random decode batches against the oracle: 1-9 requests of 1-700
    keys, 1/2/3/4/8 KV heads, GQA group 1/2/4/8, head_dim 64/128, page sizes
    that do and do not divide a tile, automatic or forced chunk lengths (so
    every heads-per-wave kernel meets ragged lengths and several chunks)."""
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(1, 10))
    hk = int(r.choice([1, 2, 3, 4, 8]))
    g = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    ps = int(r.choice([1, 5, 16, 32, 64]))
    chunk = int(r.choice([0, 64, 128, 192]))
    kv = [int(x) for x in r.integers(1, 701, B)]
    pool = sum((k + ps - 1) // ps for k in kv) + 3
    banner(f"decode random shape {seed}: B={B} hk={hk} G={g} d={d} page={ps} chunk={chunk} kv={kv}")
    w = W.make_attention(f"decode_rand_{seed}", [1] * B, kv, hk * g, hk, d, ps, pool, seed=60 + seed,
                         device="cuda", scales="amax")
    e, plan = _check(K, oracle, w, chunk_len=chunk)
    print(f"max err {e:.3g}; heads per wave {plan.heads_per_wave}, chunks {plan.max_chunks}")


@pytest.mark.parametrize("chunk_len", [64, 128, 192, 1024])
def test_decode_forced_chunks(K, oracle, chunk_len):
    """Chunks merged in order: one tile per chunk, uneven last chunks,
    requests with a single chunk next to split ones."""
    banner(f"decode chunk_len {chunk_len}")
    w = _ragged(32, 8, 128, seed=22)
    e, plan = _check(K, oracle, w, chunk_len=chunk_len)
    assert plan.chunk_len == chunk_len and plan.max_chunks == -(-2049 // chunk_len)
    _check(K, oracle, w, chunk_len=chunk_len)  # the workspace needs no reset


def test_decode_lognormal_scales_head_dim_64(K, oracle):
    banner("decode head_dim 64, lognormal scales, page 32")
    kv = [5, 70, 129, 500]
    w = W.make_attention("decode_d64_ps32", [1] * 4, kv, 8, 2, 64, 32, 40, seed=23, device="cuda",
                         scales="lognormal", lognormal=(-3.0, 0.5))
    _check(K, oracle, w, chunk_len=64)


def test_decode_batch_sampled(K, oracle):
    banner("decode 32 x 8192, 6 sampled requests")
    w = W.decode_batch("cuda")
    reqs = np.random.default_rng(5).choice(w.batch, 6, replace=False)
    e, plan = _check(K, oracle, w, reqs=reqs)
    assert plan.max_chunks > 1
    print(f"max err {e:.3g}; chunk_len {plan.chunk_len}, chunks {plan.max_chunks}")


def test_decode_agrees_with_prefill_kernel(K):
    """The decode kernel and the prefill kernel run on the same q_len = 1
    batch agree within the sum of their tolerances to the oracle."""
    w = _ragged(32, 8, 128, seed=24, kv=[1, 63, 64, 65, 200])
    out_d, cache, _ = _run(K, w)
    out_p = torch.empty_like(w.q)
    plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), 32, 8, 128, 16)
    K.paged_prefill_causal(w.q, torch.from_numpy(w.qo_indptr).cuda(), torch.from_numpy(w.kv_indptr).cuda(),
                           torch.from_numpy(w.page_table).cuda(), torch.from_numpy(w.kv_lens).cuda(), cache,
                           out_p, w.sm_scale, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    d = (out_d.float() - out_p.float()).abs()
    bound = 2e-2 + 2e-2 * out_p.float().abs()
    assert bool((d <= bound).all()), float(d.max())


def test_decode_page_id_out_of_range_sets_flag(K):
    w = _ragged(32, 8, 128, seed=25, kv=[100, 40])
    out, cache, plan = _run(K, w)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    pt = torch.from_numpy(w.page_table).cuda()
    pt[2] = w.num_pages + 3
    K.paged_decode(w.q, torch.from_numpy(w.kv_indptr).cuda(), pt, torch.from_numpy(w.kv_lens).cuda(),
                   cache, out, w.sm_scale, plan)
    assert K.read_device_error("cuda") == K.DEV_PAGE_OOB


def test_decode_does_not_synchronize(K):
    w = _ragged(32, 8, 128, seed=26, kv=[300, 900])
    out, cache, plan = _run(K, w, chunk_len=64)
    args = [torch.from_numpy(x).cuda() for x in (w.kv_indptr, w.page_table, w.kv_lens)]
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    K.paged_decode(w.q, *args, cache, out, w.sm_scale, plan)
    assert not torch.cuda.current_stream().query()
    torch.cuda.synchronize()


@pytest.mark.parametrize("ps,d,chunk_len", [(1, 128, 128), (8, 64, 0), (64, 128, 64), (5, 128, 128),
                                            (48, 64, 0), (128, 128, 192)])
def test_decode_page_sizes(K, oracle, ps, d, chunk_len):
    """Page sizes that divide the 64-key tile (a lane's key keeps its page
    slot in every tile) and page sizes that do not, with one or more chunks
    per request and lengths that end inside a tile and a page."""
    banner(f"decode page size {ps}, head_dim {d}, chunk_len {chunk_len}")
    kv = [1, 17, 63, 64, 65, 300, 1000, 700]
    pool = sum((k + ps - 1) // ps for k in kv) + 5
    w = W.make_attention(f"decode_ps{ps}_{d}", [1] * len(kv), kv, 16, 4, d, ps, pool, seed=24, device="cuda",
                         scales="amax")
    e, plan = _check(K, oracle, w, chunk_len=chunk_len)
    print(f"max err {e:.3g}; chunk_len {plan.chunk_len}, chunks {plan.max_chunks}")
