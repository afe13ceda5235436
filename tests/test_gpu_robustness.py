"""GPU checks of the attention kernels' own choices where they depart from the
plain definition:

* split Q tiles: the merge of a split tile's KV chunks is in chunk order, so
  repeated runs give the same bits whichever chunk finishes last, and every
  call zeroes its arrival counters itself, so stale counters left in the
  workspace (by an earlier call, or its first contents) change nothing;
* query rows far from N(0, 1): the kernels rescale each bf16 query row by a
  power of two (its largest magnitude to [2^14, 2^15)) before the 16-bit
  matrix instructions (bf16 in the prefill's default form, f16 in its mode 0
  and in the decode), so rows with a huge magnitude, rows of bf16
  subnormals and rows whose elements span more than 2^30 are compared with
  the fp64 oracle at the usual tolerance, in the prefill (both tile widths;
  the f16 form in test_gpu_f16_staging.py) and the decode;
* a global k/v scale that is not positive finite: the prefill and the decode
  set NVFP4KV_DEV_BAD_SCALE_ATTN and every kernel runs to its end (the next
  call with good scales is exact again).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, banner, force_tile_waves, gpu_cache, oracle_outputs, run_gpu

pytestmark = pytest.mark.gpu

Q_LENS = [1, 37, 200, 64, 3, 129]
KV_LENS = [1, 37, 333, 700, 3, 130]


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _dev_args(w):
    return [torch.from_numpy(x).cuda() for x in (w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens)]


@pytest.mark.parametrize("split_len,waves", [(1, 4), (2, 4), (3, 8), (5, 8), (7, 4)])
def test_split_merge_bitwise_repeatable(K, split_len, waves):
    banner(f"split merge repeat: chunk length {split_len}, {waves}-wave tiles")
    w = W.make_attention(f"split_repeat_{split_len}_{waves}", Q_LENS, KV_LENS, 32, 8, 128, 16, 120,
                         seed=21, device="cuda", scales="amax")
    plan = force_tile_waves(K, w, waves, split_len=split_len)
    assert plan.num_split_tiles > 0 and plan.max_chunks > 1
    first, cache, _ = run_gpu(K, w, plan=plan)
    for _ in range(4):
        again, _, _ = run_gpu(K, w, cache=cache, plan=plan)
        assert torch.equal(again, first)
    # stale arrival counters and partials: the call starts from zero anyway
    ws = plan.workspace("cuda")
    ws.fill_(0x7F)
    stale, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    assert torch.equal(stale, first)


def _wide_range_queries(q: torch.Tensor) -> torch.Tensor:
    """q with its rows rewritten by kind (row index mod 6): 0 unchanged;
    1 times 1e30; 2 bf16 subnormals only; 3 every other element times 2^-34
    (a dynamic range above 2^30); 4 one element 1e4 and the rest ~1e-6;
    5 times 1e-30 (small but normal)."""
    qf = q.float().clone()
    n = qf.shape[0] * qf.shape[1]
    flat = qf.view(n, -1)
    kind = torch.arange(n, device=q.device) % 6
    D = flat.shape[1]
    alt = torch.ones(D, device=q.device)
    alt[1::2] = 2.0 ** -34
    flat[kind == 1] *= 1e30
    flat[kind == 2] = flat[kind == 2] * 2e-39  # below bf16's smallest normal (1.18e-38)
    flat[kind == 3] *= alt
    r4 = flat[kind == 4] * 1e-6
    r4[:, 5] = 1e4
    flat[kind == 4] = r4
    flat[kind == 5] *= 1e-30
    out = qf.to(torch.bfloat16)
    sub = out.view(n, -1)[kind == 2].float()
    assert (sub != 0).any() and (sub.abs() < 1.18e-38).all()
    return out


@pytest.mark.parametrize("waves", [4, 8])
def test_prefill_wide_range_query_rows(K, oracle, waves):
    banner(f"prefill, wide-range query rows, {waves}-wave tiles")
    w = W.make_attention(f"wide_q_{waves}", Q_LENS, KV_LENS, 32, 8, 128, 16, 120, seed=22,
                         device="cuda", scales="amax")
    w.q = _wide_range_queries(w.q)
    out, cache, plan = run_gpu(K, w, plan=force_tile_waves(K, w, waves))
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(oracle, w)
    e = assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)
    print(f"max err {e:.3g}")


def test_prefill_wide_range_query_rows_head_dim_64(K, oracle):
    banner("prefill, wide-range query rows, head_dim 64")
    w = W.make_attention("wide_q_d64", Q_LENS, KV_LENS, 8, 4, 64, 16, 120, seed=23, device="cuda",
                         scales="lognormal", lognormal=(-3.0, 0.5))
    w.q = _wide_range_queries(w.q)
    out, cache, plan = run_gpu(K, w)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(oracle, w)
    assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)


@pytest.mark.parametrize("hq,hk,d", [(32, 8, 128), (8, 4, 64)])
def test_decode_wide_range_query_rows(K, oracle, hq, hk, d):
    banner(f"decode, wide-range query rows, hq={hq} hk={hk} d={d}")
    kv = [1, 17, 64, 65, 300, 1000, 2049, 130, 7, 500, 64, 1]
    pool = sum((k + 15) // 16 for k in kv) + 3
    w = W.make_attention(f"decode_wide_q_{hq}_{d}", [1] * len(kv), kv, hq, hk, d, 16, pool, seed=24,
                         device="cuda", scales="amax")
    w.q = _wide_range_queries(w.q)
    cache = gpu_cache(K, w)
    cache.append(w.k, w.v, w.slot_mapping)
    plan = K.decode_plan(torch.from_numpy(w.kv_lens), hq, hk, d, 16, chunk_len=128)
    out = torch.empty_like(w.q)
    _, kvp, pt, kvl = _dev_args(w)
    K.paged_decode(w.q, kvp, pt, kvl, cache, out, w.sm_scale, plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(oracle, w)
    assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)


BAD_SCALES = [0.0, -1.0, float("nan"), float("inf")]


@pytest.mark.parametrize("which", ["k", "v"])
def test_attention_bad_device_scale_sets_flag(K, oracle, which):
    """A bad global scale reaches the attention kernels only through the
    device scalar (the binding never reads it); each kernel reports it and
    runs to its end: the uniform prefill, the split prefill (work list,
    merge) and the chunked decode."""
    banner(f"attention with a bad {which}_scale")
    w = W.make_attention("bad_scale", Q_LENS, KV_LENS, 32, 8, 128, 16, 120, seed=25, device="cuda",
                         scales="amax")
    out, cache, plan = run_gpu(K, w)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    good = out.clone()
    split = force_tile_waves(K, w, 4, split_len=2)
    assert split.num_split_tiles > 0
    dplan = K.decode_plan(torch.from_numpy(w.kv_lens), 32, 8, 128, 16, chunk_len=64)
    assert dplan.max_chunks > 1
    qd = w.q[torch.from_numpy(w.qo_indptr[1:] - 1).cuda()].contiguous()  # each request's last row
    dout = torch.empty_like(qd)
    qo, kvp, pt, kvl = _dev_args(w)
    scale = cache.k_scale if which == "k" else cache.v_scale
    keep = scale.clone()
    for bad in BAD_SCALES:
        scale.fill_(bad)
        for p in (plan, split):
            run_gpu(K, w, cache=cache, plan=p, out=torch.empty_like(w.q))
            torch.cuda.synchronize()
            assert K.read_device_error("cuda") == K.DEV_BAD_SCALE_ATTN, (bad, p.split_len)
        K.paged_decode(qd, kvp, pt, kvl, cache, dout, w.sm_scale, dplan)
        torch.cuda.synchronize()
        assert K.read_device_error("cuda") == K.DEV_BAD_SCALE_ATTN, bad
    scale.copy_(keep)
    again, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    assert torch.equal(again, good)
