"""GPU parity of the prefill's f16 form (dequant mode 0: f16 staging tile,
f16 queries after an exact per-row power-of-two rescale, f16 probabilities,
f16 matrix instructions) on every kernel shape the default bf16 form has:
head_dim 64 and 128, GQA groups 1/2/4/8, 4- and 8-wave tiles, page sizes
that divide the 64-key tile and others, split Q tiles, the 2 x 128 small
batch, the full 2048 x 2048 batch, sampled requests of the 1024 x 1024 and
ragged batches at full size, and query rows far from N(0, 1).  Same
tolerance as the bf16 form: |err| <= 1e-2 + 1e-2 |ref| per element."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, banner, oracle_outputs, run_gpu
from test_gpu_robustness import _wide_range_queries

pytestmark = pytest.mark.gpu

Q_LENS = [1, 37, 200, 64, 3, 129]
KV_LENS = [1, 37, 333, 700, 3, 130]


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _plan(K, w, waves=0, split_len=-1):
    return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads,
                  w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr), split_len=split_len,
                  tile_waves=waves, dequant_mode=0)


def _check(K, O, w, plan, reqs=None):
    out, _, _ = run_gpu(K, w, plan=plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    ref, rows = oracle_outputs(O, w, reqs)
    e = assert_close(out.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)
    print(f"max err {e:.3g}", flush=True)
    return plan


@pytest.mark.parametrize("hq,hk,d,ps,waves,split", [
    (32, 8, 128, 16, 4, -1), (32, 8, 128, 16, 8, -1), (32, 8, 128, 16, 4, 2), (32, 8, 128, 16, 8, 3),
    (16, 8, 128, 16, 4, -1), (8, 8, 128, 16, 8, -1), (64, 8, 128, 16, 8, -1), (8, 4, 64, 16, 4, -1),
    (4, 2, 64, 16, 4, -1), (16, 2, 64, 16, 4, -1), (32, 8, 128, 48, 4, -1), (8, 4, 64, 5, 4, 2)])
def test_f16_staging_every_kernel(K, oracle, hq, hk, d, ps, waves, split):
    banner(f"f16 staging: hq={hq} hk={hk} d={d} page={ps} waves={waves} split={split}")
    pool = sum((k + ps - 1) // ps for k in KV_LENS) + 5
    w = W.make_attention(f"f16_{hq}_{hk}_{d}_{ps}", Q_LENS, KV_LENS, hq, hk, d, ps, pool, seed=41,
                         device="cuda", scales="amax")
    plan = _check(K, oracle, w, _plan(K, w, waves, split))
    assert plan.block_q * (hq // hk) == 32 * waves
    if split > 0:
        assert plan.num_split_tiles > 0


def test_f16_staging_small_batch(K, oracle):
    banner("f16 staging: 2 x 128 small batch, head_dim 64")
    _check(K, oracle, W.tiny("cuda"), _plan(K, W.tiny("cuda")))


def test_f16_staging_2k(K, oracle):
    """The f16 form on the full 2048x2048 batch (paired issue, as the plan
    picks for it)."""
    banner("f16 staging: 2048x2048")
    w = W.prefill_2k("cuda")
    plan = _check(K, oracle, w, _plan(K, w, 4, 0))
    assert plan.dequant_mode == 0 and plan.schedule == K.SCHEDULE_PAIRED


def test_f16_staging_uniform_1k_sampled(K, oracle):
    banner("f16 staging: 1024x1024 uniform, 16 sampled requests")
    w = W.uniform_batch_1k("cuda")
    reqs = np.random.default_rng(2).choice(w.batch, 16, replace=False)
    plan = _check(K, oracle, w, _plan(K, w), reqs)
    assert plan.uniform_q == 1


def test_f16_staging_ragged_chunked_sampled(K, oracle):
    banner("f16 staging: ragged chunked 256 requests, 16 sampled")
    w = W.ragged_chunked("cuda")
    order = np.argsort(w.kv_lens, kind="stable")
    reqs = np.concatenate([order[-4:], order[:4], np.random.default_rng(4).choice(order[4:-4], 8, replace=False)])
    _check(K, oracle, w, _plan(K, w), reqs)


@pytest.mark.parametrize("d,waves", [(128, 4), (128, 8), (64, 4)])
def test_f16_staging_wide_range_query_rows(K, oracle, d, waves):
    """Rows of bf16 subnormals, rows spanning more than 2^30 and rows near
    1e30: the f16 form rescales each row by a power of two (its largest
    magnitude to [2^14, 2^15)) before converting it to f16."""
    banner(f"f16 staging: wide-range query rows, d={d} waves={waves}")
    hq, hk = (32, 8) if d == 128 else (8, 4)
    w = W.make_attention(f"f16_wide_{d}_{waves}", Q_LENS, KV_LENS, hq, hk, d, 16, 120, seed=42, device="cuda",
                         scales="amax")
    w.q = _wide_range_queries(w.q)
    _check(K, oracle, w, _plan(K, w, waves))
