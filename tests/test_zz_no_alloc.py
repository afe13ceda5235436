"""paged_prefill_causal_noalloc (the entry point for callers that cannot
allocate device memory) against paged_prefill_causal with a caller-owned
workspace: two calls in a row on the library's own scratch array, the second
with a smaller batch, each bitwise equal to the workspace entry point's
output on the same inputs (the two share every kernel); a uniform batch that
needs no workspace; and the size limit, refused before any launch."""
import pytest
import torch

import workloads as W
from gpu_helpers import banner, force_tile_waves, gpu_cache, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _noalloc(K, w, cache, plan):
    dev = "cuda"
    args = [torch.from_numpy(x).to(dev) for x in (w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens)]
    out = torch.full_like(w.q, float("nan"))
    K.paged_prefill_causal_noalloc(w.q, *args, cache, out, w.sm_scale, plan, K.device_error_word(dev))
    return out


def _case(K, w, plan):
    cache = gpu_cache(K, w)
    cache.append(w.k, w.v, w.slot_mapping)
    ref, _, _ = run_gpu(K, w, cache=cache, plan=plan)
    got = _noalloc(K, w, cache, plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
    assert torch.equal(got, ref)


def test_noalloc_matches_workspace_entry_point(K):
    # 1) ragged batch with split Q tiles: work list, counters and partials
    banner("noalloc: ragged batch with split Q tiles")
    w1 = W.make_attention("noalloc_split", [1, 37, 200, 64, 3, 129], [1, 37, 333, 700, 3, 130],
                          32, 8, 128, 16, 120, seed=31, device="cuda", scales="amax")
    p1 = force_tile_waves(K, w1, 4, split_len=3)
    assert p1.num_split_tiles > 0 and 0 < p1.workspace_bytes <= K.NOALLOC_SCRATCH_BYTES
    _case(K, w1, p1)
    # 2) a smaller ragged batch right after (the array holds the first call's
    #    list, counters and partials), 8-wave tiles, automatic split
    banner("noalloc: smaller ragged batch")
    w2 = W.make_attention("noalloc_small", [17, 64, 5], [900, 64, 300], 32, 8, 128, 16, 90, seed=32,
                          device="cuda", scales="amax")
    p2 = force_tile_waves(K, w2, 8, split_len=0)
    assert 0 < p2.workspace_bytes < p1.workspace_bytes
    _case(K, w2, p2)
    # 3) a uniform batch: no workspace at all
    banner("noalloc: uniform batch")
    w3 = W.make_attention("noalloc_uniform", [96] * 3, [160] * 3, 16, 4, 64, 16, 40, seed=33,
                          device="cuda", scales="lognormal")
    p3 = K.plan(torch.from_numpy(w3.qo_indptr), torch.from_numpy(w3.kv_lens), 16, 4, 64, 16,
                split_len=-1)
    assert p3.workspace_bytes == 0
    _case(K, w3, p3)


def test_noalloc_rejects_plans_beyond_the_array(K):
    banner("noalloc: size limit")
    w = W.make_attention("noalloc_limit", [64, 37], [700, 333], 32, 8, 128, 16, 80, seed=34, device="cuda",
                         scales="amax")
    cache = gpu_cache(K, w)
    plan = force_tile_waves(K, w, 4, split_len=2)
    plan.struct.workspace_bytes = K.NOALLOC_SCRATCH_BYTES + 256
    torch.cuda.synchronize()
    with pytest.raises(K.NVFP4KVError, match="workspace"):
        _noalloc(K, w, cache, plan)
    torch.cuda.synchronize()
    assert K.read_device_error("cuda") == 0
