"""The whole step captured into one HIP graph (through torch.cuda.graph) and
replayed: append of the batch's K/V rows, the causal prefill (with split Q
tiles, so the merge counters must come back to zero between replays) and the
decode step (several chunks, so the merge kernel runs too).  Every replay
follows fresh inputs written by ordinary eager copies, and its outputs must
equal, bit for bit, the same calls made eagerly on the same inputs; the eager
results themselves are held to the oracle by the other GPU tests, and once
here on the first inputs.  The prefill's bf16 form and its two MX score
variants get the same replay check on their own."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_close, banner, gpu_cache, oracle_outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _fresh(shape, seed, stream):
    return W.normal_bf16(shape, seed, stream, "cuda")


def test_graph_replays_match_eager(K, oracle):
    banner("graph capture of append + prefill + decode, 4 replays")
    q_lens = [96, 300, 1, 517]
    kv_lens = [200, 300, 700, 1100]
    w = W.make_attention("graph_step", q_lens, kv_lens, 16, 4, 128, 16, 160, seed=31, device="cuda",
                         scales="amax")
    dev = "cuda"
    cache = gpu_cache(K, w)
    qo, kvp, pt, kvl = (torch.from_numpy(x).to(dev) for x in (w.qo_indptr, w.kv_indptr,
                                                               w.page_table, w.kv_lens))
    pplan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                   w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                   split_len=3)
    assert pplan.num_split_tiles > 0
    dplan = K.decode_plan(torch.from_numpy(w.kv_lens), w.num_q_heads, w.num_kv_heads, w.head_dim,
                          w.page_size, chunk_len=128)
    assert dplan.max_chunks > 1
    # static inputs and outputs of the captured step
    k, v, q = w.k.clone(), w.v.clone(), w.q.clone()
    qd = _fresh((w.batch, w.num_q_heads, w.head_dim), 31, 7)
    out_p = torch.empty_like(q)
    out_d = torch.empty_like(qd)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(out_prefill, out_decode):
        cache.append(k, v, w.slot_mapping, dev_error=err)
        K.paged_prefill_causal(q, qo, kvp, pt, kvl, cache, out_prefill, w.sm_scale, plan=pplan,
                               dev_error=err)
        K.paged_decode(qd, kvp, pt, kvl, cache, out_decode, w.sm_scale, dplan, dev_error=err)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside capture (workspaces allocated here)
        step(out_p, out_d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_p, out_d)
    torch.cuda.synchronize()

    eager_p, eager_d = torch.empty_like(out_p), torch.empty_like(out_d)
    prev = None
    for r in range(4):
        if r > 0:  # new inputs through eager copies between replays
            k.copy_(_fresh(k.shape, 40 + r, 1))
            v.copy_(_fresh(v.shape, 40 + r, 2))
            q.copy_(_fresh(q.shape, 40 + r, 0))
            qd.copy_(_fresh(qd.shape, 40 + r, 7))
        out_p.fill_(0)
        out_d.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        got_p, got_d = out_p.clone(), out_d.clone()
        step(eager_p, eager_d)
        torch.cuda.synchronize()
        assert K.read_device_error(word=err) == 0
        assert torch.equal(got_p.view(torch.int16), eager_p.view(torch.int16)), f"replay {r}: prefill"
        assert torch.equal(got_d.view(torch.int16), eager_d.view(torch.int16)), f"replay {r}: decode"
        if prev is not None:
            assert not torch.equal(got_p, prev), "replay produced the previous outputs"
        prev = got_p
        if r == 0:
            ref, rows = oracle_outputs(oracle, w)
            assert_close(got_p.index_select(0, torch.from_numpy(rows).cuda()), ref, w.name)
        print(f"replay {r}: bit-identical to eager", flush=True)


@pytest.mark.parametrize("mode", [3, 4, 5, "paired"])
def test_graph_prefill_other_modes(K, mode):
    """The bf16 form (mode 3) and the MX score modes (4, 5) under graph
    capture, with split Q tiles, and the paired issue order on a uniform
    batch: three replays, each after fresh queries written eagerly,
    bit-identical to the same call made eagerly."""
    banner(f"graph capture of the prefill in dequant mode {mode}, 3 replays")
    paired = mode == "paired"
    q_lens, kv_lens = ([300] * 4, [300, 500, 700, 1100]) if paired else ([96, 300, 1, 517], [200, 300, 700, 1100])
    w = W.make_attention(f"graph_mode_{mode}", q_lens, kv_lens, 16, 4, 128, 16, 180,
                         seed=32, device="cuda", scales="amax")
    dev = "cuda"
    cache = gpu_cache(K, w)
    cache.append(w.k, w.v, w.slot_mapping)
    qo, kvp, pt, kvl = (torch.from_numpy(x).to(dev) for x in (w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens))
    if paired:
        plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                      split_len=-1, tile_waves=4, schedule=K.SCHEDULE_PAIRED)
        assert plan.workspace_bytes == 0
    else:
        plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                      split_len=3, tile_waves=4, dequant_mode=mode)
        assert plan.num_split_tiles > 0
    q = w.q.clone()
    out = torch.empty_like(q)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(o):
        K.paged_prefill_causal(q, qo, kvp, pt, kvl, cache, o, w.sm_scale, plan=plan, dev_error=err)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out)
    torch.cuda.synchronize()
    eager = torch.empty_like(out)
    prev = None
    for r in range(3):
        if r > 0:
            q.copy_(_fresh(q.shape, 50 + r, 0))
        out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        step(eager)
        torch.cuda.synchronize()
        assert K.read_device_error(word=err) == 0
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        if prev is not None:
            assert not torch.equal(got, prev), "replay produced the previous outputs"
        prev = got
        print(f"replay {r}: bit-identical to eager", flush=True)
