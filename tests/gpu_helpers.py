"""Shared helpers of the GPU tests: run the HIP path through the binding and
the oracle on the same seeded inputs (the oracle always re-derives its own
cache from the bf16 inputs; nothing it reads comes from the HIP path)."""
import numpy as np
import torch

import workloads as W

SENTINEL = 0xA5
ATOL = RTOL = 1e-2  # |err| <= 1e-2 + 1e-2 * |ref| per element


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)


def gpu_cache(K, w, fill=SENTINEL):
    return K.PagedCache.empty(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim, "cuda",
                              w.k_scale, w.v_scale, fill=fill)


def run_gpu(K, w, cache=None, plan=None, out=None):
    """Append every cached position, then run the prefill.  Returns (out, cache, plan)."""
    if cache is None:
        cache = gpu_cache(K, w)
        cache.append(w.k, w.v, w.slot_mapping)
    dev = "cuda"
    if plan is None:
        plan = K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                      w.num_kv_heads, w.head_dim, w.page_size,
                      kv_indptr=torch.from_numpy(w.kv_indptr))
    if out is None:
        out = torch.empty_like(w.q)
    K.paged_prefill_causal(w.q, torch.from_numpy(w.qo_indptr).to(dev),
                           torch.from_numpy(w.kv_indptr).to(dev),
                           torch.from_numpy(w.page_table).to(dev),
                           torch.from_numpy(w.kv_lens).to(dev), cache, out, w.sm_scale, plan=plan)
    return out, cache, plan


def sub_workload(w, reqs):
    """The requests `reqs` of w as a compact host workload (own page pool,
    pages in order), with host copies of their bf16 inputs."""
    reqs = list(reqs)
    ps = w.page_size
    q_lens = w.q_lens[reqs]
    kv_lens = w.kv_lens[reqs]
    npg = (kv_lens + ps - 1) // ps
    kv_indptr = np.zeros(len(reqs) + 1, np.int32)
    kv_indptr[1:] = np.cumsum(npg)
    page_table = np.arange(kv_indptr[-1], dtype=np.int32)
    qo = np.zeros(len(reqs) + 1, np.int32)
    qo[1:] = np.cumsum(q_lens)
    q_rows = np.concatenate([np.arange(w.qo_indptr[r], w.qo_indptr[r + 1]) for r in reqs])
    kv_rows = np.concatenate([np.arange(w.kv_token_indptr[r], w.kv_token_indptr[r + 1]) for r in reqs])
    slots = np.concatenate([
        page_table[kv_indptr[i] + np.arange(kv_lens[i]) // ps] * ps + np.arange(kv_lens[i]) % ps
        for i in range(len(reqs))]).astype(np.int64)
    qi = torch.from_numpy(q_rows).to(w.q.device)
    ki = torch.from_numpy(kv_rows).to(w.k.device)
    return dict(q=W.bf16_bits(w.q.index_select(0, qi)), k=W.bf16_bits(w.k.index_select(0, ki)),
                v=W.bf16_bits(w.v.index_select(0, ki)), qo=qo, kv_indptr=kv_indptr,
                page_table=page_table, kv_lens=kv_lens.astype(np.int32), slots=slots,
                num_pages=int(kv_indptr[-1]), q_rows=q_rows)


def oracle_outputs(O, w, reqs=None):
    """fp64 oracle output rows for `reqs` (all requests if None) and their
    row indices in w's query order."""
    if reqs is None:
        reqs = range(w.batch)
    s = sub_workload(w, reqs)
    P, ps, H, D = s["num_pages"], w.page_size, w.num_kv_heads, w.head_dim
    kc = np.zeros((P, ps, H, D // 2), np.uint8)
    vc = np.zeros_like(kc)
    ksf = np.zeros((P, ps, H, D // 16), np.uint8)
    vsf = np.zeros_like(ksf)
    err = O.append(s["k"], s["v"], s["slots"], w.k_scale, w.v_scale, kc, vc, ksf, vsf, ps)
    assert err == 0
    out, err = O.prefill(s["q"], s["qo"], s["kv_indptr"], s["page_table"], s["kv_lens"], kc, vc,
                         ksf, vsf, w.k_scale, w.v_scale, w.num_q_heads, w.sm_scale)
    assert err == 0
    return out, s["q_rows"]


def assert_close(got_bf16, ref64, what):
    got = got_bf16.float().cpu().double().numpy() if isinstance(got_bf16, torch.Tensor) else got_bf16
    err = np.abs(got - ref64)
    bound = ATOL + RTOL * np.abs(ref64)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} / {bad.size} elements out of tolerance; "
                             f"max err {err.max():.3g}; first {idx.tolist()} "
                             f"got {got[tuple(idx[0])]} ref {ref64[tuple(idx[0])]}")
    return float(err.max())


def force_tile_waves(K, w, waves, split_len=-1):
    """A plan for w whose attention tiles use `waves` waves of 32 rows (the plan
    picks 4 or 8 by batch size; tests cover both kernels on every shape)."""
    return K.plan(torch.from_numpy(w.qo_indptr), torch.from_numpy(w.kv_lens), w.num_q_heads,
                  w.num_kv_heads, w.head_dim, w.page_size, kv_indptr=torch.from_numpy(w.kv_indptr),
                  split_len=split_len, tile_waves=waves)
