"""GPU parity of the NVFP4 append (bit-exact against the oracle; both the
two-block and the half-block kernels) and its boundary behaviour: device scale checks (eager and graph replay), zero rows,
padding / out-of-range slots, and no host synchronization."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import SENTINEL, banner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _oracle_cache(O, k, v, slots, ks, vs, P, ps):
    T, H, D = k.shape
    c = [np.full((P, ps, H, D // 2), SENTINEL, np.uint8), np.full((P, ps, H, D // 2), SENTINEL, np.uint8),
         np.full((P, ps, H, D // 16), SENTINEL, np.uint8), np.full((P, ps, H, D // 16), SENTINEL, np.uint8)]
    err = O.append(W.bf16_bits(k), W.bf16_bits(v), slots.cpu().numpy(), ks, vs, *c, ps)
    return c, err


def _gpu_append(K, k, v, slots, ks, vs, P, ps, err_word=None):
    T, H, D = k.shape
    cache = K.PagedCache.empty(P, ps, H, D, "cuda", fill=SENTINEL, k_scale=1.0, v_scale=1.0)
    K.nvfp4_append_paged_kv(k, v, slots, ks, vs, cache.k_cache, cache.v_cache, cache.k_sf,
                            cache.v_sf, ps, dev_error=err_word)
    return cache


def _compare(cache, ref):
    for name, got, want in zip(("k_cache", "v_cache", "k_sf", "v_sf"),
                               (cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf), ref):
        g = got.cpu().numpy()
        if not np.array_equal(g, want):
            bad = np.argwhere(g != want)
            raise AssertionError(f"{name}: {len(bad)} bytes differ, first at {bad[:3].tolist()}: "
                                 f"got {g[tuple(bad[0])]:#x} want {want[tuple(bad[0])]:#x}")


@pytest.mark.parametrize("name", ["tiny", "prefill_2k", "append_stress"])
def test_append_bitexact_full(K, oracle, name):
    banner(f"append bit-exact {name}")
    if name == "append_stress":
        w = W.append_stress("cuda")
        k, v, slots, P = w.k, w.v, w.slot_mapping, w.num_pages
    else:
        w = getattr(W, name)("cuda")
        k, v, slots, P = w.k, w.v, w.slot_mapping, w.num_pages
    err = K.device_error_word("cuda")
    err.zero_()
    cache = _gpu_append(K, k, v, slots, w.k_scale, w.v_scale, P, w.page_size, err)
    ref, oerr = _oracle_cache(oracle, k, v, slots, w.k_scale, w.v_scale, P, w.page_size)
    assert oerr == 0
    _compare(cache, ref)
    assert K.read_device_error("cuda") == 0


def test_append_bitexact_special_values(K, oracle):
    """Blocks with inf, NaN, -0, huge and tiny values (the kernel's rare path
    and saturation), with scales that push the E4M3 scale into saturation and
    into its subnormal range."""
    banner("append special values")
    g = torch.Generator().manual_seed(7)
    T, H, D = 96, 2, 64
    x = torch.randn(T, H, D, generator=g) * torch.exp(torch.randn(T, H, 1, generator=g) * 6)
    x[0, 0, 3] = float("inf")
    x[1, 1, 17] = float("nan")
    x[2, 0, :16] = float("nan")
    x[3, 0, 5] = -float("inf")
    x[4, :, :] = -0.0
    x[5, 0, :16] = 3.0e38
    k = x.to(torch.bfloat16).cuda()
    v = (-x).to(torch.bfloat16).cuda()
    P, ps = 8, 16
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64).cuda()
    for ks, vs in [(1.0, 1.0), (1e-30, 7.5), (3.0e33, 1e-5), (2.0 ** -149, 1.0e38)]:
        cache = _gpu_append(K, k, v, slots, ks, vs, P, ps)
        ref, oerr = _oracle_cache(oracle, k, v, slots, ks, vs, P, ps)
        assert oerr == 0
        _compare(cache, ref)


@pytest.mark.parametrize("name", ["uniform_batch_1k", "ragged_chunked"])
def test_append_bitexact_large_batches(K, oracle, name):
    """The largest appends, every byte of the GPU caches against the oracle's:
    1024 requests x 1024 tokens (1,048,576 rows, 2 GiB of bf16 per tensor,
    65,536 pages, lognormal global scales), and the ragged batch's whole cache
    (256 requests, kv_len ~ U[1, 4096], permuted pages)."""
    banner(f"append bit-exact {name}")
    w = getattr(W, name)("cuda")
    err = K.device_error_word("cuda")
    err.zero_()
    cache = _gpu_append(K, w.k, w.v, w.slot_mapping, w.k_scale, w.v_scale, w.num_pages, w.page_size, err)
    assert K.read_device_error("cuda") == 0
    ref, oerr = _oracle_cache(oracle, w.k, w.v, w.slot_mapping, w.k_scale, w.v_scale, w.num_pages,
                              w.page_size)
    assert oerr == 0
    _compare(cache, ref)


@pytest.mark.parametrize("H,D", [(1, 16), (3, 48), (2, 48), (5, 32)])
def test_append_bitexact_block_counts(K, oracle, H, D):
    """Token rows with an odd number of 16-element blocks (the half-block
    kernel: H=1 D=16, H=3 D=48) and with an even number whose two-block units
    straddle head boundaries (H=2 D=48, H=5 D=32)."""
    banner(f"append bit-exact H={H} D={D}")
    g = torch.Generator().manual_seed(11 + H * D)
    T, P, ps = 77, 8, 16
    k = torch.randn(T, H, D, generator=g).to(torch.bfloat16).cuda()
    v = (torch.randn(T, H, D, generator=g) * 3).to(torch.bfloat16).cuda()
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64).cuda()
    for ks, vs in [(1.0, 1.0), (0.01, 0.2)]:
        cache = _gpu_append(K, k, v, slots, ks, vs, P, ps)
        ref, oerr = _oracle_cache(oracle, k, v, slots, ks, vs, P, ps)
        assert oerr == 0
        _compare(cache, ref)


@pytest.mark.parametrize("bad", [0.0, -1.0, -0.0, float("nan"), float("inf"), float("-inf")])
def test_bad_device_scale_sets_flag_and_writes_nothing(K, bad):
    banner(f"bad device scale {bad}")
    w = W.tiny("cuda")
    for which in ("k", "v"):
        ks = torch.full((), bad if which == "k" else 1.0, device="cuda")
        vs = torch.full((), bad if which == "v" else 1.0, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        cache = _gpu_append(K, w.k, w.v, w.slot_mapping, ks, vs, w.num_pages, w.page_size, err)
        bits = K.read_device_error(word=err)
        assert bits == (K.DEV_BAD_K_SCALE if which == "k" else K.DEV_BAD_V_SCALE)
        for t in (cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf):
            assert bool((t == SENTINEL).all())


def test_host_scale_raises_value_error(K):
    w = W.tiny("cuda")
    cache = K.PagedCache.empty(w.num_pages, w.page_size, 2, 64, "cuda")
    for bad in (0.0, -1.0, float("nan"), float("inf"), torch.tensor(-2.0)):
        with pytest.raises(ValueError, match="finite and greater than zero"):
            K.nvfp4_append_paged_kv(w.k, w.v, w.slot_mapping, bad, 1.0, cache.k_cache, cache.v_cache,
                                    cache.k_sf, cache.v_sf, w.page_size)


def test_zero_rows_launch_nothing_and_check_nothing(K):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = K.PagedCache.empty(4, 16, 2, 64, "cuda", fill=SENTINEL)
    z = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    nan = torch.full((), float("nan"), device="cuda")
    K.nvfp4_append_paged_kv(z, z, torch.zeros(0, dtype=torch.int64, device="cuda"), nan, nan,
                            cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf, 16, dev_error=err)
    assert K.read_device_error(word=err) == 0


@pytest.mark.parametrize("seed", range(16))
def test_append_random_shapes(K, oracle, seed):
    """Seeded random appends, whole caches compared byte for byte: 1-700
    tokens, 1/2/3/5/8 KV heads, head_dim 16/48/64/128, page sizes 1/5/16/64,
    values N(0, s) with s spanning 2^-20 .. 2^20 and some exact zeros, a few
    padding (-1) and out-of-range slots, global scales of either kind."""
    r = np.random.default_rng(3000 + seed)
    T = int(r.integers(1, 701))
    H = int(r.choice([1, 2, 3, 5, 8]))
    D = int(r.choice([16, 48, 64, 128]))
    ps = int(r.choice([1, 5, 16, 64]))
    P = (T + ps - 1) // ps + int(r.integers(1, 6))
    g = torch.Generator().manual_seed(3000 + seed)
    scale = 2.0 ** float(r.uniform(-20, 20))
    k = (torch.randn(T, H, D, generator=g) * scale).to(torch.bfloat16)
    v = (torch.randn(T, H, D, generator=g) * scale * 7).to(torch.bfloat16)
    k[torch.rand(T, H, D, generator=g) < 0.05] = 0.0
    slots = torch.randperm(P * ps, generator=g)[:T].to(torch.int64)
    n_bad = int(r.integers(0, 4))
    if n_bad:
        idx = torch.from_numpy(r.choice(T, size=min(n_bad, T), replace=False))
        slots[idx[: len(idx) // 2 + 1]] = -1
        slots[idx[len(idx) // 2 + 1:]] = P * ps + int(r.integers(0, 100))
    ks, vs = (1.0, 1.0) if r.random() < 0.3 else (float(scale * r.uniform(0.01, 1)) / 2688.0,
                                                    float(scale * 7 * r.uniform(0.01, 1)) / 2688.0)
    banner(f"append random shape {seed}: T={T} H={H} D={D} page={ps} P={P} scale={scale:.3g} bad slots {n_bad}")
    k, v, slots = k.cuda(), v.cuda(), slots.cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = _gpu_append(K, k, v, slots, ks, vs, P, ps, err)
    ref, oerr = _oracle_cache(oracle, k, v, slots, ks, vs, P, ps)
    got_bits = K.read_device_error(word=err)
    assert got_bits == oerr
    _compare(cache, ref)


def test_padding_and_out_of_range_slots(K, oracle):
    w = W.tiny("cuda")
    slots = w.slot_mapping.clone()
    slots[0] = -1
    slots[1] = w.num_pages * w.page_size
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = _gpu_append(K, w.k, w.v, slots, w.k_scale, w.v_scale, w.num_pages, w.page_size, err)
    assert K.read_device_error(word=err) == K.DEV_SLOT_OOB
    ref, oerr = _oracle_cache(oracle, w.k, w.v, slots, w.k_scale, w.v_scale, w.num_pages, w.page_size)
    assert oerr == 4
    _compare(cache, ref)


def test_append_does_not_synchronize(K):
    """A long device spin is still running when the call returns."""
    w = W.tiny("cuda")
    cache = K.PagedCache.empty(w.num_pages, w.page_size, 2, 64, "cuda")
    ks = torch.full((), 1.0, device="cuda")
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)
    K.nvfp4_append_paged_kv(w.k, w.v, w.slot_mapping, ks, ks, cache.k_cache, cache.v_cache,
                            cache.k_sf, cache.v_sf, w.page_size)
    assert not torch.cuda.current_stream().query()
    torch.cuda.synchronize()


def test_graph_replay_checks_device_scale(K, oracle):
    """Captured once; replayed with a good scale (correct bytes) and after the
    scale tensor is overwritten with NaN (flag set, nothing written)."""
    w = W.tiny("cuda")
    ks = torch.full((), 1.0, device="cuda")
    vs = torch.full((), 0.5, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = K.PagedCache.empty(w.num_pages, w.page_size, 2, 64, "cuda", fill=SENTINEL)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up outside capture
        K.nvfp4_append_paged_kv(w.k, w.v, w.slot_mapping, ks, vs, cache.k_cache, cache.v_cache,
                                cache.k_sf, cache.v_sf, w.page_size, dev_error=err)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        K.nvfp4_append_paged_kv(w.k, w.v, w.slot_mapping, ks, vs, cache.k_cache, cache.v_cache,
                                cache.k_sf, cache.v_sf, w.page_size, dev_error=err)
    ref, _ = _oracle_cache(oracle, w.k, w.v, w.slot_mapping, 1.0, 0.5, w.num_pages, w.page_size)
    for _ in range(3):
        for t in (cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf):
            t.fill_(SENTINEL)
        graph.replay()
        torch.cuda.synchronize()
        _compare(cache, ref)
        assert K.read_device_error(word=err) == 0
    for t in (cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf):
        t.fill_(SENTINEL)
    vs.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert K.read_device_error(word=err) == K.DEV_BAD_V_SCALE
    for t in (cache.k_cache, cache.v_cache, cache.k_sf, cache.v_sf):
        assert bool((t == SENTINEL).all())
