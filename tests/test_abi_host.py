"""CPU-only checks of the HIP library's host side: the C ABI exports, the
plan step (FlashInfer PR #5043 page tests: max lengths for int32 / uint32
lengths across batch and page sizes; PR #3575 page: uniform flag and L2
gate), and a host build of the kernels' codec helpers against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def K():
    import nvfp4_paged_kv_amd as K
    K.lib()
    return K


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "nvfp4kv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol(K):
    names = _declared_functions()
    assert set(names) == set(K.ENTRY_POINTS), names
    L = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert K.lib().nvfp4kv_abi_version() == 105
    assert K.lib().nvfp4kv_status_string(-3).startswith(b"inconsistent")


def _plan(K, qo, kv, hq=32, hk=8, d=128, ps=16, cu_count=256, **kw):
    return K.plan(torch.as_tensor(qo), torch.as_tensor(kv), hq, hk, d, ps, l2_bytes=32 << 20,
                  cu_count=cu_count, **kw)


def test_plan_split_workspace_layout(K):
    """Workspace = work list (16 B per item) + 8 B of counters per split tile
    + one partial (rows x 128 fp32 O^T + rows fp32 max + rows fp32 sum) per
    chunk slot; rows = 32 x tile waves."""
    for waves in (4, 8):
        p = _plan(K, [0, 2048], [2048], split_len=5, tile_waves=waves)
        rows = 32 * waves
        part = rows * 128 * 4 + rows * 8
        lst = (p.num_items * 16 + 255) // 256 * 256
        cnt = (lst + p.num_split_tiles * 8 + 255) // 256 * 256
        assert p.block_q == rows // 4 and p.num_split_tiles > 0
        assert p.workspace_bytes == cnt + p.num_split_tiles * p.max_chunks * part


def _expected_split(qs, kvs, hk, bq, slots, split_len=0):
    """(split_len, max_chunks, num_items, num_split_tiles) by the documented
    rule: chunk length = max(total KV tiles / workgroup slots, 8), at least
    max cost / 16; Q tiles costlier than that are split evenly."""
    costs = [(kv - q + min((t + 1) * bq, q) - 1) // 64 + 1
             for q, kv in zip(qs, kvs) for t in range((q + bq - 1) // bq)]
    ntiles = len(costs) * hk
    if split_len < 0 or (split_len == 0 and ntiles >= slots) or not costs:
        return 0, 0, ntiles, 0
    total = sum(costs) * hk
    ln = split_len if split_len > 0 else max(-(-total // slots), 8)
    ln = max(ln, -(-max(costs) // 16))
    if max(costs) <= ln:
        return 0, 0, ntiles, 0
    nch = [-(-c // ln) for c in costs]
    return ln, -(-max(costs) // ln), sum(nch) * hk, sum(n > 1 for n in nch) * hk


@pytest.mark.parametrize("dtype", [torch.int32, torch.uint32])
@pytest.mark.parametrize("batch", [1, 7, 64, 1024])
@pytest.mark.parametrize("page_size", [1, 16, 64])
def test_plan_max_lens(K, dtype, batch, page_size):
    g = torch.Generator().manual_seed(batch * 131 + page_size)
    kv = torch.randint(1, 5000, (batch,), generator=g)
    q = torch.minimum(kv, torch.randint(0, 700, (batch,), generator=g))
    qo = torch.zeros(batch + 1, dtype=torch.int64)
    qo[1:] = torch.cumsum(q, 0)
    npg = (kv + page_size - 1) // page_size
    kvp = torch.zeros(batch + 1, dtype=torch.int64)
    kvp[1:] = torch.cumsum(npg, 0)
    p = K.plan(qo.to(torch.int32), kv.to(dtype), 32, 8, 128, page_size, kv_indptr=kvp.to(torch.int32),
               l2_bytes=32 << 20, cu_count=256)
    assert p.max_q_len == int((qo[1:] - qo[:-1]).max())
    assert p.max_kv_len == int(kv.max())
    assert p.total_q == int(q.sum()) and p.total_kv == int(kv.sum())
    assert p.uniform_q == int(bool((q == q.max()).all()))
    # head_dim 128: 8-wave tiles (256 rows = 64 tokens x 4 query heads) when
    # the batch has at least 4 of them per CU (256 CUs), else 4-wave tiles
    wide = 8 * int(((q + 63) // 64).sum()) >= 4 * 256
    bq = 64 if wide else 32
    assert p.block_q == bq
    assert p.num_tiles == 8 * int(((q + bq - 1) // bq).sum())
    assert p.max_tile_cost == int(((kv - 1) // 64 + 1)[q > 0].max()) if (q > 0).any() else True
    assert p.kv_bytes == int(kv.sum()) * 8 * (64 + 8) * 2
    assert p.head_first == int(2 * p.kv_bytes <= (32 << 20))
    assert (p.workspace_bytes == 0) == (bool(p.uniform_q) and p.split_len == 0)
    # issue order: heaviest first when the KV fits in L2, else stream order
    # where it is available (no split; 8 KV heads; at most 8192 requests);
    # paired instead of heaviest first for uniform batches of 4-wave tiles
    # that fill the 512 workgroup slots with nothing split
    first = K.SCHEDULE_HEAVIEST if p.head_first or p.split_len > 0 else K.SCHEDULE_STREAM
    if first == K.SCHEDULE_HEAVIEST and p.uniform_q and not wide and p.split_len == 0 \
            and p.num_tiles >= 512:
        first = K.SCHEDULE_PAIRED
    assert p.schedule == first
    assert p.cu_count == 256


def test_plan_uniform_flags_and_tiles(K):
    p = _plan(K, [0, 1024, 2048], [1024, 1024])
    assert p.uniform_q == 1 and p.uniform_kv == 1
    assert p.block_q == 32 and p.q_tiles_per_head == 32 and p.num_tiles == 2 * 8 * 32
    # one 2048-token request: 512 4-wave tiles fill the 2 x 256 slots; no split
    p = _plan(K, [0, 2048], [2048])
    assert p.head_first == 1 and p.num_tiles == 8 * 64 and p.block_q == 32
    assert p.split_len == 0 and p.num_items == p.num_tiles and p.workspace_bytes == 0
    # forced 8-wave tiles: 256 tiles, one slot each; a forced chunk length of
    # 17 splits the tiles of cost 18..32 in two
    q = _plan(K, [0, 2048], [2048], tile_waves=8)
    assert q.block_q == 64 and q.num_tiles == 256 and q.split_len == 0
    q = _plan(K, [0, 2048], [2048], tile_waves=8, split_len=17)
    assert (q.split_len, q.max_chunks, q.num_split_tiles, q.num_items) == (17, 2, 8 * 15, 8 * (17 + 2 * 15))
    q = _plan(K, [0, 2048], [2048], split_len=4)
    assert q.split_len == 4 and q.max_chunks == 8
    q = _plan(K, [0, 2048], [2048], split_len=-1, tile_waves=4)
    assert q.split_len == 0 and q.workspace_bytes == 0
    p = _plan(K, list(range(0, 1025 * 1024, 1024)), [1024] * 1024)
    assert p.block_q == 64 and p.num_tiles == 1024 * 8 * 16 and p.head_first == 0 and p.split_len == 0
    p = _plan(K, [0, 10, 20], [10, 30])
    assert p.uniform_q == 1 and p.uniform_kv == 0
    p = _plan(K, [0, 10, 25], [10, 30])
    assert p.uniform_q == 0 and p.workspace_bytes >= p.num_tiles * 8
    p = _plan(K, [0, 128, 256], [128, 128], hq=4, hk=2, d=64)
    assert p.block_q == 64 and p.num_tiles == 8 and p.split_len == 0


@pytest.mark.parametrize("qs,kvs", [([512], [8192]), ([300, 40, 1000], [9000, 40, 3000]),
                                    ([64] * 3, [20000] * 3), ([2048], [2048])])
@pytest.mark.parametrize("waves", [0, 4, 8])
def test_plan_auto_split(K, qs, kvs, waves):
    """Batches that cannot fill every workgroup slot split their heavy Q
    tiles' KV ranges (chunked prefill of a short chunk over a long cache)."""
    qo = [0] + list(np.cumsum(qs))
    p = _plan(K, qo, kvs, tile_waves=waves)
    wide = waves == 8 or (waves == 0 and 8 * sum((q + 63) // 64 for q in qs) >= 1024)
    bq, slots = (64, 256) if wide else (32, 512)
    assert p.block_q == bq
    got = (p.split_len, p.max_chunks, p.num_items, p.num_split_tiles)
    assert got == _expected_split(qs, kvs, 8, bq, slots), got
    if qs == [512]:
        assert p.split_len > 0 and p.max_chunks > 1


def test_plan_rejects_bad_lengths(K):
    with pytest.raises(ValueError):
        _plan(K, [0, 10], [9])                       # q_len > kv_len
    with pytest.raises(ValueError):
        _plan(K, [1, 10], [20])                      # qo_indptr[0] != 0
    with pytest.raises(ValueError):
        _plan(K, [0, 10], [20], kv_indptr=torch.tensor([0, 3], dtype=torch.int32))  # needs 2 pages
    with pytest.raises(K.NVFP4KVError):
        _plan(K, [0, 10], [20], d=96)
    with pytest.raises(K.NVFP4KVError):
        _plan(K, [0, 10], [20], hq=24, hk=8)
    with pytest.raises(ValueError):
        _plan(K, [0, 10], [20], tile_waves=6)
    with pytest.raises(ValueError):
        _plan(K, [0, 10], [20], hq=4, hk=2, d=64, tile_waves=8)
    p = _plan(K, [0], [])
    assert p.num_tiles == 0


def test_decode_plan_chunks_and_workspace(K):
    """Chunk length: a multiple of 64 and at least 256 keys when automatic (its
    size also depends on the CU count), or as forced; workspace = one
    (D + 4)-float partial per (request, query head, chunk) when some request
    has two chunks."""
    kv = torch.tensor([1, 300, 4096, 65], dtype=torch.int32)
    p = K.decode_plan(kv, 32, 8, 128, 16)
    assert p.chunk_len % 64 == 0 and p.chunk_len >= 256
    # two KV heads per wave (head_dim 128: 2 x 64 code bytes fill a 128-byte line)
    assert p.heads_per_wave == 2
    assert p.max_chunks == -(-4096 // p.chunk_len) and p.num_items == 4 * 4 * p.max_chunks
    assert p.max_kv_len == 4096 and p.total_kv == int(kv.sum())
    assert p.workspace_bytes == (4 * 32 * p.max_chunks * (128 + 4) * 4 if p.max_chunks > 1 else 0)
    q = K.decode_plan(kv, 32, 8, 128, 16, chunk_len=128)
    assert q.chunk_len == 128 and q.max_chunks == 32 and q.num_items == 4 * 4 * 32
    q = K.decode_plan(torch.tensor([100, 20], dtype=torch.int32), 8, 2, 64, 16, chunk_len=128)
    assert q.max_chunks == 1 and q.workspace_bytes == 0
    with pytest.raises(ValueError):
        K.decode_plan(kv, 32, 8, 128, 16, chunk_len=100)   # not a multiple of 64
    with pytest.raises(ValueError):
        K.decode_plan(torch.tensor([5, 0], dtype=torch.int32), 32, 8, 128, 16)  # kv_len < 1
    with pytest.raises(K.NVFP4KVError):
        K.decode_plan(kv, 24, 8, 128, 16)                  # GQA group 3
    p = K.decode_plan(torch.tensor([], dtype=torch.int32), 32, 8, 128, 16)
    assert p.num_items == 0 and p.workspace_bytes == 0


@pytest.mark.parametrize("hq,hk,d,hp", [
    (32, 8, 128, 2), (64, 8, 128, 2), (8, 8, 128, 2), (3, 3, 128, 1), (4, 1, 128, 1), (6, 3, 128, 1),
    (16, 8, 64, 4), (16, 4, 64, 4), (8, 8, 64, 4), (64, 8, 64, 2), (16, 2, 64, 2), (12, 6, 64, 2),
    (8, 1, 64, 1), (5, 5, 64, 1)])
def test_decode_plan_heads_per_wave(K, hq, hk, d, hp):
    """Adjacent KV heads per decode wave: as many as fill a 128-byte line of
    the code row (256 / head_dim), halved until the wave's query heads fit 16
    columns and the count divides the KV heads; the wave count follows."""
    kv = torch.tensor([700, 64, 1], dtype=torch.int32)
    p = K.decode_plan(kv, hq, hk, d, 16, chunk_len=256)
    assert p.heads_per_wave == hp
    assert p.num_items == 3 * (hk // hp) * 3


def test_decode_plan_fills_one_round_of_waves(K):
    """32 requests x 8192 keys, 32/8 heads, head_dim 128 on 256 CUs: two KV
    heads per wave, 512-key chunks, 16 chunks per request, 2,048 waves (eight
    per CU, one round of the 8-wave workgroups)."""
    p = K.decode_plan(torch.full((32,), 8192, dtype=torch.int32), 32, 8, 128, 16)
    assert (p.heads_per_wave, p.chunk_len, p.max_chunks, p.num_items) == (2, 512, 16, 2048)
    assert p.workspace_bytes == 32 * 32 * 16 * (128 + 4) * 4


@pytest.mark.parametrize("field,value", [("heads_per_wave", 1), ("heads_per_wave", 4), ("num_items", -1),
                                         ("num_items", +1)])
def test_decode_rejects_a_plan_whose_waves_do_not_match_its_shape(K, field, value):
    """paged_decode maps every wave below num_items to a (request, chunk, head
    group); a plan whose heads_per_wave or num_items differs from what its
    shape gives is refused with EINVAL before anything is launched (the
    pointers here are placeholders that are never dereferenced)."""
    kv = torch.tensor([700, 64, 1], dtype=torch.int32)
    p = K.decode_plan(kv, 32, 8, 128, 16, chunk_len=256)
    st = K.DecodePlanStruct.from_buffer_copy(p.struct)
    if field == "heads_per_wave":
        st.heads_per_wave = value
    else:
        st.num_items = st.num_items + value
    fake = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never touched
    cache = K.Cache(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 64, 16, 8, 128)
    rc = K.lib().paged_decode(fake, fake, fake, fake, ctypes.byref(cache), fake, ctypes.c_float(0.088),
                              ctypes.byref(st), fake, ctypes.c_int64(1 << 30), fake, None)
    assert rc == K.EINVAL


def test_plan_empty_requests(K):
    p = _plan(K, [0, 0, 5], [7, 5])
    assert p.max_q_len == 5 and p.total_q == 5 and p.num_tiles == 8 and p.uniform_q == 0


@pytest.fixture(scope="module")
def host_codec():
    path = os.path.join(HERE, "libcodec_host.so")
    if not os.path.exists(path):
        from nvfp4_paged_kv_amd.build import build_test_helpers
        build_test_helpers()
    return ctypes.CDLL(path)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def test_kernel_software_e2m1_matches_oracle(host_codec, oracle):
    """Every fp32 pattern of magnitude below 8 (then a stride above) through the
    kernels' software E2M1 encoder (host build) and the oracle."""
    chunk = 1 << 26
    for lo in list(range(0, 0x41000000, chunk)) + [0x41000000 + i * 0x1000000 for i in range(0x3E)]:
        pats = np.arange(lo, lo + chunk if lo < 0x41000000 else lo + (1 << 20), dtype=np.uint32)
        pats = pats[pats <= 0x7F800000]
        for sign in (0, 0x80000000):
            p = pats | np.uint32(sign)
            got = np.empty(p.size, np.uint8)
            host_codec.host_e2m1_sw(_p(p), ctypes.c_int64(p.size), _p(got))
            assert np.array_equal(got, oracle.e2m1_encode(p.view(np.float32))), hex(lo)


def test_kernel_e4m3_encode_decode_matches_oracle(host_codec, oracle):
    top = 0x7F800000
    rng = np.random.default_rng(0)
    pats = np.concatenate([np.arange(0, 0x3C800000 + 4096, 64, dtype=np.uint32),
                           np.arange(0x3A000000, 0x44000000, 3, dtype=np.uint32),
                           rng.integers(0, top + 1, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    s = pats.view(np.float32)
    got = np.empty(s.size, np.uint8)
    host_codec.host_e4m3(_p(s), ctypes.c_int64(s.size), _p(got))
    assert np.array_equal(got, oracle.e4m3_encode(s))
    codes = np.arange(0x7F, dtype=np.uint8)
    dec = np.empty(codes.size, np.float32)
    host_codec.host_e4m3_decode(_p(codes), ctypes.c_int64(codes.size), _p(dec))
    assert [float(x) for x in dec] == [oracle.e4m3_value(int(c)) for c in codes]
    host_codec.host_scale_ok.restype = ctypes.c_int
    host_codec.host_scale_ok.argtypes = [ctypes.c_float]
    for g in [1.0, 1e-40, 3e38, 0.0, -0.0, -1.0, float("nan"), float("inf"), -float("inf")]:
        assert bool(host_codec.host_scale_ok(g)) == oracle.scale_ok(g), g


def test_fastdiv(host_codec):
    rng = np.random.default_rng(1)
    n = np.concatenate([np.arange(0, 5000, dtype=np.uint32), np.array([2**32 - 1, 2**31, 2**31 - 1], np.uint32),
                        rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)])
    q = np.empty_like(n)
    for d in [1, 2, 3, 7, 8, 16, 17, 64, 100, 1000, 65535, 65536, 123457, 2**31 - 1]:
        host_codec.host_fastdiv(_p(n), ctypes.c_int64(n.size), ctypes.c_uint32(d), _p(q))
        assert np.array_equal(q, n // np.uint32(d)), d


def test_plan_bench_paths_agree(K):
    """The plan micro-benchmark's three paths compute the same maxima and
    totals on a seeded ragged batch (the benchmark asserts it before timing)."""
    import bench
    res = bench.bench_plan(K, torch, np, batches=(64,), reps=2)
    assert set(res["64"]) == {"native_us", "python_loop_us", "torch_vectorised_us"}


def test_plan_cu_count_is_an_explicit_input(K):
    """The CU count the plan sizes tiles and splits for is its own argument,
    independent of the L2 capacity given to the gate: 512 4-wave tiles fill
    the 2 x 256 slots of 256 CUs (no split) but not the 2 x 304 of 304 CUs
    (their heavy tiles are split); the L2 size alone changes neither."""
    p = _plan(K, [0, 2048], [2048], cu_count=256)
    assert p.cu_count == 256 and p.split_len == 0 and p.num_xcd == 8
    q = _plan(K, [0, 2048], [2048], cu_count=304)
    assert q.cu_count == 304 and q.split_len > 0 and q.num_xcd == 9
    expect = _expected_split([2048], [2048], 8, 32, 2 * 304)
    assert (q.split_len, q.max_chunks, q.num_items, q.num_split_tiles) == expect
    r = K.plan(torch.tensor([0, 2048]), torch.tensor([2048]), 32, 8, 128, 16, l2_bytes=1 << 40,
               cu_count=256)
    assert (r.split_len, r.num_items, r.head_first) == (0, p.num_items, 1)
    with pytest.raises(ValueError):
        K.plan(torch.tensor([0, 16]), torch.tensor([16]), 32, 8, 128, 16, cu_count=-1)
    with pytest.raises(ValueError):
        K.plan(torch.tensor([0, 16]), torch.tensor([16]), 32, 8, 128, 16, l2_bytes=-5)


def test_plan_schedule_override(K):
    """A caller-chosen issue order is kept in the plan as given."""
    p = _plan(K, [0, 2048], [2048], schedule=K.SCHEDULE_REQUEST)
    assert p.schedule == K.SCHEDULE_REQUEST
    p = _plan(K, [0, 2048], [2048], schedule=K.SCHEDULE_HEAVIEST)
    assert p.schedule == K.SCHEDULE_HEAVIEST


def test_plan_paired_choice(K):
    """The plan pairs light and heavy Q tiles (schedule 4) only for uniform
    batches of 4-wave tiles that fill every workgroup slot (two per CU)
    unsplit, with the KV in L2; otherwise it keeps its other orders."""
    p = _plan(K, [0, 2048], [2048])  # 64 Q tiles x 8 heads = 512 = 2 x 256 CUs
    assert (p.schedule, p.block_q, p.split_len, p.head_first) == (K.SCHEDULE_PAIRED, 32, 0, 1)
    assert p.dequant_mode == 3  # bf16 staging, bf16 matrix instructions
    assert _plan(K, [0, 2048], [2048], dequant_mode=0).dequant_mode == 0
    assert p.num_items == p.num_tiles == 512
    p = _plan(K, [0, 2048], [2048], cu_count=304)  # 512 < 608 slots: split instead
    assert p.split_len > 0 and p.schedule == K.SCHEDULE_HEAVIEST
    p = _plan(K, [0, 2048], [2048], cu_count=304, split_len=-1)  # unsplit, slots not filled
    assert p.schedule == K.SCHEDULE_HEAVIEST
    p = _plan(K, [0, 2048, 4100], [2048, 2052])  # ragged: work list
    assert p.schedule == K.SCHEDULE_HEAVIEST
    p = _plan(K, [0, 2048], [2048], tile_waves=8)  # 8-wave tiles
    assert p.schedule == K.SCHEDULE_HEAVIEST
    p = _plan(K, [0, 2048, 4096], [2048, 2048])  # two requests, 1024 tiles
    assert p.schedule == K.SCHEDULE_PAIRED
    p = _plan(K, [0, 2048], [1 << 20])  # KV beyond L2: stream order
    assert p.schedule == K.SCHEDULE_STREAM
    p = _plan(K, [0, 4096], [4096], hq=16, hk=8, d=64)  # head_dim 64: 64 x 8 tiles
    assert p.schedule == K.SCHEDULE_PAIRED


def test_attention_entry_points_reject_bad_sm_scale(K):
    """sm_scale must be positive and finite: checked by the C entry points
    before anything is read or enqueued (null buffers are never touched)."""
    p = _plan(K, [0, 64], [64])
    L = K.lib()
    for bad in (0.0, -0.125, float("nan"), float("inf")):
        st = L.paged_prefill_causal(None, None, None, None, None, ctypes.byref(K.Cache()), None, bad,
                                    ctypes.byref(p.struct), None, 0, None, None)
        assert st == K.EINVAL, bad
        d = K.decode_plan(torch.tensor([64], dtype=torch.int32), 32, 8, 128, 16)
        st = L.paged_decode(None, None, None, None, ctypes.byref(K.Cache()), None, bad,
                            ctypes.byref(d.struct), None, 0, None, None)
        assert st == K.EINVAL, bad


def test_binding_checks_batch_array_sizes(K):
    """The binding compares the per-request arrays with the plan before any
    launch (host-side sizes only): qo_indptr and kv_indptr need batch + 1
    entries, kv_lens batch, the page table at least the pages the requests
    own."""
    qo, kv = torch.tensor([0, 16, 48], dtype=torch.int32), torch.tensor([40, 32], dtype=torch.int32)
    kvp = torch.tensor([0, 3, 5], dtype=torch.int32)
    p = K.plan(qo, kv, 8, 2, 64, 16, kv_indptr=kvp)
    q = torch.zeros((48, 8, 64), dtype=torch.bfloat16)
    out = torch.empty_like(q)
    pt = torch.arange(5, dtype=torch.int32)
    cache = K.PagedCache(*(torch.zeros(1, dtype=torch.uint8) for _ in range(4)),
                         torch.ones(()), torch.ones(()))
    cases = [(qo[:2], kvp, kv, pt, "qo_indptr"), (qo, kvp[:2], kv, pt, "kv_indptr"),
             (qo, kvp, kv[:1], pt, "kv_lens"), (qo, kvp, kv, pt[:4], "page_table")]
    for a, b, c, d, name in cases:
        with pytest.raises(ValueError, match=name):
            K._check_batch_arrays(p, a, b, c, d)
    K._check_batch_arrays(p, qo, kvp, kv, pt)
