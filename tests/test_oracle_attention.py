"""Pins for the oracle's append (scatter) and causal paged prefill (CPU only).

References that do not come from the oracle: a dense numpy attention with an
explicit mask matrix, over K/V decoded with the OCP grid table and torch's
float8_e4m3fn decode; closed forms; and invariants (causality, GQA grouping,
page relabelling, chunked-prefill alignment).
"""
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENTINEL = 0xA5


def _grid():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt")) if l.strip() and not l.startswith("#")]
    g = np.zeros(16)
    for c, v in rows:
        g[int(c)] = float(v)
    return g


E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def empty_cache(P, ps, H, D):
    return [np.full((P, ps, H, D // 2), SENTINEL, np.uint8), np.full((P, ps, H, D // 2), SENTINEL, np.uint8),
            np.full((P, ps, H, D // 16), SENTINEL, np.uint8), np.full((P, ps, H, D // 16), SENTINEL, np.uint8)]


def fill(oracle, w):
    caches = empty_cache(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    err = oracle.append(W.bf16_bits(w.k), W.bf16_bits(w.v), w.slot_mapping.numpy(), w.k_scale,
                        w.v_scale, *caches, w.page_size)
    assert err == 0
    return caches


def decode_numpy(cache, sf, g):
    """[P, ps, H, D/2] bytes + [P, ps, H, D/16] scales -> fp64 [P, ps, H, D]."""
    grid = _grid()
    lo, hi = cache & 15, cache >> 4
    codes = np.stack([lo, hi], -1).reshape(*cache.shape[:-1], cache.shape[-1] * 2)
    S = np.repeat(E4M3[sf], 16, axis=-1)
    return grid[codes] * S * g


def dense_reference(w, caches):
    """Explicit mask-matrix attention per request and head (numpy, fp64)."""
    kc, vc, ksf, vsf = caches
    K = decode_numpy(kc, ksf, w.k_scale)
    V = decode_numpy(vc, vsf, w.v_scale)
    q = w.q.double().numpy()
    G = w.num_q_heads // w.num_kv_heads
    out = np.zeros(q.shape)
    for r in range(w.batch):
        Lq, Lk = int(w.q_lens[r]), int(w.kv_lens[r])
        pages = w.page_table[w.kv_indptr[r]:w.kv_indptr[r + 1]]
        j = np.arange(Lk)
        Kr = K[pages[j // w.page_size], j % w.page_size]  # [Lk, H, D]
        Vr = V[pages[j // w.page_size], j % w.page_size]
        mask = np.arange(Lk)[None, :] <= (Lk - Lq + np.arange(Lq))[:, None]
        for hq in range(w.num_q_heads):
            qr = q[w.qo_indptr[r]:w.qo_indptr[r + 1], hq]
            s = w.sm_scale * qr @ Kr[:, hq // G].T
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            out[w.qo_indptr[r]:w.qo_indptr[r + 1], hq] = p @ Vr[:, hq // G]
    return out


def run_oracle(oracle, w, caches, **kw):
    out, err = oracle.prefill(W.bf16_bits(w.q), w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens,
                              *caches, w.k_scale, w.v_scale, w.num_q_heads, w.sm_scale, **kw)
    assert err == 0
    return out


def small(seed=0, q=(5, 33, 17), kv=(9, 33, 50), H=(4, 2), D=32, scales="amax", std=1.0):
    return W.make_attention("t", list(q), list(kv), H[0], H[1], D, 16, 16, seed=seed,
                            device="cpu", scales=scales, std=std)


# ---------------------------------------------------------------- append ---

def test_append_gather_back_and_sentinel(oracle):
    w = small(1)
    caches = fill(oracle, w)
    slots = w.slot_mapping.numpy()
    kc, vc, ksf, vsf = [c.reshape(-1, c.shape[2], c.shape[3]) for c in caches]
    kb = W.bf16_bits(w.k)
    for t in range(0, len(slots), 7):
        for h in range(w.num_kv_heads):
            for b in range(w.head_dim // 16):
                p, sf = oracle.quantize_block(kb[t, h, 16 * b:16 * b + 16], w.k_scale)
                assert kc[slots[t], h, 8 * b:8 * b + 8].tolist() == p.tolist()
                assert ksf[slots[t], h, b] == sf
    untouched = np.setdiff1d(np.arange(kc.shape[0]), slots)
    assert untouched.size > 0
    for c in (kc, vc, ksf, vsf):
        assert (c[untouched] == SENTINEL).all()


def test_append_page_relabel_permutes_bytes(oracle):
    w = small(2)
    a = fill(oracle, w)
    perm = np.random.default_rng(0).permutation(w.num_pages)
    slots = w.slot_mapping.numpy()
    s2 = perm[slots // w.page_size] * w.page_size + slots % w.page_size
    b = empty_cache(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    assert oracle.append(W.bf16_bits(w.k), W.bf16_bits(w.v), s2.astype(np.int64), w.k_scale,
                         w.v_scale, *b, w.page_size) == 0
    for x, y in zip(a, b):
        assert np.array_equal(x, y[perm])


@pytest.mark.parametrize("bad", [0.0, -0.0, -1.0, float("nan"), float("inf"), float("-inf")])
@pytest.mark.parametrize("which", ["k", "v", "both"])
def test_append_bad_scale_writes_nothing(oracle, bad, which):
    w = small(3)
    caches = empty_cache(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    ks = bad if which in ("k", "both") else 1.0
    vs = bad if which in ("v", "both") else 1.0
    err = oracle.append(W.bf16_bits(w.k), W.bf16_bits(w.v), w.slot_mapping.numpy(), ks, vs,
                        *caches, w.page_size)
    assert err == {"k": 1, "v": 2, "both": 3}[which]
    assert all((c == SENTINEL).all() for c in caches)


def test_append_zero_rows_checks_nothing(oracle):
    caches = empty_cache(4, 16, 2, 32)
    z = np.zeros((0, 2, 32), np.uint16)
    assert oracle.append(z, z, np.zeros(0, np.int64), float("nan"), -1.0, *caches, 16) == 0
    assert all((c == SENTINEL).all() for c in caches)


def test_append_negative_slot_skipped_and_oob_flagged(oracle):
    w = small(4)
    caches = empty_cache(w.num_pages, w.page_size, w.num_kv_heads, w.head_dim)
    slots = w.slot_mapping.numpy().copy()
    slots[0] = -1
    slots[1] = w.num_pages * w.page_size  # one past the pool
    err = oracle.append(W.bf16_bits(w.k), W.bf16_bits(w.v), slots, w.k_scale, w.v_scale,
                        *caches, w.page_size)
    assert err == 4
    ref = fill(oracle, w)
    s0 = w.slot_mapping.numpy()[:2]
    for c, r in zip(caches, ref):
        cf, rf = c.reshape(-1, *c.shape[2:]), r.reshape(-1, *r.shape[2:])
        assert (cf[s0] == SENTINEL).all()
        keep = np.setdiff1d(np.arange(cf.shape[0]), s0)
        assert np.array_equal(cf[keep], rf[keep])


# --------------------------------------------------------------- prefill ---

@pytest.mark.parametrize("seed,H,D", [(0, (4, 2), 32), (1, (6, 3), 64), (2, (8, 1), 16), (3, (2, 2), 48)])
def test_prefill_vs_dense_numpy(oracle, seed, H, D):
    w = small(seed, H=H, D=D)
    caches = fill(oracle, w)
    got = run_oracle(oracle, w, caches)
    ref = dense_reference(w, caches)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_prefill_rows_sum_to_one(oracle):
    """V decoding to exactly 1 everywhere (code 2 = 1.0, scale byte 0x38 = 1.0,
    g_v = 1): every output element equals the softmax row sum."""
    w = small(5, scales="one")
    kc, vc, ksf, vsf = fill(oracle, w)
    vc[:] = 0x22
    vsf[:] = 0x38
    out = run_oracle(oracle, w, [kc, vc, ksf, vsf])
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_prefill_closed_forms(oracle):
    w = small(6, q=(1, 20, 12), kv=(1, 20, 30))
    caches = fill(oracle, w)
    out = run_oracle(oracle, w, caches)
    K = decode_numpy(caches[1], caches[3], w.v_scale)  # V decoded
    G = w.num_q_heads // w.num_kv_heads

    def vhat(r, j, h):
        page = w.page_table[w.kv_indptr[r] + j // w.page_size]
        return K[page, j % w.page_size, h]

    for hq in range(w.num_q_heads):
        # Lq = Lk = 1: the single key gets weight 1.
        np.testing.assert_allclose(out[0, hq], vhat(0, 0, hq // G), rtol=1e-15, atol=0)
        # first row of a Lq = Lk request sees only key 0.
        np.testing.assert_allclose(out[w.qo_indptr[1], hq], vhat(1, 0, hq // G), rtol=1e-15, atol=0)
    # q = 0: uniform weights -> mean of the allowed V rows.
    w.q.zero_()
    out0 = run_oracle(oracle, w, caches)
    r, Lq, Lk = 2, 12, 30
    for i in (0, 5, 11):
        n = Lk - Lq + i + 1
        for hq in range(w.num_q_heads):
            mean = np.mean([vhat(r, j, hq // G) for j in range(n)], axis=0)
            np.testing.assert_allclose(out0[w.qo_indptr[r] + i, hq], mean, rtol=1e-12, atol=1e-14)


def test_prefill_causal_future_keys_do_not_matter(oracle):
    w = small(7, q=(40,), kv=(40,))
    caches = fill(oracle, w)
    base = run_oracle(oracle, w, caches)
    # scramble every key/value at positions >= 25 (pages of the request)
    kc, vc, ksf, vsf = [c.copy() for c in caches]
    rng = np.random.default_rng(1)
    for j in range(25, 40):
        page = w.page_table[j // 16]
        for c in (kc, vc):
            c[page, j % 16] = rng.integers(0, 256, size=c[page, j % 16].shape)
        for c in (ksf, vsf):
            c[page, j % 16] = rng.integers(0, 0x7F, size=c[page, j % 16].shape)
    got = run_oracle(oracle, w, [kc, vc, ksf, vsf])
    assert np.array_equal(got[:25], base[:25])  # rows 0..24 see keys <= 24 only
    assert not np.array_equal(got[25:], base[25:])


def test_prefill_gqa_equals_replicated_mha(oracle):
    w = small(8, H=(6, 2), D=32)
    caches = fill(oracle, w)
    got = run_oracle(oracle, w, caches)
    # replicate each KV head G times -> H_kv = H_q, one Q head per KV head
    G = 3
    rep = [np.ascontiguousarray(np.repeat(c, G, axis=2)) for c in caches]
    out, err = oracle.prefill(W.bf16_bits(w.q), w.qo_indptr, w.kv_indptr, w.page_table, w.kv_lens,
                              *rep, w.k_scale, w.v_scale, 6, w.sm_scale)
    assert err == 0
    assert np.array_equal(got, out)


def test_prefill_page_relabel_invariance(oracle):
    w = small(9)
    caches = fill(oracle, w)
    got = run_oracle(oracle, w, caches)
    perm = np.random.default_rng(3).permutation(w.num_pages)  # new id of old page p is perm[p]
    moved = []
    for c in caches:
        m = np.empty_like(c)
        m[perm] = c
        moved.append(m)
    out, err = oracle.prefill(W.bf16_bits(w.q), w.qo_indptr, w.kv_indptr,
                              perm[w.page_table].astype(np.int32), w.kv_lens, *moved, w.k_scale,
                              w.v_scale, w.num_q_heads, w.sm_scale)
    assert err == 0 and np.array_equal(got, out)


def test_prefill_chunk_equals_tail_rows_of_full_prefill(oracle):
    """Bottom-right alignment: a trailing chunk of q_len rows over kv_len keys
    reproduces the last q_len rows of the full q_len = kv_len prefill."""
    Lk, Lq = 45, 13
    full = small(10, q=(Lk,), kv=(Lk,))
    caches = fill(oracle, full)
    ref = run_oracle(oracle, full, caches)
    chunk_q = full.q[Lk - Lq:].contiguous()
    out, err = oracle.prefill(W.bf16_bits(chunk_q), np.array([0, Lq], np.int32), full.kv_indptr,
                              full.page_table, full.kv_lens, *caches, full.k_scale, full.v_scale,
                              full.num_q_heads, full.sm_scale)
    assert err == 0
    assert np.array_equal(out, ref[Lk - Lq:])


def test_prefill_sampled_requests_and_errors(oracle):
    w = small(11)
    caches = fill(oracle, w)
    full = run_oracle(oracle, w, caches)
    part = run_oracle(oracle, w, caches, requests=[2])
    sl = slice(w.qo_indptr[2], w.qo_indptr[3])
    assert np.array_equal(part[sl], full[sl])
    assert np.isnan(part[:w.qo_indptr[2]]).all()
    bad_pt = w.page_table.copy()
    bad_pt[0] = w.num_pages
    _, err = oracle.prefill(W.bf16_bits(w.q), w.qo_indptr, w.kv_indptr, bad_pt, w.kv_lens, *caches,
                            w.k_scale, w.v_scale, w.num_q_heads, w.sm_scale)
    assert err & 8


def _flash_rows(q, K, V, sm_scale, nkeys, block, slack, chunks):
    """fp64 online softmax over the allowed keys of each row, in `block`-key
    tiles, with the reference max raised only when a tile's max exceeds it by
    more than `slack` (log2 units), the key range cut into `chunks` pieces
    whose (unnormalized O, max, sum) are merged in chunk order: the regrouping
    the prefill and decode kernels use (reading R26), written independently of
    the oracle."""
    out = np.zeros((q.shape[0], V.shape[1]))
    c = sm_scale / np.log(2.0)  # scores -> log2 domain
    for i in range(q.shape[0]):
        n = nkeys[i]
        bounds = [n * t // chunks for t in range(chunks + 1)]
        parts = []
        for a, b in zip(bounds[:-1], bounds[1:]):
            m, l, o = -np.inf, 0.0, np.zeros(V.shape[1])
            for t0 in range(a, b, block):
                s = (K[t0:min(t0 + block, b)] @ q[i]) * c
                mt = s.max()
                if mt > m + slack:  # lazy: raise the reference max only on large growth
                    alpha = np.exp2(m - mt) if m > -np.inf else 0.0
                    o *= alpha
                    l *= alpha
                    m = mt
                p = np.exp2(s - m)
                l += p.sum()
                o += p @ V[t0:min(t0 + block, b)]
            parts.append((m, l, o))
        mall = max(pm for pm, _, _ in parts if pm > -np.inf)
        L = sum(pl * np.exp2(pm - mall) for pm, pl, _ in parts if pm > -np.inf)
        O = sum(po * np.exp2(pm - mall) for pm, _, po in parts if pm > -np.inf)
        out[i] = O / L
    return out


@pytest.mark.parametrize("block,slack,chunks", [(64, 8.0, 1), (48, 8.0, 3), (7, 0.0, 2), (64, 8.0, 5)])
def test_online_softmax_regrouping_matches_definition(oracle, block, slack, chunks):
    """Tiled online softmax with lazy rescaling and chunk merging (the kernels'
    algorithm, in fp64) equals the oracle's plain definition to 1e-12, with
    tile sizes that do not divide the lengths and chunks that may be empty of
    tiles; scores are scaled up (std 4) so that the lazy max does lag."""
    w = small(11, q=(1, 37, 70), kv=(3, 90, 70), std=4.0)
    caches = fill(oracle, w)
    ref = run_oracle(oracle, w, caches)
    K = decode_numpy(caches[0], caches[2], w.k_scale)
    V = decode_numpy(caches[1], caches[3], w.v_scale)
    q = w.q.double().numpy()
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.batch):
        Lq, Lk = int(w.q_lens[r]), int(w.kv_lens[r])
        pages = w.page_table[w.kv_indptr[r]:w.kv_indptr[r + 1]]
        j = np.arange(Lk)
        Kr = K[pages[j // w.page_size], j % w.page_size]
        Vr = V[pages[j // w.page_size], j % w.page_size]
        nkeys = Lk - Lq + np.arange(Lq) + 1
        rows = slice(w.qo_indptr[r], w.qo_indptr[r + 1])
        for hq in range(w.num_q_heads):
            got = _flash_rows(q[rows, hq], Kr[:, hq // G], Vr[:, hq // G], w.sm_scale, nkeys, block,
                              slack, chunks)
            np.testing.assert_allclose(got, ref[rows, hq], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("D", [64, 128])
def test_dequant_rows_vs_table_decode(oracle, D):
    """oracle.dequant_rows (the helper the low-precision variant study builds
    its references from) against decode_numpy, which decodes with the OCP E2M1
    grid golden file and torch's float8_e4m3fn table: random code bytes
    (every nibble), random finite scale bytes, rows in a shuffled order with
    repeats, and a global scale that is not a power of two."""
    rng = np.random.default_rng(D)
    n_rows = 300
    cache = rng.integers(0, 256, (n_rows, D // 2), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, (n_rows, D // 16), dtype=np.uint8)  # finite E4M3FN codes
    rows = rng.integers(0, n_rows, 777).astype(np.int64)
    g = 0.0173
    got = oracle.dequant_rows(cache, sf, rows, D, g)
    ref = decode_numpy(cache, sf, g)[rows]
    assert got.shape == (rows.size, D)
    assert np.array_equal(got, ref)
    # a dropped nibble swap or a scale read from the neighbouring block would
    # show up on these hand-built rows
    c = np.zeros((1, D // 2), np.uint8)
    c[0, 0] = 0x1F  # element 0: code 0xF (-6), element 1: code 0x1 (0.5)
    s = np.full((1, D // 16), 0x38, np.uint8)  # 1.0
    s[0, 1] = 0x40  # block 1: 2.0
    c[0, 8] = 0x02  # element 16 (block 1): code 2 (1.0) -> 2.0
    one = oracle.dequant_rows(c, s, np.zeros(1, np.int64), D, 1.0)[0]
    assert one[0] == -6.0 and one[1] == 0.5 and one[16] == 2.0
    assert np.count_nonzero(one) == 3
