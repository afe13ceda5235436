"""fp64 emulation of the prefill's MX score variants (dequant modes 4 and 5),
for the tests: what the kernel's scaled matrix instruction is fed, rebuilt on
the CPU from the oracle's encoders and tables, and the attention over those
operands.

The PR #4769 page ("NVFP4 KV tile repack", code-analysis section) has a
branch for targets whose matrix cores take E2M1 operands natively.  gfx950's
scaled f8f6f4 instruction takes FP4 / FP8 elements with one power-of-two
(E8M0) scale per 32 contraction elements (the OCP MX formats), while the
cache holds E2M1 codes with one E4M3 scale per 16.  The variant therefore
requantizes both score operands; V and the probabilities stay as in the
exact path.  The recipe, as the kernel applies it:

* MX blocks: the instruction scales the product of contraction element k of
  a 64-wide K-step with the bytes of the A and B lanes of half (k / 16) % 2,
  so for both operands a block is the pair of 16-element chunks {g, g + 2}
  of a K-step: head_dim 64c + 16g + [0, 16) and 64c + 32 + 16g + [0, 16)
  (the two chunks one lane of the A operand holds);
* queries (MXFP8): each row is first rescaled by 2^-sh, sh = E - 14 for the
  row's largest bf16 magnitude of exponent E (clamped to [-100, 113]; rows
  of subnormals keep sh = 0), so that raw scores keep the exact path's bound;
  each block then takes the smallest exponent e >= -127 with its largest
  magnitude a <= 448 * 2^e, and its elements are rounded to nearest-even
  E4M3 after the exact division by 2^(sh + e): q_hat = E4M3 * 2^(sh + e).
  Nothing saturates.
* keys, mode 4 (MXFP4): the NVFP4 blocks 4c + g and 4c + 2 + g of a row
  form MX block (c, g), with e = ceil(log2 max(S_a, S_b)); every element
  e2m1 * S_b becomes the nearest-even E2M1 value of e2m1 * S_b / 2^e, times
  2^e (times the global scale g_k);
* keys, mode 5 (MXFP8): the same blocks, with the smallest e such that
  6 max(S_a, S_b) <= 448 * 2^e, and the elements rounded to nearest-even
  E4M3 instead.

Mode 4: the requantized keys are handed to the oracle as an NVFP4 cache with
block scale 2^(e - 1) and global scale 2 g_k (an E4M3 scale cannot hold 2^9,
which e reaches when S = 448), the requantized queries as bf16 (every E4M3
value times a power of two in range is a bf16 value); both conversions are
checked to be exact.  Mode 5's keys are not NVFP4 values, so its attention is
dense_prefill below: a direct fp64 transcription of the oracle's definition
(pinned against the oracle on exact operands).
"""
import numpy as np

# The variants' accuracy contracts against the oracle, per mode: (elem, rms)
# with |out - ref| <= elem * (1 + |ref|) per element and rms(out - ref) <=
# rms * rms(ref) over a batch.  On N(0,1) workloads of the prefill's shapes
# the emulation reaches 0.45 / 0.115 (mode 4) and 0.185 / 0.032 (mode 5).
MX_CONTRACT = {4: (0.75, 0.2), 5: (0.3, 0.05)}
MX_ELEM, MX_RMS = MX_CONTRACT[4]


def _tables(O):
    e2 = np.array([O.e2m1_value(c) for c in range(16)])
    e4 = np.array([O.e4m3_value(c) for c in range(256)])
    return e2, e4


def _bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64_to_bf16_exact(x):
    f = x.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), x), "value outside float32"
    b = f.view(np.uint32)
    assert not (b & 0xFFFF).any(), "value not a bf16 value"
    return (b >> 16).astype(np.uint16)


def _exponent(x):
    """floor(log2 x) and x / 2^floor for x > 0 (fp64, exact)."""
    m, ex = np.frexp(x)  # x = m 2^ex, m in [0.5, 1)
    return ex - 1, 2.0 * m


def mx_partner(j):
    """The 16-element chunk (an NVFP4 block of K) that shares chunk j's MX
    block: 4c + g <-> 4c + 2 + g."""
    return j ^ 2


def mx_query_values(O, q_bits):
    """q_hat (fp64) of bf16 queries q_bits [..., D] (uint16), and the E8M0
    exponents e [..., D/16] of their 16-element chunks (equal within a
    block)."""
    _, e4 = _tables(O)
    q = _bf16_to_f64(q_bits)
    D = q.shape[-1]
    am_bits = (q_bits & 0x7FFF).max(axis=-1, keepdims=True).astype(np.int64)
    sh = np.where(am_bits >= 0x80, np.clip((am_bits >> 7) - 127 - 14, -100, 113), 0)
    qs = q * np.exp2(-sh.astype(np.float64))
    blocks = qs.reshape(*q.shape[:-1], D // 16, 16)
    a = np.abs(blocks).max(axis=-1)
    a = np.maximum(a, a[..., [mx_partner(j) for j in range(D // 16)]])
    E, sig = _exponent(np.where(a > 0, a, 1.0))
    e = np.where(a < 2.0 ** -126, -127, np.maximum(E - 8 + (sig > 1.75), -127))
    y = blocks * np.exp2(-e.astype(np.float64))[..., None]
    assert np.abs(y).max() <= 448.0
    codes = O.e4m3_encode(np.abs(y).astype(np.float32).reshape(-1)).reshape(y.shape)
    yh = np.copysign(e4[codes], y)
    q_hat = (yh * np.exp2(e.astype(np.float64))[..., None]).reshape(q.shape) * np.exp2(sh.astype(np.float64))
    return q_hat, e


def mx_query_bits(O, q_bits):
    """bf16 bits of q_hat (checked exact)."""
    return _f64_to_bf16_exact(mx_query_values(O, q_bits)[0])


def _unpack(codes):
    """[rows, D/2] packed bytes -> [rows, D] codes (element 2i: low nibble)."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def _pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def mx_key_rows(O, codes, sf):
    """Requantize NVFP4 rows (codes [rows, D/2] uint8, scale bytes [rows,
    D/16] uint8) to MXFP4: returns (new codes [rows, D] int, MX exponent of
    each NVFP4 block [rows, D/16] int, valid where the pair's scales are not
    both zero)."""
    e2, e4 = _tables(O)
    c = _unpack(codes)
    rows, D = c.shape
    S = e4[sf.astype(np.int64)]  # [rows, D/16]
    smax = np.maximum(S, S[:, [mx_partner(b) for b in range(D // 16)]])
    E, sig = _exponent(np.where(smax > 0, smax, 1.0))
    e = np.where(smax > 0, E + (sig > 1.0), 0)
    r = S * np.exp2(-e.astype(np.float64))
    vals = e2[c] * np.repeat(r, 16, axis=1)
    assert np.abs(vals).max() <= 6.0
    new = O.e2m1_encode(vals.astype(np.float32).reshape(-1)).reshape(rows, D).astype(np.int64)
    return new, e


def mx8_key_values(O, codes, sf):
    """Requantize NVFP4 rows to MXFP8 (mode 5): values [rows, D] (without the
    global scale) and the MX exponent of each NVFP4 block [rows, D/16]."""
    e2, e4 = _tables(O)
    c = _unpack(codes)
    rows, D = c.shape
    S = e4[sf.astype(np.int64)]
    smax = np.maximum(S, S[:, [mx_partner(b) for b in range(D // 16)]])
    E, sig = _exponent(np.where(smax > 0, 6.0 * smax, 1.0))
    e = np.where(smax > 0, E - 8 + (sig > 1.75), 0)
    vals = e2[c] * np.repeat(S * np.exp2(-e.astype(np.float64)), 16, axis=1)
    assert np.abs(vals).max() <= 448.0
    codes8 = O.e4m3_encode(np.abs(vals).astype(np.float32).reshape(-1)).reshape(rows, D)
    out = np.copysign(e4[codes8.astype(np.int64)], vals) * np.repeat(np.exp2(e.astype(np.float64)), 16, axis=1)
    return out, e


def dense_prefill(q, k_rows, v_rows, qo, kv_indptr, page_table, kv_lens, page_size, num_kv_heads, sm_scale):
    """fp64 causal paged prefill over dense operands: q [total_q, H_q, D]
    values, k_rows / v_rows [(slot * H_kv + head), D] values; the oracle's
    definition (bottom-right causal alignment, query head h reads KV head
    h / (H_q / H_kv), softmax(sm_scale q.k) v) written with numpy."""
    total_q, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((total_q, Hq, D))
    for r in range(len(kv_lens)):
        Lk = int(kv_lens[r])
        q0, q1 = int(qo[r]), int(qo[r + 1])
        Lq = q1 - q0
        j = np.arange(Lk)
        slots = page_table[kv_indptr[r] + j // page_size].astype(np.int64) * page_size + j % page_size
        vis = np.arange(Lk)[None, :] <= (Lk - Lq + np.arange(Lq))[:, None]
        for h in range(Hq):
            rows = slots * num_kv_heads + h // G
            sc = np.where(vis, (q[q0:q1, h] @ k_rows[rows].T) * sm_scale, -np.inf)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            out[q0:q1, h] = (p @ v_rows[rows]) / p.sum(axis=1, keepdims=True)
    return out


def mx_key_cache(O, k_cache, k_sf, k_scale):
    """The requantized keys as an NVFP4 cache for the oracle: (codes, scale
    bytes, global scale) with values e2m1' * 2^(e - 1) * (2 g_k)."""
    shp_c, shp_s = k_cache.shape, k_sf.shape
    D = shp_c[-1] * 2
    new, e = mx_key_rows(O, k_cache.reshape(-1, D // 2), k_sf.reshape(-1, D // 16))
    e4 = _tables(O)[1]
    zero = e4[k_sf.reshape(-1, D // 16).astype(np.int64)] == 0
    zero &= zero[:, [mx_partner(b) for b in range(D // 16)]]
    assert (e[~zero] - 1 >= -9).all(), "MX exponent below what the E4M3 carrier holds"
    sfb = np.where(zero, 0, O.e4m3_encode(np.exp2((e - 1).astype(np.float64)).astype(np.float32).reshape(-1))
                   .reshape(e.shape)).astype(np.uint8)
    assert np.array_equal(e4[sfb.astype(np.int64)][~zero], np.exp2((e - 1).astype(np.float64))[~zero])
    g2 = float(np.float32(2.0 * np.float32(k_scale)))
    return _pack(new).reshape(shp_c), sfb.reshape(shp_s), g2


def mx_outputs(O, w, reqs=None, mode=4):
    """The MX variant's fp64 output rows for `reqs` of workload w (all if
    None) and their row indices in w's query order: the oracle's append of
    w's bf16 K and V, the requantized queries and keys, the attention over
    them (the oracle's for mode 4, dense_prefill for mode 5)."""
    from gpu_helpers import sub_workload
    if reqs is None:
        reqs = range(w.batch)
    s = sub_workload(w, reqs)
    P, ps, H, D = s["num_pages"], w.page_size, w.num_kv_heads, w.head_dim
    kc = np.zeros((P, ps, H, D // 2), np.uint8)
    vc = np.zeros_like(kc)
    ksf = np.zeros((P, ps, H, D // 16), np.uint8)
    vsf = np.zeros_like(ksf)
    assert O.append(s["k"], s["v"], s["slots"], w.k_scale, w.v_scale, kc, vc, ksf, vsf, ps) == 0
    if mode == 5:
        q_hat, _ = mx_query_values(O, s["q"])
        kv, _ = mx8_key_values(O, kc.reshape(-1, D // 2), ksf.reshape(-1, D // 16))
        rows = np.arange(P * ps * H)
        vv = O.dequant_rows(vc.reshape(-1, D // 2), vsf.reshape(-1, D // 16), rows, D, w.v_scale)
        out = dense_prefill(q_hat, kv * np.float64(np.float32(w.k_scale)), vv, s["qo"], s["kv_indptr"],
                            s["page_table"], s["kv_lens"], ps, H, w.sm_scale)
        return out, s["q_rows"]
    kc2, ksf2, g2 = mx_key_cache(O, kc, ksf, w.k_scale)
    out, err = O.prefill(mx_query_bits(O, s["q"]), s["qo"], s["kv_indptr"], s["page_table"], s["kv_lens"],
                         kc2, vc, ksf2, vsf, g2, w.v_scale, w.num_q_heads, w.sm_scale)
    assert err == 0
    return out, s["q_rows"]
