"""The prefill's MX score variants (dequant modes 4 and 5) on the CPU: pins
of their emulation (tests/mx_emulation.py) and the accuracy contracts derived
from it.

gfx950's scaled f8f6f4 matrix instruction takes FP4 / FP8 elements with one
power-of-two (E8M0) scale per 32 elements; the cache holds E2M1 codes with an
E4M3 scale per 16 (the PR #4769 page's NVFP4 tiles).  Mode 4 requantizes K to
MXFP4, mode 5 to MXFP8, and both Q to MXFP8; all of these round, so neither
meets the exact path's 1e-2 + 1e-2 |ref| bound.  Each mode's contract
(mx_emulation.MX_CONTRACT[mode] = (elem, rms)), measured here on the
emulation over N(0,1) workloads of the prefill's shapes and checked on the
GPU against the oracle by tests/test_gpu_mx_scores.py:

* per element: |out - ref| <= elem * (1 + |ref|);
* over a batch: rms(out - ref) <= rms * rms(ref).

The emulation reaches at most 0.45 / 0.115 (mode 4) and 0.185 / 0.032
(mode 5) on these workloads; the bounds leave a margin for other draws.
Everything here runs on the CPU.
"""
import numpy as np
import pytest
import torch

import mx_emulation as M
import workloads as W
from gpu_helpers import oracle_outputs

RAGGED_Q = [1, 37, 200, 64, 3, 129]
RAGGED_KV = [1, 37, 333, 700, 3, 130]


@pytest.fixture(scope="module")
def tables(oracle):
    return M._tables(oracle)


def _rows_of(rng, n, D=128):
    codes = rng.integers(0, 256, (n, D // 2)).astype(np.uint8)
    return codes


def test_query_blocks_use_the_smallest_unsaturated_exponent(oracle):
    """Each MX block's (16-element chunks {g, g + 2} of a 64-wide K-step)
    largest magnitude lands in (224, 448] after the division by 2^(sh + e),
    both chunks of a block share e, and every element is within half an
    E4M3 step of q: 2^-4 relative for normals, 2^-10 * 2^(sh + e) below
    them.  Chunks of one row are spread over 2^-20 .. 2^20."""
    rng = np.random.default_rng(1)
    q = W.normal_bf16((64, 4, 128), seed=3, stream=W.Q_STREAM, device="cpu").float()
    spread = np.repeat(np.exp2(rng.integers(-20, 21, (64, 4, 8)).astype(np.float64)), 16, -1)
    bits = W.bf16_bits((q * torch.from_numpy(spread).float()).to(torch.bfloat16))
    qf = M._bf16_to_f64(bits)
    q_hat, e = M.mx_query_values(oracle, bits)
    assert np.array_equal(e, e[..., [j ^ 2 for j in range(8)]])
    am = (bits & 0x7FFF).max(-1, keepdims=True).astype(np.int64)
    sh = np.where(am >= 0x80, np.clip((am >> 7) - 127 - 14, -100, 113), 0)
    unit = np.exp2((np.repeat(e, 16, -1) + sh).astype(np.float64))
    chunk = np.abs(qf.reshape(*qf.shape[:-1], 8, 16)).max(-1)
    blk = np.maximum(chunk, chunk[..., [j ^ 2 for j in range(8)]]) / np.exp2((e + sh).astype(np.float64))
    assert (e > -127).all() and ((blk > 224) & (blk <= 448)).all()
    assert (np.abs(q_hat - qf) <= np.maximum(2.0 ** -4 * np.abs(qf), 2.0 ** -10 * unit)).all()
    # values already on the grid are kept
    q2, _ = M.mx_query_values(oracle, M.mx_query_bits(oracle, bits))
    assert np.array_equal(q2, q_hat)


def _row_shift(bits):
    am = (bits & 0x7FFF).max(-1, keepdims=True).astype(np.int64)
    return np.where(am >= 0x80, np.clip((am >> 7) - 127 - 14, -100, 113), 0)


def test_query_block_pairing(oracle):
    """A chunk raised alone (x 2^10) changes the scale 2^(sh + e) of exactly
    its own block: chunk j and chunk j ^ 2."""
    bits0 = W.bf16_bits(W.normal_bf16((1, 1, 128), seed=4, stream=W.Q_STREAM, device="cpu"))
    _, e0 = M.mx_query_values(oracle, bits0)
    x0 = e0 + _row_shift(bits0)
    for j in range(8):
        x = M._bf16_to_f64(bits0).copy()
        x[..., 16 * j:16 * j + 16] *= 1024.0
        bits = M._f64_to_bf16_exact(x)
        _, e = M.mx_query_values(oracle, bits)
        xe = e + _row_shift(bits)
        assert {i for i in range(8) if xe[0, 0, i] != x0[0, 0, i]} == {j, j ^ 2}


@pytest.mark.parametrize("b", range(8))
def test_key_pairing_follows_the_operand_layout(oracle, b):
    """Block b's scale raised alone (8 while the others are 1) requantizes
    exactly one other block -- the one sharing b's MX block, head_dim
    16(b ^ 2), as one lane of the A operand holds 16h + [0, 16) and
    32 + 16h + [0, 16) of a 64-wide K-step -- and leaves b itself exact."""
    rng = np.random.default_rng(10 + b)
    codes = rng.integers(0, 256, (16, 64)).astype(np.uint8)
    codes |= 0x66  # every element has magnitude >= 2 (code 6: 4.0 or more)
    sf = np.full((16, 8), 0x38, np.uint8)  # E4M3 1.0
    sf[:, b] = 0x50  # E4M3 8.0
    new, e = M.mx_key_rows(oracle, codes, sf)
    old = M._unpack(codes)
    changed = {blk for blk in range(8) if not np.array_equal(new[:, 16 * blk:16 * blk + 16],
                                                             old[:, 16 * blk:16 * blk + 16])}
    assert changed == {b ^ 2}
    assert (e[:, [b, b ^ 2]] == 3).all() and (np.delete(e, [b, b ^ 2], axis=1) == 0).all()


def test_key_requantization_exact_for_power_of_two_pairs(oracle):
    """Pairs whose two scales are the same power of two keep their codes."""
    rng = np.random.default_rng(4)
    codes = _rows_of(rng, 64)
    ex = rng.integers(-6, 9, (64, 4))  # E4M3 normals 2^-6 .. 2^8
    sf = np.zeros((64, 8), np.uint8)
    for b in range(8):
        c, h = b // 4, b % 2
        sf[:, b] = ((ex[:, 2 * c + h] + 7) << 3).astype(np.uint8)
    new, e = M.mx_key_rows(oracle, codes, sf)
    assert np.array_equal(new, M._unpack(codes))


def test_key_requantization_error_bound(oracle, tables):
    """|k' - k| is at most one E2M1 half-step at the MX scale (2^e; the
    grid's largest half-step is 1), and k' is the nearest grid value."""
    e2, e4 = tables
    rng = np.random.default_rng(5)
    codes = _rows_of(rng, 256)
    sf = rng.integers(1, 0x7F, (256, 8)).astype(np.uint8)
    new, e = M.mx_key_rows(oracle, codes, sf)
    S = np.repeat(e4[sf.astype(np.int64)], 16, 1)
    k = e2[M._unpack(codes)] * S
    unit = np.repeat(np.exp2(e.astype(np.float64)), 16, 1)
    kq = e2[new] * unit
    assert (np.abs(kq - k) <= unit * 1.0).all()
    mags = np.array(sorted(set(np.abs(e2))))
    nearest = np.abs(np.abs(k / unit)[..., None] - mags).min(-1)
    assert np.allclose(np.abs(np.abs(kq / unit) - np.abs(k / unit)), nearest)


def test_mx8_keys_exact_when_representable(oracle):
    """MXFP8 keys: a pair with equal power-of-two scales keeps every value
    (e2m1 x 2^k has at most 2 significant bits), and any value is within
    half an E4M3 step (2^-4 relative, 2^-10 x 2^e absolute) of e2m1 x S."""
    e2, e4 = M._tables(oracle)
    rng = np.random.default_rng(6)
    codes = _rows_of(rng, 64)
    ex = rng.integers(-6, 9, (64, 4))
    sf = np.zeros((64, 8), np.uint8)
    for b in range(8):
        sf[:, b] = ((ex[:, 2 * (b // 4) + b % 2] + 7) << 3).astype(np.uint8)
    vals, _ = M.mx8_key_values(oracle, codes, sf)
    exact = e2[M._unpack(codes)] * np.repeat(e4[sf.astype(np.int64)], 16, 1)
    assert np.array_equal(vals, exact)
    sf = rng.integers(1, 0x7F, (256, 8)).astype(np.uint8)
    codes = _rows_of(rng, 256)
    vals, e = M.mx8_key_values(oracle, codes, sf)
    exact = e2[M._unpack(codes)] * np.repeat(e4[sf.astype(np.int64)], 16, 1)
    unit = np.repeat(np.exp2(e.astype(np.float64)), 16, 1)
    assert (np.abs(vals - exact) <= np.maximum(2.0 ** -4 * np.abs(exact), 2.0 ** -10 * unit)).all()
    # the exponent is the smallest with 6 max(S_a, S_b) <= 448 x 2^e
    S = e4[sf.astype(np.int64)]
    bound = 6 * np.maximum(S, S[:, [b ^ 2 for b in range(8)]]) / np.exp2(e.astype(np.float64))
    assert ((bound > 224) & (bound <= 448)).all()


def test_dense_prefill_matches_the_oracle(oracle):
    """dense_prefill (mode 5's attention) on the exact dequantized operands
    equals the oracle's prefill to fp64 rounding."""
    from gpu_helpers import sub_workload
    w = W.make_attention("ragged_amax", RAGGED_Q, RAGGED_KV, 32, 8, 128, 16, 120, seed=1, device="cpu",
                         scales="amax")
    s = sub_workload(w, range(w.batch))
    P, ps, H, D = s["num_pages"], 16, 8, 128
    kc = np.zeros((P, ps, H, D // 2), np.uint8)
    vc, ksf = np.zeros_like(kc), np.zeros((P, ps, H, D // 16), np.uint8)
    vsf = np.zeros_like(ksf)
    assert oracle.append(s["k"], s["v"], s["slots"], w.k_scale, w.v_scale, kc, vc, ksf, vsf, ps) == 0
    rows = np.arange(P * ps * H)
    kk = oracle.dequant_rows(kc.reshape(-1, 64), ksf.reshape(-1, 8), rows, D, w.k_scale)
    vv = oracle.dequant_rows(vc.reshape(-1, 64), vsf.reshape(-1, 8), rows, D, w.v_scale)
    d = M.dense_prefill(M._bf16_to_f64(s["q"]), kk, vv, s["qo"], s["kv_indptr"], s["page_table"], s["kv_lens"],
                        ps, H, w.sm_scale)
    ref, _ = oracle_outputs(oracle, w)
    assert np.abs(d - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def _ratio_stats(O, w, mode):
    ref, _ = oracle_outputs(O, w)
    emu, _ = M.mx_outputs(O, w, mode=mode)
    err = np.abs(emu - ref)
    return (err / (1 + np.abs(ref))).max(), np.sqrt((err ** 2).mean() / (ref ** 2).mean()), \
        (err / (1e-2 + 1e-2 * np.abs(ref))).max()


@pytest.mark.parametrize("shape", ["uniform_256", "ragged_amax", "ragged_lognormal"])
@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("mode", [4, 5])
def test_mx_contract_on_the_emulation(oracle, shape, seed, mode):
    """Each mode's contract holds on the emulation with a margin of 1.5, and
    both leave the exact path's 1e-2 bound (so they need their own)."""
    if shape == "uniform_256":
        w = W.make_attention(shape, [256], [256], 32, 8, 128, 16, 20, seed=seed, device="cpu", scales="amax")
    elif shape == "ragged_amax":
        w = W.make_attention(shape, RAGGED_Q, RAGGED_KV, 32, 8, 128, 16, 120, seed=seed, device="cpu",
                             scales="amax")
    else:
        w = W.make_attention(shape, RAGGED_Q, RAGGED_KV, 32, 8, 128, 16, 120, seed=seed, device="cpu",
                             scales="lognormal", lognormal=(-3.0, 0.5))
    elem, rms, tight = _ratio_stats(oracle, w, mode)
    elem_max, rms_max = M.MX_CONTRACT[mode]
    assert elem * 1.5 <= elem_max
    assert rms * 1.5 <= rms_max
    assert tight > 1.0


def test_kernel_f16_numerics_within_the_exact_bound(oracle):
    """For contrast: the exact path's own rounding (P to f16, 11 significant
    bits) keeps the output far inside 1e-2 + 1e-2 |ref| on the same data."""
    w = W.make_attention("uniform_256", [256], [256], 32, 8, 128, 16, 20, seed=1, device="cpu", scales="amax")
    ref, _ = oracle_outputs(oracle, w)
    from gpu_helpers import sub_workload
    s = sub_workload(w, range(1))
    q = M._bf16_to_f64(s["q"])
    P, ps, H, D = s["num_pages"], 16, 8, 128
    kc = np.zeros((P, ps, H, D // 2), np.uint8)
    vc, ksf = np.zeros_like(kc), np.zeros((P, ps, H, D // 16), np.uint8)
    vsf = np.zeros_like(ksf)
    assert oracle.append(s["k"], s["v"], s["slots"], w.k_scale, w.v_scale, kc, vc, ksf, vsf, ps) == 0
    rows = np.arange(256 * H)
    kh = oracle.dequant_rows(kc.reshape(-1, 64), ksf.reshape(-1, 8), rows, D, w.k_scale).reshape(256, H, D)
    vh = oracle.dequant_rows(vc.reshape(-1, 64), vsf.reshape(-1, 8), rows, D, w.v_scale).reshape(256, H, D)
    o = np.zeros_like(ref)
    causal = np.arange(256)[None, :] <= np.arange(256)[:, None]
    for h in range(32):
        sc = np.where(causal, q[:, h] @ kh[:, h // 4].T * w.sm_scale, -np.inf)
        p = np.exp(sc - sc.max(1, keepdims=True)).astype(np.float16).astype(np.float64)
        o[:, h] = (p @ vh[:, h // 4]) / p.sum(1, keepdims=True)
    assert (np.abs(o - ref) / (1e-2 + 1e-2 * np.abs(ref))).max() < 0.05
