"""GPU checks of the gfx950 builtins the kernels rely on (probe library
tests/libnvfp4kv_probes.so): the hardware FP4 conversion used by the append
against the oracle's E2M1 encoder over every fp32 pattern, the FP4 -> fp32
decode used by the attention's staging, the E4M3 pair decode of its block
scales, the MFMA lane layouts, the cross-row lane swaps, and what the MX
score variant relies on: the scaled FP4 x FP8 matrix instruction and the two
encoders that feed it."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_helpers import banner

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probes():
    path = os.path.join(HERE, "libnvfp4kv_probes.so")
    if not os.path.exists(path):
        pytest.fail("tests/libnvfp4kv_probes.so missing: run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    for f in ("probe_e2m1_scan", "probe_cvt_pairs", "probe_fp4_to_bf16", "probe_mfma32", "probe_mfma16",
              "probe_fp8_pairs", "probe_mfma_scale", "probe_fp8_from_bf16", "probe_fp4_from_f16",
              "probe_permlane_swap"):
        getattr(L, f).restype = ctypes.c_int
    return L


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def _scan(probes, sign, mode):
    cap = 4096
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.zeros(2 * cap, dtype=torch.int32, device="cuda")
    assert probes.probe_e2m1_scan(ctypes.c_uint32(sign), mode, P(count), P(buf), cap) == 0
    n = int(count.item())
    assert n <= cap
    t = buf.cpu().numpy().view(np.uint32)[: 2 * n].reshape(n, 2)
    return sorted((int(p), int(c)) for p, c in t)


@pytest.mark.parametrize("mode", [0, 1], ids=["hardware_cvt", "software"])
@pytest.mark.parametrize("sign", [0, 0x80000000], ids=["pos", "neg"])
def test_e2m1_encoder_matches_oracle_on_every_fp32(probes, oracle, mode, sign):
    banner(f"e2m1 scan mode={mode} sign={sign:#x}")
    tr = _scan(probes, sign, mode)
    # every change point p: oracle(p) == code and oracle(p-1) == previous code;
    # also the last pattern (+-inf) — the oracle is monotone (pinned on the CPU)
    pats = [p for p, _ in tr]
    assert pats[0] == 0
    codes = [c & 0xF for _, c in tr]
    assert all(c >> 4 == 0 for _, c in tr), "high nibble (second value, +0) must stay 0"
    check = np.array([sign | p for p in pats] + [sign | (p - 1) for p in pats[1:]] + [sign | 0x7F800000],
                     np.uint32).view(np.float32)
    want = oracle.e2m1_encode(check)
    n = len(pats)
    assert list(want[:n]) == codes, (tr, list(want[:n]))
    assert list(want[n:2 * n - 1]) == codes[:-1]
    assert want[-1] == codes[-1]
    assert n == 8


def test_cvt_pair_nibble_order(probes):
    vals = torch.tensor([1.0, 6.0, -0.5, 3.0, 0.0, -0.0, -6.0, 0.25], device="cuda")
    out = torch.zeros(8, dtype=torch.int32, device="cuda")
    assert probes.probe_cvt_pairs(P(vals), 4, P(out)) == 0
    o = out.cpu().numpy().view(np.uint32)
    assert o[:4].tolist() == [0x72, 0x59, 0x80, 0x0F], [hex(x) for x in o[:4]]
    assert o[4:].tolist() == [0x72 << 16, 0x59 << 16, 0x80 << 16, 0x0F << 16]


def test_fp4_to_f32_decode_and_scaled_forms(probes, oracle):
    scales = torch.tensor([1.0, 1.5, 0.001953125, 448.0, 0.75, 2.0], device="cuda")
    ob = torch.zeros(256 * 6, dtype=torch.int32, device="cuda")
    of = torch.zeros(2 * 256 * 6, dtype=torch.float32, device="cuda")
    assert probes.probe_fp4_to_bf16(P(scales), 6, P(ob), P(of)) == 0
    f = of.cpu().numpy().reshape(6, 256, 2)
    grid = np.array([oracle.e2m1_value(c) for c in range(16)])
    byte = np.arange(256)
    # scale 1.0: the exact E2M1 values, low nibble first (used by the staging)
    assert np.array_equal(f[0, :, 0], grid[byte & 15]) and np.array_equal(f[0, :, 1], grid[byte >> 4])
    bf = ob.cpu().numpy().view(np.uint32).reshape(6, 256)
    bf_lo = (bf & 0xFFFF).astype(np.uint32) << 16
    bfv = bf_lo.view(np.float32)
    # The conversions' scale operand applies only its power of two (the use
    # it is made for: E8M0 block scales), so a non-power-of-two E4M3 block
    # scale cannot be handed to it and is multiplied in separately.
    for i, s in enumerate(scales.cpu().tolist()):
        pow2 = 2.0 ** np.floor(np.log2(s))
        print(f"[probe] scale {s}: f32 form sample {f[i, 0x27, :].tolist()}, bf16 form {bfv[i, 0x27]}", flush=True)
        assert np.array_equal(f[i, :, 0], grid[byte & 15] * pow2), s
        assert np.array_equal(f[i, :, 1], grid[byte >> 4] * pow2), s
        assert np.array_equal(bfv[i], (grid[byte & 15] * pow2).astype(np.float32)), s


def test_e4m3_pair_decode_matches_oracle(probes, oracle):
    """Every finite E4M3 byte (both signs, subnormals included) decodes to the
    oracle's value in both halves of the pair and with both word selects."""
    banner("E4M3 pair decode, all 256 bytes")
    out = torch.zeros(512, dtype=torch.float32, device="cuda")
    assert probes.probe_fp8_pairs(P(out)) == 0
    f = out.cpu().numpy().reshape(128, 4)
    got = np.empty((256, 2))
    got[0::2, 0], got[1::2, 0], got[1::2, 1], got[0::2, 1] = f[:, 0], f[:, 1], f[:, 2], f[:, 3]
    for b in range(256):
        ref = oracle.e4m3_value(b)
        if np.isnan(ref):
            assert np.isnan(got[b]).all(), b
        else:
            assert got[b, 0] == ref and got[b, 1] == ref, (b, got[b], ref)


def test_mfma_32x32x16_layout(probes):
    g = torch.Generator().manual_seed(0)
    A = torch.randn(32, 16, generator=g).bfloat16().float()
    B = torch.randn(16, 32, generator=g).bfloat16().float()
    D = torch.zeros(32, 32)
    Ad, Bd, Dd = A.cuda(), B.cuda(), D.cuda()
    assert probes.probe_mfma32(P(Ad), P(Bd), P(Dd)) == 0
    torch.testing.assert_close(Dd.cpu(), A.double().mm(B.double()).float(), rtol=1e-5, atol=1e-5)


def test_permlane_swaps_exchange_rows(probes):
    """v_permlane16_swap with one register as both operands leaves lanes of
    even 16-lane rows their own value in the first result and the value of
    lane + 16 in the second (odd rows: lane - 16, then their own), so the
    pair is {x[l], x[l ^ 16]} in every lane; v_permlane32_swap likewise
    with the wave's halves, {x[l], x[l ^ 32]}."""
    x = torch.arange(1000, 1064, dtype=torch.int32)
    xd, out = x.cuda(), torch.zeros(256, dtype=torch.int32, device="cuda")
    assert probes.probe_permlane_swap(P(xd), P(out)) == 0
    o = out.cpu().view(4, 64).numpy()
    xs = x.numpy()
    lane = np.arange(64)
    even16 = (lane // 16) % 2 == 0
    np.testing.assert_array_equal(o[0], np.where(even16, xs[lane], xs[lane - 16]))
    np.testing.assert_array_equal(o[1], np.where(even16, xs[(lane + 16) % 64], xs[lane]))
    lo = lane < 32
    np.testing.assert_array_equal(o[2], np.where(lo, xs[lane], xs[lane - 32]))
    np.testing.assert_array_equal(o[3], np.where(lo, xs[(lane + 32) % 64], xs[lane]))
    for a, b, k in ((o[0], o[1], 16), (o[2], o[3], 32)):
        np.testing.assert_array_equal(np.minimum(a, b), np.minimum(xs, xs[lane ^ k]))
        np.testing.assert_array_equal(np.maximum(a, b), np.maximum(xs, xs[lane ^ k]))


def test_mfma_16x16x32_layout(probes):
    g = torch.Generator().manual_seed(1)
    A = torch.randn(16, 32, generator=g).bfloat16().float()
    B = torch.randn(32, 16, generator=g).bfloat16().float()
    Ad, Bd, Dd = A.cuda(), B.cuda(), torch.zeros(16, 16).cuda()
    assert probes.probe_mfma16(P(Ad), P(Bd), P(Dd)) == 0
    torch.testing.assert_close(Dd.cpu(), A.double().mm(B.double()).float(), rtol=1e-5, atol=1e-5)


def test_mfma_scale_fp4_fp8_layout(probes, oracle):
    """The scaled FP4 x FP8 32x32x64 product that the MX score variant uses
    for S^T = K Q^T: lane l of A holds row l%32 with two 16-element chunks
    (nibbles 0-15 and 16-31, the even element of a byte in its low nibble)
    at contraction offsets 16(l//32) and 32 + 16(l//32); lane l of B holds
    column l%32 with 32 consecutive contraction elements (byte j at offset
    32(l//32) + j); the product of contraction element k takes the E8M0
    scale (byte 0) of A lane m + 32g and of B lane n + 32g, g = (k//16)%2 --
    the A layout's halves, not B's; the result has the 32x32 layout of the
    16-bit products.  Random signed codes, random E4M3 bytes and a random
    scale per lane, against the sum computed from the oracle's E2M1 and E4M3
    decodes.  The instruction's own sum is not exact in fp32: it stays
    within 2^-10 of the largest product (measured: 4.9e-4)."""
    banner("scaled FP4 x FP8 matrix instruction layout")
    rng = np.random.default_rng(7)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    e4 = np.array([oracle.e4m3_value(c) for c in range(256)])
    codes = rng.integers(0, 16, (64, 32))
    fp8 = rng.integers(0, 256, (64, 32))
    fp8[(fp8 & 0x7F) == 0x7F] = 0x38  # no NaN encodings
    sa = rng.integers(120, 134, 64)
    sb = rng.integers(120, 134, 64)
    A = np.zeros((32, 64))
    B = np.zeros((64, 32))
    a_regs = np.zeros((64, 8), np.int64)
    b_regs = np.zeros((64, 8), np.int64)
    for l in range(64):
        h = l // 32
        for j in range(32):
            k = (0 if j < 16 else 32) + 16 * h + j % 16
            A[l % 32, k] = e2[codes[l, j]] * 2.0 ** (int(sa[l]) - 127)
            a_regs[l, j // 8] |= int(codes[l, j]) << (4 * (j % 8))
            kb = 32 * h + j
            B[kb, l % 32] = e4[fp8[l, j]] * 2.0 ** (int(sb[l % 32 + 32 * ((kb // 16) % 2)]) - 127)
            b_regs[l, j // 4] |= int(fp8[l, j]) << (8 * (j % 4))
    # (device tensors held by name until the call returns: a temporary's
    # memory could go to the next operand before the kernel reads it)
    ta, tb, tsa, tsb = (torch.from_numpy((x & 0xFFFFFFFF).astype(np.uint32).view(np.int32)).cuda()
                        for x in (a_regs, b_regs, sa, sb))
    d = torch.zeros(64 * 16, dtype=torch.float32, device="cuda")
    assert probes.probe_mfma_scale(P(ta), P(tb), P(tsa), P(tsb), P(d)) == 0
    d = d.cpu().numpy().reshape(64, 16)
    got = np.zeros((32, 32))
    for l in range(64):
        for r in range(16):
            got[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] = d[l, r]
    ref = A @ B
    largest = (np.abs(A)[:, :, None] * np.abs(B)[None, :, :]).max(axis=1)
    assert (np.abs(got - ref) <= 2.0 ** -10 * largest).all(), np.max(np.abs(got - ref) / largest)


def test_fp8_encode_of_every_bf16_matches_oracle(probes, oracle):
    """The MXFP8 query load rounds bf16-valued floats of magnitude <= 448
    (after an exact power-of-two scaling) with the pair conversion: every
    bf16 pattern in that range, both word selects, against the oracle's
    nearest-even E4M3 encoder with the sign bit on top."""
    banner("f32 -> E4M3 pair conversion, every bf16 pattern")
    out = torch.zeros(16384, dtype=torch.int32, device="cuda")
    assert probes.probe_fp8_from_bf16(P(out)) == 0
    got = out.cpu().numpy().view(np.uint32)
    got = np.stack([(got >> (8 * i)) & 0xFF for i in range(4)], 1).reshape(-1)  # byte i: pattern 4t + i
    pats = np.arange(65536, dtype=np.uint32)
    v = (pats << 16).view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    got, v = got[keep], v[keep]
    want = oracle.e4m3_encode(np.abs(v)).astype(np.uint32)
    # magnitude codes equal; the sign bit too wherever the result is not zero
    bad = np.nonzero(((got & 0x7F) != want) | ((want != 0) & ((got >> 7) != np.signbit(v))))[0]
    assert bad.size == 0, [(float(v[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]


def test_fp4_encode_of_every_f16_matches_oracle(probes, oracle):
    """The K requantization rounds exact f16 products of magnitude <= 6 with
    the f16 pair -> E2M1 conversion: every f16 pattern in that range, both
    elements of each pair and all four byte selects, against the oracle's
    nearest-even E2M1 encoder."""
    banner("f16 pair -> E2M1 conversion, every f16 pattern")
    out = torch.zeros(8192, dtype=torch.int32, device="cuda")
    assert probes.probe_fp4_from_f16(P(out)) == 0
    got = out.cpu().numpy().view(np.uint32)
    got = np.stack([(got >> (4 * i)) & 0xF for i in range(8)], 1).reshape(-1)  # nibble i: pattern 8t + i
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    keep = np.abs(v) <= 6.0
    got, v = got[keep], v[keep]
    want = oracle.e2m1_encode(v).astype(np.uint32)
    bad = np.nonzero(((got & 7) != (want & 7)) | (((want & 7) != 0) & ((got >> 3) != (want >> 3))))[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:8]]
