"""GPU checks of the gfx950 builtins the kernels rely on (probe library
tests/libnvfp4kv_probes.so): the hardware FP4 conversion used by the append
against the oracle's E2M1 encoder over every fp32 pattern, the FP4 -> fp32
decode used by the attention's staging, the E4M3 pair decode of its block
scales, and the MFMA lane layouts."""
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
              "probe_fp8_pairs"):
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


def test_mfma_16x16x32_layout(probes):
    g = torch.Generator().manual_seed(1)
    A = torch.randn(16, 32, generator=g).bfloat16().float()
    B = torch.randn(32, 16, generator=g).bfloat16().float()
    Ad, Bd, Dd = A.cuda(), B.cuda(), torch.zeros(16, 16).cuda()
    assert probes.probe_mfma16(P(Ad), P(Bd), P(Dd)) == 0
    torch.testing.assert_close(Dd.cpu(), A.double().mm(B.double()).float(), rtol=1e-5, atol=1e-5)
