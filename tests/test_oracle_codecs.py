"""Pins for the oracle's NVFP4 codecs and block quantizer (CPU only).

Nothing here compares the oracle with itself: the references are the OCP
grid table (tests/golden/e2m1_grid.txt), torch's float8_e4m3fn conversion
(a library routine), numpy's round-half-even (np.rint) on the E2M1 spacing,
closed-form tie points, hand-worked blocks (tests/golden/append_blocks.txt)
and invariants of the format.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_grid.txt")) if l.strip() and not l.startswith("#")]
    return {int(c): float(v) for c, v in rows}


def test_e2m1_decode_matches_ocp_grid(oracle):
    for code, val in _grid().items():
        got = oracle.e2m1_value(code)
        assert got == val and np.signbit(got) == np.signbit(val), code


def test_e2m1_exact_roundtrip_of_all_codes(oracle):
    vals = np.array([oracle.e2m1_value(c) for c in range(16)], np.float32)
    assert list(oracle.e2m1_encode(vals)) == list(range(16))


def _e2m1_ref_mag(y):
    """Nearest-even E2M1 magnitude via np.rint on each binade's spacing
    (0.5 below 2, 1 on [2,4), 2 on [4,6]), saturating at 6."""
    a = np.abs(y.astype(np.float64))
    v = np.where(a < 2, np.rint(a * 2) / 2, np.where(a < 4, np.rint(a), 2 * np.rint(a / 2)))
    v = np.minimum(v, 6.0)
    lut = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    return np.vectorize(lut.__getitem__)(v).astype(np.uint8)


def test_e2m1_encode_vs_rint_reference(oracle):
    rng = np.random.default_rng(11)
    pats = rng.integers(0, 0x41000000, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 2, 4, 6], np.float32)
    near = (ties.view(np.uint32)[:, None] + np.arange(-40, 41, dtype=np.int64)[None, :]).astype(np.uint32).ravel()
    y = np.concatenate([pats, near]).view(np.float32)
    got = oracle.e2m1_encode(y)
    assert np.array_equal(got & 7, _e2m1_ref_mag(y))
    assert np.array_equal(got >> 3, np.signbit(y).astype(np.uint8))
    got_neg = oracle.e2m1_encode(-y)
    assert np.array_equal(got_neg, (got & 7) | 8)


# First fp32 value (as a real number) at which each magnitude code begins,
# derived from the grid and round-half-even: a tie stays on the even code.
_E2M1_STARTS = [
    (1, np.nextafter(np.float32(0.25), np.float32(1))),   # 0.25 ties to code 0
    (2, np.float32(0.75)),                                  # 0.75 ties to code 2
    (3, np.nextafter(np.float32(1.25), np.float32(2))),   # 1.25 ties to code 2
    (4, np.float32(1.75)),                                  # 1.75 ties to code 4
    (5, np.nextafter(np.float32(2.5), np.float32(3))),    # 2.5 ties to code 4
    (6, np.float32(3.5)),                                   # 3.5 ties to code 6
    (7, np.nextafter(np.float32(5.0), np.float32(6))),    # 5 ties to code 6
]


def test_e2m1_exhaustive_nonnegative_sweep(oracle):
    """All 2^31 - 2^23 non-negative, non-NaN fp32 patterns (0 .. +inf): the
    codes never decrease and change exactly at the seven closed-form starts."""
    starts = {int(np.float32(v).view(np.uint32)): c for c, v in _E2M1_STARTS}
    chunk = 1 << 26
    prev = None
    seen = {}
    end = 0x7F800001
    for lo in range(0, end, chunk):
        hi = min(end, lo + chunk)
        pats = np.arange(lo, hi, dtype=np.uint32)
        codes = oracle.e2m1_encode(pats.view(np.float32))
        assert codes.max() <= 7
        d = np.diff(codes.astype(np.int16))
        assert d.min() >= 0
        for i in np.nonzero(d)[0]:
            seen[int(pats[i + 1])] = int(codes[i + 1])
        if prev is not None and codes[0] != prev:
            seen[lo] = int(codes[0])
        prev = codes[-1]
    assert seen == starts
    assert oracle.e2m1_encode(np.array([0.0, np.inf, -np.inf, np.nan], np.float32)).tolist() == [0, 7, 15, 0]


def test_e4m3_decode_all_codes_vs_torch(oracle):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_exhaustive_vs_torch(oracle):
    """Every positive fp32 pattern up to 464 against torch's round-to-nearest-
    even float8_e4m3fn cast; [464, inf] saturates to 448 (0x7E)."""
    top = int(np.float32(464.0).view(np.uint32))
    chunk = 1 << 26
    for lo in range(1, top + 1, chunk):
        hi = min(top + 1, lo + chunk)
        s = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
        ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3_encode(s), ref), lo
    hi_vals = np.array([464.0, 464.00003, 480.0, 1e6, 3e38, np.inf], np.float32)
    assert (oracle.e4m3_encode(hi_vals) == 0x7E).all()
    assert (oracle.e4m3_encode(np.array([0.0, -0.0, -1.0, np.nan], np.float32)) == 0).all()


def _bf16_bits(vals):
    t = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(vals, dtype=torch.float32)), "fixture value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def test_quantize_block_golden(oracle):
    n = 0
    for line in open(os.path.join(GOLDEN, "append_blocks.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        g, xs, sf, packed = [p.strip() for p in line.split("|")]
        x = [float(t) for t in xs.split()]
        got_p, got_sf = oracle.quantize_block(_bf16_bits(x), float(g))
        assert got_sf == int(sf, 16), line
        assert got_p.tolist() == [int(b, 16) for b in packed.split()], line
        n += 1
    assert n == 5


@pytest.mark.parametrize("gkind", ["pow2", "three_quarters_pow2"])
def test_quantize_block_closed_form_roundtrip(oracle, gkind):
    """x_i = e2m1(c_i) * S * g with max |c_i| = 6 and S an E4M3 value: the block
    returns exactly (c_i, sf(S)).  g = 2^e, or 0.75 * 2^e (then S*g has <= 6
    significant bits for the S used, so x stays exact in bf16)."""
    rng = np.random.default_rng(5)
    grid = _grid()
    sfs = [c for c in range(1, 0x7F) if c & 7 in ((0, 1, 2, 4) if gkind != "pow2" else range(8))]
    for trial in range(3000):
        c = rng.integers(0, 16, size=16)
        c[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
        sf = int(rng.choice(sfs))
        S = oracle.e4m3_value(sf)
        e = int(rng.integers(-20, 12))
        g = 2.0 ** e * (1.0 if gkind == "pow2" else 0.75)
        x = np.array([grid[int(ci)] * S * g for ci in c], np.float64)
        xb = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16)
        if not torch.equal(xb.double(), torch.from_numpy(x)):
            continue
        # codes of exact zeros keep their sign bit; -0 elements are written as -0
        p, got_sf = oracle.quantize_block(xb.view(torch.int16).numpy().view(np.uint16), g)
        codes = np.stack([p & 15, p >> 4], 1).ravel()
        assert got_sf == sf, (trial, sf, g)
        assert codes.tolist() == c.tolist(), (trial, c, codes)


def _blocks(rng, n, kind):
    if kind == "normal":
        x = rng.standard_normal((n, 16))
    else:  # heavy-tailed Student-t(3)
        x = rng.standard_normal((n, 16)) / np.sqrt((rng.standard_normal((n, 16, 3)) ** 2).sum(-1) / 3)
    return torch.from_numpy(x).to(torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("kind", ["normal", "t3"])
def test_quantize_block_error_bound_and_order(oracle, kind):
    """Unsaturated elements land within half an E2M1 spacing (plus fp32
    rounding slack) of x / (S g); codes are monotone in x within a block; the
    sign bit is the input's; S is the nearest-even E4M3 of amax / (6 g)."""
    rng = np.random.default_rng(7)
    grid = _grid()
    xb = _blocks(rng, 4000, kind)
    gs = np.exp(rng.normal(-4, 1.5, size=4000)).astype(np.float32)
    for x16, g in zip(xb, gs):
        bits = x16.view(torch.int16).numpy().view(np.uint16)
        p, sf = oracle.quantize_block(bits, float(g))
        codes = np.stack([p & 15, p >> 4], 1).ravel()
        x = x16.double().numpy()
        a = np.float32(np.abs(x).max())
        s = np.float32(a / np.float32(np.float32(6.0) * g))
        assert sf == int(torch.tensor([s]).to(torch.float8_e4m3fn).view(torch.uint8)) or (s > 448 and sf == 0x7E)
        S = oracle.e4m3_value(sf)
        dec = np.array([grid[int(c)] for c in codes])
        assert np.array_equal(np.signbit(dec), np.signbit(x))
        if sf == 0:
            assert (codes & 7 == 0).all()
            continue
        y = x / (S * float(g))
        ok = np.abs(y) <= 6
        spacing = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
        assert (np.abs(y - dec)[ok] <= 0.5 * spacing[ok] + 1e-5 * np.abs(y[ok]) + 1e-30).all()
        assert ((codes & 7)[~ok] == 7).all()
        order = np.argsort(x, kind="stable")
        assert (np.diff(dec[order]) >= 0).all()


def test_quantize_block_special_values(oracle):
    def q(vals, g=1.0):
        t = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
        p, sf = oracle.quantize_block(t.view(torch.int16).numpy().view(np.uint16), g)
        return np.stack([p & 15, p >> 4], 1).ravel().tolist(), sf

    # NaN is ignored by amax and quantizes to magnitude 0 (its own sign).
    codes, sf = q([float("nan"), 6.0] + [0.0] * 14)
    assert sf == 0x38 and codes[0] & 7 == 0 and codes[1] == 7
    # inf: amax = inf -> scale saturates to 448; inf -> 6, others tiny.
    codes, sf = q([float("inf"), float("-inf"), 1.0] + [0.0] * 13)
    assert sf == 0x7E and codes[:3] == [7, 15, 0]
    # huge g: s underflows to code 0; only the signs survive.
    codes, sf = q([1.0, -2.0] + [0.0] * 14, g=1e30)
    assert sf == 0 and codes[:2] == [0, 8]


def test_scale_predicate(oracle):
    for g, ok in [(1.0, True), (1e-40, True), (0.0, False), (-0.0, False), (-1.0, False),
                  (float("nan"), False), (float("inf"), False), (float("-inf"), False)]:
        assert oracle.scale_ok(g) == ok, g
