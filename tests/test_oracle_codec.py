"""Pins for the oracle's E4M3 codec, independent of the oracle itself.

The FP8 format is E4M3 with largest finite value 448 (lpnh.cn page on the FP8
block-quantised GEMM, s2.2 and s3.1); rounding is to the nearest value with
ties to even (same page, s4.2).  Independent references used here:
PyTorch's float8_e4m3fn dtype (decode table and binary32 cast), an
exact-rational nearest search (tests/exact.py), and the oracle's second
encoder, a brute-force table search written separately from the arithmetic
encoder.
"""
import concurrent.futures as cf
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_cast(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_256_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = exact.torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero of 0x80
    assert np.signbit(ours[0x80]) and ours[0x80] == 0.0


def test_decode_closed_forms(orc):
    d = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert d[0x7E] == 448.0                     # largest finite value
    assert d[0x38] == 1.0                       # exponent field 7 = bias
    assert d[0x08] == 2.0 ** -6                 # smallest normal
    assert d[0x01] == 2.0 ** -9                 # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert np.sum(np.isfinite(d)) == 254
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)             # monotone over 0x00..0x7E
    for c in range(0x7F):
        assert d[c | 0x80] == -d[c]
    # the decode table equals the exact-rational enumeration of the format
    assert [Fraction(float(v)) for v in pos] == exact.E4M3_MAG


def test_encode_roundtrip_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    for method in ("arith", "search"):
        back = orc.e4m3_encode(vals, method)
        finite = np.isfinite(vals)
        assert np.array_equal(back[finite], codes[finite])
        assert back[0x7F] == 0x7F and back[0xFF] == 0xFF   # NaN keeps its sign


def test_all_midpoints_go_to_even_code(orc):
    mags = exact.E4M3_MAG
    mids = []
    for c in range(126):
        m = (mags[c] + mags[c + 1]) / 2
        f = np.float32(float(m))
        assert Fraction(float(f)) == m           # midpoints are exact binary32
        mids.append(f)
    mids = np.array(mids, dtype=np.float32)
    for method in ("arith", "search"):
        got = orc.e4m3_encode(mids, method)
        want = np.array([c if c % 2 == 0 else c + 1 for c in range(126)], dtype=np.uint8)
        assert np.array_equal(got, want)
        assert np.array_equal(orc.e4m3_encode(-mids, method), want | 0x80)
    assert np.array_equal(orc.e4m3_encode(mids), _torch_cast(mids))


def test_saturation_and_signed_zero(orc):
    v = np.array([448.0, 455.0, 463.99, 464.0, 480.0, 1e6, 3.0e38, -464.0, -1e9,
                  0.0, -0.0, 1e-30, -1e-30, -1e-45, 2.0 ** -10, -(2.0 ** -10)],
                 dtype=np.float32)
    want = np.array([0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE,
                     0x00, 0x80, 0x00, 0x80, 0x80, 0x00, 0x80], dtype=np.uint8)
    for method in ("arith", "search"):
        assert np.array_equal(orc.e4m3_encode(v, method), want)


def _neighbourhood_values():
    """Every binary32 within 8 ulps of each E4M3 magnitude and midpoint,
    and of the powers of two in the E4M3 range, both signs."""
    mags = exact.E4M3_MAG
    pts = [float(m) for m in mags]
    pts += [float((mags[c] + mags[c + 1]) / 2) for c in range(126)]
    pts += [2.0 ** e for e in range(-14, 10)] + [464.0, 2.0 ** -10, 2.0 ** -11]
    base = np.array(pts, dtype=np.float32).view(np.int32)
    offs = np.arange(-8, 9, dtype=np.int32)
    bits = (base[:, None] + offs[None, :]).ravel()
    bits = bits[bits >= 0]
    v = bits.view(np.float32)
    v = v[np.abs(v) <= 464.0]
    return np.concatenate([v, -v])


def test_two_encoders_agree_near_every_boundary(orc):
    v = _neighbourhood_values()
    a = orc.e4m3_encode(v, "arith")
    s = orc.e4m3_encode(v, "search")
    assert np.array_equal(a, s)
    assert np.array_equal(a, _torch_cast(v))


def test_two_encoders_agree_on_random_binary32(orc):
    g = np.random.default_rng(1234)
    bits = g.integers(0, 0x43E80001, size=400_000, dtype=np.int64).astype(np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    a = orc.e4m3_encode(v, "arith")
    assert np.array_equal(a, orc.e4m3_encode(v, "search"))
    assert np.array_equal(a, _torch_cast(v))


def test_exact_rational_nearest_on_sample(orc):
    g = np.random.default_rng(7)
    bits = g.integers(0x30000000, 0x43E80001, size=3000, dtype=np.int64).astype(np.uint32)
    v = bits.view(np.float32)
    got = orc.e4m3_encode(v)
    want = [exact.nearest_even_code(Fraction(float(x)), False) for x in v]
    assert got.tolist() == want


@pytest.mark.slow
def test_arith_encoder_matches_torch_on_every_binary32(orc):
    """Every binary32 bit pattern with |v| <= 464, both signs (2.3e9 values):
    the arithmetic encoder equals PyTorch's float8_e4m3fn cast (which rounds
    to nearest-even and agrees with saturation up to 464).  Chunks of 2^24
    patterns run on host threads (the oracle's C code releases the GIL)."""
    top = 0x43E80000  # 464.0
    starts = list(range(0, top + 1, 1 << 24))

    def chunk(start):
        bits = np.arange(start, min(start + (1 << 24), top + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        for w in (v, -v):
            if not np.array_equal(orc.e4m3_encode(w), _torch_cast(w)):
                return start
        return None
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        bad = [s for s in ex.map(chunk, starts) if s is not None]
    assert not bad, [hex(b) for b in bad[:4]]


def test_search_encoder_near_every_code_and_midpoint(orc):
    """The brute-force search encoder against the arithmetic one on every
    binary32 within 64 ulps of each E4M3 value and each rounding midpoint
    (both signs), and on every 4096th pattern below 464."""
    vals = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [448.0, 456.0, 464.0]]).astype(np.float32)
    u = pts.view(np.uint32).astype(np.int64)
    near = (u[:, None] + np.arange(-64, 65)[None, :]).ravel()
    near = near[(near >= 0) & (near <= 0x43E80000)].astype(np.uint32)
    sweep = np.arange(0, 0x43E80001, 4096, dtype=np.uint32)
    v = np.concatenate([near, sweep]).view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(orc.e4m3_encode(v, "search"), orc.e4m3_encode(v, "arith"))


def test_two_step_rounding_vectors(orc):
    """The quotient is rounded to binary32 first, then to E4M3."""
    with open(os.path.join(GOLDEN, "two_step_rounding.json")) as f:
        vecs = json.load(f)["vectors"]
    for vec in vecs:
        x = np.array([int(vec["x_hex"], 16)], dtype=np.uint32).view(np.float32)
        s = np.array([int(vec["s_hex"], 16)], dtype=np.uint32).view(np.float32)
        v = x / s
        assert float(v[0]) == vec["v"]
        code = int(vec["code"], 16)
        assert orc.e4m3_encode(v)[0] == code
        assert exact.nearest_even_code(Fraction(float(v[0])), False) == code
        one = exact.nearest_even_code(Fraction(float(x[0])) / Fraction(float(s[0])), False)
        assert one == int(vec["one_step_code"], 16) and one != code
