"""The quantiser forms x / s from one reciprocal per block and a fused
multiply-add correction per element, rescaling blocks with s < 2^-62 by
2^64 first (lpnh.cn FP8 block-quantised GEMM page, s4.2 step 4: divide by
the scale, then round).  Restated in C (tests/csrc/quotient.c, compiled here
with gcc), it must equal IEEE binary32 division on the values whose E4M3
code could depend on it: inputs next to every E4M3 rounding midpoint and
random bit patterns, for scales across the whole binary32 range, subnormal
scales included.  Quotients below 2^-11 encode to zero whichever way they
are rounded; there the codes are compared."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def qlib(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("quot") / "libquot.so")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    os.path.join(HERE, "csrc", "quotient.c"), "-o", so, "-lm"], check=True)
    lib = ctypes.CDLL(so)
    for fn in (lib.quotient_fma, lib.quotient_div):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
    return lib


def run(lib, x, s):
    x = np.ascontiguousarray(x, np.float32)
    s = np.ascontiguousarray(s, np.float32)
    out = [np.empty_like(x), np.empty_like(x)]
    for fn, o in zip((lib.quotient_fma, lib.quotient_div), out):
        fn(x.ctypes.data, s.ctypes.data, o.ctypes.data, x.size)
    return out


def midpoints():
    """The 126 positive E4M3 rounding midpoints below 448 (between
    consecutive finite codes) as float64."""
    from fractions import Fraction
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else
                    (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return np.array([float((a + b) / 2) for a, b in zip(vals[:-1], vals[1:])])


def scales(rng):
    """Scales from every binade a block scale amax / 448 can take (2^-149 ..
    2^118: 448 s stays finite), subnormals included, with random mantissas,
    plus exact powers of two."""
    out = []
    for e in range(-149, 119):
        m = rng.random(6) + 1.0
        out.append(np.float32(2.0) ** np.float32(e) if e >= -126 else np.float32(2.0 ** e))
        out.extend((m * 2.0 ** e).astype(np.float32))
    s = np.array(out, np.float32)
    return s[s > 0]


def check(lib, x, s, orc):
    fma, div = run(lib, x, s)
    big = div >= np.float32(2.0 ** -11)
    assert np.array_equal(fma[big].view(np.uint32), div[big].view(np.uint32)), \
        (x[big][fma[big] != div[big]][:4], s[big][fma[big] != div[big]][:4])
    assert np.array_equal(orc.e4m3_encode(fma), orc.e4m3_encode(div))


def test_quotient_near_every_midpoint_across_the_scale_range(qlib, orc):
    rng = np.random.default_rng(1)
    mids = midpoints()
    s = scales(rng)
    xs, ss = [], []
    for sv in s:
        # the binary32 values nearest to s * midpoint, and 3 ulps either side
        t = (np.float64(sv) * mids).astype(np.float32)
        t = t[np.isfinite(t) & (t > 0)]
        u = t.view(np.uint32).astype(np.int64)
        for d in range(-3, 4):
            xs.append((u + d).astype(np.uint32).view(np.float32))
            ss.append(np.full(u.size, sv, np.float32))
    x, s = np.concatenate(xs), np.concatenate(ss)
    keep = np.isfinite(x) & (x > 0)
    assert keep.sum() > 400000
    check(qlib, x[keep], s[keep], orc)
    check(qlib, -x[keep], s[keep], orc)


def test_quotient_random_bits_across_the_scale_range(qlib, orc):
    rng = np.random.default_rng(2)
    s = scales(rng)
    s = np.repeat(s, 400)
    # |x| up to 448 s (x / s never exceeds that inside a block), random bits below
    top = (s.astype(np.float64) * 448.0).astype(np.float32).view(np.uint32)
    x = (rng.random(s.size) * top).astype(np.uint32).view(np.float32)
    check(qlib, x, s, orc)
    # and the amax element itself: x = amax = 448 s exactly representable or not
    amax = (s.astype(np.float64) * 448.0).astype(np.float32)
    ok = np.isfinite(amax)
    check(qlib, amax[ok], (amax[ok] / np.float32(448.0)).astype(np.float32), orc)
