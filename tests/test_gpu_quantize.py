"""GPU quantiser parity: codes and scales must equal the oracle bit for bit
(the quantisation recipe of the lpnh.cn FP8 block-quantised GEMM page, s3.1,
s4.2, s5.4, has a unique result).  Calls go through the C ABI."""
import json
import os

import numpy as np
import pytest
import torch

import datagen
from gpu_util import dev, need_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dg():
    need_gpu()
    import fp8_block_scaled_dg_amd as m
    return m


def gpu_quant(dg, x, br):
    q, s = dg.to_fp8(dev(x), br)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check(dg, orc, x, br, what):
    q, s = gpu_quant(dg, x, br)
    oq, os_ = orc.quantize(x, br)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32)), what + ": scales differ"
    bad = np.argwhere(q != oq)
    assert bad.size == 0, "%s: %d codes differ, first %s gpu %s oracle %s x %r" % (
        what, len(bad), bad[:3].tolist(), q[tuple(bad[0])], oq[tuple(bad[0])], x[tuple(bad[0])])


@pytest.mark.parametrize("br", [128, 1])
@pytest.mark.parametrize("rows,cols", [(128, 512), (256, 512), (1, 128), (3, 16), (200, 384),
                                       (129, 1024), (300, 144), (64, 400)])
def test_quantize_small_and_ragged(dg, orc, rows, cols, br):
    x = datagen.normal((rows, cols), 1.0, seed=rows * 7 + cols, stream=br)
    check(dg, orc, x, br, "%dx%d/%d" % (rows, cols, br))


@pytest.mark.parametrize("br", [128, 1])
def test_quantize_special_blocks(dg, orc, br):
    x = datagen.normal((256, 640), 0.02, seed=3)
    x[:128, :128] = 0.0                      # all-zero block
    x[5, 7] = -0.0
    x[:, 128:256] *= np.float32(1e-38)       # amax/448 is subnormal: IEEE division path
    x[130:, 256:384] *= np.float32(1e-30)    # tiny but normal scale
    x[:, 384:512] = np.float32(2.0) ** np.arange(-20, 108, dtype=np.float32)[None, :]
    x[3, 512:] = -np.abs(x[3, 512:])
    x[10, 300] = x[200, 20] = x[7, 600] = x[255, 639] = -0.0   # -0 inside non-zero blocks
    check(dg, orc, x, br, "special/%d" % br)


def test_two_step_rounding_vectors_on_gpu(dg, orc):
    """Blocks built so that s = binary32(amax/448) equals the vector's s and
    the block holds x: the quotient x/s rounds to an E4M3 midpoint in binary32."""
    with open(os.path.join(GOLDEN, "two_step_rounding.json")) as f:
        vecs = json.load(f)["vectors"]
    x = np.zeros((len(vecs), 128), dtype=np.float32)
    expect = []
    for r, v in enumerate(vecs):
        xv = np.array([int(v["x_hex"], 16)], np.uint32).view(np.float32)[0]
        sv = np.array([int(v["s_hex"], 16)], np.uint32).view(np.float32)[0]
        amax = np.float32(sv * np.float32(448.0))
        for _ in range(64):                  # nudge amax until amax/448 gives s exactly
            got = amax / np.float32(448.0)
            if got == sv:
                break
            amax = np.nextafter(amax, np.float32(np.inf) if got < sv else np.float32(0))
        assert amax / np.float32(448.0) == sv
        x[r, 0] = amax
        x[r, 1] = xv
        expect.append(int(v["code"], 16))
    q, s = gpu_quant(dg, x, 1)
    assert q[:, 1].tolist() == expect
    check(dg, orc, x, 1, "r3")


@pytest.mark.parametrize("amax", [448.0, 56.0, 448.0 * 2.0 ** -70])
def test_quantize_every_midpoint_and_its_neighbours(dg, orc, amax):
    """Every block holds its amax (so s = amax/448 is a power of two and x/s
    is exact) and then quotients at every E4M3 rounding midpoint -- between
    consecutive magnitudes, subnormal range and the midpoint below the
    smallest subnormal included -- and at the binary32 neighbours on both
    sides, with both signs: the encoder's ties-to-even and its binade edges
    are checked on every code boundary."""
    mags = np.array(sorted({float(v) for v in orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))}))
    mids = (mags[:-1] + mags[1:]) / 2.0
    s = np.float32(amax) / np.float32(448.0)
    vals = []
    for m in mids.astype(np.float32):
        for v in (np.nextafter(m, np.float32(0)), m, np.nextafter(m, np.float32(np.inf))):
            vals += [v, -v]
    unscaled = np.array(vals, np.float32)
    vals = unscaled * s                   # exact: s is a power of two, no underflow
    assert np.array_equal(vals / s, unscaled)
    per_row = 127
    rows = -(-len(vals) // per_row)
    x = np.zeros((rows, 128), np.float32)
    x[:, 0] = np.float32(amax)
    flat = np.zeros(rows * per_row, np.float32)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(rows, per_row)
    for br in (1, 128):
        check(dg, orc, x, br, "midpoints amax=%g br=%d" % (amax, br))


@pytest.mark.parametrize("amax_bits", [0x054FE4BA,    # s = amax/448 ~ 1.86 * 2^-126
                                       0x05ABF09A,    # s ~ 1.27 * 2^-125
                                       0x069A8AC6,    # s ~ 1.10 * 2^-123
                                       0x13100000,    # s ~ 1.29 * 2^-98
                                       0x04DBC887,    # s subnormal, ~1.96 * 2^-127
                                       0x00C2A000])   # s subnormal, ~2^-135
def test_quantize_midpoints_with_tiny_scales(dg, orc, amax_bits):
    """Scales far below 1 that are not powers of two.  A quotient formed as
    x * RN(1/s) plus one FMA correction is misrounded there when the
    correction's remainder falls below binary32's smallest subnormal; the
    first three blocks were picked because that formula, evaluated without
    rescaling, gives a different E4M3 code than x / s for 14 to 19 of their
    values.  Each block holds the amax, then the binary32 values nearest to
    s times every E4M3 rounding midpoint and their neighbours two ulps either
    way, both signs; codes and scales must match the oracle bit for bit."""
    amax = np.array([amax_bits], np.uint32).view(np.float32)[0]
    s = np.float32(amax / np.float32(448.0))
    mags = np.array(sorted({float(v) for v in orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))}))
    mids = (mags[:-1] + mags[1:]) / 2.0
    vals = []
    for m in mids:
        v = np.float32(m * float(s))           # nearest binary32 to m*s
        cand = [v]
        for _ in range(2):
            cand = [np.nextafter(cand[0], np.float32(0))] + cand + \
                   [np.nextafter(cand[-1], np.float32(np.inf))]
        for c in cand:
            if np.abs(c) <= amax:
                vals += [c, -c]
    per_row = 127
    rows = -(-len(vals) // per_row)
    x = np.zeros((rows, 128), np.float32)
    x[:, 0] = amax
    flat = np.zeros(rows * per_row, np.float32)
    flat[:len(vals)] = np.array(vals, np.float32)
    x[:, 1:] = flat.reshape(rows, per_row)
    for br in (1, 128):
        check(dg, orc, x, br, "tiny scale, amax 0x%08x br=%d" % (amax_bits, br))


@pytest.mark.parametrize("what,rows,cols,br", [
    ("C2a A", 4096, 2048, 128), ("C2c B", 8192, 8192, 128), ("C3 A M=64", 64, 16384, 1),
    ("C4 down A", 2816, 11008, 1)])
def test_quantize_full_size(dg, orc, what, rows, cols, br):
    x = datagen.normal((rows, cols), 1.0 if br == 1 else 0.02, seed=0, stream=1)
    check(dg, orc, x, br, what)


def test_quantize_outlier_activations(dg, orc):
    x, hot = datagen.student_t_outliers(1024, 8192, seed=0, stream=5)
    check(dg, orc, x, 1, "C5 A rows")
    check(dg, orc, x, 128, "C5 A rows global-ish")


def test_quantize_deterministic(dg):
    x = dev(datagen.normal((1024, 2048), 1.0, seed=4))
    q1, s1 = dg.to_fp8(x, 128)
    q2, s2 = dg.to_fp8(x, 128)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


@pytest.mark.parametrize("rows,cols,br", [(65535 * 32, 128, 1), (65535 * 128, 16, 128)])
def test_quantize_at_grid_limit(dg, orc, rows, cols, br):
    """The largest row counts the quantiser's launch accepts (65535 workgroup
    rows); one more block row is rejected on the host.  Sampled blocks (rows
    are independent across blocks) are compared with the oracle bit for bit."""
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    x = torch.randn((rows, cols), device="cuda", generator=g)
    q, s = dg.to_fp8(x, br)
    torch.cuda.synchronize()
    for blk in (0, 1, rows // br // 2, rows // br - 1):
        r0 = blk * br
        xs = x[r0:r0 + br].cpu().numpy()
        oq, os_ = orc.quantize(xs, br)
        assert np.array_equal(q[r0:r0 + br].cpu().numpy(), oq), blk
        got_s = s[:, blk:blk + 1].cpu().numpy()
        assert np.array_equal(got_s.view(np.uint32), os_.view(np.uint32)), blk
    bad = torch.empty((rows + (32 if br == 1 else 128), cols), device="cuda")
    qb = torch.empty(bad.shape, dtype=torch.uint8, device="cuda")
    sb = torch.empty((-(-cols // 128), bad.shape[0] // br), device="cuda")
    with pytest.raises(dg.DGError):
        dg.dg_quantize_fp8_block(qb, sb, bad, br)
