"""Pins for the oracle's fused epilogue (bjdmk.com.cn DeepGEMM page s3.2:
activation and residual applied to the product before it is written; pzsr.cn
DeepGEMM page s2.3: SwiGLU), checked against textbook values and identities:
SiLU(1) = 1/(1 + e^-1), GELU(+-1) = +-Phi(+-1), SiLU(-x) = SiLU(x) - x,
GELU(x) - GELU(-x) = x, SwiGLU with unit up = SiLU of the gate, and the
residual added exactly from its BF16 bits."""
import math

import numpy as np
import pytest


def test_textbook_values(orc):
    a = np.array([[1.0, -1.0, 0.0, 3.5]])
    silu = orc.epilogue(a, "silu")[0]
    gelu = orc.epilogue(a, "gelu")[0]
    assert silu[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert silu[2] == 0.0
    assert gelu[0] == pytest.approx(0.8413447460685429, rel=1e-15)     # Phi(1)
    assert gelu[1] == pytest.approx(-0.15865525393145707, rel=1e-14)   # -Phi(-1)
    assert gelu[2] == 0.0
    assert list(orc.epilogue(a, "relu")[0]) == [1.0, 0.0, 0.0, 3.5]
    assert list(orc.epilogue(a, "none")[0]) == [1.0, -1.0, 0.0, 3.5]


def test_symmetry_identities(orc):
    x = np.linspace(-30.0, 30.0, 241)[None, :]
    s_pos, s_neg = orc.epilogue(x, "silu"), orc.epilogue(-x, "silu")
    assert np.allclose(s_neg, s_pos - x, rtol=0, atol=1e-12)
    g_pos, g_neg = orc.epilogue(x, "gelu"), orc.epilogue(-x, "gelu")
    assert np.allclose(g_pos - g_neg, x, rtol=0, atol=1e-12)
    assert np.all(orc.epilogue(x, "relu") == np.maximum(x, 0.0))


def test_swiglu_pairs_interleaved_columns(orc):
    g = np.random.default_rng(2)
    gate = g.standard_normal((5, 6))
    up = g.standard_normal((5, 6))
    acc = np.empty((5, 12))
    acc[:, 0::2], acc[:, 1::2] = gate, up
    out = orc.epilogue(acc, "swiglu")
    assert out.shape == (5, 6)
    # unit up gives the gate's SiLU; unit gate gives SiLU(1) times up
    acc_u = acc.copy(); acc_u[:, 1::2] = 1.0
    assert np.array_equal(orc.epilogue(acc_u, "swiglu"), orc.epilogue(gate, "silu"))
    acc_g = acc.copy(); acc_g[:, 0::2] = 1.0
    assert np.allclose(orc.epilogue(acc_g, "swiglu"), up / (1.0 + math.exp(-1.0)),
                       rtol=1e-15, atol=0)


@pytest.mark.parametrize("act", ["none", "relu", "silu", "gelu", "swiglu"])
def test_residual_is_added_exactly(orc, act):
    g = np.random.default_rng(3)
    acc = g.standard_normal((4, 16))
    n_out = 8 if act == "swiglu" else 16
    r_f32 = g.standard_normal((4, n_out)).astype(np.float32)
    r_bits = (r_f32.view(np.uint32) >> 16).astype(np.uint16)         # truncated to BF16
    r_val = (r_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with_r = orc.epilogue(acc, act, residual=r_bits)
    assert np.array_equal(with_r, orc.epilogue(acc, act) + r_val)
