"""Pins of the oracle's precision configurations (oracle/layer.py, FourTune §4 "Impact
of Precision Configurations").

- closed form: with a weight on the E2M1 grid (block exponents 0, so deq Q(R) = R),
  the A16 forward is bf16(X) R^T + XL U^T and the G16 backward bf16(G) R + GB D,
  evaluated here with plain matmuls;
- finite differences: with the bf16 roundings off, the A16 forward is linear in X and
  the G16 backward's dX is its gradient of <Y, G> (the weight read transposed);
- the 16-bit and 4-bit configurations differ on ordinary data (the switch is live).
"""
import numpy as np

from oracle import layer, mx4
from oracle.layer import Linear, Prec
from tests.test_oracle_layer import _fd, _lin


def _on_grid(rng, rows, cols):
    v = mx4.E2M1_GRID[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    v[::32, ::32] = 6.0
    return v


def test_prec_closed_form_on_grid_weight():
    rng = np.random.default_rng(50)
    M, N, K, r, s = 40, 64, 96, 16, 16
    lin = _lin(rng, N, K, r, s)
    lin = Linear(R=_on_grid(rng, N, K), A=lin.A, B=lin.B, L1=lin.L1, L2=lin.L2)
    assert np.array_equal(mx4.fake_quant(lin.R), lin.R)
    X, G = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    Y, XL = layer.linear_forward_prec(X, lin, a16=True)
    XLw = mx4.bf16_round(mx4.bf16_round(X) @ lin.D().T)
    np.testing.assert_allclose(Y, mx4.bf16_round(X) @ lin.R.T + XLw @ lin.U().T, rtol=1e-12, atol=1e-12)
    dX, dA, dB, GB = layer.linear_backward_prec(G, X, XL, lin, g16=True)
    GBw = mx4.bf16_round(mx4.bf16_round(G) @ lin.U())
    np.testing.assert_allclose(dX, mx4.bf16_round(G) @ lin.R + GBw @ lin.D(), rtol=1e-12, atol=1e-12)


def test_prec_g16_is_gradient_of_a16():
    rng = np.random.default_rng(51)
    M, N, K, r, s = 5, 64, 32, 2, 2
    lin = _lin(rng, N, K, r, s, scale=0.5)
    X, G = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    p = Prec(quant=True, bf16=False)

    def loss():
        Y, _ = layer.linear_forward_prec(X, lin, a16=True, prec=p)
        return float(np.sum(Y * G))

    _, XL = layer.linear_forward_prec(X, lin, a16=True, prec=p)
    dX, dA, dB, _ = layer.linear_backward_prec(G, X, XL, lin, g16=True, prec=p)
    np.testing.assert_allclose(dX, _fd(loss, X, 1e-6), rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(dA, _fd(loss, lin.A, 1e-6), rtol=1e-7, atol=1e-8)


def test_prec_configurations_differ():
    rng = np.random.default_rng(52)
    lin = _lin(rng, 64, 64, 16, 16)
    X = rng.standard_normal((32, 64))
    Y4, _ = layer.linear_forward_prec(X, lin, a16=False)
    Y16, _ = layer.linear_forward_prec(X, lin, a16=True)
    Yref, _ = layer.linear_forward(X, lin)
    assert np.array_equal(Y4, Yref)
    assert np.abs(Y16 - Y4).max() > 0
