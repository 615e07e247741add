"""Pins of the oracle's layer arithmetic (oracle/layer.py).

- brute force: a pure-Python Fraction triple loop over the codes equals the oracle's
  4-bit product exactly;
- library special case: on-grid operands reduce the quantized product to numpy.matmul;
- closed form: with quantization and bf16 rounding off, the three branches equal one
  linear with the merged weight R + L2 L1 + B A (FourTune §3.1);
- finite differences: the backward (dX, dA, dB; and through GELU for the MLP) is the
  derivative of <Y, G> (FourTune §3.2);
- GELU identities;
- hand-computed cases with quantization and bf16 rounding on: the MLP pair on on-grid
  operands whose FC1 output lands on an E2M1 tie (the fp32 decision precision of Q(H)
  and Q(dP), the rounding of P^, GELU' in dP), and an fp32-input linear whose bf16
  roundings (X^, G^, XL, GB) survive cancellation, so each rounding point changes an
  output value.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import layer, mx4
from oracle.layer import Linear, Prec

OFF = Prec(quant=False, bf16=False)


def _lin(rng, N, K, r, s, scale=0.05):
    return Linear(R=rng.standard_normal((N, K)) * scale,
                  A=rng.standard_normal((r, K)) * scale,
                  B=rng.standard_normal((N, r)) * scale,
                  L1=rng.standard_normal((s, K)) * scale,
                  L2=rng.standard_normal((N, s)) * scale)


# ---------------------------------------------------------------- 4-bit product
def _frac_deq(codes, scales):
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    rows, cols = codes.shape
    out = [[None] * cols for _ in range(rows)]
    for i in range(rows):
        for j in range(cols):
            c = int(codes[i, j])
            v = grid[c & 7] * (-1 if c & 8 else 1)
            e = int(scales[i // 32, j // 32]) - 127
            out[i][j] = v * (Fraction(2) ** e)
    return out


def test_gemm_brute_force_fraction():
    rng = np.random.default_rng(10)
    M, N, K = 64, 64, 64
    X = rng.standard_normal((M, K)) * np.ldexp(1.0, rng.integers(-3, 3, (M, 1)))
    R = rng.standard_t(3, (N, K)) * 0.02
    cx, sx = mx4.quantize(X)
    cr, sr = mx4.quantize(R)
    fx, fr = _frac_deq(cx, sx), _frac_deq(cr, sr)
    lin = Linear(R=R, A=np.zeros((0, K)), B=np.zeros((N, 0)), L1=np.zeros((0, K)),
                 L2=np.zeros((N, 0)))
    Y, XL = layer.linear_forward(X, lin)
    assert XL.shape == (M, 0)
    for i in range(M):
        for j in range(N):
            exact = sum(fx[i][k] * fr[j][k] for k in range(K))
            assert Y[i, j] == float(exact), (i, j)


def test_gemm_on_grid_equals_matmul():
    rng = np.random.default_rng(11)
    M, N, K = 64, 96, 128

    def on_grid(rows, cols):
        v = mx4.E2M1_GRID[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
        v[::32, ::32] = 6.0  # pins every block's exponent at 0
        return v

    X, R = on_grid(M, K), on_grid(N, K)
    lin = Linear(R=R, A=np.zeros((0, K)), B=np.zeros((N, 0)), L1=np.zeros((0, K)),
                 L2=np.zeros((N, 0)))
    Y, _ = layer.linear_forward(X, lin)
    assert np.array_equal(Y, np.matmul(X, R.T))
    G = on_grid(M, N)
    dX, dA, dB, _ = layer.linear_backward(G, X, np.zeros((M, 0)), lin)
    assert np.array_equal(dX, np.matmul(G, R))


# ---------------------------------------------------------------- triple branch
def test_forward_equals_merged_weight():
    rng = np.random.default_rng(12)
    M, N, K, r, s = 40, 48, 64, 8, 4
    lin = _lin(rng, N, K, r, s)
    X = rng.standard_normal((M, K))
    Y, XL = layer.linear_forward(X, lin, OFF)
    W_eff = lin.R + lin.L2 @ lin.L1 + lin.B @ lin.A
    np.testing.assert_allclose(Y, X @ W_eff.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(XL[:, :r], X @ lin.A.T, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(XL[:, r:], X @ lin.L1.T, rtol=1e-12, atol=1e-13)


def test_rank_zero_is_plain_quantized_gemm():
    rng = np.random.default_rng(13)
    M, N, K = 64, 64, 96
    X, R = rng.standard_normal((M, K)), rng.standard_normal((N, K)) * 0.02
    lin = Linear(R=R, A=np.zeros((0, K)), B=np.zeros((N, 0)), L1=np.zeros((0, K)),
                 L2=np.zeros((N, 0)))
    Y, _ = layer.linear_forward(X, lin)
    assert np.array_equal(Y, mx4.fake_quant(X) @ mx4.fake_quant(R).T)


def _fd(f, x, eps):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_linear_backward_finite_differences():
    rng = np.random.default_rng(14)
    M, N, K, r, s = 6, 10, 8, 3, 2
    lin = _lin(rng, N, K, r, s, scale=0.5)
    X = rng.standard_normal((M, K))
    G = rng.standard_normal((M, N))

    def loss():
        Y, _ = layer.linear_forward(X, lin, OFF)
        return float(np.sum(Y * G))

    _, XL = layer.linear_forward(X, lin, OFF)
    dX, dA, dB, GB = layer.linear_backward(G, X, XL, lin, OFF)
    np.testing.assert_allclose(dX, _fd(loss, X, 1e-6), rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(dA, _fd(loss, lin.A, 1e-6), rtol=1e-7, atol=1e-8)
    np.testing.assert_allclose(dB, _fd(loss, lin.B, 1e-6), rtol=1e-7, atol=1e-8)
    # the frozen branches are used in dX (a dropped stabilizer term would fail here)
    assert np.abs(_fd(loss, lin.L1, 1e-6)).max() > 1e-3
    np.testing.assert_allclose(GB, G @ lin.U(), rtol=1e-12)


def test_backward_backbone_uses_quantized_operands():
    """With quantization on and bf16 off, dX - GB D is the 4-bit product Q(G) Q(R)."""
    rng = np.random.default_rng(15)
    M, N, K, r, s = 64, 64, 96, 4, 4
    lin = _lin(rng, N, K, r, s)
    X, G = rng.standard_normal((M, K)), rng.standard_normal((M, N)) * 1e-3
    prec = Prec(quant=True, bf16=False)
    _, XL = layer.linear_forward(X, lin, prec)
    dX, _, _, GB = layer.linear_backward(G, X, XL, lin, prec)
    np.testing.assert_allclose(dX - GB @ lin.D(), mx4.fake_quant(G) @ mx4.fake_quant(lin.R),
                               rtol=1e-12, atol=1e-15)


def test_bf16_rounding_points_are_small():
    rng = np.random.default_rng(16)
    M, N, K, r, s = 64, 64, 64, 8, 8
    lin = _lin(rng, N, K, r, s)
    X = rng.standard_normal((M, K))
    _, XL_on = layer.linear_forward(X, lin, Prec(quant=False, bf16=True))
    _, XL_off = layer.linear_forward(X, lin, Prec(quant=False, bf16=False))
    # bf16 keeps 8 significant bits: the roundings of X and XL move XL by ~2^-9 relative
    rel = np.linalg.norm(XL_on - XL_off) / np.linalg.norm(XL_off)
    assert 2 ** -14 < rel < 2 ** -7
    assert np.array_equal(mx4.bf16_round(XL_on), XL_on)  # the saved XL holds bf16 values


# ---------------------------------------------------------------- GELU and MLP
def test_gelu_identities():
    x = np.linspace(-8, 8, 4001)
    g = layer.gelu_tanh(x)
    assert layer.gelu_tanh(0.0) == 0.0 and layer.gelu_tanh_grad(0.0) == 0.5
    np.testing.assert_allclose(g - layer.gelu_tanh(-x), x, atol=1e-12)  # g(x) - g(-x) = x
    np.testing.assert_allclose(layer.gelu_tanh(np.array([20.0, 40.0])), [20.0, 40.0])
    assert np.all(np.abs(layer.gelu_tanh(np.array([-20.0, -40.0]))) < 1e-30)
    h = 1e-5
    np.testing.assert_allclose(layer.gelu_tanh_grad(x),
                               (layer.gelu_tanh(x + h) - layer.gelu_tanh(x - h)) / (2 * h),
                               atol=1e-8)
    # the tanh form approximates x * Phi(x) to about 1e-3
    from scipy.special import erf
    assert np.max(np.abs(g - 0.5 * x * (1 + erf(x / np.sqrt(2))))) < 1e-3


def test_mlp_backward_finite_differences():
    rng = np.random.default_rng(17)
    M, D, F, r, s = 5, 8, 12, 2, 2
    fc1 = _lin(rng, F, D, r, s, scale=0.4)
    fc2 = _lin(rng, D, F, r, s, scale=0.4)
    X = rng.standard_normal((M, D))
    G = rng.standard_normal((M, D))

    def loss():
        return float(np.sum(layer.mlp_forward(X, fc1, fc2, OFF)["Y"] * G))

    saved = layer.mlp_forward(X, fc1, fc2, OFF)
    g = layer.mlp_backward(G, X, saved, fc1, fc2, OFF)
    kw = dict(rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(g["dX"], _fd(loss, X, 1e-6), **kw)
    np.testing.assert_allclose(g["dA1"], _fd(loss, fc1.A, 1e-6), **kw)
    np.testing.assert_allclose(g["dB1"], _fd(loss, fc1.B, 1e-6), **kw)
    np.testing.assert_allclose(g["dA2"], _fd(loss, fc2.A, 1e-6), **kw)
    np.testing.assert_allclose(g["dB2"], _fd(loss, fc2.B, 1e-6), **kw)


def test_mlp_epilogue_decision_in_fp32():
    """Q(H) is decided on fp32(GELU(P)). With P bf16, GELU(P) rounds to P in fp32 for
    P above ~5.3, so an element P = 7 in a block whose maximum is 12 (scale 2) sits on
    the 3 | 4 threshold (7 / 2 = 3.5) and rounds to the even code (4, i.e. 8.0); the
    fp64 value GELU(7) = 7 - 3e-15 would fall just below it (3, i.e. 6.0)."""
    P = np.zeros((32, 32))
    P[0, 0], P[5, 7] = 12.0, 7.0
    H = layer.gelu_tanh(P)
    assert H[5, 7] < 7.0 and layer.fp32(H)[5, 7] == 7.0
    assert mx4.fake_quant(layer.fp32(H))[5, 7] == 8.0
    assert mx4.fake_quant(H)[5, 7] == 6.0


# ---------------------------------------------------------------- quantized MLP, by hand
# On-grid operands, no low-rank branches: every product below is exact, so the expected
# outputs are written down by hand (FourTune §3.3 "MLP Fusion": FC2's 4-bit operand is
# the quantized GELU of FC1's output; §3.2: FC1's backward takes the quantized gradient
# dP = dH * GELU'(P^)). Shapes: M = 32, d = 64, f = 32.
#   R1 [f x d]: R1[j, j] = R1[j, (j+16) % 32] = R1[j, 32+j] = 1, so
#               P[i, j] = X[i, j] + X[i, (j+16) % 32] + X[i, 32+j];
#   R2 [d x f] = [I; I], so Y[i, c] = Hq[i, c % 32] and dH[i, j] = G[i, j] + G[i, 32+j].
# Every block of X, R1, R2 and G holds its amax exactly on a power-of-two multiple of 4
# or 6 or is otherwise representable, so Q() leaves them unchanged.
def _mlp_hand_case():
    M, d, f = 32, 64, 32
    R1 = np.zeros((f, d))
    for j in range(f):
        R1[j, j] = R1[j, (j + 16) % 32] = R1[j, 32 + j] = 1.0
    R2 = np.vstack([np.eye(f), np.eye(f)])
    X = np.zeros((M, d))
    X[0, 0] = X[0, 16] = 6.0                         # P[0, 0] = P[0, 16] = 12
    X[5, 7], X[5, 23] = 4.0, 3.0                     # P[5, 7] = P[5, 23] = 7: a tie after GELU
    X[9, 3], X[9, 19], X[9, 35] = 4.0, 3.0, -2.0 ** -8   # P[9, 3] = 7 - 2^-8, P^ = bf16 -> 7
    G = np.zeros((M, d))
    G[0, 0] = G[0, 32] = 3.0                         # dH[0, 0] = 6, GELU'(12) = 1
    G[5, 7], G[5, 39] = 1.0, 0.25                    # dH[5, 7] = 1.25, GELU'(7) = 1 + 3e-14
    G[9, 10] = 3.0                                   # dH[9, 10] = 3, GELU'(0) = 1/2
    empty = dict(A=np.zeros((0, d)), B=np.zeros((f, 0)), L1=np.zeros((0, d)), L2=np.zeros((f, 0)))
    fc1 = Linear(R=R1, **empty)
    fc2 = Linear(R=R2, A=np.zeros((0, f)), B=np.zeros((d, 0)), L1=np.zeros((0, f)), L2=np.zeros((d, 0)))
    return X, G, fc1, fc2


def test_mlp_quantized_forward_by_hand():
    """P^ = bf16(FC1 out) holds 12 (block max: scale 2) and 7 = 3.5 * 2, a tie that the
    fp32 value of GELU(7) sits on (rounds to the even code: 4 * 2 = 8) and fp64's
    GELU(7) = 7 - 3e-15 misses (3 * 2 = 6); P[9, 3] = 7 - 2^-8 rounds to P^ = 7 first.
    A wrong decision precision, a skipped rounding of P or a missing Q(H) each change Y."""
    X, G, fc1, fc2 = _mlp_hand_case()
    assert np.array_equal(mx4.fake_quant(X), X) and np.array_equal(mx4.fake_quant(fc1.R), fc1.R)
    out = layer.mlp_forward(X, fc1, fc2)
    P = np.zeros((32, 32))
    P[0, 0] = P[0, 16] = 12.0
    P[5, 7] = P[5, 23] = P[9, 3] = P[9, 19] = 7.0
    assert np.array_equal(out["P"], P)
    Hq = np.zeros((32, 32))
    Hq[0, 0] = Hq[0, 16] = 12.0
    Hq[5, 7] = Hq[5, 23] = Hq[9, 3] = Hq[9, 19] = 8.0
    assert np.array_equal(out["Y"], np.hstack([Hq, Hq]))


def test_mlp_quantized_backward_by_hand():
    """dP = dH * GELU'(P^): dP[5, 7] = 1.25 (1 + 3e-14) in fp64, exactly 1.25 in fp32, the
    1 | 1.5 tie in a block of maximum 6 (scale 1): the fp32 decision rounds to the even
    code (1); dP[9, 10] = 3 * GELU'(0) = 1.5. dX = Q(dP) Q(R1) spreads each code to its
    three input columns."""
    X, G, fc1, fc2 = _mlp_hand_case()
    saved = layer.mlp_forward(X, fc1, fc2)
    g = layer.mlp_backward(G, X, saved, fc1, fc2)
    dPq = np.zeros((32, 32))
    dPq[0, 0], dPq[5, 7], dPq[9, 10] = 6.0, 1.0, 1.5
    dX = np.zeros((32, 64))
    for i, j in ((0, 0), (5, 7), (9, 10)):
        dX[i, j] = dX[i, (j + 16) % 32] = dX[i, 32 + j] = dPq[i, j]
    assert np.array_equal(g["dX"], dX)
    assert g["dP32"][5, 7] == 1.25 and g["dP"][5, 7] > 1.25


# ---------------------------------------------------------------- bf16 rounding points
def test_bf16_rounding_points_by_hand():
    """fp32 input and gradient whose bf16 roundings survive cancellation (the c1 input is
    fp32): X^ = bf16(X) before the down-projection and in dA, G^ = bf16(G) in GB and dB,
    and the single roundings of XL and GB. x = 1 + 3 * 2^-9 rounds to 1 + 2^-7 and
    1 + 2^-8 (a tie) rounds to 1. Rank 1, no stabilizer, R = 0."""
    K = N = 32
    X = np.zeros((2, K))
    X[0, 0], X[0, 1] = 1.0 + 3 * 2.0 ** -9, -1.0     # X^ A^T = 2^-7 (exact: 3 * 2^-9)
    X[1, 0], X[1, 1] = 1.0, 2.0 ** -8                # X^ A^T = 1 + 2^-8 -> bf16 1
    G = np.zeros((2, N))
    G[0, 0], G[0, 1] = 1.0 + 3 * 2.0 ** -9, -1.0     # G^ B = 2^-7
    G[1, 0], G[1, 1] = 1.0, 2.0 ** -8                # G^ B = 1 + 2^-8 -> bf16 1
    A = np.zeros((1, K))
    A[0, 0] = A[0, 1] = 1.0
    B = np.zeros((N, 1))
    B[0, 0] = B[1, 0] = 1.0
    lin = Linear(R=np.zeros((N, K)), A=A, B=B, L1=np.zeros((0, K)), L2=np.zeros((N, 0)))
    Y, XL = layer.linear_forward(X, lin)
    e7, e8, e14 = 2.0 ** -7, 2.0 ** -8, 2.0 ** -14
    assert np.array_equal(XL, np.array([[e7], [1.0]]))
    Yw = np.zeros((2, N))
    Yw[0, :2], Yw[1, :2] = e7, 1.0
    assert np.array_equal(Y, Yw)
    dX, dA, dB, GB = layer.linear_backward(G, X, XL, lin)
    assert np.array_equal(GB, np.array([[e7], [1.0]]))
    dXw = np.zeros((2, K))
    dXw[0, :2], dXw[1, :2] = e7, 1.0
    assert np.array_equal(dX, dXw)
    dAw = np.zeros((1, K))
    dAw[0, 0], dAw[0, 1] = e7 * (1 + e7) + 1.0, -e7 + e8   # GB^T X^
    assert np.array_equal(dA, dAw)
    dBw = np.zeros((N, 1))
    dBw[0, 0], dBw[1, 0] = (1 + e7) * e7 + 1.0, -e7 + e8   # G^^T XL
    assert np.array_equal(dB, dBw)
    assert dA[0, 0] == 1.0 + e7 + e14
