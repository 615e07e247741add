"""Pins of the oracle's unfused forms (oracle/layer.py, FourTune §4 "Kernel Fusion
Breakdown"), which the fusion ablation's GPU path is compared against.

- closed forms: with quantization and bf16 rounding off, the unfused linear equals one
  linear with the merged weight R + L2 L1 + B A, and its backward is that linear's
  gradient (dX = G W, dA = (G B)^T X, dB = G^T (X A^T)); the unfused MLP equals
  GELU(X W1^T) W2^T, and its backward matches finite differences of <Y, dY>;
- brute force: with quantization and rounding on, the unfused forward minus its
  low-rank term is the exact 4-bit product (a Fraction triple loop) rounded to the
  nearest bf16, i.e. the one extra rounding sits on the backbone product alone;
- the MLP's stored H is bf16 GELU(P), and the fused and unfused forms agree to within
  those roundings.
"""
from fractions import Fraction

import numpy as np

from oracle import layer, mx4
from oracle.layer import Linear, Prec
from tests.test_oracle_layer import _fd, _frac_deq, _lin

OFF = Prec(quant=False, bf16=False)


def _merged(lin):
    return lin.R + lin.L2 @ lin.L1 + lin.B @ lin.A


def test_unfused_linear_closed_form():
    rng = np.random.default_rng(30)
    M, N, K, r, s = 24, 40, 64, 8, 8
    lin = _lin(rng, N, K, r, s)
    X, G = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    Y, XL = layer.linear_forward_unfused(X, lin, OFF)
    W = _merged(lin)
    np.testing.assert_allclose(Y, X @ W.T, rtol=1e-12, atol=1e-12)
    dX, dA, dB, GB = layer.linear_backward_unfused(G, X, XL, lin, OFF)
    np.testing.assert_allclose(dX, G @ W, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dA, (G @ lin.B).T @ X, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dB, G.T @ (X @ lin.A.T), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(GB[:, r:], G @ lin.L2, rtol=1e-12, atol=1e-13)


def _bf16_nearest(q: Fraction) -> float:
    """Nearest bf16 to an exact rational, ties to even, by search over the candidates
    around float(q) (independent of the oracle's bf16 rounder)."""
    f = float(q)
    if f == 0.0:
        return 0.0
    bits = np.float32(f).view(np.uint32)
    lo = np.uint32(bits & 0xFFFF0000)
    cands = [lo, np.uint32(lo + 0x10000)]
    if lo >= 0x10000 and (lo & 0x7FFFFFFF) != 0:
        cands.append(np.uint32(lo - 0x10000))
    best = None
    for c in cands:
        v = float(np.array([c], dtype=np.uint32).view(np.float32)[0])
        d = abs(Fraction(v) - q)
        key = (d, int((c >> 16) & 1))  # ties: the even bf16 (low mantissa bit 0)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_unfused_rounding_sits_on_the_backbone_product():
    rng = np.random.default_rng(31)
    M, N, K, r, s = 32, 32, 1024, 16, 16
    lin = _lin(rng, N, K, r, s)
    # a long reduction over blocks of different magnitudes: the exact 4-bit product then
    # needs more significant bits than bf16 holds (E2M1 products carry few bits, so a
    # short reduction is often exact in bf16 and would not show the rounding)
    X = rng.standard_normal((M, K)) * np.ldexp(1.0, rng.integers(-3, 3, (1, K // 32))).repeat(32, axis=1)
    Y, XL = layer.linear_forward_unfused(X, lin)
    Y0 = Y - XL @ lin.U().T
    cx, sx = mx4.quantize(X)
    cr, sr = mx4.quantize(lin.R)
    fx, fr = _frac_deq(cx, sx), _frac_deq(cr, sr)
    # the low-rank term is added in fp64 after the rounding, so Y0 is recovered to
    # within fp64 rounding of that addition
    worst = 0.0
    for i in range(0, M, 3):
        for j in range(0, N, 5):
            exact = sum(fx[i][k] * fr[j][k] for k in range(K))
            want = _bf16_nearest(exact)
            worst = max(worst, abs(Y0[i, j] - want) / max(abs(want), 1e-30))
    assert worst < 1e-12
    # and the fused form does not round there
    Yf, _ = layer.linear_forward(X, lin)
    assert np.mean(Yf != Y) > 0.5


def test_unfused_mlp_closed_form_and_gradients():
    rng = np.random.default_rng(32)
    M, D, F, r, s = 5, 8, 12, 2, 2
    fc1, fc2 = _lin(rng, F, D, r, s, scale=0.4), _lin(rng, D, F, r, s, scale=0.4)
    X, dY = rng.standard_normal((M, D)), rng.standard_normal((M, D))
    for fused in (False, True):
        fwd = layer.mlp_forward_unfused(X, fc1, fc2, OFF, lora_fused=fused)
        P = X @ _merged(fc1).T
        np.testing.assert_allclose(fwd["Y"], layer.gelu_tanh(P) @ _merged(fc2).T, rtol=1e-12, atol=1e-12)
        bwd = layer.mlp_backward_unfused(dY, X, fwd, fc1, fc2, OFF, lora_fused=fused)

        def loss():
            f = layer.mlp_forward_unfused(X, fc1, fc2, OFF, lora_fused=fused)
            return float(np.sum(f["Y"] * dY))

        np.testing.assert_allclose(bwd["dX"], _fd(loss, X, 1e-6), rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose(bwd["dA1"], _fd(loss, fc1.A, 1e-6), rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose(bwd["dB2"], _fd(loss, fc2.B, 1e-6), rtol=1e-6, atol=1e-8)


def test_unfused_mlp_stores_bf16_h_and_tracks_fused():
    rng = np.random.default_rng(33)
    M, D, F, r, s = 64, 64, 128, 16, 16
    fc1, fc2 = _lin(rng, F, D, r, s, scale=0.1), _lin(rng, D, F, r, s, scale=0.1)
    X, dY = rng.standard_normal((M, D)), rng.standard_normal((M, D)) * 1e-3
    f = layer.mlp_forward_unfused(X, fc1, fc2)
    assert np.array_equal(f["H"], mx4.bf16_round(f["H"]))
    assert np.array_equal(f["H"], mx4.bf16_round(layer.gelu_tanh(f["P"])))
    ref = layer.mlp_forward(X, fc1, fc2)
    rel = np.linalg.norm(f["Y"] - ref["Y"]) / np.linalg.norm(ref["Y"])
    assert 0 < rel < 5e-2
    b = layer.mlp_backward_unfused(dY, X, f, fc1, fc2)
    assert np.array_equal(b["dP"], mx4.bf16_round(b["dP"]))
    rb = layer.mlp_backward(dY, X, ref, fc1, fc2)
    rel = np.linalg.norm(b["dX"] - rb["dX"]) / np.linalg.norm(rb["dX"])
    assert 0 < rel < 5e-2


def test_unfused_without_low_rank_branches_is_the_plain_quantized_gemm():
    rng = np.random.default_rng(34)
    M, N, K = 48, 64, 96
    lin = Linear(R=rng.standard_normal((N, K)) * 0.02, A=np.zeros((0, K)), B=np.zeros((N, 0)),
                 L1=np.zeros((0, K)), L2=np.zeros((N, 0)))
    X, G = rng.standard_normal((M, K)), rng.standard_normal((M, N))
    Y, XL = layer.linear_forward_unfused(X, lin)
    assert np.array_equal(Y, mx4.fake_quant(X) @ mx4.fake_quant(lin.R).T)
    dX, _, _, _ = layer.linear_backward_unfused(G, X, XL, lin)
    assert np.array_equal(dX, mx4.fake_quant(G) @ mx4.fake_quant(lin.R))
