"""fp64 reference of the triple-branch W4A4G4 linear and the GELU MLP pair.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation (nn.Linear convention, Y = X W^T):
  X [M x K] input, W [N x K] frozen weight, G = dL/dY [M x N].
  Stabilizer (frozen, low rank s): L1 [s x K] (down), L2 [N x s] (up).
  LoRA adapter (trainable, rank r): A [r x K] (down), B [N x r] (up).
  Residual R = W - L2 L1, quantized once and frozen.
  D = [A; L1] [rt x K], U = [B | L2] [N x rt], rt = r + s.

What is computed and why:
* Forward [FourTune, §3.1 "Triple-Branch Hybrid-Precision Pipeline"; §3.3 "LoRA
  Fusion"]: a 4-bit backbone on the residual plus a full-precision low-rank
  stabilizer plus the trainable LoRA branch. The section's equations are missing from
  the pages; the reading taken is Y = Q(X) Q(R)^T + X L1^T L2^T + X A^T B^T, the
  low-rank branches reading the unquantized input (all three branches share the same
  input in the quantization/down-projection phase, §3.3).
* Backward [FourTune, §3.2]: gradient propagation through all three branches,
  parameter updates for the adapter only. The backbone term of dX is the 4-bit
  product of Q(G) with Q(R) (same codes and scales as the forward). The quantizer is
  passed straight through (identity in the backward).
* MLP [FourTune, §3.3 "MLP Fusion"]: FC1 -> GELU (tanh form) -> FC2, FC2's 4-bit
  operand being Q(GELU(FC1 output)).

Precision contract (the points where the GPU rounds to bf16 because its low-rank
products run on bf16 matrix units; the pages call bf16 LoRA "full precision"):
  Xh = bf16(X), XL = bf16(Xh D^T), Gh = bf16(G), GB = bf16(Gh U), Ph = bf16(pre),
  Hh = bf16(GELU(Ph)), dPh = bf16(dP). All products here are fp64.
Decision precision of the fused epilogues (reading 10 of the design notes): the MLP's
Q(H) and Q(dP) quantize values the GPU forms in fp32 inside a GEMM epilogue, so the
code decisions here are taken on those values rounded to fp32 (H32 = fp32(GELU(Ph)),
dP32 = fp32(dP)). This matters at ties: Ph is bf16, so GELU(Ph) = Ph in fp32 for
Ph > ~5.3, and bf16 values such as 7 = 3.5 * 2 sit exactly on an E2M1 threshold,
which fp64's GELU(7) = 7 - 3e-15 misses.
``Prec(quant=False)`` replaces Q by the identity and ``Prec(bf16=False)`` removes the
bf16 roundings; with both off the layer is exactly linear, which the tests use for
finite-difference checks.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import mx4

SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)
GELU_C = 0.044715


@dataclass(frozen=True)
class Prec:
    quant: bool = True
    bf16: bool = True


EXACT = Prec()


def _b(x, prec: Prec):
    return mx4.bf16_round(x) if prec.bf16 else np.asarray(x, dtype=np.float64)


def _q(T, prec: Prec):
    return mx4.fake_quant(T) if prec.quant else np.asarray(T, dtype=np.float64)


@dataclass
class Linear:
    """Frozen residual R (fp32 values), frozen stabilizer L1/L2, LoRA A/B (bf16 values)."""
    R: np.ndarray
    A: np.ndarray
    B: np.ndarray
    L1: np.ndarray
    L2: np.ndarray

    @property
    def rank(self):
        return self.A.shape[0]

    def D(self):
        return np.vstack([self.A, self.L1]).astype(np.float64)

    def U(self):
        return np.hstack([self.B, self.L2]).astype(np.float64)


# ----------------------------------------------------------------------------------
# Linear layer
# ----------------------------------------------------------------------------------
def linear_forward(X, lin: Linear, prec: Prec = EXACT, Xq=None, Rq=None):
    """Returns (Y, XL). Y = deq Q(X) deq Q(R)^T + XL U^T, XL = bf16(bf16(X) D^T).

    ``Xq``/``Rq`` optionally supply already-dequantized 4-bit operands (for checks that
    feed the GPU's own codes in, "identical quantized operands").
    """
    X = np.asarray(X, dtype=np.float64)
    Xd = _q(X, prec) if Xq is None else Xq
    Rd = _q(lin.R, prec) if Rq is None else Rq
    XL = _b(_b(X, prec) @ lin.D().T, prec)
    Y = Xd @ Rd.T + XL @ lin.U().T
    return Y, XL


def linear_backward(G, X, XL, lin: Linear, prec: Prec = EXACT, Gq=None, Rq=None):
    """Returns (dX, dA, dB, GB).

    GB = bf16(bf16(G) U); dX = deq Q(G) deq Q(R) + GB D;
    dA = GB[:, :r]^T bf16(X); dB = bf16(G)^T XL[:, :r]. No gradient for R, L1, L2.
    """
    G = np.asarray(G, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    r = lin.rank
    Gh = _b(G, prec)
    Gd = _q(G, prec) if Gq is None else Gq
    Rd = _q(lin.R, prec) if Rq is None else Rq
    GB = _b(Gh @ lin.U(), prec)
    dX = Gd @ Rd + GB @ lin.D()
    dA = GB[:, :r].T @ _b(X, prec)
    dB = Gh.T @ XL[:, :r]
    return dX, dA, dB, GB


# ----------------------------------------------------------------------------------
# GELU (tanh form) and the MLP pair
# ----------------------------------------------------------------------------------
def gelu_tanh(p):
    p = np.asarray(p, dtype=np.float64)
    return 0.5 * p * (1.0 + np.tanh(SQRT_2_OVER_PI * (p + GELU_C * p ** 3)))


def gelu_tanh_grad(p):
    p = np.asarray(p, dtype=np.float64)
    u = SQRT_2_OVER_PI * (p + GELU_C * p ** 3)
    t = np.tanh(u)
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_C * p ** 2)
    return 0.5 * (1.0 + t) + 0.5 * p * (1.0 - t * t) * du


def fp32(x):
    """Round to fp32 (returned as fp64 values)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def mlp_forward(X, fc1: Linear, fc2: Linear, prec: Prec = EXACT, Hq=None):
    """Returns dict(Y, XL1, P, H, H32, HL2).

    pre = FC1(X); P = bf16(pre) (the saved tensor); H = GELU(P); Y = FC2(H), FC2's
    4-bit operand being Q(H32), H32 = fp32(H) (the epilogue's decision precision), and
    its low-rank input bf16(H). ``Hq`` optionally gives deq Q(H) computed from the
    GPU's own H.
    """
    pre, XL1 = linear_forward(X, fc1, prec)
    P = _b(pre, prec)
    H = gelu_tanh(P)
    H32 = fp32(H)
    if Hq is None and prec.quant:
        Hq = mx4.fake_quant(H32)
    Y, HL2 = linear_forward(H, fc2, prec, Xq=Hq)
    return dict(Y=Y, XL1=XL1, P=P, H=H, H32=H32, HL2=HL2)


def mlp_backward(dY, X, saved: dict, fc1: Linear, fc2: Linear, prec: Prec = EXACT,
                 dPq=None, H=None):
    """Returns dict(dX, dA1, dB1, dA2, dB2, dH, dP, dP32).

    FC2 backward with G = dY and input H; dP = dH * GELU'(P); FC1 backward with G = dP,
    its 4-bit operand Q(dP32), dP32 = fp32(dP).
    ``dPq`` optionally gives deq Q(dP) computed from the GPU's own dP; ``H`` optionally
    overrides the recomputed GELU(P).
    """
    P = saved["P"]
    Hv = gelu_tanh(P) if H is None else H
    dH, dA2, dB2, _ = linear_backward(dY, Hv, saved["HL2"], fc2, prec)
    dP = dH * gelu_tanh_grad(P)
    dP32 = fp32(dP)
    if dPq is None and prec.quant:
        dPq = mx4.fake_quant(dP32)
    dX, dA1, dB1, _ = linear_backward(dP, X, saved["XL1"], fc1, prec, Gq=dPq)
    return dict(dX=dX, dA1=dA1, dB1=dB1, dA2=dA2, dB2=dB2, dH=dH, dP=dP, dP32=dP32)



# ----------------------------------------------------------------------------------
# Unfused forms (FourTune §4 "Kernel Fusion Breakdown": the fusions taken apart)
# ----------------------------------------------------------------------------------
# Reading: without fusion every step is its own pass and its result is stored in HBM
# in bf16 before the next step reads it. Compared with the fused forms above, this
# adds exactly these roundings: the 4-bit product before the up-projection is added
# (Y0, dX0; a layer without low-rank branches has no up-projection, its 4-bit product
# is the output itself and is not rounded in between), the MLP's GELU output H, and
# FC2's input gradient dH.
def linear_forward_unfused(X, lin: Linear, prec: Prec = EXACT):
    """Returns (Y, XL). Y = bf16(deq Q(X) deq Q(R)^T) + XL U^T, XL = bf16(bf16(X) D^T)."""
    X = np.asarray(X, dtype=np.float64)
    XL = _b(_b(X, prec) @ lin.D().T, prec)
    Y0 = _q(X, prec) @ _q(lin.R, prec).T
    if XL.shape[1] == 0:
        return Y0, XL
    return _b(Y0, prec) + XL @ lin.U().T, XL


def linear_backward_unfused(G, X, XL, lin: Linear, prec: Prec = EXACT):
    """Returns (dX, dA, dB, GB). dX = bf16(deq Q(G) deq Q(R)) + GB D; GB, dA, dB as in
    the fused form (the LoRA gradients are separate kernels in both)."""
    G = np.asarray(G, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    r = lin.rank
    Gh = _b(G, prec)
    GB = _b(Gh @ lin.U(), prec)
    dX0 = _q(G, prec) @ _q(lin.R, prec)
    dX = dX0 if GB.shape[1] == 0 else _b(dX0, prec) + GB @ lin.D()
    dA = GB[:, :r].T @ _b(X, prec)
    dB = Gh.T @ XL[:, :r]
    return dX, dA, dB, GB


def mlp_forward_unfused(X, fc1: Linear, fc2: Linear, prec: Prec = EXACT, lora_fused=False):
    """Returns dict(Y, XL1, P, H, HL2). P = bf16(FC1(X)); H = bf16(GELU(P)) is stored and
    is FC2's input (its 4-bit operand Q(H) and its down-projection both read it).
    ``lora_fused`` builds the MLP from the fused linears, otherwise from the unfused."""
    fwd = linear_forward if lora_fused else linear_forward_unfused
    pre, XL1 = fwd(X, fc1, prec)
    P = _b(pre, prec)
    H = _b(gelu_tanh(P), prec)
    Y, HL2 = fwd(H, fc2, prec)
    return dict(Y=Y, XL1=XL1, P=P, H=H, HL2=HL2)


def mlp_backward_unfused(dY, X, saved: dict, fc1: Linear, fc2: Linear, prec: Prec = EXACT,
                         lora_fused=False):
    """Returns dict(dX, dA1, dB1, dA2, dB2, dH, dP). dH = bf16(FC2 backward with input H);
    dP = bf16(dH GELU'(P)); FC1 backward with G = dP."""
    bwd = linear_backward if lora_fused else linear_backward_unfused
    dH, dA2, dB2, _ = bwd(dY, saved["H"], saved["HL2"], fc2, prec)
    dH = _b(dH, prec)
    dP = _b(dH * gelu_tanh_grad(saved["P"]), prec)
    dX, dA1, dB1, _ = bwd(dP, X, saved["XL1"], fc1, prec)
    return dict(dX=dX, dA1=dA1, dB1=dB1, dA2=dA2, dB2=dB2, dH=dH, dP=dP)


# ----------------------------------------------------------------------------------
# Precision configurations (FourTune §4 "Impact of Precision Configurations")
# ----------------------------------------------------------------------------------
# W4A16 keeps the activation in 16 bits in the forward's backbone product, G16 the
# gradient in the backward's; the weight is Q(R) throughout. The 16-bit type is bf16,
# the pipeline's activation type (the pages name only the bit widths).
def linear_forward_prec(X, lin: Linear, a16: bool, prec: Prec = EXACT):
    """Returns (Y, XL): Y = A deq Q(R)^T + XL U^T with A = bf16(X) (a16) or deq Q(X)."""
    X = np.asarray(X, dtype=np.float64)
    return linear_forward(X, lin, prec, Xq=_b(X, prec) if a16 else None)


def linear_backward_prec(G, X, XL, lin: Linear, g16: bool, prec: Prec = EXACT):
    """Returns (dX, dA, dB, GB): dX = Gv deq Q(R) + GB D with Gv = bf16(G) (g16) or
    deq Q(G); dA, dB, GB as in the W4A4G4 backward."""
    G = np.asarray(G, dtype=np.float64)
    return linear_backward(G, X, XL, lin, prec, Gq=_b(G, prec) if g16 else None)
