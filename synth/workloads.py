"""Seeded synthetic DiT-shaped inputs for the W4A4G4 linear and MLP.

This module only draws data: activations, weights, adapters, incoming gradients, and
the frozen stabilizer/residual split of each weight. It holds none of the hot path's
arithmetic (no quantizer, no GEMM, no rounding rule of the method) and imports
nothing from either the GPU package or the oracle; both sides receive the arrays it
returns.

Workloads (shapes of FLUX.1-dev-like and video-DiT-like layers; the pages name a
3072x12288 MLP intermediate, FourTune §3.3 "MLP Fusion", and LoRA rank 64, §4.1):

  c1  tiny single linear: X fp32 [256 x 512], W [512 x 512], 4 outlier input
      channels x50, r = s = 16, dY fp32 ~N(0, 1e-3)
  c2  attention projection: X bf16 [4608 x 3072], W [3072 x 3072], 1% of input
      channels (31) x30, r = s = 32, dY bf16 ~N(0, 1e-3)
  c3  MLP 3072 -> 12288 -> 3072 on the c2-shaped X, r = s = 32 on both linears
  c4  the four linears of a DiT block at batch 2 (M = 9216): QKV [9216 x 3072],
      out-proj [3072 x 3072] on an attention output O ~N(0, 1), MLP 3072 -> 12288 ->
      3072; X ~ Student-t(3); r = 64, s = 32
  c5  video-DiT large M: X bf16 [32760 x 5120], 0.5% of channels (26) x50, QKV
      [15360 x 5120] and MLP 5120 -> 13824 -> 5120, r = s = 64, dY ~N(0, 1e-4)

Distributions: N(mu, sd) names the standard deviation. W ~ N(0, 0.02), A, B ~
N(0, 0.01), all stored as bf16. Outlier channels are drawn without replacement and
scaled after drawing, the same channels for every token.

Stabilizer split (frozen, computed once): the top-s singular triplets of W give
L1 = sqrt(S) V^T [s x K] and L2 = U sqrt(S) [N x s], both cast to bf16, and the
residual R = W - L2 L1 (fp64, stored fp32) is what the 4-bit backbone quantizes
[FourTune §3.1; the low-rank outlier absorption is the SVDQuant idea it cites]. The
exact SVD is used when W has at most 3072 x 3072 entries; larger weights use seeded
randomized subspace iteration (6 power iterations, oversampling 32), which yields a
rank-s factor pair close to the truncated SVD. The hot path consumes (R, L1, L2) as
given, so this choice only shapes the data.

Every tensor has its own PCG64 stream, seeded from (seed, layer index, tensor index),
so any one tensor can be regenerated alone. Arrays come back as float32 numpy arrays
whose values are exactly representable in the stated dtype (bf16 values are rounded
to nearest-even on creation).
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 0

# tensor indices inside a layer's stream family
_T_X, _T_O, _T_W, _T_A, _T_B, _T_DY, _T_SVD = 0, 1, 2, 3, 4, 5, 6


def _rng(seed, layer, tensor):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tensor])))


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage dtype ('fp32' or 'bf16'), returned as float32 values."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16).to(torch.float32)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return t.numpy()


@dataclass
class LinearSpec:
    name: str
    n: int            # out features
    k: int            # in features
    r: int            # LoRA rank
    s: int            # stabilizer rank
    inp: str = "x"    # which activation feeds it


@dataclass
class MlpSpec:
    name: str
    d: int            # model width
    f: int            # intermediate width
    r: int
    s: int
    inp: str = "x"


@dataclass
class Workload:
    key: str
    title: str
    m: int
    k: int
    x_dtype: str
    dy_dtype: str
    x_dist: str                    # 'normal' or 't3'
    outliers: tuple                # (count, factor)
    dy_std: float
    layers: list = field(default_factory=list)
    seed: int = SEED


WORKLOADS = {
    "c1": Workload("c1", "tiny single linear", 256, 512, "fp32", "fp32", "normal", (4, 50.0),
                   1e-3, [LinearSpec("lin", 512, 512, 16, 16)]),
    "c2": Workload("c2", "FLUX attention projection", 4608, 3072, "bf16", "bf16", "normal",
                   (31, 30.0), 1e-3, [LinearSpec("proj", 3072, 3072, 32, 32)]),
    "c3": Workload("c3", "FLUX MLP", 4608, 3072, "bf16", "bf16", "normal", (31, 30.0), 1e-3,
                   [MlpSpec("mlp", 3072, 12288, 32, 32)]),
    "c4": Workload("c4", "DiT block linears, batch 2", 9216, 3072, "bf16", "bf16", "t3", (0, 1.0),
                   1e-3, [LinearSpec("qkv", 9216, 3072, 64, 32),
                          LinearSpec("o", 3072, 3072, 64, 32, inp="o"),
                          MlpSpec("mlp", 3072, 12288, 64, 32)]),
    "c5": Workload("c5", "video-DiT large M", 32760, 5120, "bf16", "bf16", "normal", (26, 50.0),
                   1e-4, [LinearSpec("qkv", 15360, 5120, 64, 64),
                          MlpSpec("mlp", 5120, 13824, 64, 64)]),
}


# ----------------------------------------------------------------------------- draws
def draw_activation(wl: Workload, which: str = "x", m: int | None = None) -> np.ndarray:
    m = wl.m if m is None else m
    if which == "o":   # stand-in for the attention output feeding the out-projection
        x = _rng(wl.seed, 0, _T_O).standard_normal((m, wl.k), dtype=np.float32)
        return to_dtype(x, wl.x_dtype)
    g = _rng(wl.seed, 0, _T_X)
    if wl.x_dist == "t3":
        x = g.standard_t(3, (m, wl.k)).astype(np.float32)
    else:
        x = g.standard_normal((m, wl.k), dtype=np.float32)
    cnt, fac = wl.outliers
    if cnt:
        idx = g.choice(wl.k, cnt, replace=False)
        x[:, idx] *= np.float32(fac)
    return to_dtype(x, wl.x_dtype)


def _top_svd(W: np.ndarray, s: int, g: np.random.Generator):
    if s == 0:
        return np.zeros((W.shape[0], 0)), np.zeros(0), np.zeros((0, W.shape[1]))
    if W.size <= 3072 * 3072:
        U, S, Vt = np.linalg.svd(W, full_matrices=False)
        return U[:, :s], S[:s], Vt[:s]
    p = 32
    Y = W @ g.standard_normal((W.shape[1], s + p))
    Q, _ = np.linalg.qr(Y)
    for _ in range(6):
        Q, _ = np.linalg.qr(W.T @ Q)
        Q, _ = np.linalg.qr(W @ Q)
    Ub, S, Vt = np.linalg.svd(Q.T @ W, full_matrices=False)
    return (Q @ Ub)[:, :s], S[:s], Vt[:s]


def draw_linear(wl: Workload, layer_idx: int, n: int, k: int, r: int, s: int,
                m: int | None = None, dy: bool = True) -> dict:
    """W, its stabilizer split (R, L1, L2), the adapter (A, B) and the incoming dY."""
    m = wl.m if m is None else m
    L = layer_idx + 1
    W64 = to_dtype(_rng(wl.seed, L, _T_W).standard_normal((n, k), dtype=np.float32) * 0.02,
                   "bf16").astype(np.float64)
    A = to_dtype(_rng(wl.seed, L, _T_A).standard_normal((r, k), dtype=np.float32) * 0.01, "bf16")
    B = to_dtype(_rng(wl.seed, L, _T_B).standard_normal((n, r), dtype=np.float32) * 0.01, "bf16")
    U, S, Vt = _top_svd(W64, s, _rng(wl.seed, L, _T_SVD))
    rs = np.sqrt(S)
    L1 = to_dtype((rs[:, None] * Vt).astype(np.float32), "bf16")
    L2 = to_dtype((U * rs[None, :]).astype(np.float32), "bf16")
    R = (W64 - L2.astype(np.float64) @ L1.astype(np.float64)).astype(np.float32)
    out = dict(W=W64.astype(np.float32), R=R, A=A, B=B, L1=L1, L2=L2, n=n, k=k, r=r, s=s)
    if dy:
        out["dY"] = to_dtype(_rng(wl.seed, L, _T_DY).standard_normal((m, n), dtype=np.float32)
                             * np.float32(wl.dy_std), wl.dy_dtype)
    return out


def linear_case(key: str, layer: str | None = None, m: int | None = None) -> dict:
    """Inputs of one linear of a workload: X (or O), R, L1, L2, A, B, dY."""
    wl = WORKLOADS[key]
    for i, spec in enumerate(wl.layers):
        if isinstance(spec, LinearSpec) and (layer is None or spec.name == layer):
            d = draw_linear(wl, i, spec.n, spec.k, spec.r, spec.s, m=m)
            d["X"] = draw_activation(wl, spec.inp, m=m)
            d["x_dtype"], d["dy_dtype"] = wl.x_dtype, wl.dy_dtype
            return d
    raise KeyError((key, layer))


def mlp_case(key: str, layer: str | None = None, m: int | None = None) -> dict:
    """Inputs of one MLP of a workload: X, fc1 and fc2 parameter sets, dY."""
    wl = WORKLOADS[key]
    for i, spec in enumerate(wl.layers):
        if isinstance(spec, MlpSpec) and (layer is None or spec.name == layer):
            fc1 = draw_linear(wl, 10 * (i + 1), spec.f, spec.d, spec.r, spec.s, m=m, dy=False)
            fc2 = draw_linear(wl, 10 * (i + 1) + 1, spec.d, spec.f, spec.r, spec.s, m=m)
            dY = fc2.pop("dY")
            return dict(X=draw_activation(wl, spec.inp, m=m), fc1=fc1, fc2=fc2, dY=dY,
                        x_dtype=wl.x_dtype, dy_dtype=wl.dy_dtype)
    raise KeyError((key, layer))


def random_linear(m: int, n: int, k: int, r: int, s: int, seed: int = 1,
                  x_dtype: str = "bf16", dy_dtype: str = "bf16", outliers=(2, 30.0),
                  dy_std: float = 1e-3) -> dict:
    """A small case of arbitrary shape (ragged M, several tiles) for parity tests."""
    wl = Workload("adhoc", "adhoc", m, k, x_dtype, dy_dtype, "normal", outliers, dy_std,
                  [LinearSpec("lin", n, k, r, s)], seed=seed)
    d = draw_linear(wl, 0, n, k, r, s)
    d["X"] = draw_activation(wl, "x")
    d["x_dtype"], d["dy_dtype"] = x_dtype, dy_dtype
    return d


def random_mlp(m: int, d: int, f: int, r: int, s: int, seed: int = 2,
               x_dtype: str = "bf16", dy_dtype: str = "bf16", dy_std: float = 1e-3) -> dict:
    wl = Workload("adhoc", "adhoc", m, d, x_dtype, dy_dtype, "normal", (2, 30.0), dy_std,
                  [MlpSpec("mlp", d, f, r, s)], seed=seed)
    fc1 = draw_linear(wl, 10, f, d, r, s, dy=False)
    fc2 = draw_linear(wl, 11, d, f, r, s)
    dY = fc2.pop("dY")
    return dict(X=draw_activation(wl, "x"), fc1=fc1, fc2=fc2, dY=dY, x_dtype=x_dtype,
                dy_dtype=dy_dtype)
