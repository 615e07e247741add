"""Element-by-element parity of GPU outputs against the fp64 oracle.

Every GPU product here is a sum accumulated in fp32 (the MFMA accumulators, split
reductions added in a fixed order), every oracle product the same sum in fp64 on the
same operands. For a sum of n terms t_i accumulated in fp32 in any order,
|fl32(sum) - sum| <= gamma(n) * sum |t_i| with gamma(n) = (n + 1) 2^-24 (the standard
recursive-summation bound, rounded up). The bounds below are that term, computed from
the oracle's operands with absolute values (|A| |B|), plus the propagation of the
intermediates that both sides round to bf16 (XL, GB, P^, H^, dP^, HL2): where the
oracle's exact value lies within its bound of a bf16 rounding point the two sides may
round it to neighbouring bf16 values, one ulp apart, which then enters the next
product; elsewhere both round it to the same value. bf16 outputs are compared with the oracle rounded to bf16
(one more bf16 ulp). On top of the elementwise bound every output must also meet the
relative Frobenius bar of 1e-3.

Quantized operands: the codes of Q(X), Q(dY), Q(R) are compared bit for bit. The MLP's
Q(H) and Q(dP) quantize fp32 values that the GPU computes; those values are exported
(h_debug, dp_debug) and the oracle quantizer applied to them must reproduce the GPU's
codes bit for bit. Against the oracle's own decisions (from its own fp64 chain) a code
may differ only where the oracle's value lies within the derived bound of a rounding
threshold, a scale byte only where the block maximum lies within it of a power of two.
"""
from __future__ import annotations

import numpy as np

from oracle import layer, mx4
from tests.gpu_util import log, rel_fro

TOL = 1e-3
U32 = 2.0 ** -24
# E2M1 rounding thresholds (midpoints of the grid 0, .5, 1, 1.5, 2, 3, 4, 6)
THRESH = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
# bound on the absolute error of the GPU's fp32 GELU' (values <= 1.13; a few tens of
# fp32 ulps where its two terms cancel)
GELU_GRAD_ERR = 2.0 ** -18


def gamma(n: int) -> float:
    return (n + 1) * U32


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (2^-133 at zero and among subnormals)."""
    x = np.abs(_f64(x))
    _, e = np.frexp(x)
    return np.where(x == 0.0, 2.0 ** -133, np.ldexp(1.0, np.maximum(e, -125) - 8))


def ulp_f32(x):
    """Spacing of fp32 numbers at |x| (2^-149 at zero and among subnormals)."""
    x = np.abs(_f64(x))
    _, e = np.frexp(x)
    return np.where(x == 0.0, 2.0 ** -149, np.ldexp(1.0, np.maximum(e, -125) - 24))


def amm(a, b):
    """|a| @ |b|."""
    return np.abs(_f64(a)) @ np.abs(_f64(b))


def bf16_step(w, b):
    """Bound on |bf16(s) - bf16(w)| given |s - w| <= b. Rounding is monotone, so when
    w - b and w + b round to the same bf16 value every s between them does too and the
    two roundings agree exactly; otherwise they differ by at most b plus one bf16 ulp."""
    w, b = _f64(w), _f64(b)
    straddle = mx4.bf16_round(w - b) != mx4.bf16_round(w + b)
    return np.where(straddle, b + ulp_bf16(np.abs(w) + b), 0.0)


def check_values(name, got, want, bound, out_bf16=False):
    """got (GPU) against want (fp64, unrounded) with |got - want| <= bound (+ the
    output rounding) everywhere, and the relative Frobenius bar."""
    got, want, bound = _f64(got), _f64(want), np.broadcast_to(_f64(bound), np.shape(want))
    if out_bf16:
        wr, lim = mx4.bf16_round(want), bf16_step(want, bound)
    else:
        wr, lim = want, bound + ulp_f32(np.abs(want) + bound)
    err = np.abs(got - wr)
    fro = rel_fro(got, wr)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = float(np.max(np.where(lim > 0, err / np.where(lim > 0, lim, 1.0), 0.0))) if err.size else 0.0
    log(f"  {name}: rel Frobenius {fro:.2e}, max |err| / bound {ratio:.2e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert fro <= TOL, (name, fro)
    bad = err > lim
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} elements beyond the bound; first {i}: "
                             f"got {got[i]!r}, oracle {wr[i]!r}, bound {lim[i]!r}")
    return fro


# ------------------------------------------------------------------ quantized operands
def unpack(codes_packed):
    return mx4.unpack_codes(np.asarray(codes_packed, dtype=np.uint8))


def quant_exact(name, codes_packed, scales, T):
    """GPU codes (packed) and scales equal the oracle's Q(T) bit for bit."""
    wc, ws_ = mx4.quantize(_f64(T))
    assert np.array_equal(np.asarray(scales), ws_), f"{name}: scale bytes"
    assert np.array_equal(np.asarray(codes_packed), mx4.pack_codes(wc)), f"{name}: codes"


def _grid_index(c):
    return (c & 7).astype(np.int64) * np.where(c & 8, -1, 1)


def quant_near_threshold(name, codes_packed, scales, T, delta):
    """GPU Q(T') against the oracle's Q(T) where |T' - T| <= delta elementwise: a scale
    byte may differ only in a block whose amax lies within the block's largest delta of a
    power of two; in the other blocks a code may differ only where |T| / 2^E lies within
    delta / 2^E of a rounding threshold, and then by one grid step."""
    T, delta = _f64(T), np.broadcast_to(_f64(delta), np.shape(T))
    gc, gs = unpack(codes_packed), np.asarray(scales)
    wc, ws_ = mx4.quantize(T)
    rows, cols = T.shape
    nbr, nbc = ws_.shape
    pad = np.zeros((nbr * 32, cols))
    pad[:rows] = np.abs(T)
    dpad = np.zeros((nbr * 32, cols))
    dpad[:rows] = delta
    amax = pad.reshape(nbr, 32, nbc, 32).max(axis=(1, 3))
    dmax = dpad.reshape(nbr, 32, nbc, 32).max(axis=(1, 3))
    with np.errstate(divide="ignore"):
        p2 = np.exp2(np.round(np.log2(np.where(amax > 0, amax, 1.0))))
    near_p2 = np.abs(amax - p2) <= dmax
    sdiff = gs != ws_
    assert not np.any(sdiff & ~near_p2), f"{name}: a scale byte differs away from a power-of-two amax"
    same = np.kron(~sdiff, np.ones((32, 32), dtype=bool))[:rows, :cols]
    E = np.kron(ws_.astype(np.float64) - 127.0, np.ones((32, 32)))[:rows, :cols]
    y, dy = np.abs(T) / np.exp2(E), delta / np.exp2(E)
    near_t = np.min(np.abs(y[..., None] - THRESH), axis=-1) <= dy
    zero_both = ((gc & 7) == 0) & ((wc & 7) == 0)
    diff = same & (gc != wc) & ~zero_both
    assert not np.any(diff & ~near_t), f"{name}: a code differs away from a rounding threshold"
    assert np.all(np.abs(_grid_index(gc) - _grid_index(wc))[diff] <= 1), f"{name}: a code differs by >1 step"
    log(f"  {name}: {int(sdiff.sum())} of {sdiff.size} scale bytes and {int(diff.sum())} of {T.size} codes "
        f"differ from the oracle's own chain, each within the bound of a decision point")


# ------------------------------------------------------------------ GELU on the GPU
def gelu_bound(P):
    """Bound on |GELU_gpu(p) - GELU(p)|: the GPU forms GELU(p) = p / (1 + 2^a) with
    a = p (A0 + A1 p^2) from the hardware base-2 exponential and reciprocal, whose
    relative error grows with |a| (the argument's own rounding is amplified by
    ln 2 |a|); plus the fp64 reference's absolute error where 1 + tanh cancels."""
    P = _f64(P)
    a = np.abs(P) * (2.303 + 0.103 * P * P)
    H = layer.gelu_tanh(P)
    return (np.minimum(a, 200.0) + 8.0) * 2.0 ** -23 * np.abs(H) + np.abs(P) * 2.0 ** -50 + 2.0 ** -146


def _bf(a):
    return mx4.bf16_round(_f64(a))


# ------------------------------------------------------------------ one linear
def linear_expect(lin, X, G, got, rows=None, ncols=None, kcols=None, jsel=None, m_chunk=4096):
    """Oracle values and elementwise bounds of one linear's outputs (FourTune §3.1
    forward, §3.2 backward), each stage on the operands it consumes: XL from X; Y on
    `rows` (whole 32-row blocks) x `ncols` from Q(X), Q(R) and the GPU's saved XL
    (got['XL'], all M rows; checked itself as the first stage); dX on rows x `kcols`
    from Q(dY), Q(R) and GB = bf16(dY^ [B|L2]); dA [jsel x kcols] and dB [ncols x
    jsel] as full reductions over all M rows. None selects everything. Returns
    {name: (want, bound)}."""
    M = X.shape[0]
    N, K = lin.R.shape
    rows = np.arange(M) if rows is None else np.asarray(rows)
    ncols = np.arange(N) if ncols is None else np.asarray(ncols)
    kcols = np.arange(K) if kcols is None else np.asarray(kcols)
    D, U = lin.D(), lin.U()
    r, rt = lin.rank, D.shape[0]
    jsel = np.arange(r) if jsel is None else np.asarray(jsel)
    Rd = mx4.fake_quant(lin.R)
    XLg = _f64(got["XL"])
    out = {}
    Xr, Gr = _f64(X[rows]), _f64(G[rows])
    Xh, Gh = _bf(Xr), _bf(Gr)
    Xd, Gd = mx4.fake_quant(Xr), mx4.fake_quant(Gr)
    out["XL"] = (Xh @ D.T, gamma(K) * amm(Xh, D.T))
    Rn, Un, XLr = Rd[ncols], U[ncols], XLg[rows]
    out["Y"] = (Xd @ Rn.T + XLr @ Un.T, gamma(K + rt) * (amm(Xd, Rn.T) + amm(XLr, Un.T)))
    GBw = Gh @ U
    GB, eGB = _bf(GBw), bf16_step(GBw, gamma(N) * amm(Gh, U))
    Rk, Dk = Rd[:, kcols], D[:, kcols]
    out["dX"] = (Gd @ Rk + GB @ Dk,
                 gamma(N + rt) * (amm(Gd, Rk) + amm(GB, Dk)) + eGB @ np.abs(Dk))
    if r > 0 and len(jsel):
        dA = np.zeros((len(jsel), len(kcols)))
        bdA = np.zeros_like(dA)
        dB = np.zeros((len(ncols), len(jsel)))
        bdB = np.zeros_like(dB)
        Uj = U[:, jsel]
        for lo in range(0, M, m_chunk):
            hi = min(M, lo + m_chunk)
            Xc, Gc = _bf(X[lo:hi]), _bf(G[lo:hi])
            GBw_c = Gc @ Uj
            GBc, eGBc = _bf(GBw_c), bf16_step(GBw_c, gamma(N) * amm(Gc, Uj))
            XLc = XLg[lo:hi][:, jsel]
            Xk, Gn = Xc[:, kcols], Gc[:, ncols]
            dA += GBc.T @ Xk
            bdA += gamma(M) * amm(GBc.T, Xk) + eGBc.T @ np.abs(Xk)
            dB += Gn.T @ XLc
            bdB += gamma(M) * amm(Gn.T, XLc)
        out["dA"], out["dB"] = (dA, bdA), (dB, bdB)
    return out


# ------------------------------------------------------------------ the MLP pair
def mlp_expect(l1, l2, X, G, got, rows=None, dcols=None, fcols=None, j1=None, j2=None, m_chunk=2048):
    """Oracle values and bounds of the MLP pair (FourTune §3.3 "MLP Fusion"), each stage
    on the operands it consumes, the GPU's own where a stage consumes a GPU result:
      XL1 from X;  P^ from Q(X), Q(R1), XL1;  H = GELU(P^);  HL2 from bf16(H);
      Y from Q(H), HL2;  dP = dH GELU'(P^) with dH from Q(dY), Q(R2), GB2;
      dX from Q(dP), GB1 = bf16(bf16(dP) [B1|L2_1]);
      dA2 = GB2^T bf16(H), dB2 = dY^^T HL2, dA1 = GB1^T X^, dB1 = bf16(dP)^T XL1.
    Q(H), Q(dP) are compared bit for bit with the oracle quantizer applied to the GPU's
    H and dP, and with the oracle's own fp64 chain within the bound of a decision point.
    `got` holds the GPU's arrays: on `rows` (whole block rows) 'P', 'H', 'dP',
    'hq' / 'dpq' (packed codes, scales); on all M rows 'XL1', 'HL2', 'Hf' (H on fcols)
    and 'dPa' (dP, every column; needed only when fc1 has a LoRA branch). Gradients are
    full reductions over M: dA2 [j2 x fcols], dB1 [fcols x j1], dB2 [dcols x j2],
    dA1 [j1 x dcols]. Returns {name: (want, bound)}."""
    M, d = X.shape
    F = l1.R.shape[0]
    dout = l2.R.shape[0]
    rows = np.arange(M) if rows is None else np.asarray(rows)
    dcols = np.arange(dout) if dcols is None else np.asarray(dcols)
    fcols = np.arange(F) if fcols is None else np.asarray(fcols)
    D1, U1, D2, U2 = l1.D(), l1.U(), l2.D(), l2.U()
    r1, r2 = l1.rank, l2.rank
    rt1, rt2 = D1.shape[0], D2.shape[0]
    j1 = np.arange(r1) if j1 is None else np.asarray(j1)
    j2 = np.arange(r2) if j2 is None else np.asarray(j2)
    Rd1, Rd2 = mx4.fake_quant(l1.R), mx4.fake_quant(l2.R)
    XL1g, HL2g = _f64(got["XL1"]), _f64(got["HL2"])
    out = {}

    # ---- forward on the sampled rows
    Xr, Gr = _f64(X[rows]), _f64(G[rows])
    Xh, Xd = _bf(Xr), mx4.fake_quant(Xr)
    XL1w = Xh @ D1.T
    bXL1 = gamma(d) * amm(Xh, D1.T)
    out["XL1"] = (XL1w, bXL1)
    XL1r = XL1g[rows]
    Pw = Xd @ Rd1.T + XL1r @ U1.T
    bP = gamma(d + rt1) * (amm(Xd, Rd1.T) + amm(XL1r, U1.T))
    out["P"] = (Pw, bP)
    P_g = _f64(got["P"])
    out["H"] = (layer.gelu_tanh(P_g), gelu_bound(P_g))
    quant_exact("Q(H) from the GPU's H", *got["hq"], got["H"])
    Hh_g = _bf(got["H"])
    out["HL2"] = (Hh_g @ D2.T, gamma(F) * amm(Hh_g, D2.T))
    Hq_g = mx4.dequantize(unpack(got["hq"][0]), got["hq"][1])
    R2n, U2n, HL2r = Rd2[dcols], U2[dcols], HL2g[rows]
    out["Y"] = (Hq_g @ R2n.T + HL2r @ U2n.T, gamma(F + rt2) * (amm(Hq_g, R2n.T) + amm(HL2r, U2n.T)))
    # the oracle's own chain: its P^ within eP of the GPU's, its H within eH
    _, eXL1 = _bf(XL1w), bf16_step(XL1w, bXL1)
    P_o, eP = _bf(Pw), bf16_step(Pw, bP + eXL1 @ np.abs(U1.T))
    H_o = layer.gelu_tanh(P_o)
    dH_ = 1.13 * eP + gelu_bound(P_o)              # |GELU'| <= 1.13
    quant_near_threshold("Q(H) vs the oracle's own chain", *got["hq"], layer.fp32(H_o),
                         dH_ + ulp_f32(np.abs(H_o) + dH_))

    # ---- backward on the sampled rows
    Gh, Gd = _bf(Gr), mx4.fake_quant(Gr)
    GB2w = Gh @ U2
    GB2, eGB2 = _bf(GB2w), bf16_step(GB2w, gamma(dout) * amm(Gh, U2))
    dHw = Gd @ Rd2 + GB2 @ D2
    bdH = gamma(dout + rt2) * (amm(Gd, Rd2) + amm(GB2, D2)) + eGB2 @ np.abs(D2)
    gp_g = layer.gelu_tanh_grad(P_g)
    out["dP"] = (dHw * gp_g, np.abs(gp_g) * bdH + np.abs(dHw) * GELU_GRAD_ERR)
    quant_exact("Q(dP) from the GPU's dP", *got["dpq"], got["dP"])
    gp_o = layer.gelu_tanh_grad(P_o)
    ddP = np.abs(gp_o) * bdH + np.abs(dHw) * (GELU_GRAD_ERR + eP)   # |GELU''| <= 1
    dP_o = dHw * gp_o
    quant_near_threshold("Q(dP) vs the oracle's own chain", *got["dpq"], layer.fp32(dP_o),
                         ddP + ulp_f32(np.abs(dP_o) + ddP))
    dPh_g = _bf(got["dP"])
    GB1w = dPh_g @ U1
    GB1, eGB1 = _bf(GB1w), bf16_step(GB1w, gamma(F) * amm(dPh_g, U1))
    dPq_g = mx4.dequantize(unpack(got["dpq"][0]), got["dpq"][1])
    R1k, D1k = Rd1[:, dcols], D1[:, dcols]
    out["dX"] = (dPq_g @ R1k + GB1 @ D1k,
                 gamma(F + rt1) * (amm(dPq_g, R1k) + amm(GB1, D1k)) + eGB1 @ np.abs(D1k))

    # ---- LoRA gradients: reductions over all M rows, chunked
    acc = {}

    def add(name, v, b):
        acc[name] = (acc[name][0] + v, acc[name][1] + b) if name in acc else (v, b)

    for lo in range(0, M, m_chunk):
        hi = min(M, lo + m_chunk)
        Xh_c, Gh_c = _bf(X[lo:hi]), _bf(G[lo:hi])
        if r2 > 0:
            Uj = U2[:, j2]
            GB2w_c = Gh_c @ Uj
            GB2_c, eGB2_c = _bf(GB2w_c), bf16_step(GB2w_c, gamma(dout) * amm(Gh_c, Uj))
            Hh_c = _bf(got["Hf"][lo:hi])
            add("dA2", GB2_c.T @ Hh_c, gamma(M) * amm(GB2_c.T, Hh_c) + eGB2_c.T @ np.abs(Hh_c))
            Gn, HL2_c = Gh_c[:, dcols], HL2g[lo:hi][:, j2]
            add("dB2", Gn.T @ HL2_c, gamma(M) * amm(Gn.T, HL2_c))
        if r1 > 0:
            dPh_c = _bf(got["dPa"][lo:hi])
            B = XL1g[lo:hi][:, j1]
            dPf = dPh_c[:, fcols]
            add("dB1", dPf.T @ B, gamma(M) * amm(dPf.T, B))
            Uj = U1[:, j1]
            GB1w_c = dPh_c @ Uj
            GB1_c, eGB1_c = _bf(GB1w_c), bf16_step(GB1w_c, gamma(F) * amm(dPh_c, Uj))
            Xk = Xh_c[:, dcols]
            add("dA1", GB1_c.T @ Xk, gamma(M) * amm(GB1_c.T, Xk) + eGB1_c.T @ np.abs(Xk))
    out.update(acc)
    return out
