"""GPU parity of the precision configurations (fourtune_linear_fwd_prec / _bwd_prec,
FourTune §4 "Impact of Precision Configurations") against the oracle's
linear_forward_prec / linear_backward_prec: Y, XL, dX, dA, dB within a relative
Frobenius error of 1e-3 (bf16 outputs against the oracle rounded to bf16), over every
configuration, ragged rows, a reduction length that is an odd multiple of 32, every
low-rank configuration, fp32 inputs, and c2 at full size on sampled rows."""
import zlib

import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from synth import workloads as wl
from tests.gpu_util import dev, host, log, rel_fro
from tests.sampling import _bf, _block_rows, _chunked, _col_blocks, _errs_ok, _f64, _gpu_lin, _lin64, _rows

pytestmark = pytest.mark.gpu
TOL = 1e-3
PRECS = ["W4A4G4", "W4A16G4", "W4A4G16", "W4A16G16"]

CASES = [
    # m, n, k, r, s, x_dtype, out_dtype
    (256, 512, 512, 16, 16, "fp32", torch.float32),
    (200, 352, 480, 32, 0, "bf16", torch.float32),    # ragged M, no stabilizer
    (96, 256, 320, 0, 32, "bf16", torch.bfloat16),    # no LoRA, K % 64 = 0
    (64, 128, 160, 0, 0, "bf16", torch.float32),      # backbone alone, K % 64 = 32
    (130, 384, 288, 32, 32, "bf16", torch.bfloat16),  # N % 128 != 0, K % 64 = 32
    (300, 640, 384, 64, 64, "bf16", torch.float32),   # widest low-rank part
    (160, 384, 352, 32, 16, "bf16", torch.float32),   # rank + stab_rank = 48 (16 mod 32)
]


def _run(d, prec, odt):
    m, n, k = d["X"].shape[0], d["R"].shape[0], d["R"].shape[1]
    r, s = d["A"].shape[0], d["L1"].shape[0]
    L = _gpu_lin(d)
    x, dy = dev(d["X"], d["x_dtype"]), dev(d["dY"], d["dy_dtype"])
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))
    y = torch.empty((m, n), dtype=odt, device="cuda")
    xl = torch.empty((m, r + s), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((m, k), dtype=odt, device="cuda")
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((n, r), dtype=torch.float32, device="cuda")
    abi.fourtune_linear_fwd_prec(L, prec, x, y, xl, ws)
    abi.fourtune_linear_bwd_prec(L, prec, dy, x, xl, dx, da, db, ws)
    torch.cuda.synchronize()
    return dict(Y=host(y), XL=host(xl), dX=host(dx), dA=host(da), dB=host(db))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("m,n,k,r,s,xdt,odt", CASES)
def test_prec_small(m, n, k, r, s, xdt, odt, prec):
    log(f"prec {prec} m={m} n={n} k={k} r={r} s={s} x={xdt} out={odt}")
    d = wl.random_linear(m, n, k, r, s, seed=m + 2 * n + k, x_dtype=xdt, dy_dtype=xdt)
    got = _run(d, prec, odt)
    lin = _lin64(d)
    X, G = _f64(d["X"]), _f64(d["dY"])
    Y, XL = layer.linear_forward_prec(X, lin, a16="A16" in prec)
    dX, dA, dB, _ = layer.linear_backward_prec(G, X, XL, lin, g16="G16" in prec)
    rnd = _bf if odt == torch.bfloat16 else (lambda a: a)
    errs = dict(Y=rel_fro(got["Y"], rnd(Y)), dX=rel_fro(got["dX"], rnd(dX)))
    if r + s:
        errs["XL"] = rel_fro(got["XL"], XL)
    if r:
        errs["dA"] = rel_fro(got["dA"], dA)
        errs["dB"] = rel_fro(got["dB"], dB)
    log(f"  rel errors {errs}")
    for key, e in errs.items():
        assert e <= TOL, (key, e)


def test_prec_weight_scales_far_from_one():
    """Weight blocks with scale bytes far below and above 127 (values ~2^-60 and 2^40):
    the weight's dequantization to bf16 applies the block scale exactly."""
    rng = np.random.default_rng(7)
    d = wl.random_linear(128, 256, 256, 16, 16, seed=77)
    R = d["R"].astype(np.float64)
    R[:128] *= 2.0 ** -60
    R[128:] *= 2.0 ** 40
    d["R"] = R.astype(np.float32)
    got = _run(d, "W4A16G16", torch.float32)
    lin = _lin64(d)
    X, G = _f64(d["X"]), _f64(d["dY"])
    Y, XL = layer.linear_forward_prec(X, lin, a16=True)
    dX, _, _, _ = layer.linear_backward_prec(G, X, XL, lin, g16=True)
    e = dict(Y_lo=rel_fro(got["Y"][:, :128], Y[:, :128]), Y_hi=rel_fro(got["Y"][:, 128:], Y[:, 128:]),
             dX=rel_fro(got["dX"], dX))
    log(f"  rel errors {e}")
    for key, v in e.items():
        assert v <= TOL, (key, v)


@pytest.mark.timeout(600)
def test_prec_c2_full_size_sampled():
    log("W4A16G16 linear c2, full size")
    d = wl.linear_case("c2")
    X, G, R = d["X"], d["dY"], d["R"]
    m, k = X.shape
    n, r = R.shape[0], d["A"].shape[0]
    L = _gpu_lin(d)
    x, dy = dev(X, d["x_dtype"]), dev(G, d["dy_dtype"])
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))
    bf = dict(dtype=torch.bfloat16, device="cuda")
    y, xl, dx = torch.empty((m, n), **bf), torch.empty((m, r + d["L1"].shape[0]), **bf), torch.empty((m, k), **bf)
    da = torch.empty((r, k), dtype=torch.float32, device="cuda")
    db = torch.empty((n, r), dtype=torch.float32, device="cuda")
    abi.fourtune_linear_fwd_prec(L, "W4A16G16", x, y, xl, ws)
    abi.fourtune_linear_bwd_prec(L, "W4A16G16", dy, x, xl, dx, da, db, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(zlib.crc32(b"prec/c2"))
    _, rows = _block_rows(m, rng)
    ncols, kcols = _col_blocks(n, rng), _col_blocks(k, rng)
    lin = _lin64(d)
    D, U = lin.D(), lin.U()
    Xr, Gr = _f64(X[rows]), _f64(G[rows])
    XL_o = _bf(_bf(Xr) @ D.T)
    Y_o = _bf(Xr) @ mx4.fake_quant(R[ncols]).T + XL_o @ U[ncols].T
    GB_o = _bf(_bf(Gr) @ U)
    dX_o = _bf(Gr) @ mx4.fake_quant(R[:, kcols]) + GB_o @ D[:, kcols]
    errs = dict(XL=rel_fro(_rows(xl, rows), XL_o), Y=rel_fro(_rows(y, rows)[:, ncols], _bf(Y_o)),
                dX=rel_fro(_rows(dx, rows)[:, kcols], _bf(dX_o)))
    jsel = np.unique([0, r // 2, r - 1])
    GBA = _chunked(lambda lo, hi: _bf(_bf(G[lo:hi]) @ U[:, jsel]), m)
    XLA = _chunked(lambda lo, hi: _bf(_bf(X[lo:hi]) @ D[jsel].T), m)
    errs["dA"] = rel_fro(host(da)[jsel][:, kcols], GBA.T @ _bf(X[:, kcols]))
    errs["dB"] = rel_fro(host(db)[ncols][:, jsel], _f64(G[:, ncols]).T @ XLA)
    _errs_ok(errs)
