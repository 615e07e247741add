"""GPU parity at the workloads' full sizes (c3, c4, c5), in the launch configuration the
bench uses for c2: the whole layer runs on the GPU at full size; the oracle then
computes sampled outputs one by one from the same seeded inputs.

What is sampled (block rows are 32-row groups, so every sampled row brings its whole
quantization blocks; the first, a middle and the last, possibly partial, block row):
* Q(X), Q(dY), Q(H), Q(dP): the sampled block rows' codes and scales (Q(X), Q(dY)
  bit-exact; the fused-epilogue codes Q(H), Q(dP) as in the small MLP tests: scale
  bytes within one, codes within one grid step, differences rare).
* Y, XL, P^, HL2 on the sampled rows (Y on sampled output-column blocks); dX on the
  sampled rows and input-column blocks. In the MLP, Y and dX consume the epilogue
  codes Q(H), Q(dP): they are compared on the sampled rows whose codes all equal the
  oracle's (a code whose value lies within the two sides' accumulation difference of a
  threshold may validly go either way).
* LoRA gradients: sampled (rank, column) entries, each a full reduction over all M
  rows that the oracle evaluates for just those entries. For the c5 MLP the entries
  of dA1 and dB2 would need GELU'(P) or H over the whole [M x F] intermediate (2.3
  TFLOP in fp64): they are left to the smaller MLP cases, where the same kernels run.
Bar: relative Frobenius error <= 1e-3 over each sampled set.
"""
import zlib

import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from synth import workloads as wl
from tests.gpu_util import dev, host, log, oracle_packed, rel_fro
from tests.test_gpu_mlp import check_quant_close, rows_with_oracle_codes

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _block_rows(m, rng):
    nb = (m + 31) // 32
    picks = sorted({0, int(rng.integers(1, max(nb - 1, 2))), nb - 1})
    return picks, np.concatenate([np.arange(32 * b, min(32 * b + 32, m)) for b in picks])


def _col_blocks(n, rng, count=3):
    nb = n // 32
    picks = sorted(set([0, nb - 1] + [int(v) for v in rng.integers(0, nb, count)]))
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in picks])


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _bf(a):
    return mx4.bf16_round(_f64(a))


def _chunked(fn, m, step=4096):
    """Row-chunked evaluation of fn(lo, hi) -> array, stacked (bounds fp64 temporaries)."""
    return np.concatenate([fn(lo, min(m, lo + step)) for lo in range(0, m, step)], axis=0)


def _rows(t, idx):
    return host(t.index_select(0, torch.as_tensor(idx, device=t.device)))


def _check_codes(got_mx4, T_rows, rows, brows, name, exact=True):
    """Exact: codes and scales equal the oracle's. Otherwise (fused-epilogue codes) the
    close check, returning the mask of sampled rows whose codes all equal the oracle's."""
    codes = got_mx4.codes.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    scales = got_mx4.scales.index_select(0, torch.as_tensor(brows, device="cuda")).cpu().numpy()
    if exact:
        wc, ws_ = oracle_packed(T_rows)
        assert np.array_equal(scales, ws_), f"{name}: scale bytes"
        assert np.array_equal(codes, wc), f"{name}: codes"
        return np.ones(len(rows), dtype=bool)
    check_quant_close((codes, scales), _f64(T_rows), name)
    ok = rows_with_oracle_codes((codes, scales), _f64(T_rows))
    log(f"  {name}: sampled rows with every code equal: {int(ok.sum())}/{ok.size}")
    assert ok.mean() >= 0.5
    return ok


def _lin64(d):
    return layer.Linear(R=_f64(d["R"]), A=_f64(d["A"]), B=_f64(d["B"]), L1=_f64(d["L1"]), L2=_f64(d["L2"]))


def _gpu_lin(d):
    return abi.make_linear(dev(d["R"], "fp32"), dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))


def _errs_ok(errs):
    log(f"  rel errors {errs}")
    for k_, e in errs.items():
        assert e <= TOL, (k_, e)


# ------------------------------------------------------------------------------ linear
LINEARS = [("c4", "qkv"), ("c4", "o"), ("c5", "qkv")]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key,name", LINEARS)
def test_linear_full_size_sampled(key, name):
    log(f"full-size linear {key}/{name}: drawing inputs")
    d = wl.linear_case(key, name)
    X, G, R = d["X"], d["dY"], d["R"]
    m, k = X.shape
    n, r = R.shape[0], d["A"].shape[0]
    log(f"  m={m} n={n} k={k} r={r} s={d['L1'].shape[0]}: GPU fwd+bwd")
    L = _gpu_lin(d)
    x, dy = dev(X, d["x_dtype"]), dev(G, d["dy_dtype"])
    xq, gq = abi.Mx4.empty(m, k), abi.Mx4.empty(m, n)
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))
    y, xl = abi.linear_forward(L, x, y_dtype=torch.bfloat16, ws=ws, xq_out=xq)
    dx, da, db = abi.linear_backward(L, dy, x, xl, dx_dtype=torch.bfloat16, ws=ws, gq_out=gq)
    torch.cuda.synchronize()
    del x, dy

    rng = np.random.default_rng(zlib.crc32(f"{key}/{name}".encode()))
    brows, rows = _block_rows(m, rng)
    ncols, kcols = _col_blocks(n, rng), _col_blocks(k, rng)
    lin = _lin64(d)
    D, U = lin.D(), lin.U()
    log("  oracle: codes of the sampled block rows")
    _check_codes(xq, X[rows], rows, brows, "Q(X)")
    _check_codes(gq, G[rows], rows, brows, "Q(dY)")

    log("  oracle: sampled rows of Y, XL, dX")
    Xr, Gr = _f64(X[rows]), _f64(G[rows])
    XL_o = _bf(_bf(Xr) @ D.T)
    Y_o = mx4.fake_quant(Xr) @ mx4.fake_quant(R[ncols]).T + XL_o @ U[ncols].T
    GB_o = _bf(_bf(Gr) @ U)
    dX_o = mx4.fake_quant(Gr) @ mx4.fake_quant(R[:, kcols]) + GB_o @ D[:, kcols]
    errs = dict(XL=rel_fro(_rows(xl, rows), XL_o),
                Y=rel_fro(_rows(y, rows)[:, ncols], _bf(Y_o)),
                dX=rel_fro(_rows(dx, rows)[:, kcols], _bf(dX_o)))

    if r > 0:
        log("  oracle: sampled LoRA-gradient entries (reductions over all rows)")
        jsel = np.unique([0, r // 2, r - 1])
        GBA = _chunked(lambda lo, hi: _bf(_bf(G[lo:hi]) @ U[:, jsel]), m)       # GB[:, jsel]
        dA_o = GBA.T @ _bf(X[:, kcols])
        XLA = _chunked(lambda lo, hi: _bf(_bf(X[lo:hi]) @ D[jsel].T), m)        # XL[:, jsel]
        dB_o = _f64(G[:, ncols]).T @ XLA
        errs["dA"] = rel_fro(host(da)[jsel][:, kcols], dA_o)
        errs["dB"] = rel_fro(host(db)[ncols][:, jsel], dB_o)
    _errs_ok(errs)


# --------------------------------------------------------------------------------- MLP
MLPS = ["c3", "c4", "c5"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", MLPS)
def test_mlp_full_size_sampled(key):
    log(f"full-size MLP {key}: drawing inputs")
    case = wl.mlp_case(key)
    X, G = case["X"], case["dY"]
    p1, p2 = case["fc1"], case["fc2"]
    m, dm = X.shape
    f = p1["R"].shape[0]
    r1, r2 = p1["A"].shape[0], p2["A"].shape[0]
    log(f"  m={m} d={dm} f={f} r={r1}: GPU fwd+bwd")
    fc1, fc2 = _gpu_lin(p1), _gpu_lin(p2)
    x, dy = dev(X, case["x_dtype"]), dev(G, case["dy_dtype"])
    hq, dpq = abi.Mx4.empty(m, f), abi.Mx4.empty(m, f)
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2))
    y, saved = abi.mlp_forward(fc1, fc2, x, y_dtype=torch.bfloat16, ws=ws, hq_out=hq)
    g = abi.mlp_backward(fc1, fc2, dy, x, saved, dx_dtype=torch.bfloat16, ws=ws, dpq_out=dpq)
    torch.cuda.synchronize()
    del x, dy

    rng = np.random.default_rng(zlib.crc32(key.encode()))
    brows, rows = _block_rows(m, rng)
    dcols, fcols = _col_blocks(dm, rng), _col_blocks(f, rng)
    l1, l2 = _lin64(p1), _lin64(p2)
    D1, U1, D2, U2 = l1.D(), l1.U(), l2.D(), l2.U()
    log("  oracle: Q(R1), Q(R2)")
    Rd1, Rd2 = mx4.fake_quant(p1["R"]), mx4.fake_quant(p2["R"])

    log("  oracle: sampled rows, forward")
    Xr, Gr = _f64(X[rows]), _f64(G[rows])
    XL1_o = _bf(_bf(Xr) @ D1.T)
    P_o = _bf(mx4.fake_quant(Xr) @ Rd1.T + XL1_o @ U1.T)
    H_o = layer.gelu_tanh(P_o)
    H32 = layer.fp32(H_o)  # the epilogue decides Q(H) on fp32 values
    h_ok = _check_codes(hq, H32, rows, brows, "Q(H)", exact=False)
    HL2_o = _bf(_bf(H_o) @ D2.T)
    Y_o = mx4.fake_quant(H32) @ Rd2[dcols].T + HL2_o @ U2[dcols].T

    log("  oracle: sampled rows, backward")
    GB2_o = _bf(_bf(Gr) @ U2)
    dH_o = mx4.fake_quant(Gr) @ Rd2 + GB2_o @ D2
    dP_o = dH_o * layer.gelu_tanh_grad(P_o)
    dP32 = layer.fp32(dP_o)
    p_ok = _check_codes(dpq, dP32, rows, brows, "Q(dP)", exact=False)
    GB1_o = _bf(_bf(dP_o) @ U1)
    kcols = dcols  # FC1's input columns are the model width
    dX_o = mx4.fake_quant(dP32) @ Rd1[:, kcols] + GB1_o @ D1[:, kcols]
    errs = dict(XL1=rel_fro(_rows(saved["xl1"], rows), XL1_o),
                P=rel_fro(_rows(saved["pre"], rows), P_o),
                HL2=rel_fro(_rows(saved["hl2"], rows), HL2_o),
                Y=rel_fro(_rows(y, rows)[:, dcols][h_ok], _bf(Y_o)[h_ok]),
                dX=rel_fro(_rows(g["dX"], rows)[:, kcols][p_ok], _bf(dX_o)[p_ok]))

    log("  oracle: sampled LoRA-gradient entries (reductions over all rows)")
    # P, H and GELU'(P) on the sampled intermediate columns, every row
    Xd_all = _chunked(lambda lo, hi: mx4.fake_quant(X[lo:hi]), m, step=2048)
    XL1_all = _chunked(lambda lo, hi: _bf(_bf(X[lo:hi]) @ D1.T), m)
    Pf = _bf(Xd_all @ Rd1[fcols].T + XL1_all @ U1[fcols].T)
    Gd_all = _chunked(lambda lo, hi: mx4.fake_quant(G[lo:hi]), m, step=2048)
    GB2_all = _chunked(lambda lo, hi: _bf(_bf(G[lo:hi]) @ U2), m)
    dPf = (Gd_all @ Rd2[:, fcols] + GB2_all @ D2[:, fcols]) * layer.gelu_tanh_grad(Pf)
    if r2 > 0:
        j2 = np.unique([0, r2 // 2, r2 - 1])
        errs["dA2"] = rel_fro(host(g["dA2"])[j2][:, fcols], GB2_all[:, j2].T @ _bf(layer.gelu_tanh(Pf)))
    if r1 > 0:
        j1 = np.unique([0, r1 // 2, r1 - 1])
        errs["dB1"] = rel_fro(host(g["dB1"])[fcols][:, j1], _bf(dPf).T @ XL1_all[:, j1])
    heavy = m * dm * f > 1e12
    if not heavy:
        # the whole intermediate is affordable: dA1 and dB2 too
        P_all = _bf(Xd_all @ Rd1.T + XL1_all @ U1.T)
        if r2 > 0:
            HL2_all = _bf(_bf(layer.gelu_tanh(P_all)) @ D2.T)
            errs["dB2"] = rel_fro(host(g["dB2"])[dcols][:, j2], _f64(G[:, dcols]).T @ HL2_all[:, j2])
        if r1 > 0:
            dP_all = (Gd_all @ Rd2 + GB2_all @ D2) * layer.gelu_tanh_grad(P_all)
            GB1_all = _bf(_bf(dP_all) @ U1[:, j1])
            errs["dA1"] = rel_fro(host(g["dA1"])[j1][:, kcols], GB1_all.T @ _bf(X[:, kcols]))
    _errs_ok(errs)


# ------------------------------------------------------------------ DiT text stream
@pytest.mark.timeout(600)
def test_dit_text_stream_linears_full():
    """The whole-DiT step's smallest stream (the 512 text tokens of a double-stream
    block) at its real shapes and ranks (LoRA 64, stabilizer 32): QKV, the output
    projection and the MLP pair, every output against the full oracle."""
    from tests.test_gpu_linear import _check_full, _run as run_linear
    from tests.test_gpu_mlp import _check_all, _oracle as mlp_oracle, _run as run_mlp
    for n, k in ((9216, 3072), (3072, 3072)):
        log(f"DiT text stream linear m=512 n={n} k={k}")
        d = wl.random_linear(512, n, k, 64, 32, seed=n + k)
        _check_full(d, run_linear(d))
    log("DiT text stream MLP m=512 d=3072 f=12288")
    case = wl.random_mlp(512, 3072, 12288, 64, 32, seed=512)
    got = run_mlp(case)
    fwd, bwd = mlp_oracle(case)
    _check_all(case, got, fwd, bwd)
