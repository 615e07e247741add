"""GPU parity of fourtune_mlp_fwd / fourtune_mlp_bwd against the oracle's MLP pair.

Bars (see the module-level helpers):
* P^ (saved FC1 output), XL1, HL2, Y, dX and the four LoRA gradients: relative
  Frobenius error <= 1e-3 against the fp64 oracle on the same seeded inputs.
* Q(H) and Q(dP), the 4-bit operands the fused epilogues quantize from fp32 values the
  GPU computes (GELU of P^, dH * GELU'(P^)): the oracle decides on its values rounded
  to fp32; in general cases almost all scale bytes and codes equal the oracle's and
  every difference is one grid step (the fp32 accumulations of the two sides differ
  near a threshold, where both codes are valid). Y and dX, which consume those codes,
  are compared on the rows whose codes all equal the oracle's (at least half of them).
* Exact-epilogue cases: with on-grid operands and no low-rank branches, FC1's output
  and dH are exact on both sides, so every code and scale byte must equal the
  oracle's except where the oracle's value lies within 2^-16 (relative) of a rounding
  threshold or its block maximum within 2^-16 of a power of two.
"""
import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from synth import workloads as wl
from tests.gpu_util import dev, host, host_u8, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-3
THRESH = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _lin(d):
    return layer.Linear(R=d["R"].astype(np.float64), A=d["A"].astype(np.float64),
                        B=d["B"].astype(np.float64), L1=d["L1"].astype(np.float64),
                        L2=d["L2"].astype(np.float64))


def _gpu_lin(d):
    return abi.make_linear(dev(d["R"], "fp32"), dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))


def _run(case, out_dtype=torch.float32):
    m = case["X"].shape[0]
    fc1, fc2 = _gpu_lin(case["fc1"]), _gpu_lin(case["fc2"])
    x, dy = dev(case["X"], case["x_dtype"]), dev(case["dY"], case["dy_dtype"])
    f = fc1.n
    hq, dpq = abi.Mx4.empty(m, f), abi.Mx4.empty(m, f)
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2))
    y, saved = abi.mlp_forward(fc1, fc2, x, y_dtype=out_dtype, ws=ws, hq_out=hq)
    g = abi.mlp_backward(fc1, fc2, dy, x, saved, dx_dtype=out_dtype, ws=ws, dpq_out=dpq)
    torch.cuda.synchronize()
    out = dict(Y=host(y), XL1=host(saved["xl1"]), P=host(saved["pre"]), HL2=host(saved["hl2"]),
               hq=(host_u8(hq.codes), host_u8(hq.scales)), dpq=(host_u8(dpq.codes), host_u8(dpq.scales)))
    out.update({k: host(v) for k, v in g.items()})
    return out


def _oracle(case):
    fc1, fc2 = _lin(case["fc1"]), _lin(case["fc2"])
    X, G = case["X"].astype(np.float64), case["dY"].astype(np.float64)
    fwd = layer.mlp_forward(X, fc1, fc2)
    bwd = layer.mlp_backward(G, X, fwd, fc1, fc2)
    return fwd, bwd


def _codes_scales(got, T):
    """Oracle codes (unpacked) and scales of T; GPU codes unpacked."""
    wc, wsc = mx4.quantize(T)
    gc = mx4.unpack_codes(got[0])
    return gc, got[1], wc, wsc


def _grid_index(c):
    return (c & 7).astype(np.int64) * np.where(c & 8, -1, 1)


def check_quant_close(got, T, name, max_frac=1e-3):
    """Scale bytes within +-1 and codes within one grid step of the oracle's, with few
    differences; deq within TOL."""
    gc, gs, wc, ws_ = _codes_scales(got, T)
    ds = gs.astype(np.int64) - ws_.astype(np.int64)
    assert np.all(np.abs(ds) <= 1), f"{name}: scale bytes differ by more than 1"
    frac_s = np.mean(ds != 0)
    same_blk = np.kron(ds == 0, np.ones((32, 32), dtype=bool))[: gc.shape[0], : gc.shape[1]]
    mag_g, mag_w = gc & 7, wc & 7
    zero_both = (mag_g == 0) & (mag_w == 0)
    diff = (gc != wc) & same_blk & ~zero_both
    step = np.abs(_grid_index(gc) - _grid_index(wc))
    assert np.all(step[diff] <= 1), f"{name}: a code differs by more than one grid step"
    frac_c = np.mean(diff)
    deq_err = rel_fro(mx4.dequantize(gc, gs), mx4.dequantize(wc, ws_))
    log(f"  {name}: scale bytes differing {frac_s:.2e}, codes differing {frac_c:.2e}, deq rel {deq_err:.2e}")
    # (a single legitimate one-step flip of a block's largest element can move deq Q by
    # ~1e-3 in Frobenius on these small tensors, so the deq figure is logged, not barred)
    assert frac_s <= max_frac and frac_c <= max_frac, name


def check_quant_exact(got, T, name):
    """Codes and scales equal the oracle's except where the oracle's value is within
    2^-16 of a rounding threshold (or its block max within 2^-16 of a power of two)."""
    gc, gs, wc, ws_ = _codes_scales(got, T)
    rows, cols = T.shape
    nb_r, nb_c = ws_.shape
    Tp = np.zeros((nb_r * 32, cols))
    Tp[:rows] = T
    amax = np.abs(Tp.reshape(nb_r, 32, nb_c, 32)).max(axis=(1, 3))
    with np.errstate(divide="ignore"):
        lg = np.log2(np.where(amax > 0, amax, 1.0))
    near_pow2 = (amax > 0) & (np.abs(amax / np.exp2(np.round(lg)) - 1.0) < 2.0 ** -16)
    ok_blk = ~near_pow2
    assert np.array_equal(gs[ok_blk], ws_[ok_blk]), f"{name}: scale bytes differ away from boundaries"
    E = ws_.astype(np.float64) - 127.0
    y = np.abs(T) / np.exp2(np.kron(E, np.ones((32, 32)))[:rows, :cols])
    near_t = np.min(np.abs(y[..., None] - THRESH) / THRESH, axis=-1) < 2.0 ** -16
    blk_ok = np.kron(ok_blk, np.ones((32, 32), dtype=bool))[:rows, :cols]
    zero_both = ((gc & 7) == 0) & ((wc & 7) == 0)
    must = blk_ok & ~near_t & ~zero_both
    bad = must & (gc != wc)
    flips = blk_ok & ~must & ~zero_both & (gc != wc)
    log(f"  {name}: {int(np.sum(~must))} of {T.size} codes near a decision boundary or zero on both sides, "
        f"{int(np.sum(flips))} of those differ, {int(np.sum(bad))} mismatches elsewhere")
    assert not np.any(bad), f"{name}: codes differ away from rounding thresholds"
    step = np.abs(_grid_index(gc) - _grid_index(wc))
    assert np.all(step[flips] <= 1), f"{name}: a near-threshold code differs by more than one grid step"


def rows_with_oracle_codes(got, T):
    """Rows whose GPU codes and block scales all equal the oracle's Q(T). Where the two
    sides' fp32-vs-fp64 values straddle a rounding threshold both codes are valid
    (check_quant_close bounds how many and by how much); products that consume those
    codes are unique only on the other rows, which is where they are compared."""
    gc, gs, wc, ws_ = _codes_scales(got, T)
    zero_both = ((gc & 7) == 0) & ((wc & 7) == 0)  # +0 and -0 are the same value
    same = np.all((gc == wc) | zero_both, axis=1)
    blk_same = np.all(gs == ws_, axis=1)
    return same & np.repeat(blk_same, 32)[: gc.shape[0]]


def _check_all(case, got, fwd, bwd):
    h_ok = rows_with_oracle_codes(got["hq"], fwd["H32"])
    p_ok = rows_with_oracle_codes(got["dpq"], bwd["dP32"])
    log(f"  rows with every Q(H) code equal: {int(h_ok.sum())}/{h_ok.size}, Q(dP): {int(p_ok.sum())}/{p_ok.size}")
    assert h_ok.mean() >= 0.5 and p_ok.mean() >= 0.5
    errs = {"P": rel_fro(got["P"], fwd["P"]),
            "XL1": rel_fro(got["XL1"], fwd["XL1"]), "HL2": rel_fro(got["HL2"], fwd["HL2"]),
            "Y": rel_fro(got["Y"][h_ok], fwd["Y"][h_ok]), "dX": rel_fro(got["dX"][p_ok], bwd["dX"][p_ok])}
    for k in ("dA1", "dB1", "dA2", "dB2"):
        errs[k] = rel_fro(got[k], bwd[k]) if bwd[k].size else 0.0
    log(f"  rel errors {errs}")
    for k, e in errs.items():
        assert e <= TOL, (k, e)
    check_quant_close(got["hq"], fwd["H32"], "Q(H)")
    check_quant_close(got["dpq"], bwd["dP32"], "Q(dP)")


MLP_CASES = [
    # m, d, f, r, s, x_dtype
    (200, 256, 512, 32, 32, "bf16"),
    (300, 384, 768, 16, 16, "bf16"),    # r % 32 == 16: padded low-rank tiles
    (96, 256, 512, 32, 0, "fp32"),
    (130, 320, 640, 0, 32, "bf16"),
    # the pass over FC1's output in four column ranges, one range's last chunk pair
    # reaching into the next, the last chunk half past F
    (640, 512, 2080, 32, 32, "bf16"),
]


@pytest.mark.parametrize("m,d,f,r,s,xdt", MLP_CASES)
def test_mlp_small(m, d, f, r, s, xdt):
    log(f"mlp m={m} d={d} f={f} r={r} s={s} x={xdt}")
    case = wl.random_mlp(m, d, f, r, s, seed=m + d + f, x_dtype=xdt, dy_dtype=xdt)
    got = _run(case)
    fwd, bwd = _oracle(case)
    _check_all(case, got, fwd, bwd)


def test_mlp_bf16_outputs_deterministic():
    log("mlp bf16 outputs, twice")
    case = wl.random_mlp(160, 256, 512, 32, 32, seed=77)
    a, b = _run(case, torch.bfloat16), _run(case, torch.bfloat16)
    for k in ("Y", "P", "HL2", "dX", "dA1", "dB1", "dA2", "dB2"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("hq", "dpq"):
        assert np.array_equal(a[k][0], b[k][0]) and np.array_equal(a[k][1], b[k][1]), k
    fwd, bwd = _oracle(case)
    assert rel_fro(a["Y"], mx4.bf16_round(fwd["Y"])) <= TOL
    assert rel_fro(a["dX"], mx4.bf16_round(bwd["dX"])) <= TOL


def test_mlp_split_reductions_any_workspace_and_graph_replay():
    """The MLP pair's split reductions keep their fp32 partials in the workspace: any
    prior contents (all-ones bytes, random bytes, the previous call's state) give the
    same bits, and so do replays of a captured forward + backward with eager calls on
    the same workspace between them."""
    m, d, f = 640, 512, 2080
    log(f"mlp split reductions m={m} d={d} f={f}: workspace contents, graph replay")
    case = wl.random_mlp(m, d, f, 32, 32, seed=31)
    fc1, fc2 = _gpu_lin(case["fc1"]), _gpu_lin(case["fc2"])
    x, dy = dev(case["X"], case["x_dtype"]), dev(case["dY"], case["dy_dtype"])
    hq, dpq = abi.Mx4.empty(m, f), abi.Mx4.empty(m, f)
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2))

    def step():
        y, saved = abi.mlp_forward(fc1, fc2, x, y_dtype=torch.float32, ws=ws, hq_out=hq)
        g = abi.mlp_backward(fc1, fc2, dy, x, saved, dx_dtype=torch.float32, ws=ws, dpq_out=dpq)
        return dict(Y=y, XL1=saved["xl1"], P=saved["pre"], HL2=saved["hl2"], **g)

    def fetch(o):
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in o.items()}
        got["hq"] = (host_u8(hq.codes), host_u8(hq.scales))
        got["dpq"] = (host_u8(dpq.codes), host_u8(dpq.scales))
        return got

    def same(a, b, what):
        for k in ("Y", "XL1", "P", "HL2", "dX", "dA1", "dB1", "dA2", "dB2"):
            assert np.array_equal(a[k], b[k]), (what, k)
        for k in ("hq", "dpq"):
            assert np.array_equal(a[k][0], b[k][0]) and np.array_equal(a[k][1], b[k][1]), (what, k)

    ws.fill_(0xFF)
    ref = fetch(step())
    fwd, bwd = _oracle(case)
    _check_all(case, ref, fwd, bwd)
    same(ref, fetch(step()), "second call, same workspace")
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    same(ref, fetch(step()), "random workspace bytes")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        graph.replay()
        same(ref, fetch(outs), f"graph replay {rep}")
        same(ref, fetch(step()), f"eager call after replay {rep}")


def _on_grid(rng, rows, cols, e_lo, e_hi):
    """A tensor each of whose 32x32 blocks holds E2M1 grid values times one power of
    two 2^e (e uniform in [e_lo, e_hi]) with a +-6 element, so that quantizing it is
    exact and its block exponent is e."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    v = grid[rng.integers(0, 8, size=(rows, cols))] * rng.choice([-1.0, 1.0], size=(rows, cols))
    nb_r, nb_c = (rows + 31) // 32, cols // 32
    e = rng.integers(e_lo, e_hi + 1, size=(nb_r, nb_c)).astype(np.float64)
    v[::32, ::32] = 6.0 * rng.choice([-1.0, 1.0], size=(nb_r, nb_c))
    return (v * np.exp2(np.kron(e, np.ones((32, 32)))[:rows, :cols])).astype(np.float32)


@pytest.mark.parametrize("m", [128, 200])
def test_mlp_exact_epilogue_codes(m):
    """On-grid X, R1, R2, dY and no low-rank branches: FC1's output and dH are exact in
    fp32, so the epilogues' Q(H) and Q(dP) must match the oracle's decisions."""
    d, f = 256, 512
    log(f"mlp exact epilogue m={m} d={d} f={f}")
    rng = np.random.default_rng(1000 + m)

    def linear(n, k):
        return dict(R=_on_grid(rng, n, k, -6, -4), A=np.zeros((0, k), np.float32), B=np.zeros((n, 0), np.float32),
                    L1=np.zeros((0, k), np.float32), L2=np.zeros((n, 0), np.float32))
    case = dict(X=_on_grid(rng, m, d, -2, 0), fc1=linear(f, d), fc2=linear(d, f),
                dY=_on_grid(rng, m, d, -9, -7), x_dtype="bf16", dy_dtype="bf16")
    got = _run(case)
    fwd, bwd = _oracle(case)
    assert np.array_equal(got["P"], fwd["P"]), "P^ must be exact here"
    check_quant_exact(got["hq"], fwd["H32"], "Q(H)")
    check_quant_exact(got["dpq"], bwd["dP32"], "Q(dP)")
    # (Y and dX are not barred here: on-grid FC1 outputs put many GELU values within
    # an fp32 ulp of a rounding tie, where either adjacent code is correct)


def test_mlp_argument_errors():
    case = wl.random_mlp(64, 256, 512, 16, 16, seed=5)
    fc1, fc2 = _gpu_lin(case["fc1"]), _gpu_lin(case["fc2"])
    x = dev(case["X"])
    y = torch.empty((64, 256), dtype=torch.float32, device="cuda")
    xl1 = torch.empty((64, 32), dtype=torch.bfloat16, device="cuda")
    pre = torch.empty((64, 512), dtype=torch.bfloat16, device="cuda")
    hl2 = torch.empty((64, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(abi.FourTuneError) as e:
        abi.fourtune_mlp_fwd(fc1, fc2, x, y, xl1, pre, hl2, abi.workspace(64))
    assert e.value.name == "FT_ERR_WORKSPACE"
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(64, fc1, fc2))
    with pytest.raises(abi.FourTuneError) as e:
        abi.fourtune_mlp_fwd(fc2, fc2, x, y, xl1, pre, hl2, ws)  # fc1.n != fc2.k
    assert e.value.name == "FT_ERR_SHAPE"
    with pytest.raises(abi.FourTuneError) as e:
        abi.fourtune_mlp_fwd(fc1, fc2, x, y, xl1, None, hl2, ws)
    assert e.value.name == "FT_ERR_NULL"
