"""GPU parity of fourtune_mlp_fwd / fourtune_mlp_bwd against the oracle's MLP pair
(FourTune §3.3 "MLP Fusion"; the bounds are derived in tests/parity.py).

Every output is compared element by element, on every row:
* XL1, P^ (saved FC1 output), HL2: the oracle's products within the fp32-accumulation
  bound plus one bf16 ulp per rounded intermediate;
* H and dP, the fp32 values the fused steps quantize (exported through h_debug and
  dp_debug): the oracle's GELU / GELU' of the GPU's own P^ within the fp32 function
  error; the oracle quantizer applied to them reproduces Q(H) and Q(dP) bit for bit;
  and against the oracle's own fp64 chain a code or scale byte differs only within
  the derived bound of a rounding threshold or power of two;
* Y and dX given the GPU's own Q(H) and Q(dP) ("identical quantized operands"), and the
  four LoRA gradients, within their bounds and the relative Frobenius bar of 1e-3.
"""
import ctypes

import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from synth import workloads as wl
from tests import parity
from tests.gpu_util import dev, host, host_u8, log

pytestmark = pytest.mark.gpu


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
    hdbg = torch.empty((m, f), dtype=torch.float32, device="cuda")
    dpdbg = torch.empty((m, f), dtype=torch.float32, device="cuda")
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2))
    y, saved = abi.mlp_forward(fc1, fc2, x, y_dtype=out_dtype, ws=ws, hq_out=hq, h_debug=hdbg)
    g = abi.mlp_backward(fc1, fc2, dy, x, saved, dx_dtype=out_dtype, ws=ws, dpq_out=dpq, dp_debug=dpdbg)
    torch.cuda.synchronize()
    out = dict(Y=host(y), XL1=host(saved["xl1"]), P=host(saved["pre"]), HL2=host(saved["hl2"]),
               H=host(hdbg), dP=host(dpdbg),
               hq=(host_u8(hq.codes), host_u8(hq.scales)), dpq=(host_u8(dpq.codes), host_u8(dpq.scales)))
    out.update({k: host(v) for k, v in g.items()})
    out["Hf"], out["dPa"] = out["H"], out["dP"]
    return out


def _check_all(case, got, out_bf16=False):
    fc1, fc2 = _lin(case["fc1"]), _lin(case["fc2"])
    ex = parity.mlp_expect(fc1, fc2, case["X"], case["dY"], got)
    for k in ("XL1", "P", "HL2"):
        parity.check_values(k, got[k], *ex[k], out_bf16=True)
    for k in ("H", "dP", "dA1", "dB1", "dA2", "dB2"):
        if k in ex:
            parity.check_values(k, got[k], *ex[k])
    for k in ("Y", "dX"):
        parity.check_values(k, got[k], *ex[k], out_bf16=out_bf16)


MLP_CASES = [
    # m, d, f, r, s, x_dtype
    (200, 256, 512, 32, 32, "bf16"),
    (300, 384, 768, 16, 16, "bf16"),    # each factor 16 wide
    (96, 256, 512, 32, 0, "fp32"),
    (130, 320, 640, 0, 32, "bf16"),
    (200, 256, 512, 16, 32, "bf16"),    # rank + stab_rank = 48: a padding tile
    (130, 320, 640, 48, 32, "bf16"),    # width 80: the register kernel's pass over P^
    # the pass over FC1's output in four column ranges, one range's last chunk pair
    # reaching into the next, the last chunk half past F
    (640, 512, 2080, 32, 32, "bf16"),
    # many rows at widths above 64: the row-split kernel's pass over P^ (GELU, Q(H))
    # and its down-projection of dP, with a ragged last stripe
    (16400, 128, 256, 64, 64, "bf16"),
    (16390, 128, 288, 48, 32, "bf16"),  # width 80: a padding tile
    (4160, 256, 2080, 64, 32, "bf16"),  # pass over P^ in column ranges, 33 stripes
]


@pytest.mark.parametrize("m,d,f,r,s,xdt", MLP_CASES)
def test_mlp_small(m, d, f, r, s, xdt):
    log(f"mlp m={m} d={d} f={f} r={r} s={s} x={xdt}")
    case = wl.random_mlp(m, d, f, r, s, seed=m + d + f, x_dtype=xdt, dy_dtype=xdt)
    _check_all(case, _run(case))


def test_mlp_bf16_outputs_deterministic():
    log("mlp bf16 outputs, twice")
    case = wl.random_mlp(160, 256, 512, 32, 32, seed=77)
    a, b = _run(case, torch.bfloat16), _run(case, torch.bfloat16)
    for k in ("Y", "P", "HL2", "dX", "dA1", "dB1", "dA2", "dB2"):
        assert np.array_equal(a[k], b[k]), k
    for k in ("hq", "dpq"):
        assert np.array_equal(a[k][0], b[k][0]) and np.array_equal(a[k][1], b[k][1]), k
    _check_all(case, a, out_bf16=True)


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
    hdbg = torch.empty((m, f), dtype=torch.float32, device="cuda")
    dpdbg = torch.empty((m, f), dtype=torch.float32, device="cuda")
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(m, fc1, fc2))

    def step():
        y, saved = abi.mlp_forward(fc1, fc2, x, y_dtype=torch.float32, ws=ws, hq_out=hq, h_debug=hdbg)
        g = abi.mlp_backward(fc1, fc2, dy, x, saved, dx_dtype=torch.float32, ws=ws, dpq_out=dpq, dp_debug=dpdbg)
        return dict(Y=y, XL1=saved["xl1"], P=saved["pre"], HL2=saved["hl2"], H=hdbg, dP=dpdbg, **g)

    def fetch(o):
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in o.items()}
        got["Hf"], got["dPa"] = got["H"], got["dP"]
        got["hq"] = (host_u8(hq.codes), host_u8(hq.scales))
        got["dpq"] = (host_u8(dpq.codes), host_u8(dpq.scales))
        return got

    def same(a, b, what):
        for k in ("Y", "XL1", "P", "HL2", "H", "dP", "dX", "dA1", "dB1", "dA2", "dB2"):
            assert np.array_equal(a[k], b[k]), (what, k)
        for k in ("hq", "dpq"):
            assert np.array_equal(a[k][0], b[k][0]) and np.array_equal(a[k][1], b[k][1]), (what, k)

    ws.fill_(0xFF)
    ref = fetch(step())
    _check_all(case, ref)
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
    fp32 on both sides, so P^ equals the oracle's bit for bit, and many GELU values sit
    on or next to E2M1 rounding ties (the decisions the fused steps must take in fp32)."""
    d, f = 256, 512
    log(f"mlp exact epilogue m={m} d={d} f={f}")
    rng = np.random.default_rng(1000 + m)

    def linear(n, k):
        return dict(R=_on_grid(rng, n, k, -6, -4), A=np.zeros((0, k), np.float32), B=np.zeros((n, 0), np.float32),
                    L1=np.zeros((0, k), np.float32), L2=np.zeros((n, 0), np.float32))
    case = dict(X=_on_grid(rng, m, d, -2, 0), fc1=linear(f, d), fc2=linear(d, f),
                dY=_on_grid(rng, m, d, -9, -7), x_dtype="bf16", dy_dtype="bf16")
    got = _run(case)
    fwd = layer.mlp_forward(case["X"].astype(np.float64), _lin(case["fc1"]), _lin(case["fc2"]))
    assert np.array_equal(got["P"], fwd["P"]), "P^ must be exact here"
    _check_all(case, got)


def test_mlp_empty_batch():
    """m = 0: the MLP calls (fused and unfused) succeed and set all four LoRA gradients
    to zero."""
    case = wl.random_mlp(64, 256, 512, 32, 16, seed=7)
    fc1, fc2 = _gpu_lin(case["fc1"]), _gpu_lin(case["fc2"])
    d, f, r = 256, 512, 32
    bf = dict(dtype=torch.bfloat16, device="cuda")
    x, dy, y, dx = (torch.empty((0, d), **bf), torch.empty((0, d), **bf), torch.empty((0, d), **bf),
                    torch.empty((0, d), **bf))
    xl1, pre, h, hl2 = torch.empty((0, 48), **bf), torch.empty((0, f), **bf), torch.empty((0, f), **bf), \
        torch.empty((0, 48), **bf)
    ws = abi.workspace(abi.fourtune_mlp_workspace_bytes(64, fc1, fc2))
    abi.fourtune_mlp_fwd(fc1, fc2, x, y, xl1, pre, hl2, ws)

    def grads():
        return [torch.full(sh, float("nan"), device="cuda") for sh in ((r, d), (f, r), (r, f), (d, r))]

    for name in ("mlp_bwd", "mlp_bwd_unfused"):
        g = grads()
        if name == "mlp_bwd":
            abi.fourtune_mlp_bwd(fc1, fc2, dy, x, xl1, pre, hl2, dx, *g, ws)
        else:
            abi.fourtune_mlp_bwd_unfused(fc1, fc2, False, dy, x, xl1, pre, h, hl2, dx, *g, ws)
        torch.cuda.synchronize()
        log(f"  {name}: m = 0")
        for t in g:
            assert torch.equal(t, torch.zeros_like(t)), name


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
    with pytest.raises(ValueError):  # fc1.n != fc2.k, caught by the binding
        abi.fourtune_mlp_fwd(fc2, fc2, x, y, xl1, pre, hl2, ws)
    with pytest.raises(ValueError):
        abi.fourtune_mlp_fwd(fc1, fc2, x, y, xl1, None, hl2, ws)
    # the library's own checks, reached with raw pointers
    s1, s2 = fc1.struct(), fc2.struct()
    st = abi.lib().fourtune_mlp_fwd(ctypes.byref(s2), ctypes.byref(s2), abi._ptr(x), abi.FT_BF16, 64, abi._ptr(y),
                                    abi.FT_F32, abi._ptr(xl1), abi._ptr(pre), abi._ptr(hl2), None, None,
                                    abi._ptr(ws), ws.numel(), None)
    assert abi.STATUS[st] == "FT_ERR_SHAPE"
    st = abi.lib().fourtune_mlp_fwd(ctypes.byref(s1), ctypes.byref(s2), abi._ptr(x), abi.FT_BF16, 64, abi._ptr(y),
                                    abi.FT_F32, abi._ptr(xl1), None, abi._ptr(hl2), None, None,
                                    abi._ptr(ws), ws.numel(), None)
    assert abi.STATUS[st] == "FT_ERR_NULL"
