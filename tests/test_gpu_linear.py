"""GPU parity of fourtune_linear_fwd / fourtune_linear_bwd against the oracle.

Bar: Q(X), Q(dY) codes and scales bit-exact; XL, Y, dX, dA, dB element by element
within the bounds derived in tests/parity.py (fp32 accumulation plus one bf16 ulp per
rounded intermediate), each stage on the operands it consumes; and, end to end, the
oracle's own chain from the same seeded inputs within a relative Frobenius error of
1e-3 (bf16 outputs against the oracle rounded to bf16).
"""
import ctypes

import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from synth import workloads as wl
from tests import parity
from tests.gpu_util import dev, host, host_u8, log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _gpu_linear(d):
    R = dev(d["R"], "fp32")
    L = abi.make_linear(R, dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))
    return L


def _oracle_linear(d):
    return layer.Linear(R=d["R"].astype(np.float64), A=d["A"].astype(np.float64),
                        B=d["B"].astype(np.float64), L1=d["L1"].astype(np.float64),
                        L2=d["L2"].astype(np.float64))


def _run(d, out_dtype=torch.float32):
    """Forward + backward on the GPU; returns host arrays."""
    m, n, k = d["X"].shape[0], d["R"].shape[0], d["R"].shape[1]
    L = _gpu_linear(d)
    x = dev(d["X"], d["x_dtype"])
    dy = dev(d["dY"], d["dy_dtype"])
    xq = abi.Mx4.empty(m, k)
    gq = abi.Mx4.empty(m, n)
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))
    y, xl = abi.linear_forward(L, x, y_dtype=out_dtype, ws=ws, xq_out=xq)
    dx, da, db = abi.linear_backward(L, dy, x, xl, dx_dtype=out_dtype, ws=ws, gq_out=gq)
    torch.cuda.synchronize()
    return dict(Y=host(y), XL=host(xl), dX=host(dx), dA=host(da), dB=host(db),
                xq=(host_u8(xq.codes), host_u8(xq.scales)), gq=(host_u8(gq.codes), host_u8(gq.scales)))


def _check_full(d, got, out_bf16=False):
    lin = _oracle_linear(d)
    X, G = d["X"], d["dY"]
    parity.quant_exact("Q(X)", *got["xq"], X)
    parity.quant_exact("Q(dY)", *got["gq"], G)
    ex = parity.linear_expect(lin, X, G, got)
    parity.check_values("XL", got["XL"], *ex["XL"], out_bf16=True)
    for k_ in ("Y", "dX"):
        parity.check_values(k_, got[k_], *ex[k_], out_bf16=out_bf16)
    for k_ in ("dA", "dB"):
        if k_ in ex:
            parity.check_values(k_, got[k_], *ex[k_])
    # end to end: the oracle's own chain
    X64, G64 = X.astype(np.float64), G.astype(np.float64)
    Y, XL = layer.linear_forward(X64, lin)
    dX, dA, dB, _ = layer.linear_backward(G64, X64, XL, lin)
    rnd = mx4.bf16_round if out_bf16 else (lambda a: a)
    errs = dict(Y=rel_fro(got["Y"], rnd(Y)), dX=rel_fro(got["dX"], rnd(dX)),
                dA=rel_fro(got["dA"], dA) if dA.size else 0.0, dB=rel_fro(got["dB"], dB) if dB.size else 0.0)
    log(f"  end to end rel errors {errs}")
    for k_, e in errs.items():
        assert e <= TOL, (k_, e)
    return errs


CASES = [
    # m, n, k, r, s, x_dtype
    (64, 256, 256, 16, 16, "bf16"),
    (300, 544, 384, 32, 32, "bf16"),     # ragged M (partial block, partial tile), N tail
    (257, 512, 416, 64, 32, "bf16"),     # K % 128 != 0 (scale bytes one by one)
    (200, 320, 288, 0, 32, "bf16"),      # no LoRA
    (200, 320, 288, 32, 0, "fp32"),      # no stabilizer, fp32 input
    (96, 256, 512, 0, 0, "bf16"),        # plain 4-bit GEMM
    (520, 768, 640, 64, 64, "fp32"),
    # two column ranges per row block in the fused quantize + down-projection, the first
    # range's last chunk pair reaching into the second, the last chunk half past K
    (640, 1056, 1056, 32, 32, "bf16"),
    (600, 1120, 1088, 16, 16, "bf16"),
    # tiny: a single reduction block (K = 32), a partial first row block, ragged tiles
    (7, 96, 32, 16, 16, "bf16"),
    # rank + stab_rank = 16 (mod 32): the fused kernels add a padding tile of zeros
    (300, 544, 384, 16, 32, "bf16"),     # staged kernel, LoRA tile alone in its pair
    (257, 512, 416, 32, 16, "fp32"),     # register kernel, stabilizer tile alone
    (200, 320, 288, 16, 0, "bf16"),      # width 16
    (200, 320, 288, 0, 48, "bf16"),
    (130, 384, 320, 48, 32, "bf16"),     # width 80: register kernel, six tiles
    (96, 256, 512, 64, 48, "bf16"),      # width 112: eight tiles
    (640, 1056, 1056, 16, 32, "bf16"),   # width 48 with split reductions
    (33, 64, 96, 0, 32, "bf16"),
    # more than 256 LoRA-gradient tiles (N = 16384): four row ranges and their reduction
    (1024, 16384, 512, 32, 32, "bf16"),
]


@pytest.mark.parametrize("m,n,k,r,s,xdt", CASES)
def test_small_cases(m, n, k, r, s, xdt):
    log(f"linear m={m} n={n} k={k} r={r} s={s} x={xdt}")
    d = wl.random_linear(m, n, k, r, s, seed=m + n + k, x_dtype=xdt, dy_dtype=xdt)
    _check_full(d, _run(d))


ROW_SPLIT_CASES = [
    # m >= 4096 with rank + stab_rank above 64: the row-split quantize + down-projection
    # (128 rows per workgroup, a ring of stages shared by its four waves)
    (16400, 256, 416, 64, 32, "bf16"),   # width 96; last stripe 16 rows, last chunk half past K
    (16384, 256, 1056, 64, 64, "bf16"),  # width 128 in two column ranges (128 stripes)
    (16416, 320, 288, 48, 32, "bf16"),   # width 80: a padding tile
    (16390, 256, 256, 64, 48, "bf16"),   # width 112: a padding tile, a 6-row last stripe
    (16384, 256, 1024, 64, 64, "fp32"),  # fp32 input: the register kernel, two ranges
    (4100, 256, 2080, 64, 32, "bf16"),   # 33 stripes in 4 column ranges of 9 chunks (odd)
    (4100, 256, 320, 0, 96, "bf16"),     # width 96 from the stabilizer alone (empty first factor)
    (4100, 256, 320, 96, 0, "bf16"),     # width 96 from LoRA alone (empty second factor)
]


@pytest.mark.parametrize("m,n,k,r,s,xdt", ROW_SPLIT_CASES)
def test_row_split_cases(m, n, k, r, s, xdt):
    log(f"linear m={m} n={n} k={k} r={r} s={s} x={xdt} (row-split range)")
    d = wl.random_linear(m, n, k, r, s, seed=m + n + k + 1, x_dtype=xdt, dy_dtype=xdt)
    _check_full(d, _run(d))


@pytest.mark.parametrize("n,k", [(512, 16384), (16384, 512)])
def test_longest_reductions(n, k):
    """The longest reductions this build accepts (16384 elements: the forward's over K,
    the backward's over N), where the GEMMs stage the most block scales, against the
    whole oracle."""
    log(f"linear m=96 n={n} k={k} r=16 s=16 (longest reduction)")
    d = wl.random_linear(96, n, k, 16, 16, seed=n + 3 * k)
    _check_full(d, _run(d))


def _nan(shape, dtype=torch.float32):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def test_empty_batch():
    """m = 0: nothing is read, the calls succeed, and the LoRA gradients of the empty
    batch are zero (every backward entry point), not left as they were."""
    d = wl.random_linear(64, 256, 320, 32, 16, seed=5)
    L = _gpu_linear(d)
    n, k, r, rt = 256, 320, 32, 48
    x, dy = torch.empty((0, k), dtype=torch.bfloat16, device="cuda"), torch.empty((0, n), dtype=torch.bfloat16,
                                                                                  device="cuda")
    y, xl, dx = torch.empty((0, n), device="cuda"), torch.empty((0, rt), dtype=torch.bfloat16, device="cuda"), \
        torch.empty((0, k), device="cuda")
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(64, L))
    abi.fourtune_linear_fwd(L, x, y, xl, ws)
    for name, call in (
            ("linear_bwd", lambda da, db: abi.fourtune_linear_bwd(L, dy, x, xl, dx, da, db, ws)),
            ("linear_bwd_unfused", lambda da, db: abi.fourtune_linear_bwd_unfused(L, dy, x, xl, dx, da, db, ws)),
            ("linear_bwd_prec W4A4G16", lambda da, db: abi.fourtune_linear_bwd_prec(L, "W4A4G16", dy, x, xl, dx, da,
                                                                                     db, ws))):
        da, db = _nan((r, k)), _nan((n, r))
        call(da, db)
        torch.cuda.synchronize()
        log(f"  {name}: m = 0")
        assert torch.equal(da, torch.zeros_like(da)) and torch.equal(db, torch.zeros_like(db)), name


def test_bf16_outputs():
    log("linear bf16 outputs")
    d = wl.random_linear(300, 544, 384, 32, 32, seed=9)
    _check_full(d, _run(d, out_dtype=torch.bfloat16), out_bf16=True)


def test_c1_tiny_layer():
    log("linear c1")
    d = wl.linear_case("c1")
    _check_full(d, _run(d))


def test_c2_attention_projection():
    log("linear c2 (full size, full oracle), fp32 outputs")
    d = wl.linear_case("c2")
    _check_full(d, _run(d))


def test_c2_attention_projection_bf16_outputs():
    """c2 in the launch configuration the benchmark times (bf16 Y and dX), against the
    full oracle."""
    log("linear c2 (full size, full oracle), bf16 outputs")
    d = wl.linear_case("c2")
    _check_full(d, _run(d, out_dtype=torch.bfloat16), out_bf16=True)


def test_deterministic():
    d = wl.random_linear(300, 544, 384, 32, 32, seed=5)
    a, b = _run(d), _run(d)
    for key in ("Y", "XL", "dX", "dA", "dB"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("xdt", ["bf16", "fp32"])  # staged / register quantize kernels
def test_split_reductions_any_workspace_and_graph_replay(xdt):
    """The split reductions (fused quantize + down-projection over column ranges, LoRA
    gradients over row ranges) keep their fp32 partials in the workspace. Whatever the
    workspace held before (all-ones bytes, random bytes, the previous call's state) the
    bits come out the same, and so do replays of a captured graph with eager calls on
    the same workspace between them."""
    m, n, k = 1024, 3072, 3072  # 16 row stripes x 6 column ranges, 96 tiles x 2 row ranges
    log(f"linear split reductions m={m} n={n} k={k} x={xdt}: workspace contents, graph replay")
    d = wl.random_linear(m, n, k, 32, 32, seed=21, x_dtype=xdt, dy_dtype=xdt)
    L = _gpu_linear(d)
    x, dy = dev(d["X"], d["x_dtype"]), dev(d["dY"], d["dy_dtype"])
    xq, gq = abi.Mx4.empty(m, k), abi.Mx4.empty(m, n)
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))

    def step():
        y, xl = abi.linear_forward(L, x, y_dtype=torch.float32, ws=ws, xq_out=xq)
        dx, da, db = abi.linear_backward(L, dy, x, xl, dx_dtype=torch.float32, ws=ws, gq_out=gq)
        return dict(Y=y, XL=xl, dX=dx, dA=da, dB=db)

    def fetch(o):
        torch.cuda.synchronize()
        got = {key: host(t) for key, t in o.items()}
        got["xq"] = (host_u8(xq.codes), host_u8(xq.scales))
        got["gq"] = (host_u8(gq.codes), host_u8(gq.scales))
        return got

    def same(a, b, what):
        for key in ("Y", "XL", "dX", "dA", "dB"):
            assert np.array_equal(a[key], b[key]), (what, key)

    ws.fill_(0xFF)
    ref = fetch(step())
    _check_full(d, ref)
    same(ref, fetch(step()), "second call, same workspace")
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    same(ref, fetch(step()), "random workspace bytes")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        g.replay()
        same(ref, fetch(outs), f"graph replay {rep}")
        same(ref, fetch(step()), f"eager call after replay {rep}")


def test_workspace_and_argument_errors():
    d = wl.random_linear(64, 256, 256, 16, 16, seed=3)
    L = _gpu_linear(d)
    x = dev(d["X"])
    y = torch.empty((64, 256), dtype=torch.float32, device="cuda")
    xl = torch.empty((64, 32), dtype=torch.bfloat16, device="cuda")
    small = abi.workspace(64)
    with pytest.raises(abi.FourTuneError) as e:
        abi.fourtune_linear_fwd(L, x, y, xl, small)
    assert e.value.name == "FT_ERR_WORKSPACE"
    ws = abi.workspace(abi.fourtune_linear_workspace_bytes(64, L))
    with pytest.raises(ValueError):  # the binding checks every tensor before the call
        abi.fourtune_linear_fwd(L, x, y, None, ws)
    with pytest.raises(ValueError):
        abi.fourtune_linear_fwd(L, x[:, 1:], y, xl, ws)
    # the library's own checks, reached with raw pointers
    s = L.struct()
    lib = abi.lib()
    st = lib.fourtune_linear_fwd(ctypes.byref(s), abi._ptr(x), abi.FT_BF16, 64, abi._ptr(y), abi.FT_F32, None,
                                 None, abi._ptr(ws), ws.numel(), None)
    assert abi.STATUS[st] == "FT_ERR_NULL"
    st = lib.fourtune_linear_fwd(ctypes.byref(s), ctypes.c_void_p(x.data_ptr() + 2), abi.FT_BF16, 64, abi._ptr(y),
                                 abi.FT_F32, abi._ptr(xl), None, abi._ptr(ws), ws.numel(), None)
    assert abi.STATUS[st] == "FT_ERR_ALIGN"


def test_gemm_entry_points():
    """fourtune_gemm_fwd / fourtune_gemm_bwd on their own: the forward GEMM given Q(X)
    and XL reproduces linear_fwd's Y bitwise; the backward GEMM given Q(dY) and a GB
    drawn on the host matches the oracle's 4-bit product plus GB [A;L1]."""
    log("gemm entry points m=300 n=544 k=384 r=32 s=32")
    d = wl.random_linear(300, 544, 384, 32, 32, seed=21)
    L = _gpu_linear(d)
    x = dev(d["X"])
    y_ref, xl = abi.linear_forward(L, x, y_dtype=torch.float32)
    xq = abi.quantize(x)
    y = torch.empty_like(y_ref)
    abi.fourtune_gemm_fwd(L, xq, xl, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)

    rng = np.random.default_rng(22)
    GB = wl.to_dtype(rng.standard_normal((300, 64)) * 1e-2, "bf16")
    gq = abi.quantize(dev(d["dY"]))
    dx = torch.empty((300, 384), dtype=torch.float32, device="cuda")
    abi.fourtune_gemm_bwd(L, gq, dev(GB), dx)
    torch.cuda.synchronize()
    lin = _oracle_linear(d)
    want = mx4.fake_quant(d["dY"].astype(np.float64)) @ mx4.fake_quant(lin.R) + GB.astype(np.float64) @ lin.D()
    e = rel_fro(host(dx), want)
    log(f"  gemm_bwd rel error {e:.3g}")
    assert e <= TOL
