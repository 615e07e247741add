"""fourtune_linear_fwd_noalloc (no workspace argument; the library allocates nothing and
keeps the split reduction's partial sums in its own device array) against
fourtune_linear_fwd on the same inputs: Q(X) codes and scales bit for bit, XL and Y
identical, on two calls in a row whose second has a smaller input (the array then still
holds the first call's partial sums), for both quantize + down-projection kernels."""
import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from synth import workloads as wl
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu


def _pair(d, out_dtype):
    m, n, k = d["X"].shape[0], d["R"].shape[0], d["R"].shape[1]
    rt = d["A"].shape[0] + d["L1"].shape[0]
    L = abi.make_linear(dev(d["R"], "fp32"), dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))
    x = dev(d["X"], d["x_dtype"])
    outs = []
    for noalloc in (False, True):
        y = torch.full((m, n), float("nan"), dtype=out_dtype, device="cuda")
        xl = torch.full((m, rt), float("nan"), dtype=torch.bfloat16, device="cuda")
        xq = abi.Mx4.empty(m, k)
        xq.codes.fill_(0xAA)
        xq.scales.fill_(0xAA)
        if noalloc:
            abi.fourtune_linear_fwd_noalloc(L, x, y, xl, xq)
        else:
            ws = abi.workspace(abi.fourtune_linear_workspace_bytes(m, L))
            abi.fourtune_linear_fwd(L, x, y, xl, ws, xq_out=xq)
        outs.append((y, xl, xq))
    torch.cuda.synchronize()
    (y0, xl0, q0), (y1, xl1, q1) = outs
    assert torch.equal(q0.scales, q1.scales) and torch.equal(q0.codes, q1.codes), "Q(X)"
    assert torch.equal(xl0, xl1), "XL"
    assert torch.equal(y0, y1), "Y"
    assert not torch.isnan(y1.float()).any()


@pytest.mark.parametrize("xdt,out_dtype", [("bf16", torch.bfloat16), ("fp32", torch.float32)])
def test_noalloc_forward_equals_workspace_forward(xdt, out_dtype):
    # first a c2-sized call (three column ranges: partial sums in the array), then a
    # smaller one with another split and rank
    log(f"noalloc forward: m=4608 n=k=3072 r=s=32 x={xdt}")
    d = wl.random_linear(4608, 3072, 3072, 32, 32, seed=41, x_dtype=xdt, dy_dtype=xdt)
    _pair(d, out_dtype)
    log(f"noalloc forward: m=600 n=1120 k=1088 r=s=16 x={xdt}")
    d = wl.random_linear(600, 1120, 1088, 16, 16, seed=42, x_dtype=xdt, dy_dtype=xdt)
    _pair(d, out_dtype)


def test_noalloc_forward_largest_partials():
    """Width 128 over 72 row stripes of 128 rows takes three column ranges: partial
    sums near the largest the array holds for rank + stab_rank <= 128 (14 MiB here, at
    most 16 MiB), then a smaller call on the same array."""
    log("noalloc forward: m=9216 n=256 k=8192 r=s=64 (three ranges)")
    d = wl.random_linear(9216, 256, 8192, 64, 64, seed=44, x_dtype="bf16", dy_dtype="bf16")
    _pair(d, torch.bfloat16)
    log("noalloc forward: m=600 n=1120 k=1088 r=32 s=64")
    d = wl.random_linear(600, 1120, 1088, 32, 64, seed=45, x_dtype="bf16", dy_dtype="bf16")
    _pair(d, torch.float32)


def test_noalloc_argument_errors():
    d = wl.random_linear(64, 256, 256, 16, 16, seed=43)
    L = abi.make_linear(dev(d["R"], "fp32"), dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))
    x = dev(d["X"])
    y = torch.empty((64, 256), dtype=torch.float32, device="cuda")
    xl = torch.empty((64, 32), dtype=torch.bfloat16, device="cuda")
    s = L.struct()
    import ctypes
    st = abi.lib().fourtune_linear_fwd_noalloc(ctypes.byref(s), abi._ptr(x), abi.FT_BF16, 64, abi._ptr(y),
                                               abi.FT_F32, abi._ptr(xl), None, None)
    assert abi.STATUS[st] == "FT_ERR_NULL" and "xq_out" in abi.fourtune_last_error()
