"""The LoRA gradients' row-range sum in the backward GEMM's launch.

The fused linear backward runs the LoRA gradients (FourTune §3.2: parameter updates
for the adapter only) before the transposed GEMM and lets extra workgroups of that
GEMM's launch add the gradients' row-range partials. The fusion-ablation backward runs
the same gradient kernel and adds the partials with a launch of its own; both add the
ranges in range order from the same partials, so dA and dB must agree bit for bit.

Shapes: the GEMM's tiles (256 x 256 over M x K) leaving most CUs idle (the extra
workgroups run beside the tiles), exactly 256 tiles (none idle: the extra workgroups
start as tiles finish), the 128-column gradient tiles used from 8192 rows, and fp32 X
with bf16 dY (the dA and dB tiles are then two launches sharing one sum). rank +
stab_rank <= 64 keeps both backward forms on the same down-projection kernel, so GB,
and with it the partials, are identical.
The values themselves are checked against the oracle by the linear parity tests.
"""
import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from synth import workloads as wl
from tests.gpu_util import dev, log
from tests.sampling import _gpu_lin

pytestmark = pytest.mark.gpu

CASES = [
    # m, n, k, r, s, x dtype: the backward GEMM's tiles (m/256 x k/256) and the gradient split
    (1024, 1024, 1024, 32, 32, "bf16"),   # 16 tiles, 240 CUs idle; 6 row ranges
    (2048, 512, 8192, 32, 32, "bf16"),    # 256 tiles, none idle; 2 row ranges
    (8192, 512, 1024, 32, 32, "bf16"),    # 128-column gradient tiles (from 8192 rows)
    (1024, 512, 768, 16, 16, "fp32"),     # fp32 X, bf16 dY: dA and dB tiles in two launches
]


@pytest.mark.parametrize("m,n,k,r,s,xdt", CASES)
def test_lora_sum_in_gemm_launch_matches_own_launch(m, n, k, r, s, xdt):
    log(f"lora-gradient sum in the GEMM launch: m={m} n={n} k={k} r={r} s={s} x={xdt}")
    d = wl.random_linear(m, n, k, r, s, seed=7 + m + k, x_dtype=xdt)
    L = _gpu_lin(d)
    x, dy = dev(d["X"], xdt), dev(d["dY"])
    _, xl = abi.linear_forward(L, x)
    dx, da, db = abi.linear_backward(L, dy, x, xl)

    ws = abi.workspace(abi.fourtune_ablation_workspace_bytes(m, L))
    dx_u = torch.empty_like(dx)
    da_u, db_u = torch.empty_like(da), torch.empty_like(db)
    abi.fourtune_linear_bwd_unfused(L, dy, x, xl, dx_u, da_u, db_u, ws)
    torch.cuda.synchronize()
    for name, a, b in (("dA", da, da_u), ("dB", db, db_u)):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        diff = int(np.count_nonzero(a.view(np.uint32) != b.view(np.uint32)))
        log(f"  {name}: {diff} of {a.size} differ")
        assert np.all(np.isfinite(a)) and np.abs(a).max() > 0, name
        assert diff == 0, name
