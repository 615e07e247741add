"""GPU parity of fourtune_quantize_groups (1x32 groups) against the oracle's group
quantizer: codes and scales bit-exact, over ragged shapes, both input types, strided
rows, random bit patterns (every exponent, subnormals, signed zeros) and non-finite
groups, and the c4 activation at full size."""
import numpy as np
import pytest
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import mx4
from synth import workloads as wl
from tests.gpu_util import dev, host_u8, log

pytestmark = pytest.mark.gpu


def _check(T: np.ndarray, dtype: str, ld_pad: int = 0, name: str = ""):
    log(f"quantize_groups {name} {T.shape} {dtype} ld_pad={ld_pad}")
    rows, cols = T.shape
    if ld_pad:
        big = np.zeros((rows, cols + ld_pad), dtype=np.float32)
        big[:, :cols] = T
        x = dev(big, dtype)[:, :cols]
    else:
        x = dev(T, dtype)
    q = abi.Mx4.empty_groups(rows, cols)
    abi.fourtune_quantize_groups(x, q)
    torch.cuda.synchronize()
    wc, ws = mx4.quantize_groups(T)
    got_c, got_s = host_u8(q.codes), host_u8(q.scales)
    assert np.array_equal(got_s, ws), f"scales differ at {np.argwhere(got_s != ws)[:5]}"
    assert np.array_equal(got_c, mx4.pack_codes(wc)), "codes differ"


@pytest.mark.parametrize("rows,cols", [(1, 32), (31, 64), (100, 160), (257, 544), (96, 2080)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_group_ragged_shapes(rows, cols, dtype):
    rng = np.random.default_rng(rows * 5 + cols)
    T = wl.to_dtype(rng.standard_normal((rows, cols)) * np.ldexp(1.0, rng.integers(-8, 8, (rows, 1))), dtype)
    _check(T, dtype, name="ragged")


def test_group_strided_rows():
    rng = np.random.default_rng(4)
    T = wl.to_dtype(rng.standard_normal((70, 256)), "bf16")
    _check(T, "bf16", ld_pad=64, name="strided")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_group_random_bit_patterns(dtype):
    rng = np.random.default_rng(12)
    rows, cols = 96, 512
    if dtype == "bf16":
        bits = rng.integers(0, 1 << 16, (rows, cols), dtype=np.uint32) << 16
    else:
        bits = rng.integers(0, 1 << 32, (rows, cols), dtype=np.uint64).astype(np.uint32)
    exp_band = rng.integers(0, 255, (rows, 1))
    bits = (bits & 0x807FFFFF) | (np.minimum(exp_band + rng.integers(0, 6, (rows, cols)), 254).astype(np.uint32) << 23)
    T = bits.view(np.float32).copy()
    T[0, :32] = 0.0
    T[1, 32] = -0.0
    T[2, 64] = np.nan
    T[3, 100] = -np.inf
    if dtype == "bf16":
        T = wl.to_dtype(T, "bf16")
    _check(T, dtype, name="bits")


def test_group_c4_activation_full_size():
    d = wl.linear_case("c4", "qkv")
    _check(d["X"], d["x_dtype"], name="c4 X")
