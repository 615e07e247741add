"""Host-side checks of the C ABI library (no GPU needed).

The library must load, export every function include/fourtune.h declares, and reject
bad arguments before touching the GPU.
"""
import ctypes
import os
import re

import pytest

from bit_quantized_lora_fp4_amd import abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "fourtune.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ["fourtune_quantize", "fourtune_linear_fwd", "fourtune_linear_bwd",
                 "fourtune_mlp_fwd", "fourtune_mlp_bwd", "fourtune_linear_workspace_bytes",
                 "fourtune_mlp_workspace_bytes", "ft_mx4_codes_bytes", "ft_mx4_scales_bytes",
                 "fourtune_status_string", "fourtune_last_error"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(abi.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert sorted(abi.exported_symbols()) == _declared_functions()


def test_size_helpers():
    assert abi.ft_mx4_codes_bytes(4608, 3072) == 4608 * 1536
    assert abi.ft_mx4_scales_bytes(4608, 3072) == 144 * 96
    assert abi.ft_mx4_scales_bytes(32760, 5120) == 1024 * 160  # partial last block row
    assert abi.ft_mx4_codes_bytes(0, 64) == 0


def test_status_strings():
    assert abi.fourtune_status_string(0) == "ok"
    assert abi.fourtune_status_string(5) == "workspace too small"


def _q(x_ptr, dt, rows, cols, ld, out):
    L = abi.lib()
    return L.fourtune_quantize(x_ptr, dt, rows, cols, ld, ctypes.byref(out) if out else None, None)


def test_quantize_validation_before_launch():
    out = abi.FtMx4(ctypes.c_void_p(4096), ctypes.c_void_p(8192), 64, 64)
    x = ctypes.c_void_p(1 << 20)
    assert _q(x, 7, 64, 64, 64, out) == 3                      # unknown dtype
    assert _q(x, abi.FT_BF16, 64, 48, 48, out) == 2            # cols % 32
    assert _q(x, abi.FT_BF16, 64, 64, 32, out) == 2            # ld < cols
    assert _q(x, abi.FT_BF16, 64, 64, 68, out) == 4            # row stride not 16 B
    assert _q(None, abi.FT_BF16, 64, 64, 64, out) == 1         # NULL x
    assert _q(ctypes.c_void_p((1 << 20) + 2), abi.FT_BF16, 64, 64, 64, out) == 4
    assert _q(x, abi.FT_BF16, 64, 64, 64, None) == 1           # NULL out
    bad = abi.FtMx4(ctypes.c_void_p(4096), ctypes.c_void_p(8192), 32, 64)
    assert _q(x, abi.FT_BF16, 64, 64, 64, bad) == 2            # out shape mismatch
    assert "rows" in abi.fourtune_last_error() or "expected" in abi.fourtune_last_error()
    assert _q(None, abi.FT_BF16, 0, 64, 64, None) == 0         # empty: no-op


def _fake_linear(n=256, k=256, r=16, s=16, codes=4096):
    rq = abi.FtMx4(ctypes.c_void_p(codes), ctypes.c_void_p(codes + (1 << 20)), n, k)
    p = ctypes.c_void_p(1 << 24)
    return abi.FtLinear(rq, p, p, p, p, n, k, r, s)


def test_new_entry_points_validate_before_launch():
    """The ablation, precision and group-quantizer entry points reject bad arguments
    with FT_ERR_* codes before touching the GPU (fake device addresses are never used)."""
    L = abi.lib()
    lin = _fake_linear()
    x, y, xl, ws = (ctypes.c_void_p(1 << 26), ctypes.c_void_p(1 << 27), ctypes.c_void_p(1 << 28),
                    ctypes.c_void_p(1 << 29))
    # precision variants: unknown configuration, NULL input, small workspace, bad dtype
    assert L.fourtune_linear_fwd_prec(ctypes.byref(lin), 9, x, abi.FT_BF16, 64, y, abi.FT_BF16, xl, ws, 1 << 30,
                                      None) == 6
    assert L.fourtune_linear_fwd_prec(ctypes.byref(lin), 1, None, abi.FT_BF16, 64, y, abi.FT_BF16, xl, ws, 1 << 30,
                                      None) == 1
    assert L.fourtune_linear_bwd_prec(ctypes.byref(lin), 3, x, abi.FT_BF16, x, abi.FT_BF16, xl, 64, y, abi.FT_BF16,
                                      y, y, ws, 16, None) == 5
    assert L.fourtune_linear_fwd_prec(ctypes.byref(lin), 1, x, 5, 64, y, abi.FT_BF16, xl, ws, 1 << 30, None) == 3
    # unfused linear: misaligned input, NULL saved XL, workspace too small
    assert L.fourtune_linear_fwd_unfused(ctypes.byref(lin), ctypes.c_void_p((1 << 26) + 8), abi.FT_BF16, 64, y,
                                         abi.FT_BF16, xl, ws, 1 << 30, None) == 4
    assert L.fourtune_linear_fwd_unfused(ctypes.byref(lin), x, abi.FT_BF16, 64, y, abi.FT_BF16, None, ws, 1 << 30,
                                         None) == 1
    assert L.fourtune_linear_bwd_unfused(ctypes.byref(lin), x, abi.FT_BF16, x, abi.FT_BF16, xl, 64, y, abi.FT_BF16,
                                         y, y, ws, 16, None) == 5
    # unfused MLP: fc1's outputs must match fc2's inputs
    fc2 = _fake_linear(n=256, k=512)
    assert L.fourtune_mlp_fwd_unfused(ctypes.byref(lin), ctypes.byref(fc2), 0, x, abi.FT_BF16, 64, y, abi.FT_BF16,
                                      xl, y, y, xl, ws, 1 << 30, None) == 2
    # ranks that are not multiples of 16
    odd = _fake_linear(r=8, s=24)
    assert L.fourtune_linear_fwd_prec(ctypes.byref(odd), 1, x, abi.FT_BF16, 64, y, abi.FT_BF16, xl, ws, 1 << 30,
                                      None) == 2
    # multiples of 16 wider than 128 in all: valid layers the fused kernels are not built for
    for r, s in ((64, 80), (128, 16), (0, 144)):
        wide = _fake_linear(r=r, s=s)
        assert L.fourtune_linear_fwd(ctypes.byref(wide), x, abi.FT_BF16, 64, y, abi.FT_BF16, xl, None, ws,
                                     1 << 30, None) == 6, (r, s)
        assert "> 128" in abi.fourtune_last_error()
        assert L.fourtune_mlp_bwd(ctypes.byref(wide), ctypes.byref(_fake_linear(n=256, k=256)), x, abi.FT_BF16, x,
                                  abi.FT_BF16, xl, y, xl, 64, y, abi.FT_BF16, y, y, y, y, None, None, ws, 1 << 30,
                                  None) == 6
    # group quantizer: as the block quantizer
    out = abi.FtMx4(ctypes.c_void_p(4096), ctypes.c_void_p(8192), 64, 64)
    assert L.fourtune_quantize_groups(x, abi.FT_BF16, 64, 48, 48, ctypes.byref(out), None) == 2
    assert L.fourtune_quantize_groups(None, abi.FT_BF16, 64, 64, 64, ctypes.byref(out), None) == 1
    assert L.fourtune_quantize_groups(None, abi.FT_BF16, 0, 64, 64, None, None) == 0
    # workspace sizes are well defined without a GPU
    assert abi.fourtune_ablation_workspace_bytes(4608, abi.Linear(
        abi.Mx4(None, None, 3072, 3072), *[_FakeT((32, 3072))] * 4)) > 0


class _FakeT:
    """Stand-in for a tensor in the workspace-size query (only its shape is read)."""

    def __init__(self, shape):
        self.shape = shape
        self.is_cuda = True

    def data_ptr(self):
        return 1 << 24
