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
