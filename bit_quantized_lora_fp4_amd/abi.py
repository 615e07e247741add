"""ctypes binding of libfourtune.so (the C ABI declared in include/fourtune.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream. Functions named like the
C entry points take preallocated tensors; the short helpers below them allocate
outputs and workspace with torch and call those.

If the library is missing or cannot load, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfourtune.so")

FT_F32, FT_BF16 = 0, 1
STATUS = {0: "FT_OK", 1: "FT_ERR_NULL", 2: "FT_ERR_SHAPE", 3: "FT_ERR_DTYPE", 4: "FT_ERR_ALIGN",
          5: "FT_ERR_WORKSPACE", 6: "FT_ERR_UNSUPPORTED", 7: "FT_ERR_HIP"}

c_i64, c_vp, c_sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class FtMx4(ctypes.Structure):
    _fields_ = [("codes", c_vp), ("scales", c_vp), ("rows", c_i64), ("cols", c_i64)]


class FtLinear(ctypes.Structure):
    _fields_ = [("r", FtMx4), ("lora_a", c_vp), ("lora_b", c_vp), ("stab_down", c_vp),
                ("stab_up", c_vp), ("n", c_i64), ("k", c_i64), ("rank", c_i64),
                ("stab_rank", c_i64)]


class FourTuneError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.name = STATUS.get(status, str(status))
        self.detail = detail


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "ft_mx4_codes_bytes": (c_sz, [c_i64, c_i64]),
    "ft_mx4_scales_bytes": (c_sz, [c_i64, c_i64]),
    "fourtune_quantize": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64,
                                         ctypes.POINTER(FtMx4), c_vp]),
    "fourtune_quantize_groups": (ctypes.c_int, [c_vp, ctypes.c_int, c_i64, c_i64, c_i64,
                                                ctypes.POINTER(FtMx4), c_vp]),
    "fourtune_linear_workspace_bytes": (c_sz, [c_i64, ctypes.POINTER(FtLinear)]),
    "fourtune_linear_fwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), c_vp, ctypes.c_int, c_i64,
                                           c_vp, ctypes.c_int, c_vp, ctypes.POINTER(FtMx4),
                                           c_vp, c_sz, c_vp]),
    "fourtune_linear_bwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), c_vp, ctypes.c_int, c_vp,
                                           ctypes.c_int, c_vp, c_i64, c_vp, ctypes.c_int, c_vp,
                                           c_vp, ctypes.POINTER(FtMx4), c_vp, c_sz, c_vp]),
    "fourtune_gemm_fwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtMx4), c_vp,
                                         c_i64, c_vp, ctypes.c_int, c_vp]),
    "fourtune_gemm_bwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtMx4), c_vp,
                                         c_i64, c_vp, ctypes.c_int, c_vp]),
    "fourtune_mlp_workspace_bytes": (c_sz, [c_i64, ctypes.POINTER(FtLinear),
                                            ctypes.POINTER(FtLinear)]),
    "fourtune_mlp_fwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear), c_vp,
                                        ctypes.c_int, c_i64, c_vp, ctypes.c_int, c_vp, c_vp, c_vp,
                                        ctypes.POINTER(FtMx4), c_vp, c_vp, c_sz, c_vp]),
    "fourtune_mlp_bwd": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear), c_vp,
                                        ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_vp, c_vp, c_i64,
                                        c_vp, ctypes.c_int, c_vp, c_vp, c_vp, c_vp,
                                        ctypes.POINTER(FtMx4), c_vp, c_vp, c_sz, c_vp]),
    "fourtune_ablation_workspace_bytes": (c_sz, [c_i64, ctypes.POINTER(FtLinear),
                                                 ctypes.POINTER(FtLinear)]),
    "fourtune_linear_fwd_unfused": (ctypes.c_int, [ctypes.POINTER(FtLinear), c_vp, ctypes.c_int,
                                                   c_i64, c_vp, ctypes.c_int, c_vp, c_vp, c_sz,
                                                   c_vp]),
    "fourtune_linear_bwd_unfused": (ctypes.c_int, [ctypes.POINTER(FtLinear), c_vp, ctypes.c_int,
                                                   c_vp, ctypes.c_int, c_vp, c_i64, c_vp,
                                                   ctypes.c_int, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "fourtune_mlp_fwd_unfused": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear),
                                                ctypes.c_int, c_vp, ctypes.c_int, c_i64, c_vp,
                                                ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                                c_vp]),
    "fourtune_mlp_bwd_unfused": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.POINTER(FtLinear),
                                                ctypes.c_int, c_vp, ctypes.c_int, c_vp,
                                                ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp,
                                                ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                                c_vp]),
    "fourtune_linear_fwd_prec": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.c_int, c_vp,
                                                ctypes.c_int, c_i64, c_vp, ctypes.c_int, c_vp, c_vp,
                                                c_sz, c_vp]),
    "fourtune_linear_bwd_prec": (ctypes.c_int, [ctypes.POINTER(FtLinear), ctypes.c_int, c_vp,
                                                ctypes.c_int, c_vp, ctypes.c_int, c_vp, c_i64, c_vp,
                                                ctypes.c_int, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "fourtune_linear_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(FtLinear), c_vp, ctypes.c_int, c_i64, c_vp,
                                                   ctypes.c_int, c_vp, ctypes.POINTER(FtMx4), c_vp]),
    "fourtune_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fourtune_last_error": (ctypes.c_char_p, []),
}


def lib():
    """Load libfourtune.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FourTuneError(-1, f"{LIB_PATH} is not built; run "
                                    "`python -m bit_quantized_lora_fp4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(status: int):
    if status != 0:
        raise FourTuneError(status, lib().fourtune_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FT_F32
    if t.dtype == torch.bfloat16:
        return FT_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------- argument checks
# The C side sees raw pointers and sizes only, so the shape, dtype and layout of every
# tensor argument are checked here, before any pointer is taken.
_F32_BF16 = (torch.float32, torch.bfloat16)
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _need(t, name: str, shape, dtypes, optional: bool = False):
    """t must be a contiguous tensor of `shape` and one of `dtypes` (or None when
    `optional`)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_mx4(q, name: str, rows: int, cols: int, optional: bool = False, groups: bool = False):
    if q is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(q, Mx4):
        raise TypeError(f"{name} must be an Mx4")
    if (q.rows, q.cols) != (rows, cols):
        raise ValueError(f"{name} is [{q.rows} x {q.cols}], expected [{rows} x {cols}]")
    _need(q.codes, f"{name}.codes", (rows, cols // 2), _U8)
    _need(q.scales, f"{name}.scales", (rows if groups else (rows + 31) // 32, cols // 32), _U8)


def _need_linear(L, name: str = "L"):
    if not isinstance(L, Linear):
        raise TypeError(f"{name} must be a Linear")
    n, k = L.rq.rows, L.rq.cols
    _need_mx4(L.rq, f"{name}.rq", n, k)
    for t, nm in ((L.A, "A"), (L.B, "B"), (L.L1, "L1"), (L.L2, "L2")):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError(f"{name}.{nm} must be a 2-D tensor")
    r, s = L.A.shape[0], L.L1.shape[0]
    _need(L.A, f"{name}.A", (r, k), _BF16)
    _need(L.B, f"{name}.B", (n, r), _BF16)
    _need(L.L1, f"{name}.L1", (s, k), _BF16)
    _need(L.L2, f"{name}.L2", (n, s), _BF16)


def _rt(L) -> int:
    return L.A.shape[0] + L.L1.shape[0]


def _need_low(t, name: str, m: int, rt: int):
    """A saved [m x rt] bf16 low-rank activation (may be omitted when rt is 0)."""
    _need(t, name, (m, rt), _BF16, optional=rt == 0)


def _need_ws(ws):
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous 1-D uint8 tensor")


def _need_linear_fwd(L, x, y, xl_saved, ws):
    _need_linear(L)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, L.k), _F32_BF16)
    _need(y, "y", (m, L.n), _F32_BF16)
    _need_low(xl_saved, "xl_saved", m, _rt(L))
    _need_ws(ws)


def _need_linear_bwd(L, dy, x, xl_saved, dx, d_lora_a, d_lora_b, ws):
    _need_linear(L)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, L.k), _F32_BF16)
    _need(dy, "dy", (m, L.n), _F32_BF16)
    _need_low(xl_saved, "xl_saved", m, _rt(L))
    _need(dx, "dx", (m, L.k), _F32_BF16)
    _need(d_lora_a, "d_lora_a", (L.rank, L.k), _F32, optional=L.rank == 0)
    _need(d_lora_b, "d_lora_b", (L.n, L.rank), _F32, optional=L.rank == 0)
    _need_ws(ws)


def _need_mlp(fc1, fc2):
    _need_linear(fc1, "fc1")
    _need_linear(fc2, "fc2")
    if fc1.n != fc2.k:
        raise ValueError(f"fc1 has {fc1.n} outputs, fc2 {fc2.k} inputs")


def _need_mlp_bwd(fc1, fc2, m, dy, x, xl1_saved, pre_saved, hl2_saved, dx, d_a1, d_b1, d_a2, d_b2):
    _need(x, "x", (m, fc1.k), _F32_BF16)
    _need(dy, "dy", (m, fc2.n), _F32_BF16)
    _need_low(xl1_saved, "xl1_saved", m, _rt(fc1))
    _need(pre_saved, "pre_saved", (m, fc1.n), _BF16)
    _need_low(hl2_saved, "hl2_saved", m, _rt(fc2))
    _need(dx, "dx", (m, fc1.k), _F32_BF16)
    _need(d_a1, "d_a1", (fc1.rank, fc1.k), _F32, optional=fc1.rank == 0)
    _need(d_b1, "d_b1", (fc1.n, fc1.rank), _F32, optional=fc1.rank == 0)
    _need(d_a2, "d_a2", (fc2.rank, fc2.k), _F32, optional=fc2.rank == 0)
    _need(d_b2, "d_b2", (fc2.n, fc2.rank), _F32, optional=fc2.rank == 0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------------------- types
@dataclass
class Mx4:
    """An MXFP4 tensor: codes [rows x cols/2] uint8, scales [ceil(rows/32) x cols/32] uint8."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    @staticmethod
    def empty(rows: int, cols: int, device="cuda") -> "Mx4":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty(((rows + 31) // 32, cols // 32), dtype=torch.uint8, device=device)
        return Mx4(codes, scales, rows, cols)

    @staticmethod
    def empty_groups(rows: int, cols: int, device="cuda") -> "Mx4":
        """Storage for the 1x32 group form: scales [rows x cols/32]."""
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=device)
        return Mx4(codes, scales, rows, cols)

    def struct(self) -> FtMx4:
        return FtMx4(_ptr(self.codes), _ptr(self.scales), self.rows, self.cols)


@dataclass
class Linear:
    """One W4A4G4 linear: Q(R) [n x k] and the bf16 low-rank factors A, B, L1, L2."""
    rq: Mx4
    A: torch.Tensor   # [r x k]
    B: torch.Tensor   # [n x r]
    L1: torch.Tensor  # [s x k]
    L2: torch.Tensor  # [n x s]

    @property
    def n(self):
        return self.rq.rows

    @property
    def k(self):
        return self.rq.cols

    @property
    def rank(self):
        return self.A.shape[0]

    @property
    def stab_rank(self):
        return self.L1.shape[0]

    def struct(self) -> FtLinear:
        return FtLinear(self.rq.struct(), _ptr(self.A), _ptr(self.B), _ptr(self.L1),
                        _ptr(self.L2), self.n, self.k, self.rank, self.stab_rank)


# ----------------------------------------------------------------------------- C calls
def ft_mx4_codes_bytes(rows: int, cols: int) -> int:
    return lib().ft_mx4_codes_bytes(rows, cols)


def ft_mx4_scales_bytes(rows: int, cols: int) -> int:
    return lib().ft_mx4_scales_bytes(rows, cols)


def _need_rows(x, name="x"):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    if x.dtype not in _F32_BF16:
        raise ValueError(f"{name} has dtype {x.dtype}, expected one of {list(_F32_BF16)}")
    if x.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")


def fourtune_quantize(x: torch.Tensor, out: Mx4, stream=None, ld: Optional[int] = None):
    _need_rows(x)
    rows, cols = x.shape
    ld = x.stride(0) if ld is None else ld
    _need_mx4(out, "out", rows, cols)
    s = out.struct()
    _check(lib().fourtune_quantize(_ptr(x), _dt(x), rows, cols, ld, ctypes.byref(s),
                                   _stream(stream)))


def fourtune_quantize_groups(x: torch.Tensor, out: Mx4, stream=None, ld: Optional[int] = None):
    """1x32 groups: out.scales must be [rows x cols/32] (see Mx4.empty_groups)."""
    _need_rows(x)
    rows, cols = x.shape
    ld = x.stride(0) if ld is None else ld
    _need_mx4(out, "out", rows, cols, groups=True)
    s = out.struct()
    _check(lib().fourtune_quantize_groups(_ptr(x), _dt(x), rows, cols, ld, ctypes.byref(s),
                                          _stream(stream)))


def fourtune_linear_workspace_bytes(m: int, L: Linear) -> int:
    s = L.struct()
    return lib().fourtune_linear_workspace_bytes(m, ctypes.byref(s))


def fourtune_linear_fwd(L: Linear, x: torch.Tensor, y: torch.Tensor, xl_saved: torch.Tensor,
                        ws: torch.Tensor, xq_out: Optional[Mx4] = None, stream=None):
    _need_linear(L)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, L.k), _F32_BF16)
    _need(y, "y", (m, L.n), _F32_BF16)
    _need_low(xl_saved, "xl_saved", m, _rt(L))
    _need_mx4(xq_out, "xq_out", m, L.k, optional=True)
    _need_ws(ws)
    s = L.struct()
    xq = xq_out.struct() if xq_out is not None else None
    _check(lib().fourtune_linear_fwd(ctypes.byref(s), _ptr(x), _dt(x), x.shape[0], _ptr(y),
                                     _dt(y), _ptr(xl_saved),
                                     ctypes.byref(xq) if xq is not None else None,
                                     _ptr(ws), ws.numel() if ws is not None else 0,
                                     _stream(stream)))


def fourtune_linear_bwd(L: Linear, dy: torch.Tensor, x: torch.Tensor, xl_saved: torch.Tensor,
                        dx: torch.Tensor, d_lora_a: Optional[torch.Tensor],
                        d_lora_b: Optional[torch.Tensor], ws: torch.Tensor,
                        gq_out: Optional[Mx4] = None, stream=None):
    _need_linear(L)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, L.k), _F32_BF16)
    _need(dy, "dy", (m, L.n), _F32_BF16)
    _need_low(xl_saved, "xl_saved", m, _rt(L))
    _need(dx, "dx", (m, L.k), _F32_BF16)
    _need(d_lora_a, "d_lora_a", (L.rank, L.k), _F32, optional=L.rank == 0)
    _need(d_lora_b, "d_lora_b", (L.n, L.rank), _F32, optional=L.rank == 0)
    _need_mx4(gq_out, "gq_out", m, L.n, optional=True)
    _need_ws(ws)
    s = L.struct()
    gq = gq_out.struct() if gq_out is not None else None
    _check(lib().fourtune_linear_bwd(ctypes.byref(s), _ptr(dy), _dt(dy), _ptr(x), _dt(x),
                                     _ptr(xl_saved), x.shape[0], _ptr(dx), _dt(dx),
                                     _ptr(d_lora_a), _ptr(d_lora_b),
                                     ctypes.byref(gq) if gq is not None else None,
                                     _ptr(ws), ws.numel() if ws is not None else 0,
                                     _stream(stream)))


def fourtune_linear_fwd_noalloc(L: Linear, x: torch.Tensor, y: torch.Tensor, xl_saved: torch.Tensor,
                                xq_out: Mx4, stream=None):
    """The forward without a workspace (the library allocates nothing; Q(X) goes to
    xq_out, the split reduction's partial sums to the library's own device array)."""
    _need_linear(L)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, L.k), _F32_BF16)
    _need(y, "y", (m, L.n), _F32_BF16)
    _need_low(xl_saved, "xl_saved", m, _rt(L))
    _need_mx4(xq_out, "xq_out", m, L.k)
    s, q = L.struct(), xq_out.struct()
    _check(lib().fourtune_linear_fwd_noalloc(ctypes.byref(s), _ptr(x), _dt(x), m, _ptr(y), _dt(y), _ptr(xl_saved),
                                             ctypes.byref(q), _stream(stream)))


def fourtune_gemm_fwd(L: Linear, xq: Mx4, xl: Optional[torch.Tensor], y: torch.Tensor,
                      stream=None):
    _need_linear(L)
    if not isinstance(xq, Mx4):
        raise TypeError("xq must be an Mx4")
    _need_mx4(xq, "xq", xq.rows, L.k)
    _need_low(xl, "xl", xq.rows, _rt(L))
    _need(y, "y", (xq.rows, L.n), _F32_BF16)
    s, q = L.struct(), xq.struct()
    _check(lib().fourtune_gemm_fwd(ctypes.byref(s), ctypes.byref(q), _ptr(xl), xq.rows, _ptr(y),
                                   _dt(y), _stream(stream)))


def fourtune_gemm_bwd(L: Linear, gq: Mx4, gb: Optional[torch.Tensor], dx: torch.Tensor,
                      stream=None):
    _need_linear(L)
    if not isinstance(gq, Mx4):
        raise TypeError("gq must be an Mx4")
    _need_mx4(gq, "gq", gq.rows, L.n)
    _need_low(gb, "gb", gq.rows, _rt(L))
    _need(dx, "dx", (gq.rows, L.k), _F32_BF16)
    s, q = L.struct(), gq.struct()
    _check(lib().fourtune_gemm_bwd(ctypes.byref(s), ctypes.byref(q), _ptr(gb), gq.rows, _ptr(dx),
                                   _dt(dx), _stream(stream)))


def fourtune_mlp_workspace_bytes(m: int, fc1: Linear, fc2: Linear) -> int:
    s1, s2 = fc1.struct(), fc2.struct()
    return lib().fourtune_mlp_workspace_bytes(m, ctypes.byref(s1), ctypes.byref(s2))


def fourtune_mlp_fwd(fc1: Linear, fc2: Linear, x: torch.Tensor, y: torch.Tensor,
                     xl1_saved: torch.Tensor, pre_saved: torch.Tensor, hl2_saved: torch.Tensor,
                     ws: torch.Tensor, hq_out: Optional[Mx4] = None,
                     h_debug: Optional[torch.Tensor] = None, stream=None):
    _need_mlp(fc1, fc2)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, fc1.k), _F32_BF16)
    _need(y, "y", (m, fc2.n), _F32_BF16)
    _need_low(xl1_saved, "xl1_saved", m, _rt(fc1))
    _need(pre_saved, "pre_saved", (m, fc1.n), _BF16)
    _need_low(hl2_saved, "hl2_saved", m, _rt(fc2))
    _need_mx4(hq_out, "hq_out", m, fc1.n, optional=True)
    _need(h_debug, "h_debug", (m, fc1.n), _F32, optional=True)
    _need_ws(ws)
    s1, s2 = fc1.struct(), fc2.struct()
    hq = hq_out.struct() if hq_out is not None else None
    _check(lib().fourtune_mlp_fwd(ctypes.byref(s1), ctypes.byref(s2), _ptr(x), _dt(x),
                                  x.shape[0], _ptr(y), _dt(y), _ptr(xl1_saved), _ptr(pre_saved),
                                  _ptr(hl2_saved), ctypes.byref(hq) if hq is not None else None,
                                  _ptr(h_debug), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)))


def fourtune_mlp_bwd(fc1: Linear, fc2: Linear, dy: torch.Tensor, x: torch.Tensor,
                     xl1_saved: torch.Tensor, pre_saved: torch.Tensor, hl2_saved: torch.Tensor,
                     dx: torch.Tensor, d_a1, d_b1, d_a2, d_b2, ws: torch.Tensor,
                     dpq_out: Optional[Mx4] = None, dp_debug: Optional[torch.Tensor] = None,
                     stream=None):
    _need_mlp(fc1, fc2)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need_mlp_bwd(fc1, fc2, m, dy, x, xl1_saved, pre_saved, hl2_saved, dx, d_a1, d_b1, d_a2, d_b2)
    _need_mx4(dpq_out, "dpq_out", m, fc1.n, optional=True)
    _need(dp_debug, "dp_debug", (m, fc1.n), _F32, optional=True)
    _need_ws(ws)
    s1, s2 = fc1.struct(), fc2.struct()
    dq = dpq_out.struct() if dpq_out is not None else None
    _check(lib().fourtune_mlp_bwd(ctypes.byref(s1), ctypes.byref(s2), _ptr(dy), _dt(dy), _ptr(x),
                                  _dt(x), _ptr(xl1_saved), _ptr(pre_saved), _ptr(hl2_saved),
                                  x.shape[0], _ptr(dx), _dt(dx), _ptr(d_a1), _ptr(d_b1),
                                  _ptr(d_a2), _ptr(d_b2), ctypes.byref(dq) if dq is not None else None,
                                  _ptr(dp_debug), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)))


def fourtune_ablation_workspace_bytes(m: int, fc1: Linear, fc2: Optional[Linear] = None) -> int:
    s1 = fc1.struct()
    s2 = fc2.struct() if fc2 is not None else None
    return lib().fourtune_ablation_workspace_bytes(m, ctypes.byref(s1),
                                                   ctypes.byref(s2) if s2 is not None else None)


def fourtune_linear_fwd_unfused(L: Linear, x: torch.Tensor, y: torch.Tensor,
                                xl_saved: torch.Tensor, ws: torch.Tensor, stream=None):
    _need_linear_fwd(L, x, y, xl_saved, ws)
    s = L.struct()
    _check(lib().fourtune_linear_fwd_unfused(ctypes.byref(s), _ptr(x), _dt(x), x.shape[0], _ptr(y),
                                             _dt(y), _ptr(xl_saved), _ptr(ws), ws.numel(),
                                             _stream(stream)))


def fourtune_linear_bwd_unfused(L: Linear, dy: torch.Tensor, x: torch.Tensor,
                                xl_saved: torch.Tensor, dx: torch.Tensor,
                                d_lora_a: Optional[torch.Tensor], d_lora_b: Optional[torch.Tensor],
                                ws: torch.Tensor, stream=None):
    _need_linear_bwd(L, dy, x, xl_saved, dx, d_lora_a, d_lora_b, ws)
    s = L.struct()
    _check(lib().fourtune_linear_bwd_unfused(ctypes.byref(s), _ptr(dy), _dt(dy), _ptr(x), _dt(x),
                                             _ptr(xl_saved), x.shape[0], _ptr(dx), _dt(dx),
                                             _ptr(d_lora_a), _ptr(d_lora_b), _ptr(ws), ws.numel(),
                                             _stream(stream)))


def fourtune_mlp_fwd_unfused(fc1: Linear, fc2: Linear, lora_fused: bool, x: torch.Tensor,
                             y: torch.Tensor, xl1_saved: torch.Tensor, pre_saved: torch.Tensor,
                             h_saved: torch.Tensor, hl2_saved: torch.Tensor, ws: torch.Tensor,
                             stream=None):
    _need_mlp(fc1, fc2)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need(x, "x", (m, fc1.k), _F32_BF16)
    _need(y, "y", (m, fc2.n), _F32_BF16)
    _need_low(xl1_saved, "xl1_saved", m, _rt(fc1))
    _need(pre_saved, "pre_saved", (m, fc1.n), _BF16)
    _need(h_saved, "h_saved", (m, fc1.n), _BF16)
    _need_low(hl2_saved, "hl2_saved", m, _rt(fc2))
    _need_ws(ws)
    s1, s2 = fc1.struct(), fc2.struct()
    _check(lib().fourtune_mlp_fwd_unfused(ctypes.byref(s1), ctypes.byref(s2), int(bool(lora_fused)),
                                          _ptr(x), _dt(x), x.shape[0], _ptr(y), _dt(y),
                                          _ptr(xl1_saved), _ptr(pre_saved), _ptr(h_saved),
                                          _ptr(hl2_saved), _ptr(ws), ws.numel(), _stream(stream)))


def fourtune_mlp_bwd_unfused(fc1: Linear, fc2: Linear, lora_fused: bool, dy: torch.Tensor,
                             x: torch.Tensor, xl1_saved: torch.Tensor, pre_saved: torch.Tensor,
                             h_saved: torch.Tensor, hl2_saved: torch.Tensor, dx: torch.Tensor,
                             d_a1, d_b1, d_a2, d_b2, ws: torch.Tensor, stream=None):
    _need_mlp(fc1, fc2)
    m = x.shape[0] if isinstance(x, torch.Tensor) and x.dim() == 2 else -1
    _need_mlp_bwd(fc1, fc2, m, dy, x, xl1_saved, pre_saved, hl2_saved, dx, d_a1, d_b1, d_a2, d_b2)
    _need(h_saved, "h_saved", (m, fc1.n), _BF16)
    _need_ws(ws)
    s1, s2 = fc1.struct(), fc2.struct()
    _check(lib().fourtune_mlp_bwd_unfused(ctypes.byref(s1), ctypes.byref(s2), int(bool(lora_fused)),
                                          _ptr(dy), _dt(dy), _ptr(x), _dt(x), _ptr(xl1_saved),
                                          _ptr(pre_saved), _ptr(h_saved), _ptr(hl2_saved),
                                          x.shape[0], _ptr(dx), _dt(dx), _ptr(d_a1), _ptr(d_b1),
                                          _ptr(d_a2), _ptr(d_b2), _ptr(ws), ws.numel(),
                                          _stream(stream)))


PREC = {"W4A4G4": 0, "W4A16G4": 1, "W4A4G16": 2, "W4A16G16": 3}


def fourtune_linear_fwd_prec(L: Linear, prec: str, x: torch.Tensor, y: torch.Tensor,
                             xl_saved: torch.Tensor, ws: torch.Tensor, stream=None):
    _need_linear_fwd(L, x, y, xl_saved, ws)
    s = L.struct()
    _check(lib().fourtune_linear_fwd_prec(ctypes.byref(s), PREC[prec], _ptr(x), _dt(x), x.shape[0],
                                          _ptr(y), _dt(y), _ptr(xl_saved), _ptr(ws), ws.numel(),
                                          _stream(stream)))


def fourtune_linear_bwd_prec(L: Linear, prec: str, dy: torch.Tensor, x: torch.Tensor,
                             xl_saved: torch.Tensor, dx: torch.Tensor,
                             d_lora_a: Optional[torch.Tensor], d_lora_b: Optional[torch.Tensor],
                             ws: torch.Tensor, stream=None):
    _need_linear_bwd(L, dy, x, xl_saved, dx, d_lora_a, d_lora_b, ws)
    s = L.struct()
    _check(lib().fourtune_linear_bwd_prec(ctypes.byref(s), PREC[prec], _ptr(dy), _dt(dy), _ptr(x),
                                          _dt(x), _ptr(xl_saved), x.shape[0], _ptr(dx), _dt(dx),
                                          _ptr(d_lora_a), _ptr(d_lora_b), _ptr(ws), ws.numel(),
                                          _stream(stream)))


def fourtune_status_string(status: int) -> str:
    return lib().fourtune_status_string(status).decode()


def fourtune_last_error() -> str:
    return lib().fourtune_last_error().decode()


# ----------------------------------------------------------------------------- helpers
def quantize(x: torch.Tensor, stream=None) -> Mx4:
    out = Mx4.empty(x.shape[0], x.shape[1], device=x.device)
    fourtune_quantize(x, out, stream=stream)
    return out


def make_linear(R: torch.Tensor, A: torch.Tensor, B: torch.Tensor, L1: torch.Tensor,
                L2: torch.Tensor, stream=None) -> Linear:
    """Quantize the frozen residual R once and bundle it with the low-rank factors."""
    return Linear(quantize(R, stream=stream), A, B, L1, L2)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def linear_forward(L: Linear, x: torch.Tensor, y_dtype=torch.bfloat16, ws=None, xq_out=None,
                   stream=None):
    m = x.shape[0]
    y = torch.empty((m, L.n), dtype=y_dtype, device=x.device)
    xl = torch.empty((m, L.rank + L.stab_rank), dtype=torch.bfloat16, device=x.device)
    ws = workspace(fourtune_linear_workspace_bytes(m, L), x.device) if ws is None else ws
    fourtune_linear_fwd(L, x, y, xl, ws, xq_out=xq_out, stream=stream)
    return y, xl


def linear_backward(L: Linear, dy: torch.Tensor, x: torch.Tensor, xl: torch.Tensor,
                    dx_dtype=torch.bfloat16, ws=None, gq_out=None, stream=None):
    m = x.shape[0]
    dx = torch.empty((m, L.k), dtype=dx_dtype, device=x.device)
    da = torch.empty((L.rank, L.k), dtype=torch.float32, device=x.device)
    db = torch.empty((L.n, L.rank), dtype=torch.float32, device=x.device)
    ws = workspace(fourtune_linear_workspace_bytes(m, L), x.device) if ws is None else ws
    fourtune_linear_bwd(L, dy, x, xl, dx, da, db, ws, gq_out=gq_out, stream=stream)
    return dx, da, db


def mlp_forward(fc1: Linear, fc2: Linear, x: torch.Tensor, y_dtype=torch.bfloat16, ws=None,
                hq_out=None, h_debug=None, stream=None):
    """Allocating helper: returns (y, saved) with saved = dict(xl1, pre, hl2)."""
    m, dev = x.shape[0], x.device
    y = torch.empty((m, fc2.n), dtype=y_dtype, device=dev)
    saved = dict(xl1=torch.empty((m, fc1.rank + fc1.stab_rank), dtype=torch.bfloat16, device=dev),
                 pre=torch.empty((m, fc1.n), dtype=torch.bfloat16, device=dev),
                 hl2=torch.empty((m, fc2.rank + fc2.stab_rank), dtype=torch.bfloat16, device=dev))
    ws = workspace(fourtune_mlp_workspace_bytes(m, fc1, fc2), dev) if ws is None else ws
    fourtune_mlp_fwd(fc1, fc2, x, y, saved["xl1"], saved["pre"], saved["hl2"], ws, hq_out=hq_out,
                     h_debug=h_debug, stream=stream)
    return y, saved


def mlp_backward(fc1: Linear, fc2: Linear, dy: torch.Tensor, x: torch.Tensor, saved: dict,
                 dx_dtype=torch.bfloat16, ws=None, dpq_out=None, dp_debug=None, stream=None):
    """Allocating helper: returns dict(dX, dA1, dB1, dA2, dB2)."""
    m, dev = x.shape[0], x.device
    dx = torch.empty((m, fc1.k), dtype=dx_dtype, device=dev)
    g = dict(dA1=torch.empty((fc1.rank, fc1.k), dtype=torch.float32, device=dev),
             dB1=torch.empty((fc1.n, fc1.rank), dtype=torch.float32, device=dev),
             dA2=torch.empty((fc2.rank, fc2.k), dtype=torch.float32, device=dev),
             dB2=torch.empty((fc2.n, fc2.rank), dtype=torch.float32, device=dev))
    ws = workspace(fourtune_mlp_workspace_bytes(m, fc1, fc2), dev) if ws is None else ws
    fourtune_mlp_bwd(fc1, fc2, dy, x, saved["xl1"], saved["pre"], saved["hl2"], dx, g["dA1"], g["dB1"],
                     g["dA2"], g["dB2"], ws, dpq_out=dpq_out, dp_debug=dp_debug, stream=stream)
    g["dX"] = dx
    return g
