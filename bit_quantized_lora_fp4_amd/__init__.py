"""MI355X-native W4A4G4 quantized linear layer (FourTune) behind a C ABI.

The kernels live in libfourtune.so (csrc/, built by ``build.py``); ``abi`` is the
ctypes binding with the C entry points' names.
"""
from . import abi  # noqa: F401
from .abi import (FourTuneError, Linear, Mx4, fourtune_gemm_bwd, fourtune_gemm_fwd, fourtune_linear_bwd, fourtune_linear_fwd,  # noqa: F401
                  fourtune_linear_workspace_bytes, fourtune_mlp_bwd, fourtune_mlp_fwd,
                  fourtune_mlp_workspace_bytes, fourtune_quantize, ft_mx4_codes_bytes,
                  ft_mx4_scales_bytes, fourtune_status_string, fourtune_last_error)
