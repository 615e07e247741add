"""CPU oracle for the W4A4G4 quantized linear layer and its MLP pairing.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, fp64 statement of what
the GPU path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It imports nothing from the
GPU package and the GPU package imports nothing from it; the two share no code.

Method source: "FourTune: Towards Fully 4-Bit Efficient Post-Training for Diffusion
Models" (the pages), §2.3 (quantizer form and MXFP4), §3.1 (triple-branch
hybrid-precision linear), §3.2 (block-wise quantization, 4-bit backward),
§3.3 (LoRA fusion, MLP fusion). The E8M0 scale rule comes from the Microscaling
formats paper the pages cite for MXFP4 (Rouhani et al., 2023).

Modules:
  mx4    -- bf16 rounding, the 32x32-block E2M1+E8M0 quantizer, dequantization.
  layer  -- triple-branch linear forward/backward and the GELU MLP pair.
"""
from . import mx4, layer  # noqa: F401
