"""Helpers for the GPU parity tests: host<->device moves and packed-code views."""
import numpy as np
import torch

from oracle import mx4

TORCH_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def dev(a: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    """float32 numpy array (values exact in `dtype`) -> contiguous CUDA tensor of `dtype`."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(TORCH_DT[dtype])


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def oracle_packed(T: np.ndarray):
    codes, scales = mx4.quantize(np.asarray(T, dtype=np.float64))
    return mx4.pack_codes(codes), scales


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def log(msg: str):
    print(msg, flush=True)
