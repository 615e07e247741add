"""Row / column sampling helpers of the full-size ablation and precision tests (which
compare sampled outputs of the unfused and 16-bit forms with the oracle by relative
Frobenius error)."""
import numpy as np
import torch

from bit_quantized_lora_fp4_amd import abi
from oracle import layer, mx4
from tests.gpu_util import dev, host, log

TOL = 1e-3


def _block_rows(m, rng):
    """The first, a middle and the last (possibly partial) 32-row block row."""
    nb = (m + 31) // 32
    picks = sorted({0, int(rng.integers(1, max(nb - 1, 2))), nb - 1})
    return picks, np.concatenate([np.arange(32 * b, min(32 * b + 32, m)) for b in picks])


def _col_blocks(n, rng, count=3):
    nb = n // 32
    picks = sorted(set([0, nb - 1] + [int(v) for v in rng.integers(0, nb, count)]))
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in picks])


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _bf(a):
    return mx4.bf16_round(_f64(a))


def _chunked(fn, m, step=4096):
    """Row-chunked evaluation of fn(lo, hi) -> array, stacked (bounds fp64 temporaries)."""
    return np.concatenate([fn(lo, min(m, lo + step)) for lo in range(0, m, step)], axis=0)


def _rows(t, idx):
    return host(t.index_select(0, torch.as_tensor(idx, device=t.device)))


def _lin64(d):
    return layer.Linear(R=_f64(d["R"]), A=_f64(d["A"]), B=_f64(d["B"]), L1=_f64(d["L1"]), L2=_f64(d["L2"]))


def _gpu_lin(d):
    return abi.make_linear(dev(d["R"], "fp32"), dev(d["A"]), dev(d["B"]), dev(d["L1"]), dev(d["L2"]))


def _errs_ok(errs):
    log(f"  rel errors {errs}")
    for k_, e in errs.items():
        assert e <= TOL, (k_, e)
