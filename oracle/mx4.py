"""fp64 reference of the 32x32-block MXFP4 quantizer (E2M1 codes, E8M0 scales).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where it comes from:

* Quantizer form: a tensor is mapped to low-bit values as Round(W / s) with a group
  scale s; MXFP4 is one of the group-scaled formats named [FourTune, §2.3 "Model
  Quantization"].
* Block structure: scales are bound to small independent 2-D blocks, so a block and
  its scale are fetched together in either orientation [FourTune, §3.2]. The pages use
  16x16 blocks (§4.3, "Impact of Quantization Granularity"); this build uses 32x32
  blocks, the smallest square block in which every run of 32 consecutive elements
  along either axis shares one E8M0 scale, as an MX block-scaled matrix unit needs.
* Scale rule (MX, Rouhani et al. 2023, cited by the pages in §2.3): the shared
  exponent of a block is floor(log2(amax)) - emax, emax = 2 for E2M1, clamped to the
  E8M0 range [-127, 127]; stored as the biased byte E + 127.
* Element rounding: round-to-nearest onto the E2M1 magnitude grid
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even code index, saturating at 6.

Readings where the pages are silent (each is listed with its reason in the design
notes): an all-zero block gets E = -127; a block holding a non-finite value gets
scale byte 0xFF and all-zero codes; the sign bit is kept for values that round to
zero (code 0x8); a partial last block row takes its maximum over the valid rows
only; two codes per byte with the even column in the low nibble; scales row-major
over blocks.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
NAN_SCALE = 0xFF
E_MIN, E_MAX = -127, 127
EMAX_E2M1 = 2  # exponent of the largest E2M1 magnitude, 6 = 1.5 * 2^2


# ----------------------------------------------------------------------------------
# bf16 round-to-nearest-even, applied where the GPU rounds (bf16 MFMA operands)
# ----------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range: normal numbers down to
    2^-126, subnormals with quantum 2^-133. The quantum of x is 2^(e-8) where
    x = m * 2^e, m in [0.5, 1), floored at the subnormal quantum; x / quantum is then
    rounded half-to-even with np.rint and scaled back (all steps exact in fp64).
    Results of magnitude >= 2^128 overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    if np.any(fin):
        _, e = np.frexp(x[fin])
        q_exp = np.maximum(e, -125) - 8
        r = np.ldexp(np.rint(np.ldexp(x[fin], -q_exp)), q_exp)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
        out[fin] = r
    return out


# ----------------------------------------------------------------------------------
# E2M1 rounding: three independent routines (midpoint table, grid search, np.rint)
# ----------------------------------------------------------------------------------
# Midpoints between neighbouring grid values, and whether a value exactly on the
# midpoint goes up (the upper neighbour has the even index) or down.
_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_TIE_GOES_UP = np.array([False, True, False, True, False, True, False])


def e2m1_index_threshold(mag: np.ndarray) -> np.ndarray:
    """Code index (0..7) of nonnegative magnitudes via the midpoint table.

    Index = number of midpoints passed; a value equal to a midpoint passes it only
    when the upper neighbour has the even index. Values above 6 land on index 7
    (saturation).
    """
    mag = np.asarray(mag, dtype=np.float64)
    idx = np.zeros(mag.shape, dtype=np.uint8)
    for mid, up in zip(_MIDPOINTS, _TIE_GOES_UP):
        passed = (mag >= mid) if up else (mag > mid)
        idx += passed.astype(np.uint8)
    return idx


def e2m1_index_nearest(mag: np.ndarray) -> np.ndarray:
    """Code index (0..7) of nonnegative magnitudes by searching the grid.

    The nearest grid value wins; among equally near values the even index wins.
    Values beyond 6 are nearest to 6 (saturation falls out of the search).
    """
    # Any value >= 6 has 6 as its nearest grid point; clipping huge values to 16 keeps
    # the distances below exact in fp64 without changing which grid point is nearest.
    mag = np.minimum(np.asarray(mag, dtype=np.float64), 16.0)
    dist = np.abs(mag[..., None] - E2M1_GRID)  # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    # prefer an even index among the tied candidates
    even = cand & (np.arange(8) % 2 == 0)
    pick_even = even.any(axis=-1)
    first_even = np.argmax(even, axis=-1)
    first_any = np.argmax(cand, axis=-1)
    return np.where(pick_even, first_even, first_any).astype(np.uint8)


def e2m1_index_binade(mag: np.ndarray) -> np.ndarray:
    """Code index via np.rint on each binade of the grid (a third, library route).

    On [0, 2) the grid spacing is 0.5, on [2, 4) it is 1, on [4, 8) it is 2; within
    each, round-half-to-even on the scaled value picks the even index. 8 saturates
    to 6.
    """
    mag = np.asarray(mag, dtype=np.float64)
    val = np.where(mag < 2.0, np.rint(mag * 2.0) / 2.0,
                   np.where(mag < 4.0, np.rint(mag), 2.0 * np.rint(mag / 2.0)))
    val = np.minimum(val, 6.0)
    return np.searchsorted(E2M1_GRID, val).astype(np.uint8)


# ----------------------------------------------------------------------------------
# Scale rule
# ----------------------------------------------------------------------------------
def shared_exponent(amax) -> np.ndarray:
    """E = clamp(floor(log2(amax)) - 2, -127, 127); E = -127 for amax == 0.

    floor(log2) is taken exactly from frexp: amax = m * 2^e with m in [0.5, 1)
    gives floor(log2(amax)) = e - 1.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    E = np.clip(e.astype(np.int64) - 1 - EMAX_E2M1, E_MIN, E_MAX)
    return np.where(amax == 0.0, E_MIN, E)


# ----------------------------------------------------------------------------------
# The block quantizer
# ----------------------------------------------------------------------------------
def _blocks(T: np.ndarray):
    rows, cols = T.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    nbr = -(-rows // BLOCK)
    pad = np.zeros((nbr * BLOCK, cols), dtype=np.float64)
    pad[:rows] = T
    return pad.reshape(nbr, BLOCK, cols // BLOCK, BLOCK), nbr


def quantize(T, rounder=e2m1_index_threshold):
    """Quantize a 2-D tensor in 32x32 blocks.

    Returns (codes, scales): codes is uint8 [rows, cols], one 4-bit code per element
    (bit 3 = sign, bits 0..2 = grid index); scales is uint8 [ceil(rows/32), cols/32],
    the biased E8M0 byte of each block. Zero rows pad the last block row (they change
    neither the block maximum nor its finiteness) and are dropped from the codes.
    """
    T = np.asarray(T, dtype=np.float64)
    rows, cols = T.shape
    blk, nbr = _blocks(T)                                   # [nbr, 32, nbc, 32]
    finite = np.isfinite(blk).all(axis=(1, 3))              # [nbr, nbc]
    amax = np.where(finite, np.abs(np.where(np.isfinite(blk), blk, 0.0)).max(axis=(1, 3)), 0.0)
    E = shared_exponent(amax)                               # [nbr, nbc]
    scales = np.where(finite, E + 127, NAN_SCALE).astype(np.uint8)
    y = np.ldexp(np.where(np.isfinite(blk), blk, 0.0), -E[:, None, :, None])
    idx = rounder(np.abs(y))
    sign = np.signbit(y).astype(np.uint8) << 3
    codes = (idx | sign) * finite[:, None, :, None].astype(np.uint8)
    codes = codes.reshape(nbr * BLOCK, cols)[:rows]
    return codes.astype(np.uint8), scales


def quantize_groups(T, rounder=e2m1_index_threshold):
    """Quantize a 2-D tensor in 1x32 groups: each row's 32 consecutive columns share one
    scale (the group-wise granularity FourTune §4 "Impact of Quantization Granularity"
    compares the block-wise one against; the MX rule applies per group unchanged).

    Returns (codes, scales): codes uint8 [rows, cols] as in ``quantize``; scales uint8
    [rows, cols/32].
    """
    T = np.asarray(T, dtype=np.float64)
    rows, cols = T.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    g = T.reshape(rows, cols // BLOCK, BLOCK)                 # [rows, ngroups, 32]
    finite = np.isfinite(g).all(axis=2)                       # [rows, ngroups]
    amax = np.where(finite, np.abs(np.where(np.isfinite(g), g, 0.0)).max(axis=2), 0.0)
    E = shared_exponent(amax)
    scales = np.where(finite, E + 127, NAN_SCALE).astype(np.uint8)
    y = np.ldexp(np.where(np.isfinite(g), g, 0.0), -E[:, :, None])
    idx = rounder(np.abs(y))
    sign = np.signbit(y).astype(np.uint8) << 3
    codes = (idx | sign) * finite[:, :, None].astype(np.uint8)
    return codes.reshape(rows, cols).astype(np.uint8), scales


def dequantize_groups(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact values of 1x32-group codes (scale byte 0xFF: NaN)."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    sc = np.repeat(scales.astype(np.int64), BLOCK, axis=1)
    out = np.ldexp(val, sc - 127)
    return np.where(sc == NAN_SCALE, np.nan, out)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: column 2j in the low nibble, column 2j+1 in the high one."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact value of every code: (-1)^bit3 * grid[bits 0..2] * 2^(scale - 127).

    A block with scale byte 0xFF dequantizes to NaN.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    sc = np.repeat(np.repeat(scales.astype(np.int64), BLOCK, axis=0), BLOCK, axis=1)[:rows, :cols]
    out = np.ldexp(val, sc - 127)
    return np.where(sc == NAN_SCALE, np.nan, out)


def fake_quant(T) -> np.ndarray:
    """deq(Q(T)): the values a 4-bit GEMM sees."""
    codes, scales = quantize(T)
    return dequantize(codes, scales)
