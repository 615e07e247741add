"""Pins of the oracle's quantizer against facts outside the oracle itself.

Each test pins one part of oracle/mx4.py to a hand-worked example, an exhaustive
comparison with an independent routine, a library routine, or an invariant the
method states (block-local scales make transposition free, FourTune §3.2).
"""
import os

import numpy as np
import pytest
import torch

from oracle import mx4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx4_blocks.txt")


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)].astype(np.float64)


def _read_golden():
    blocks, packs = [], []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "PACK":
                packs.append((int(parts[1], 16), int(parts[2], 16), int(parts[3], 16)))
                continue
            name, scale = parts[0], int(parts[1], 16)
            items = [(float(p.split(":")[0]), int(p.split(":")[1], 16)) for p in parts[2:]]
            blocks.append((name, scale, items))
    return blocks, packs


# ---------------------------------------------------------------- hand-worked examples
def test_golden_blocks():
    blocks, _ = _read_golden()
    assert [b[0] for b in blocks] == ["A", "B", "C", "D", "E"]
    for name, scale, items in blocks:
        T = np.zeros((32, 32))
        pos = [(3 * i % 32, 5 * i % 32) for i in range(len(items))]
        for (r, c), (v, _) in zip(pos, items):
            T[r, c] = v
        codes, scales = mx4.quantize(T)
        assert scales.shape == (1, 1) and scales[0, 0] == scale, name
        for (r, c), (v, code) in zip(pos, items):
            assert codes[r, c] == code, (name, v, codes[r, c], code)
        mask = np.ones((32, 32), bool)
        for r, c in pos:
            mask[r, c] = False
        assert np.all(codes[mask] == 0), name


def test_golden_packing():
    _, packs = _read_golden()
    for lo, hi, byte in packs:
        codes = np.array([[lo, hi] + [0] * 30], dtype=np.uint8)
        assert mx4.pack_codes(codes)[0, 0] == byte
        assert np.array_equal(mx4.unpack_codes(mx4.pack_codes(codes)), codes)


# ---------------------------------------------------------------- E2M1 rounding
def test_rounders_agree_exhaustively():
    """All finite bf16 values x all E8M0 exponents: three independent routines agree."""
    v = np.abs(_all_bf16_values())
    for e0 in range(-127, 128, 16):
        Es = np.arange(e0, min(e0 + 16, 128))
        y = np.ldexp(v[None, :], -Es[:, None]).ravel()
        a = mx4.e2m1_index_threshold(y)
        b = mx4.e2m1_index_nearest(y)
        c = mx4.e2m1_index_binade(y)
        assert np.array_equal(a, b), e0
        assert np.array_equal(a, c), e0


def test_rounding_midpoints_and_saturation():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    # expected: the even index of the two neighbours
    assert list(mx4.e2m1_index_threshold(mids)) == [0, 2, 2, 4, 4, 6, 6]
    eps = 2.0 ** -40
    assert list(mx4.e2m1_index_threshold(mids + eps)) == [1, 2, 3, 4, 5, 6, 7]
    assert list(mx4.e2m1_index_threshold(mids - eps)) == [0, 1, 2, 3, 4, 5, 6]
    assert list(mx4.e2m1_index_threshold(np.array([6.0, 7.9, 1e30]))) == [7, 7, 7]
    assert np.array_equal(mx4.E2M1_GRID[mx4.e2m1_index_threshold(mx4.E2M1_GRID)], mx4.E2M1_GRID)


# ---------------------------------------------------------------- scale rule
def _brute_exponent(amax):
    """Largest E in [-127, 127] with 2^(E+2) <= amax, else -127 (search over all E)."""
    out = np.full(amax.shape, -127, dtype=np.int64)
    for E in range(-127, 128):
        out = np.where(np.ldexp(1.0, E + 2) <= amax, E, out)
    return out


def test_scale_rule_exhaustive_bf16():
    v = _all_bf16_values()
    amax = np.unique(np.abs(v))
    assert np.array_equal(mx4.shared_exponent(amax), _brute_exponent(amax))


def test_scale_rule_random_and_powers():
    rng = np.random.default_rng(1)
    x = np.abs(rng.standard_normal(1 << 16).astype(np.float32).astype(np.float64))
    x *= np.ldexp(1.0, rng.integers(-140, 120, x.shape))
    p = np.ldexp(1.0, np.arange(-149, 128))
    p = np.concatenate([p, np.nextafter(p, 0), np.nextafter(p, np.inf)])
    for arr in (x, p):
        assert np.array_equal(mx4.shared_exponent(arr), _brute_exponent(arr))


def test_scale_keeps_block_in_range():
    """After scaling, every magnitude of a block lies below 8 and the maximum at >= 4
    unless the exponent was clamped: the block's largest value uses the top binade."""
    rng = np.random.default_rng(2)
    T = rng.standard_normal((64, 64)) * np.ldexp(1.0, rng.integers(-20, 20, (64, 1)))
    codes, scales = mx4.quantize(T)
    E = scales.astype(np.int64) - 127
    for bi in range(2):
        for bj in range(2):
            blk = T[32 * bi:32 * bi + 32, 32 * bj:32 * bj + 32]
            y = np.abs(blk) / 2.0 ** E[bi, bj]
            assert y.max() < 8 and y.max() >= 4


# ---------------------------------------------------------------- quantizer invariants
def _random_tensors():
    rng = np.random.default_rng(3)
    yield rng.standard_normal((96, 128))
    yield rng.standard_t(3, (64, 96)) * 0.02
    t = rng.standard_normal((64, 64))
    t[:, 5] *= 50
    yield t
    yield np.ldexp(rng.standard_normal((32, 64)), rng.integers(-130, 120, (32, 64)))


def test_idempotent():
    for T in _random_tensors():
        c1, s1 = mx4.quantize(T)
        c2, s2 = mx4.quantize(mx4.dequantize(c1, s1))
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_exact_round_trip():
    """Tensors built from codes, with a +-4 or +-6 in every block, come back exactly."""
    rng = np.random.default_rng(4)
    rows, cols = 96, 128
    idx = rng.integers(0, 8, (rows, cols))
    sign = rng.integers(0, 2, (rows, cols))
    E = rng.integers(-100, 100, (3, 4))
    val = mx4.E2M1_GRID[idx] * np.where(sign, -1.0, 1.0)
    for bi in range(3):
        for bj in range(4):
            val[32 * bi + 1, 32 * bj + 2] = rng.choice([4.0, -4.0, 6.0, -6.0])
    T = np.ldexp(val, np.repeat(np.repeat(E, 32, 0), 32, 1))
    codes, scales = mx4.quantize(T)
    assert np.array_equal(scales.astype(np.int64) - 127, E)
    assert np.array_equal(mx4.dequantize(codes, scales), T)


def test_transpose_invariance():
    """Block-local scales: Q(T^T) is Q(T) with codes and scales transposed (§3.2)."""
    for T in _random_tensors():
        r = (T.shape[0] // 32) * 32
        T = T[:r]
        c, s = mx4.quantize(T)
        ct, st = mx4.quantize(T.T)
        assert np.array_equal(ct, c.T) and np.array_equal(st, s.T)


def test_row_stripes_are_independent():
    """Quantizing a 32-row stripe alone gives the same rows as quantizing the whole."""
    T = next(_random_tensors())
    c, s = mx4.quantize(T)
    for bi in range(T.shape[0] // 32):
        cs, ss = mx4.quantize(T[32 * bi:32 * bi + 32])
        assert np.array_equal(cs, c[32 * bi:32 * bi + 32]) and np.array_equal(ss[0], s[bi])


def test_special_blocks():
    T = np.zeros((32, 96))
    T[:, 32:64] = np.nan
    T[0, 64] = np.inf
    T[1, 65] = 3.0
    c, s = mx4.quantize(T)
    assert list(s[0]) == [0x00, 0xFF, 0xFF]
    assert np.all(c == 0)
    d = mx4.dequantize(c, s)
    assert np.all(d[:, :32] == 0) and np.all(np.isnan(d[:, 32:]))


def test_partial_block_rows():
    rng = np.random.default_rng(5)
    T = rng.standard_normal((56, 64))
    c, s = mx4.quantize(T)
    assert c.shape == (56, 64) and s.shape == (2, 2)
    pad = np.zeros((64, 64))
    pad[:56] = T
    cp, sp = mx4.quantize(pad)
    assert np.array_equal(c, cp[:56]) and np.array_equal(s, sp)
    # the maximum is taken over the 24 valid rows of the last block row only
    T2 = T.copy()
    T2[32:] *= 1e-3
    _, s2 = mx4.quantize(T2)
    amax = np.abs(T2[32:, :32]).max()
    assert s2[1, 0] == int(np.floor(np.log2(amax))) - 2 + 127


def test_negative_zero_and_sign():
    T = np.zeros((32, 32))
    T[0, 0] = -0.0
    T[0, 1] = -1e-30
    T[0, 2] = 1.0
    c, _ = mx4.quantize(T)
    assert c[0, 0] == 8 and c[0, 1] == 8 and c[0, 3] == 0


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_matches_torch_on_fp32():
    rng = np.random.default_rng(6)
    bits = rng.integers(0, 2 ** 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = mx4.bf16_round(x.astype(np.float64))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    # exact ties: fp32 values halfway between two bf16 values
    t = ((np.arange(1, 4096, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ref_t = torch.from_numpy(t.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mx4.bf16_round(t.astype(np.float64)), ref_t)


def test_bf16_nearest_for_fp64_values():
    """fp64 inputs (no fp32 step): the result is the nearest of the two bf16 neighbours."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4096) * np.ldexp(1.0, rng.integers(-135, 100, 4096))
    got = mx4.bf16_round(x)
    x32 = x.astype(np.float32)  # neighbours are found from the truncated bf16 pattern
    lo_bits = (np.abs(x32).view(np.uint32) & 0xFFFF0000).astype(np.uint32)
    cands = []
    for d in (-1, 0, 1, 2):
        b = (lo_bits.astype(np.int64) + (d << 16)).clip(0, 0x7F7F0000).astype(np.uint32)
        cands.append(b.view(np.float32).astype(np.float64) * np.sign(x))
    cands = np.stack(cands)
    dist = np.abs(cands - x)
    assert np.all(np.abs(got - x) <= dist.min(axis=0))
