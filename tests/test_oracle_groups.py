"""Pins of the oracle's 1x32 group quantizer (oracle/mx4.py: quantize_groups), used for
the granularity comparison (FourTune §4 "Impact of Quantization Granularity").

- reduction to the pinned block quantizer: a one-row tensor is a single partial block
  row, whose block maximum is that row's group maximum, so row i of the group form
  equals the block form of row i alone (codes and scale bytes), over random, zero,
  subnormal, huge and non-finite rows;
- hand-worked blocks (the MX rule by hand, the same two rows as worked blocks A and B
  of the block tests): in one 32x32 block they share the larger row's scale and the
  small row's values round to zero; as groups each row keeps its own scale;
- dequantize_groups inverts on-grid rows exactly.
"""
import numpy as np

from oracle import mx4


def test_group_rows_equal_one_row_blocks():
    rng = np.random.default_rng(40)
    T = rng.standard_normal((37, 128)) * np.ldexp(1.0, rng.integers(-20, 20, (37, 1)))
    T[3] = 0.0
    T[5, :32] = np.ldexp(1.0, -140)            # subnormal group
    T[7, 40] = np.nan                           # non-finite group
    T[8, 70] = np.inf
    T[9, 96:] = 1e38
    c, s = mx4.quantize_groups(T)
    assert c.shape == T.shape and s.shape == (37, 4)
    for i in range(T.shape[0]):
        cb, sb = mx4.quantize(T[i:i + 1])
        assert np.array_equal(c[i:i + 1], cb), i
        assert np.array_equal(s[i], sb[0]), i
    assert s[7, 1] == 0xFF and np.all(c[7, 32:64] == 0)
    assert s[3, 0] == 0 and np.all(c[3] == 0)


def test_hand_worked_block_versus_groups():
    T = np.zeros((32, 32))
    T[0, 0], T[0, 1] = 7.0, -3.5          # row amax 7 -> E = 0, byte 0x7F
    T[1, 0], T[1, 1] = 0.1, 0.05          # row amax 0.1 -> E = -6, byte 0x79
    cb, sb = mx4.quantize(T)
    assert sb[0, 0] == 0x7F
    assert cb[0, 0] == 0x7 and cb[0, 1] == 0xE   # 7 saturates to 6; -3.5 ties to -4
    assert cb[1, 0] == 0x0 and cb[1, 1] == 0x0   # 0.1, 0.05 round to zero at scale 1
    cg, sg = mx4.quantize_groups(T)
    assert sg[0, 0] == 0x7F and sg[1, 0] == 0x79 and sg[2, 0] == 0x00
    assert cg[0, 0] == 0x7 and cg[0, 1] == 0xE
    assert cg[1, 0] == 0x7 and cg[1, 1] == 0x5   # 6.4 saturates to 6; 3.2 -> 3


def test_dequantize_groups_round_trip_on_grid():
    rng = np.random.default_rng(41)
    rows, cols = 20, 96
    vals = mx4.E2M1_GRID[rng.integers(0, 8, (rows, cols))] * rng.choice([-1.0, 1.0], (rows, cols))
    vals[:, ::32] = 6.0                          # pins each group's exponent at 0
    e = rng.integers(-10, 10, (rows, cols // 32))
    T = vals * np.ldexp(1.0, np.repeat(e, 32, axis=1))
    c, s = mx4.quantize_groups(T)
    assert np.array_equal(mx4.dequantize_groups(c, s), T)
