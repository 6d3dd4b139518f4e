"""Oracle MXFP4 dequantisation pinned to the E2M1 table and the E8M0 closed form."""
import math

import numpy as np

import oracle
from mx_encode import e2m1_table, random_mx_matrix


def test_all_16_e2m1_codes():
    table = e2m1_table()
    assert len(table) == 16
    for c, v in table.items():
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (c, got, v)


def test_all_e8m0_codes():
    for e in range(255):
        assert oracle.e8m0_scale(e) == 2.0 ** (e - 127)
    assert math.isnan(oracle.e8m0_scale(255))


def test_nibble_order_low_is_even():
    codes = np.array([0x72, 0x0F], dtype=np.uint8)   # elements: 2, 7, 15, 0
    scales = np.array([127], dtype=np.uint8)
    row = np.concatenate([codes, np.zeros(14, np.uint8)])
    out = oracle.dequant_row(row, scales, 32)
    assert list(out[:4]) == [1.0, 6.0, -6.0, 0.0]
    out = oracle.dequant_row(row, np.array([124], np.uint8), 32)
    assert list(out[:4]) == [0.125, 0.75, -0.75, 0.0]


def test_dequant_inverts_encoder():
    rng = np.random.default_rng(1)
    dense, codes, scales = random_mx_matrix(rng, 8, 256)
    for r in range(8):
        np.testing.assert_array_equal(oracle.dequant_row(codes[r], scales[r], 256), dense[r])
