"""Test-side MXFP4 encoder (the inverse of dequantisation), independent of the oracle.

Builds random dense matrices whose 32-element row blocks are exactly representable
(value from the E2M1 table times 2^s), and packs them into the logical blob layout
(low nibble = even element; one E8M0 byte per 32 elements along the row).
"""
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))


def e2m1_table():
    vals = {}
    with open(os.path.join(_HERE, "golden", "e2m1_codes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def random_mx_matrix(rng, rows, K, exp_lo=-4, exp_hi=0):
    """(dense float64 [rows][K], codes [rows][K/2] u8, scales [rows][K/32] u8)."""
    table = e2m1_table()
    codes4 = rng.integers(0, 16, size=(rows, K))
    sexp = rng.integers(exp_lo, exp_hi + 1, size=(rows, K // 32))
    vals = np.vectorize(table.get)(codes4).astype(np.float64)
    dense = vals * np.repeat(np.ldexp(1.0, sexp), 32, axis=1)
    codes = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    scales = (127 + sexp).astype(np.uint8)
    return dense, codes, scales


def pack_blob(parts):
    """parts: [(codes, scales)] for gate, up, down -> logical blob bytes."""
    return np.concatenate([np.concatenate([c.ravel(), s.ravel()]) for c, s in parts]).astype(np.uint8)


def random_expert(rng, H, I):
    g, gc, gs = random_mx_matrix(rng, I, H)
    u, uc, us = random_mx_matrix(rng, I, H)
    d, dc, ds = random_mx_matrix(rng, H, I)
    return (g, u, d), pack_blob([(gc, gs), (uc, us), (dc, ds)])
