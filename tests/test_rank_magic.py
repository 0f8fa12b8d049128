"""The per-rank layout maps an expert id e to its rank e / L (L = experts per
rank) with one multiply: (e * ceil(2^32 / L)) >> 32.  Checked here
exhaustively over every id the kernel can see (0 <= e < E <= 2048, ids are
validated against E first) and every L = E / R with R <= 32, and over a range
of larger ids, against integer division.
"""
import numpy as np


def _magic(L):
    return ((1 << 32) + L - 1) // L  # ceil(2^32 / L), as the host computes it


def test_rank_of_every_valid_id():
    Ls = sorted({E // R for E in range(1, 2049) for R in range(1, 33) if E % R == 0})
    e = np.arange(2048, dtype=np.uint64)
    for L in Ls:
        got = (e * np.uint64(_magic(L))) >> np.uint64(32)
        assert np.array_equal(got, e // np.uint64(L)), L


def test_rank_of_ids_below_2_pow_21():
    # the error of the rounded-up reciprocal stays below one step of e / L
    # while e * (ceil(2^32/L) * L - 2^32) < 2^32, i.e. for e < 2^32 / L
    e = np.arange(1 << 21, dtype=np.uint64)
    for L in (1, 2, 3, 5, 7, 8, 32, 75, 96, 127, 255, 256, 600 // 8, 1023, 2047, 2048):
        got = (e * np.uint64(_magic(L))) >> np.uint64(32)
        assert np.array_equal(got, e // np.uint64(L)), L
