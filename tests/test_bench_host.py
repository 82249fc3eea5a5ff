"""Host-side figures of bench.py (no GPU): the useful-FLOP pair count and the tile valid counts."""
import os
import sys

import numpy as np
import pytest

import oracle
from bit_vector_block_amd import workloads as W

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _brute_pairs(case, rp, ci):
    from oracle import encoder as E
    valid = E.valid_tokens(case)
    G = valid.size // 64
    n = 0
    for row in range(rp.size - 1):
        g = row % G
        for t in ci[rp[row]:rp[row + 1]]:
            q = np.nonzero(valid[64 * g:64 * g + 64])[0] + 64 * g
            k = np.nonzero(valid[64 * t:64 * t + 64])[0] + 64 * int(t)
            n += int((k[None, :] <= q[:, None]).sum())
    return n


@pytest.mark.parametrize("seed", range(4))
def test_useful_pairs_equal_brute_force(seed):
    case = W.random_small_case(seed, d=64, hq=2, hkv=1)
    rp, ci = oracle.decode(case)
    rp, ci = np.asarray(rp, np.int64), np.asarray(ci)
    assert bench.useful_pairs(case, rp, ci) == _brute_pairs(case, rp, ci)


def test_full_tiles_count_whole_or_half_diagonal():
    case = W.config_case(2)
    tv = bench.tile_valid_counts(case)
    assert tv.size == 162 and (tv == 64).all()
    # one row holding one off-diagonal and one diagonal full tile
    rp = np.array([0, 2] + [2] * (32 * 162 - 1), np.int64)
    ci = np.array([0, 0], np.int64)
    # row 0 is (head 0, tile 0): both entries are its diagonal tile
    assert bench.useful_pairs(case, rp, ci) == 2 * 64 * 65 // 2
    rp2 = np.array([0] * 2 + [2] * (32 * 162 - 1), np.int64)  # row 1 = (head 0, tile 1)
    ci2 = np.array([0, 1], np.int64)
    assert bench.useful_pairs(case, rp2, ci2) == 64 * 64 + 64 * 65 // 2
