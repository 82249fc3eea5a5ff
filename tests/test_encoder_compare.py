"""The margin comparison of encoder bits (tests/encoder_compare.py) on the CPU: the oracle's own
bits pass, bits selected from masses perturbed inside the mass tolerance pass, and planted
wrong selections are caught."""
import numpy as np
import pytest

from bit_vector_block_amd import workloads as W
from oracle import encoder as E

import encoder_compare as C


def _case(seed):
    return W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=4, hq=4, hkv=2, d=16)


@pytest.mark.parametrize("seed", range(4))
def test_oracle_bits_pass_and_perturbed_masses_stay_inside_the_margin(seed):
    case = _case(seed)
    M = E.tile_masses(case)
    la, ca = E.select_bits(case, M, 0.9, 0.9)
    res = C.compare(case, M, la, ca, 0.9, 0.9)
    assert res["differ"] == 0
    rng = np.random.default_rng(seed)
    for _ in range(5):
        Mp = M * (1 + rng.uniform(-C.RTOL, C.RTOL, M.shape)) + rng.uniform(-C.ATOL, C.ATOL, M.shape) * (M > 0)
        la2, ca2 = E.select_bits(case, Mp, 0.9, 0.9)
        C.compare(case, M, la2, ca2, 0.9, 0.9)  # raises on a robust row that differs


def test_fragile_rows_near_a_tie_may_differ():
    """Two candidates whose masses differ by less than the tolerance: either one may be kept."""
    m = np.array([0.5, 0.30000, 0.30001, 0.05])
    eps = C.la_eps(m)
    assert not C.robust(m, eps, 0.6, {0})
    assert C.valid_within_margin(m, eps, 0.6, {0}, {0, 1})
    assert C.valid_within_margin(m, eps, 0.6, {0}, {0, 2})
    assert not C.valid_within_margin(m, eps, 0.6, {0}, {0, 3})     # too little mass
    assert not C.valid_within_margin(m, eps, 0.6, {0}, {0, 1, 2})  # not minimal
    m2 = np.array([0.5, 0.3, 0.15, 0.05])
    assert C.robust(m2, C.la_eps(m2), 0.6, {0})


@pytest.mark.parametrize("plant", ["lower_p", "drop_forced", "swap_tile", "ca_from_own_doc"])
def test_planted_wrong_selections_are_caught(plant):
    case = W.make_case("cmp", 3, [3], [256, 192, 256], [64], 2, 1, 16, np.full((1, 2), 0.5), np.full((1, 2), 0.5))
    M = E.tile_masses(case)
    p_la = 0.9
    la, ca = E.select_bits(case, M, p_la, 0.9)
    if plant == "lower_p":
        la, ca = E.select_bits(case, M, 0.6, 0.6)
    elif plant == "drop_forced":
        la[1][0, 2, 0] = False
    elif plant == "swap_tile":
        # at p_la = 0.5 some rows drop candidates: swap a kept free tile for a dropped one
        p_la = 0.5
        la, ca = E.select_bits(case, M, p_la, 0.9)
        done = False
        for d in range(len(la)):
            for r in range(la[d].shape[1]):
                row = la[d][0, r, :r + 1]
                kept = [c for c in range(r + 1) if row[c] and c not in (0, r)]
                dropped = [c for c in range(r + 1) if not row[c]]
                if kept and dropped and not done:
                    row[kept[0]], row[dropped[0]] = False, True
                    done = True
        assert done
    elif plant == "ca_from_own_doc":
        # CA pages chosen from the document's own rows instead of the later documents'
        _, _, _, _, doc_first, doc_T = E._segments(case)
        t0, T = doc_first[0], doc_T[0]
        own = M[:, t0:t0 + T, t0:t0 + T].sum(axis=1)
        for h in range(2):
            keep = E.select_top_p(own[h], 0.9, {0})
            ca[0][h] = False
            ca[0][h, sorted(keep)] = True
        assert not all(np.array_equal(a, b) for a, b in zip(ca, E.select_bits(case, M, 0.9, 0.9)[1]))
    with pytest.raises(AssertionError):
        C.compare(case, M, la, ca, p_la, 0.9)


def test_forced_tile_outside_the_prefix():
    """A forced candidate that is not part of the top-p prefix (it is added after the cut) must
    not count towards the prefix when a near-tie at the cut is judged (seen on the Qwen3-shape
    workload: CA page 0, 31st of 32 by mass, beside a 1e-6-relative tie at the cut)."""
    m = np.array([0.28, 0.5, 0.30000, 0.30001, 0.25])
    eps = C.la_eps(m)
    assert E.select_top_p(m, 0.45, {0}) == {0, 1, 3}
    assert not C.robust(m, eps, 0.45, {0})
    assert C.valid_within_margin(m, eps, 0.45, {0}, {0, 1, 2})
    assert not C.valid_within_margin(m, eps, 0.45, {0}, {0, 1, 4})
