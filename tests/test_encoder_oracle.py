"""Pins of the encoder oracle (oracle/encoder.py): closed forms, special cases, hand-worked
selections and invariants."""
import itertools
import math

import numpy as np
import pytest

from bit_vector_block_amd import workloads as W
from oracle import encoder as E


def _small(seed, **kw):
    return W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=3, hq=2, hkv=1, d=16, **kw)


@pytest.mark.parametrize("seed", range(4))
def test_masses_rows_sum_to_valid_query_count(seed):
    case = _small(seed)
    M = E.tile_masses(case)
    valid = E.valid_tokens(case).reshape(-1, 64).sum(axis=1)
    for h in range(case.num_q_heads):
        assert np.allclose(M[h].sum(axis=1), valid, rtol=0, atol=1e-9)


def test_masses_zero_queries_give_uniform_attention():
    """Q = 0: every query attends uniformly to its valid causal keys, so a tile pair's mass is a
    count ratio summed over the query tile (no softmax involved)."""
    case = _small(7)
    case.q[:] = 0
    M = E.tile_masses(case)
    tile_req, _, _, req_first, _, _ = E._segments(case)
    valid = E.valid_tokens(case)
    G = len(tile_req)
    for g in range(G):
        b = tile_req[g]
        t0 = req_first[b]
        for c in range(t0, g + 1):
            want = 0.0
            for qt in range(64 * g, 64 * g + 64):
                if not valid[qt]:
                    continue
                keys = [kt for kt in range(64 * t0, qt + 1) if valid[kt]]
                want += sum(1 for kt in keys if kt // 64 == c) / len(keys)
            assert abs(M[0, g, c] - want) < 1e-9 and abs(M[1, g, c] - want) < 1e-9


def test_masses_outside_request_or_future_are_zero():
    case = _small(3)
    M = E.tile_masses(case)
    tile_req, *_ = E._segments(case)
    G = len(tile_req)
    for g in range(G):
        for c in range(G):
            if c > g or tile_req[c] != tile_req[g]:
                assert M[:, g, c].max() == 0.0


@pytest.mark.parametrize("masses,p,forced,want", [
    ([0.5, 0.3, 0.2], 0.7, set(), {0, 1}),
    ([0.2, 0.3, 0.5], 0.7, set(), {2, 1}),
    ([0.25, 0.25, 0.25, 0.25], 0.5, set(), {0, 1}),
    ([0.5, 0.5, 0.0], 1.0, set(), {0, 1}),
    ([0.0, 0.0, 0.0], 0.9, {0}, {0}),
    ([0.1, 0.6, 0.3], 0.5, {2, 0}, {1, 2, 0}),
    ([1.0], 0.9, set(), {0}),
])
def test_select_top_p_hand_worked(masses, p, forced, want):
    assert E.select_top_p(masses, p, forced) == want


@pytest.mark.parametrize("seed", range(20))
def test_select_top_p_is_the_minimal_sorted_prefix(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 65))
    m = rng.random(n) ** 3
    p = float(rng.uniform(0.1, 1.0))
    keep = E.select_top_p(m, p, set())
    order = sorted(range(n), key=lambda i: (-float(m[i]), i))
    k = len(keep)
    assert keep == set(order[:k])
    tot = math.fsum(m.tolist())
    # reaches the threshold, and one fewer does not (exactly rounded sums)
    assert math.fsum(m[order[:k]].tolist()) >= p * tot
    if k > 1:
        assert math.fsum(m[order[:k - 1]].tolist()) < p * tot


@pytest.mark.parametrize("seed", range(30))
def test_select_top_p_brute_force_over_all_subsets(seed):
    """Brute force over every subset of up to 10 candidates: the size of the kept set is the
    smallest size of any subset whose mass reaches p x total, and among the subsets of that
    size the kept one has the largest mass (ties: the smaller indices).  Masses are multiples of
    1/8 half of the time, so exact ties and exact hits of the threshold occur."""
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(1, 11))
    m = rng.integers(0, 6, size=n) / 8.0 if seed % 2 else rng.random(n)
    p = [0.25, 0.5, 0.75, 1.0, float(rng.uniform(0.05, 1.0))][seed % 5]
    tot = math.fsum(m.tolist())
    best = None
    for size in range(1, n + 1):
        reach = [s for s in itertools.combinations(range(n), size) if math.fsum(m[list(s)].tolist()) >= p * tot]
        if reach:
            top = max(math.fsum(m[list(s)].tolist()) for s in reach)
            cands = [s for s in reach if math.fsum(m[list(s)].tolist()) == top]
            # among equal masses the tie order prefers smaller indices: the lexicographically
            # smallest sorted-index tuple of the top subsets that is also a top-by-mass prefix
            best = (size, cands)
            break
    keep = E.select_top_p(m, p, set())
    assert best is not None and len(keep) == best[0]
    assert any(set(c) == keep for c in best[1])
    # every kept mass is >= every dropped mass; equal masses are kept smaller index first
    drop = set(range(n)) - keep
    for i in keep:
        for j in drop:
            assert m[i] > m[j] or (m[i] == m[j] and i < j)


def test_select_bits_forced_and_last_document():
    case = _small(11)
    M = E.tile_masses(case)
    la, ca = E.select_bits(case, M, 0.5, 0.5)
    tile_req, tile_doc, _, _, doc_first, doc_T = E._segments(case)
    for d, (la_d, ca_d) in enumerate(zip(la, ca)):
        T = doc_T[d]
        for r in range(T):
            assert la_d[:, r, r].all() and la_d[:, r, 0].all()
            assert not la_d[:, r, r + 1:].any()
        assert ca_d[:, 0].all()
        b = tile_req[doc_first[d]]
        if not any(tile_req[g] == b and tile_doc[g] > d for g in range(len(tile_req))):
            assert ca_d[:, 1:].sum() == 0, "nothing attends to the last document's pages"


@pytest.mark.parametrize("seed", range(3))
def test_mass_row_sums_to_the_valid_query_count_and_matches_the_full_matrix(seed):
    """The one-row evaluation: each query's probabilities sum to one (so the row sums to the
    tile's valid query count), and it agrees with the whole-request evaluation."""
    case = W.random_small_case(20 + seed, max_requests=2, max_docs=3, max_tiles=3, hq=4, hkv=2, d=16)
    M = E.tile_masses(case)
    valid = E.valid_tokens(case).reshape(-1, 64).sum(axis=1)
    for h in range(case.num_q_heads):
        for g in range(M.shape[1]):
            row = E.tile_mass_row(case, h, g)
            assert abs(row.sum() - valid[g]) < 1e-9
            assert np.allclose(row, M[h, g], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_masses_equal_sdpa_probabilities(seed):
    """torch's scaled_dot_product_attention (fp64, CPU) with V = the identity returns the softmax
    probability matrix itself.  The GQA map repeats each KV head over its q heads, and the mask is
    causal over the valid keys.  Summed over 64 x 64 blocks, these must be the oracle's masses."""
    import torch
    case = W.random_small_case(40 + seed, max_requests=2, max_docs=3, max_tiles=3, hq=4, hkv=2, d=16)
    M = E.tile_masses(case)
    tile_req, _, _, req_first, _, _ = E._segments(case)
    valid = torch.from_numpy(E.valid_tokens(case))
    q = torch.from_numpy(W.bf16_bits_to_f32(case.q).astype(np.float64))
    k = torch.from_numpy(W.bf16_bits_to_f32(case.k).astype(np.float64))
    group = case.num_q_heads // case.num_kv_heads
    for b in range(len(case.req_num_docs)):
        t0 = int(req_first[b])
        nt = int((tile_req == b).sum())
        s0, s1 = 64 * t0, 64 * (t0 + nt)
        n = s1 - s0
        qb = q[s0:s1].permute(1, 0, 2)
        kb = k[s0:s1].permute(1, 0, 2).repeat_interleave(group, dim=0)
        vb = torch.eye(n, dtype=torch.float64).expand(case.num_q_heads, n, n)
        ok = valid[s0:s1]
        mask = torch.tril(torch.ones(n, n, dtype=torch.bool)) & ok[None, :]
        mask |= ~ok[:, None]  # padded queries: any non-empty row (zeroed below)
        p = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask)
        p[:, ~ok, :] = 0.0
        want = p.reshape(case.num_q_heads, nt, 64, nt, 64).sum(dim=(2, 4)).numpy()
        assert np.allclose(M[:, t0:t0 + nt, t0:t0 + nt], want, rtol=0, atol=1e-10)


def test_select_bits_hand_worked():
    """Two documents of 3 and 2 tiles, one question tile, one head; dyadic masses (exact in
    float32), p_la = 0.5, p_ca = 0.4.  Worked by hand:
      doc 0, LA row 1: 0.625 | 0.375 -> c0 reaches 0.5 -> {0}, plus the diagonal -> {0, 1};
      doc 0, LA row 2: 0.125 | 0.25 | 0.625 -> c2 alone reaches 0.5 -> {2}, plus tile 0 -> {0, 2};
      doc 0, CA: the later document's query tiles 3 and 4 give pages 0.25 | 0.625 | 0.75
                 (total 1.625, threshold 0.65): page 2 alone reaches it -> {2} plus page 0;
                 the question tile (2.0 on page 1) and doc 0's own rows do not count;
      doc 1: rows of at most two tiles are all forced; its CA pages have no reader -> {0}."""
    case = W.make_case("hand", 1, [2], [192, 128], [64], 1, 1, 64, np.full((1, 1), 0.5), np.full((1, 1), 0.5))
    M = np.zeros((1, 6, 6))
    M[0, 0, 0] = 3.0
    M[0, 1, :2] = [0.625, 0.375]
    M[0, 2, :3] = [0.125, 0.25, 0.625]
    M[0, 3, :4] = [0.125, 0.5, 0.25, 0.125]
    M[0, 4, :5] = [0.125, 0.125, 0.5, 0.25, 0.75]
    M[0, 5, :6] = [0.0, 2.0, 0.0, 0.5, 0.5, 1.0]
    la, ca = E.select_bits(case, M, 0.5, 0.4)
    want_la0 = np.array([[1, 0, 0], [1, 1, 0], [1, 0, 1]], bool)
    want_la1 = np.array([[1, 0], [1, 1]], bool)
    np.testing.assert_array_equal(la[0][0], want_la0)
    np.testing.assert_array_equal(la[1][0], want_la1)
    np.testing.assert_array_equal(ca[0][0], [True, False, True])
    np.testing.assert_array_equal(ca[1][0], [True, False])


@pytest.mark.parametrize("seed,hq,hkv", [(60, 4, 2), (61, 3, 1), (62, 2, 2), (63, 8, 2)])
def test_masses_by_tile_equal_the_whole_request_evaluation(seed, hq, hkv):
    """The per-(query tile, KV head) evaluation used at full size gives the whole-request
    matrices (ragged documents and questions, padded queries and keys, GQA)."""
    case = W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=4, hq=hq, hkv=hkv, d=16)
    np.testing.assert_allclose(E.tile_masses_by_tile(case, threads=3), E.tile_masses(case), rtol=0, atol=1e-12)
