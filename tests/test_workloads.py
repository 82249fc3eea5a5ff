"""The seeded generator: shapes, determinism and realised statistics (P9)."""
import numpy as np
import pytest

from bit_vector_block_amd import workloads as W
from helpers import TokenMap, expected_counts_closed_form


def test_config_shapes_small():
    c = W.config_case(1)
    assert c.dtype == "fp32" and c.q.shape == (576, 1, 64) and c.k.shape == (576, 1, 64)
    assert c.la_words.size == 2 * 1 and c.ca_words.size == 2
    assert c.la_bool[0].shape == (1, 4, 4)


def test_config2_shapes_and_determinism():
    a = W.config_case(2)
    assert a.q.shape == (10368, 32, 128) and a.k.shape == (10368, 8, 128)
    assert a.q.dtype == np.uint16
    # 10 docs x 32 heads x ceil(136/32)=5 LA words; 1 CA word each
    assert a.la_words.size == 10 * 32 * 5 and a.ca_words.size == 10 * 32
    b = W.config_case(2)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.la_words, b.la_words)


def test_config2_realised_density_near_expectation():
    """P9: LA bits ~ Bernoulli(0.25) off the diagonal, CA ~ Bernoulli(0.2) off page 0, and the
    realised nnz lies within a few sigma of its expectation."""
    c = W.config_case(2)
    la_off = np.concatenate([x[:, np.tril_indices(16, -1)[0], np.tril_indices(16, -1)[1]].ravel() for x in c.la_bool])
    ca_off = np.concatenate([x[:, 1:].ravel() for x in c.ca_bool])
    for arr, p in ((la_off, 0.25), (ca_off, 0.20)):
        sigma = np.sqrt(p * (1 - p) / arr.size)
        assert abs(arr.mean() - p) < 5 * sigma
    tm = TokenMap(c)
    nnz = int(expected_counts_closed_form(c, tm).sum())
    # expectation: per head, doc rows sum_r (1 + 0.25 r) + sum_d 16 d (1 + 0.2*15)/16 ... (see DESIGN)
    e_la = 16 + 0.25 * 120
    e_ca_doc = 1 + 0.2 * 15
    e_row_doc = 10 * e_la + sum(16 * d * e_ca_doc for d in range(10))
    e_q = sum(160 + j + 1 for j in range(2))
    expected = 32 * (e_row_doc + e_q)
    assert expected == pytest.approx(117216, abs=1)
    # variance: CA bit of doc i (i < 9) counts in the 16*(9-i) rows of later docs; LA bits once
    var_head = sum((16 * (9 - i)) ** 2 * 15 * 0.2 * 0.8 for i in range(9)) + 10 * 120 * 0.25 * 0.75
    sigma = np.sqrt(32 * var_head)
    assert abs(nnz - expected) < 5 * sigma


def test_ragged_config_layout_rules():
    c = W.config_case(5)
    assert len(c.req_num_docs) == 4
    d = 0
    for b, k in enumerate(c.req_num_docs):
        assert 1 <= k <= 40
        lens = c.doc_len[d:d + k]
        assert np.all((lens >= 300) & (lens <= 3000))
        assert 64 <= c.question_len[b] <= 512
        total = sum(64 * -(-int(n) // 64) for n in lens) + 64 * -(-int(c.question_len[b]) // 64)
        assert total <= 65536
        d += k
    assert c.q.shape[0] == W.padded_total(c.req_num_docs, c.doc_len, c.question_len)
