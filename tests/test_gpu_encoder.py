"""GPU parity of the offline encoder (sift_tile_masses, sift_select_bits) against oracle/encoder.py.

Masses: fp32 kernel vs the fp64 oracle.  Both sides take the same bf16 operands.  The scores are
exact products summed in fp32 and the probabilities come from exp2 in fp32.  A tile mass sums at
most 64 x 64 probabilities, and each query's probabilities sum to one.  So the absolute error of
a mass is bounded by about (valid queries) x (a few fp32 ulps of 1): atol 2e-5 plus rtol 1e-4.

Bits: the selection is an integer decision made from fp32 sums, so the oracle takes the GPU's
fp32 masses as its input.  It makes the decision in the kernel's precision and summation order,
and the words must be equal bit for bit.
"""
import numpy as np
import pytest
import torch

import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from oracle import encoder as E

from gpu_common import DEV, config, values_tensor

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-5, 1e-4


def _gpu_masses(case):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    q, k = values_tensor(case, case.q), values_tensor(case, case.k)
    m = sift.tile_masses(lay, q, k, plan=plan)
    torch.cuda.synchronize()
    return lay, plan, m


def _full(case, m_rt):
    """Scatter [Hq, G, RT] (entry c - first tile of the request) into [Hq, G, G]; only the causal
    entries of each request are defined."""
    tile_req, _, _, req_first, _, _ = E._segments(case)
    hq, G = m_rt.shape[0], len(tile_req)
    M = np.zeros((hq, G, G), np.float32)
    for g in range(G):
        t0 = int(req_first[tile_req[g]])
        M[:, g, t0:g + 1] = m_rt[:, g, : g + 1 - t0]
    return M


def _gpu_select(lay, plan, masses, p_la, p_ca):
    la, ca = sift.select_bits(lay, masses, p_la, p_ca, plan=plan)
    torch.cuda.synchronize()
    la = la.cpu().numpy().view(np.uint32)[: lay.la_words]
    ca = ca.cpu().numpy().view(np.uint32)[: lay.ca_words]
    return la, ca


def _small(seed, d, hq=4, hkv=2, **kw):
    return W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=4, hq=hq, hkv=hkv, d=d, **kw)


@pytest.mark.parametrize("seed,d", [(0, 64), (1, 128), (2, 64), (3, 128), (4, 128)])
def test_masses_and_bits_small(seed, d):
    case = _small(seed, d)
    print(f"encoder small seed={seed} d={d}", flush=True)
    lay, plan, m = _gpu_masses(case)
    got = _full(case, m.cpu().numpy())
    want = E.tile_masses(case)
    tile_req, _, _, req_first, _, _ = E._segments(case)
    for g in range(len(tile_req)):
        t0 = int(req_first[tile_req[g]])
        np.testing.assert_allclose(got[:, g, t0:g + 1], want[:, g, t0:g + 1], rtol=RTOL, atol=ATOL)
    for p_la, p_ca in ((0.9, 0.9), (0.5, 0.3), (1.0, 1.0)):
        la_b, ca_b = E.select_bits(case, got, p_la, p_ca)
        want_la, want_ca = W.pack_bits(la_b, ca_b)
        la, ca = _gpu_select(lay, plan, m, p_la, p_ca)
        np.testing.assert_array_equal(la, want_la)
        np.testing.assert_array_equal(ca, want_ca)


@pytest.mark.parametrize("seed,hq,hkv,d", [(10, 3, 1, 128), (11, 2, 2, 64), (12, 8, 1, 64), (13, 4, 1, 128),
                                          (14, 1, 1, 128), (15, 16, 2, 64)])
def test_masses_gqa_groupings(seed, hq, hkv, d):
    """Workgroups take 1, 2 or 4 q heads of a KV head (and several groups when the GQA group is
    larger than 4): every grouping gives the oracle's masses."""
    case = _small(seed, d, hq=hq, hkv=hkv)
    print(f"encoder groups seed={seed} hq={hq} hkv={hkv} d={d}", flush=True)
    lay, plan, m = _gpu_masses(case)
    got = _full(case, m.cpu().numpy())
    want = E.tile_masses(case)
    tile_req, _, _, req_first, _, _ = E._segments(case)
    for g in range(len(tile_req)):
        t0 = int(req_first[tile_req[g]])
        np.testing.assert_allclose(got[:, g, t0:g + 1], want[:, g, t0:g + 1], rtol=RTOL, atol=ATOL)


def _long_doc_case(doc_tiles, seed=5):
    """One request, documents of the given tile counts (the last one ragged), a short question."""
    lens = [64 * t for t in doc_tiles]
    lens[-1] -= 17
    rng = np.random.default_rng(seed)
    return W.make_case(f"long-{seed}", seed, [len(lens)], lens, [70], 2, 1, 64,
                       np.full((1, 2), 0.3), np.full((1, 2), 0.3), rng=rng)


def test_select_bits_long_documents_and_ties():
    """Documents of up to 64 tiles (65 LA words per vector).  Synthetic masses have many exact
    ties, which exercises the tie order (smaller tile first) and the fp32 scan."""
    case = _long_doc_case([64, 40, 9])
    print("encoder select long docs", flush=True)
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    rt = sift.encode_masses_bytes(lay) // (4 * lay.num_q_heads * lay.num_tiles)
    rng = np.random.default_rng(77)
    m_rt = (rng.integers(0, 9, size=(lay.num_q_heads, lay.num_tiles, rt)) / 8.0).astype(np.float32)
    m_rt[0, 5, :] = 0.0   # a row of zeros: only the forced tiles
    masses = torch.from_numpy(m_rt).to(DEV)
    M = _full(case, m_rt)
    for p_la, p_ca in ((0.9, 0.9), (0.25, 0.6), (1.0, 1.0)):
        la_b, ca_b = E.select_bits(case, M, p_la, p_ca)
        want_la, want_ca = W.pack_bits(la_b, ca_b)
        la, ca = _gpu_select(lay, plan, masses, p_la, p_ca)
        np.testing.assert_array_equal(la, want_la)
        np.testing.assert_array_equal(ca, want_ca)


def test_encoder_config2_sampled_rows_and_all_bits():
    """The 10 x 1024-token workload (32 q heads, 8 KV heads, D 128).  The masses are checked on
    sampled (head, query tile) rows.  The bits are checked on every head and document, and their
    CSR must decode."""
    case = config(2)
    print("encoder config 2", flush=True)
    lay, plan, m = _gpu_masses(case)
    m_np = m.cpu().numpy()
    got = _full(case, m_np)
    rng = np.random.default_rng(2024)
    G = lay.num_tiles
    samples = [(0, 0), (31, G - 1), (5, 16), (17, 150)] + [
        (int(rng.integers(0, 32)), int(rng.integers(0, G))) for _ in range(4)]
    for h, g in samples:
        want = E.tile_mass_row(case, h, g)
        np.testing.assert_allclose(got[h, g, : g + 1], want[: g + 1], rtol=RTOL, atol=ATOL,
                                   err_msg=f"row h={h} g={g}")
    la_b, ca_b = E.select_bits(case, got, 0.9, 0.9)
    want_la, want_ca = W.pack_bits(la_b, ca_b)
    la, ca = _gpu_select(lay, plan, m, 0.9, 0.9)
    np.testing.assert_array_equal(la, want_la)
    np.testing.assert_array_equal(ca, want_ca)


def test_encoder_config4_sampled_rows_and_all_bits():
    """The Qwen3-235B shape (64 q heads, 4 KV heads: four groups of four q heads per KV head,
    20 documents of 2048 tokens): masses on sampled rows, every head's bits."""
    case = config(4)
    print("encoder config 4", flush=True)
    lay, plan, m = _gpu_masses(case)
    got = _full(case, m.cpu().numpy())
    rng = np.random.default_rng(4044)
    G = lay.num_tiles
    samples = [(0, 0), (63, G - 1), (17, 40), (46, 333)] + [
        (int(rng.integers(0, 64)), int(rng.integers(0, G))) for _ in range(4)]
    for h, g in samples:
        want = E.tile_mass_row(case, h, g)
        np.testing.assert_allclose(got[h, g, : g + 1], want[: g + 1], rtol=RTOL, atol=ATOL,
                                   err_msg=f"row h={h} g={g}")
    la_b, ca_b = E.select_bits(case, got, 0.9, 0.9)
    want_la, want_ca = W.pack_bits(la_b, ca_b)
    la, ca = _gpu_select(lay, plan, m, 0.9, 0.9)
    np.testing.assert_array_equal(la, want_la)
    np.testing.assert_array_equal(ca, want_ca)
