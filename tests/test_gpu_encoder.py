"""GPU parity of the offline encoder (sift_tile_masses, sift_select_bits) against oracle/encoder.py.

Masses: fp32 kernel vs the fp64 oracle, on every causal entry.  Both sides take the same bf16
operands.  The scores are exact products summed in fp32 and the probabilities come from exp2
in fp32.  A tile mass sums at most 64 x 64 probabilities, and each query's probabilities sum to
one.  So the absolute error of a mass is about (valid queries) x (a few fp32 ulps of 1):
atol 2e-5 plus rtol 1e-4.

Bits, against the oracle: the oracle selects in fp64 from its own fp64 masses.  The GPU selects
from its fp32 masses.  Rows are compared one by one with tests/encoder_compare.py.  A row whose
decision cannot move under any mass error inside the asserted tolerance (plus the fp32
rounding of the threshold test) must match exactly.  A row inside that margin may differ, but
only as another top-p selection within the margin.  At most 0.1 % of the rows may differ.

Bits, kernel unit test: tests/encoder_kernel_model.py replays the selection kernel's fp32
arithmetic (sort, Hillis-Steele scan, cut, forced tiles) on the GPU's own masses and must give
the same words.  This isolates the selection kernel; it is not the oracle check.
"""
import numpy as np
import pytest
import torch

import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from oracle import encoder as E

import encoder_compare as C
import encoder_kernel_model as KM
from gpu_common import DEV, config, values_tensor

pytestmark = pytest.mark.gpu

ATOL, RTOL = C.ATOL, C.RTOL


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


def _assert_masses(case, got, want):
    tile_req, _, _, req_first, _, _ = E._segments(case)
    worst = 0.0
    for g in range(len(tile_req)):
        t0 = int(req_first[tile_req[g]])
        a, b = got[:, g, t0:g + 1].astype(np.float64), want[:, g, t0:g + 1]
        np.testing.assert_allclose(a, b, rtol=RTOL, atol=ATOL, err_msg=f"masses of query tile {g}")
        worst = max(worst, float(np.max(np.abs(a - b) / (ATOL + RTOL * np.abs(b)), initial=0.0)))
    return worst


def _gpu_select(lay, plan, masses, p_la, p_ca):
    la, ca = sift.select_bits(lay, masses, p_la, p_ca, plan=plan)
    torch.cuda.synchronize()
    la = la.cpu().numpy().view(np.uint32)[: lay.la_words]
    ca = ca.cpu().numpy().view(np.uint32)[: lay.ca_words]
    return la, ca


def _unpack(case, la_words, ca_words):
    """GPU words -> per-doc booleans ([Hq, T, T], [Hq, T]) in the input bit format."""
    _, _, _, _, _, doc_T = E._segments(case)
    hq = case.num_q_heads
    la, ca, lo, co = [], [], 0, 0
    for T in doc_T:
        T = int(T)
        nla, nca = -(-(T * (T + 1) // 2) // 32), -(-T // 32)
        rows, cols = np.tril_indices(T)
        la_d = np.zeros((hq, T, T), bool)
        ca_d = np.zeros((hq, T), bool)
        for h in range(hq):
            w = la_words[lo:lo + nla]
            bits = np.unpackbits(w.astype("<u4").view(np.uint8), bitorder="little")[: rows.size].astype(bool)
            la_d[h][rows, cols] = bits
            w = ca_words[co:co + nca]
            ca_d[h] = np.unpackbits(w.astype("<u4").view(np.uint8), bitorder="little")[:T].astype(bool)
            lo += nla
            co += nca
        la.append(la_d)
        ca.append(ca_d)
    return la, ca


def _check_bits_against_oracle(case, M_oracle, la_w, ca_w, p_la, p_ca, what):
    la_b, ca_b = _unpack(case, la_w, ca_w)
    res = C.compare(case, M_oracle, la_b, ca_b, p_la, p_ca)
    print(f"{what} p=({p_la}, {p_ca}): {res['rows']} rows, {res['fragile']} inside the margin, "
          f"{res['differ']} differ from the oracle", flush=True)
    assert res["differ"] <= res["rows"] // 1000, f"{what}: too many rows differ: {res}"
    return res


def _check_bits_kernel_model(case, M_gpu, la_w, ca_w, p_la, p_ca):
    la_b, ca_b = KM.select_bits_fp32(case, M_gpu, p_la, p_ca)
    want_la, want_ca = W.pack_bits(la_b, ca_b)
    np.testing.assert_array_equal(la_w, want_la)
    np.testing.assert_array_equal(ca_w, want_ca)


def _small(seed, d, hq=4, hkv=2, **kw):
    return W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=4, hq=hq, hkv=hkv, d=d, **kw)


@pytest.mark.parametrize("seed,d", [(0, 64), (1, 128), (2, 64), (3, 128), (4, 128)])
def test_masses_and_bits_small(seed, d):
    case = _small(seed, d)
    print(f"encoder small seed={seed} d={d}", flush=True)
    lay, plan, m = _gpu_masses(case)
    got = _full(case, m.cpu().numpy())
    want = E.tile_masses(case)
    _assert_masses(case, got, want)
    for p_la, p_ca in ((0.9, 0.9), (0.5, 0.3), (1.0, 1.0)):
        la, ca = _gpu_select(lay, plan, m, p_la, p_ca)
        _check_bits_against_oracle(case, want, la, ca, p_la, p_ca, f"small {seed}")
        _check_bits_kernel_model(case, got, la, ca, p_la, p_ca)


@pytest.mark.parametrize("seed,hq,hkv,d", [(10, 3, 1, 128), (11, 2, 2, 64), (12, 8, 1, 64), (13, 4, 1, 128),
                                          (14, 1, 1, 128), (15, 16, 2, 64)])
def test_masses_gqa_groupings(seed, hq, hkv, d):
    """Workgroups take 1, 2 or 4 q heads of a KV head (and several groups when the GQA group is
    larger than 4): every grouping gives the oracle's masses."""
    case = _small(seed, d, hq=hq, hkv=hkv)
    print(f"encoder groups seed={seed} hq={hq} hkv={hkv} d={d}", flush=True)
    lay, plan, m = _gpu_masses(case)
    _assert_masses(case, _full(case, m.cpu().numpy()), E.tile_masses(case))


@pytest.mark.parametrize("hq,hkv", [(4, 1), (2, 1), (1, 1)])
def test_masses_with_score_jumps(hq, hkv):
    """Key tiles scaled by powers of two (exact in bf16): a query's largest score jumps by far
    more than 64 (in log2 units) from one tile to the next and falls back after, so the kernel
    moves its reference several times within a row, scales the entries it already holds (some of
    them to zero), and the masses still match the oracle's.  Pairs of neighbouring tiles share a
    scale, so the mass of a row splits between tiles stored before and after a move.  One request
    of 11 tiles, two documents and a question."""
    rng = np.random.default_rng(31)
    case = W.make_case("jumps", 31, [2], [64 * 5, 64 * 4 - 9], [90], hq, hkv, 64,
                       np.full((1, hq), 0.3), np.full((1, hq), 0.3), rng=rng)
    k = W.bf16_bits_to_f32(case.k)
    for t, f in enumerate([1, 64, 1, 256, 256, 1, 1024, 1024, 4, 1, 1]):
        k[64 * t:64 * (t + 1)] *= f
    case.k = W.f32_to_bf16_bits(k)
    assert np.array_equal(W.bf16_bits_to_f32(case.k), k)  # the scaling is exact
    print(f"encoder score jumps hq={hq} hkv={hkv}", flush=True)
    lay, plan, m = _gpu_masses(case)
    _assert_masses(case, _full(case, m.cpu().numpy()), E.tile_masses(case))


def _long_doc_case(doc_tiles, seed=5):
    """One request, documents of the given tile counts (the last one ragged), a short question."""
    lens = [64 * t for t in doc_tiles]
    lens[-1] -= 17
    rng = np.random.default_rng(seed)
    return W.make_case(f"long-{seed}", seed, [len(lens)], lens, [70], 2, 1, 64,
                       np.full((1, 2), 0.3), np.full((1, 2), 0.3), rng=rng)


def test_select_bits_long_documents_and_ties():
    """Documents of up to 64 tiles (65 LA words per vector).  The masses are given: multiples of
    1/8, exact in fp32, and so is every partial sum of them here (all below 2^13).  The p values
    are dyadic, so p x total is exact in fp32 and fp64 alike, and the fp32 kernel and the fp64
    oracle must make the same decisions word for word, exact hits of the threshold included.
    The many exact ties exercise the tie order (smaller tile first)."""
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
    for p_la, p_ca in ((0.875, 0.875), (0.25, 0.625), (1.0, 1.0)):
        la_b, ca_b = E.select_bits(case, M.astype(np.float64), p_la, p_ca)
        want_la, want_ca = W.pack_bits(la_b, ca_b)
        la, ca = _gpu_select(lay, plan, masses, p_la, p_ca)
        np.testing.assert_array_equal(la, want_la)
        np.testing.assert_array_equal(ca, want_ca)
        _check_bits_kernel_model(case, M, la, ca, p_la, p_ca)


@pytest.mark.parametrize("cid", [2, 4])
def test_encoder_full_size_all_masses_and_bits(cid):
    """Config 2 (32 q / 8 KV heads, 10 x 1024 tokens) and config 4 (64 q / 4 KV heads, 20 x 2048
    tokens): every causal mass against the fp64 oracle, and every head's and document's bits
    against the oracle's own fp64 selection, row by row with the decision margin."""
    case = config(cid)
    print(f"encoder config {cid}: GPU masses", flush=True)
    lay, plan, m = _gpu_masses(case)
    got = _full(case, m.cpu().numpy())
    print(f"encoder config {cid}: oracle masses", flush=True)
    want = E.tile_masses_by_tile(case)
    worst = _assert_masses(case, got, want)
    print(f"encoder config {cid}: masses within tolerance (worst {worst:.3f} of the bound)", flush=True)
    for p_la, p_ca in ((0.9, 0.9), (0.5, 0.5)):
        la, ca = _gpu_select(lay, plan, m, p_la, p_ca)
        _check_bits_against_oracle(case, want, la, ca, p_la, p_ca, f"config {cid}")
        _check_bits_kernel_model(case, got, la, ca, p_la, p_ca)
