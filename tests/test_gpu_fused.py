"""GPU: sparse prefill with the decode fused in (sift_sparse_prefill_bits) gives exactly the
result of sift_decode_bits + sift_sparse_prefill on the same bits, and matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from gpu_common import (DEV, assert_close, assert_full_parity, config, gpu_prefill, oracle_full,
                        valid_tokens, values_tensor, words_tensor)

pytestmark = pytest.mark.gpu


def fused_prefill(case, want_lse=True):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    la, ca = words_tensor(case.la_words), words_tensor(case.ca_words)
    q, k, v = (values_tensor(case, x) for x in (case.q, case.k, case.v))
    out, lse = sift.sparse_prefill_bits(lay, la, ca, q, k, v, plan=plan, want_lse=want_lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def _same_as_csr_path(case):
    out_f, lse_f = fused_prefill(case)
    out_c, lse_c = gpu_prefill(case)
    assert np.array_equal(out_f, out_c), "fused output differs from the CSR path"
    assert np.array_equal(lse_f, lse_c), "fused LSE differs from the CSR path"
    return out_f, lse_f


@pytest.mark.parametrize("seed", range(8))
def test_fused_random_small(seed):
    d = 64 if seed % 2 else 128
    hq, hkv = [(1, 1), (4, 2), (8, 8), (6, 3)][seed % 4]
    case = W.random_small_case(400 + seed, max_requests=3, max_docs=4, max_tiles=6, hq=hq, hkv=hkv, d=d)
    out, _ = _same_as_csr_path(case)
    ref, _ = oracle.attention(case)
    valid = valid_tokens(case)
    assert_close(out[valid], ref[valid], case.name)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_fused_configs_same_as_csr(cid):
    _same_as_csr_path(config(cid))


def test_fused_config2_every_element_against_the_oracle():
    """The fused call on workload 2 against the fp64 oracle directly (every valid output and
    LSE), not only against the CSR path."""
    case = config(2)
    out, lse = fused_prefill(case)
    ref, ref_lse = oracle_full(2)
    assert_full_parity(case, out, lse, ref, ref_lse, "fused, config 2")


def test_fused_long_documents_multiword_rows():
    """A 150-tile document: LA rows span up to 5 words and rows list more than 64 tiles, so the
    kernel crosses list chunks it builds itself; two more documents give CA prefixes."""
    case = W.make_case("long-docs", 1500, [3], [150 * 64 - 17, 80 * 64, 900], [300], 4, 2, 128,
                       np.full((1, 4), 0.5), np.full((1, 4), 0.4))
    rp, _ = oracle.decode(case)
    assert np.diff(rp).max() > 128
    out, lse = _same_as_csr_path(case)
    rng = np.random.default_rng(3)
    valid = np.where(valid_tokens(case))[0]
    toks = np.concatenate([rng.choice(valid, 600), valid[-64:]]).astype(np.int64)
    heads = rng.integers(0, case.num_q_heads, size=toks.size).astype(np.int32)
    ref, _ = oracle.attention(case, heads=heads, tokens=toks)
    assert_close(out[toks, heads], ref, "long docs")


@pytest.mark.parametrize("name,req_num_docs,doc_tiles,question_len,hq", [
    ("at_bounds", [512], [4] * 512, [0], 1),             # G 2048, 512 documents: the single launch
    ("ca_words_past_bound", [300], [1] * 300, [64], 8),  # 2400 CA words: transpose + two launches
])
def test_fused_at_and_past_the_single_launch_bounds(name, req_num_docs, doc_tiles, question_len, hq):
    """The fused call's decode at the single-launch decode's limits (its workgroups then share the
    launch with the V^T transpose) and just past one of them: equal to the CSR path, and sampled
    rows match the oracle."""
    doc_len = [64 * t - (i % 7) for i, t in enumerate(doc_tiles)]
    r = len(req_num_docs)
    case = W.make_case(name, 12, req_num_docs, doc_len, question_len, hq, 1, 64,
                       np.full((r, hq), 0.3), np.full((r, hq), 0.2))
    print(f"fused {name}: G={case.q.shape[0] // 64} docs={len(doc_len)}", flush=True)
    out, _ = _same_as_csr_path(case)
    rng = np.random.default_rng(7)
    valid = np.where(valid_tokens(case))[0]
    toks = np.concatenate([rng.choice(valid, 300), valid[-64:]]).astype(np.int64)
    heads = rng.integers(0, case.num_q_heads, size=toks.size).astype(np.int32)
    ref, _ = oracle.attention(case, heads=heads, tokens=toks)
    assert_close(out[toks, heads], ref, name)


def test_fused_long_document():
    """A document of 2,000 tiles (its decode takes the two-launch path): the fused call equals the
    CSR path, and sampled rows match the oracle."""
    case = W.make_case("doc-limit", 1984, [1], [2000 * 64], [64], 2, 1, 64,
                       np.full((1, 2), 0.02), np.full((1, 2), 0.02))
    out, _ = _same_as_csr_path(case)
    rng = np.random.default_rng(5)
    valid = np.where(valid_tokens(case))[0]
    toks = np.concatenate([rng.choice(valid, 200), valid[-128:]]).astype(np.int64)
    heads = rng.integers(0, case.num_q_heads, size=toks.size).astype(np.int32)
    ref, _ = oracle.attention(case, heads=heads, tokens=toks)
    assert_close(out[toks, heads], ref, "long document")


def test_fused_empty_and_dense_bits():
    case = W.random_small_case(450, max_requests=2, max_docs=3, max_tiles=5, hq=4, hkv=2, d=64)
    empty = W.with_bits(case, [np.zeros_like(x) for x in case.la_bool], [np.zeros_like(x) for x in case.ca_bool])
    _same_as_csr_path(empty)
    dense = W.with_bits(case, *W.all_ones_bits(case))
    out, _ = _same_as_csr_path(dense)
    ref, _ = oracle.attention(dense)
    valid = valid_tokens(dense)
    assert_close(out[valid], ref[valid], "dense")


def test_fused_fp32_inputs():
    case = config(1)
    out, _ = _same_as_csr_path(case)
