"""GPU: seeded random layouts beyond the hand-picked cases -- ragged documents and questions, one to
four requests, up to 150 tiles per document, GQA groups of 1 to 8, head_dim 64 and 128, keys that
grow along the sequence (so the running max rises mid-row) -- through the decode (bit-exact against
the oracle), the CSR prefill (against the fp64 oracle: output, LSE, zero padded rows) and the fused
call (identical to the CSR path)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from gpu_common import (DEV, LSE_ABS, MAX_ABS, MEAN_ABS, gpu_decode, gpu_prefill, valid_tokens, values_tensor,
                        words_tensor)

pytestmark = pytest.mark.gpu

GROUPS = [(1, 1), (2, 1), (4, 2), (8, 2), (8, 8), (6, 3), (16, 4), (4, 4)]


def _fused(case):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    q, k, v = (values_tensor(case, x) for x in (case.q, case.k, case.v))
    out, lse = sift.sparse_prefill_bits(lay, words_tensor(case.la_words), words_tensor(case.ca_words), q, k, v,
                                        plan=plan, want_lse=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("block", range(4))
def test_random_layouts_attention_against_the_oracle(block):
    """Ten small random layouts per block; every third with keys scaled up along the sequence."""
    for seed in range(10 * block, 10 * block + 10):
        rng = np.random.default_rng(seed)
        d = int(rng.choice([64, 128]))
        hq, hkv = GROUPS[seed % len(GROUPS)]
        case = W.random_small_case(5000 + seed, max_requests=int(rng.integers(1, 4)),
                                   max_docs=int(rng.integers(1, 6)), max_tiles=int(rng.integers(1, 9)),
                                   hq=hq, hkv=hkv, d=d)
        if seed % 3 == 1:
            n = case.k.shape[0]
            grow = (1.0 + (3 + seed % 11) * np.arange(n) / n).astype(np.float32)
            case = dataclasses.replace(case, k=W.f32_to_bf16_bits(W.bf16_bits_to_f32(case.k) * grow[:, None, None]))
        print(f"random attention seed {seed}: d={d} hq={hq} hkv={hkv} tokens={case.q.shape[0]}", flush=True)
        rp, ci = gpu_decode(case)
        orp, oci = oracle.decode(case)
        assert np.array_equal(rp, orp) and np.array_equal(ci, oci), f"seed {seed}: CSR differs"
        out, lse = gpu_prefill(case)
        fo, fl = _fused(case)
        assert np.array_equal(fo, out) and np.array_equal(fl, lse), f"seed {seed}: fused differs from the CSR path"
        ref, ref_lse = oracle.attention(case)
        valid = valid_tokens(case)
        err = np.abs(out[valid] - ref[valid])
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, f"seed {seed}: {err.max():.2e} / {err.mean():.2e}"
        assert np.all(out[~valid] == 0), f"seed {seed}: padded rows not zero"
        finite = np.isfinite(ref_lse) & valid[None, :]
        assert np.array_equal(np.isfinite(lse), finite), f"seed {seed}: LSE finiteness differs"
        assert np.abs(lse[finite] - ref_lse[finite]).max() <= LSE_ABS, f"seed {seed}: LSE"


@pytest.mark.parametrize("block", range(3))
def test_random_long_layouts_decode_and_fused(block):
    """Larger random layouts (up to 150-tile documents, up to 11 documents per request), some past
    the single-launch decode's bounds: CSR bit-exact, and the fused call equal to the CSR path."""
    for seed in range(8 * block, 8 * block + 8):
        rng = np.random.default_rng(seed)
        hq, hkv = [(1, 1), (4, 1), (8, 2), (16, 2), (32, 8)][seed % 5]
        max_tiles = int(rng.choice([8, 40, 70, 150]))
        case = W.random_small_case(20000 + seed, max_requests=int(rng.integers(1, 5)),
                                   max_docs=int(rng.integers(1, 12)), max_tiles=max_tiles, hq=hq, hkv=hkv, d=64)
        print(f"random long layout seed {seed}: hq={hq} G={case.q.shape[0] // 64} docs={len(case.doc_len)}", flush=True)
        rp, ci = gpu_decode(case)
        orp, oci = oracle.decode(case)
        assert np.array_equal(rp, orp) and np.array_equal(ci, oci), f"seed {seed}: CSR differs"
        if seed % 2 == 0:
            out, lse = gpu_prefill(case)
            fo, fl = _fused(case)
            assert np.array_equal(fo, out) and np.array_equal(fl, lse), f"seed {seed}: fused differs"
