"""GPU: the allocation-free decode (sift_decode_bits_noalloc, through the C ABI) against
sift_decode_bits on the same bits, bit for bit, on calls in a row whose sizes shrink.  Its scratch
is one array per GPU that keeps the last call's contents, so a smaller call after a larger one
must not see the larger one's leftovers."""
import numpy as np
import pytest
import torch

import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from gpu_common import DEV, config, words_tensor

pytestmark = pytest.mark.gpu


def _both(case):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    la, ca = words_tensor(case.la_words), words_tensor(case.ca_words)
    rp_ref, ci_ref = sift.decode_bits(lay, la, ca, plan=plan)
    rp = torch.full((lay.num_rows + 1,), -3, dtype=torch.int32, device=DEV)
    ci = torch.full((max(lay.csr_max_nnz, 1),), -3, dtype=torch.int32, device=DEV)
    sift.decode_bits_noalloc(lay, la, ca, plan, rp, ci)
    torch.cuda.synchronize()
    nnz = int(rp_ref[-1])
    assert torch.equal(rp, rp_ref), f"{case.name}: row_ptr differs"
    assert torch.equal(ci[:nnz], ci_ref[:nnz]), f"{case.name}: col_idx differs"
    return nnz


def test_noalloc_decode_equals_decode_on_shrinking_calls():
    cases = [config(5), config(2),
             W.random_small_case(77, max_requests=3, max_docs=4, max_tiles=5, hq=3, hkv=1, d=64),
             config(1)]
    for case in cases:
        print(f"noalloc decode: {case.name} (G={case.q.shape[0] // 64}, Hq={case.num_q_heads})", flush=True)
        nnz = _both(case)
        print(f"  nnz {nnz}: identical", flush=True)
