"""GPU: the multi-layer pipeline (per-layer bits from pinned host memory, copied one layer ahead
on a side stream) gives, layer by layer, exactly the single-layer result, which matches the oracle."""
import numpy as np
import pytest
import torch

import oracle
import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from bit_vector_block_amd.pipeline import LayerPipeline
from gpu_common import DEV, assert_close, gpu_prefill, valid_tokens, values_tensor

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1])
def test_pipeline_layers_match_single_layer_and_oracle(seed):
    base = W.random_small_case(300 + seed, max_requests=2, max_docs=3, max_tiles=5, hq=4, hkv=2, d=128)
    L = 4
    layer_bits = [W.layer_bits(base, layer, 0.4, 0.3) for layer in range(L)]
    packed = [W.pack_bits(la, ca) for la, ca in layer_bits]
    lay = sift.Layout.from_case(base)
    pipe = LayerPipeline(lay, DEV, [p[0] for p in packed], [p[1] for p in packed])
    q, k, v = (values_tensor(base, x) for x in (base.q, base.k, base.v))
    outs, _ = pipe.run([q] * L, [k] * L, [v] * L)
    torch.cuda.synchronize()
    valid = valid_tokens(base)
    results = []
    for layer in range(L):
        case = W.with_bits(base, *layer_bits[layer])
        single, _ = gpu_prefill(case, want_lse=False)
        got = outs[layer].cpu().numpy()
        assert np.array_equal(got, single), f"layer {layer}: pipeline differs from the single-layer call"
        ref, _ = oracle.attention(case)
        assert_close(got[valid], ref[valid], f"layer {layer}")
        results.append(got)
    assert not np.array_equal(results[0], results[1]), "layers with different bits must differ"
