"""GPU: the multi-layer pipeline (per-layer bits from pinned host memory, copied ahead on a side
stream) gives, layer by layer, exactly the single-layer result, which matches the oracle."""
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


def test_pipeline_single_layer_and_reuse():
    """A one-layer stack (no look-ahead copies or decodes), and one pipeline run three times in a
    row with different output buffers: the slots reused across runs must give the same outputs."""
    base = W.random_small_case(310, max_requests=2, max_docs=3, max_tiles=5, hq=4, hkv=2, d=64)
    lay = sift.Layout.from_case(base)
    q, k, v = (values_tensor(base, x) for x in (base.q, base.k, base.v))
    bits1 = W.pack_bits(*W.layer_bits(base, 0, 0.5, 0.4))
    one = LayerPipeline(lay, DEV, [bits1[0]], [bits1[1]])
    outs, _ = one.run([q], [k], [v])
    torch.cuda.synchronize()
    single, _ = gpu_prefill(W.with_bits(base, *W.layer_bits(base, 0, 0.5, 0.4)), want_lse=False)
    assert np.array_equal(outs[0].cpu().numpy(), single)

    L = 5
    packed = [W.pack_bits(*W.layer_bits(base, layer, 0.35, 0.3)) for layer in range(L)]
    pipe = LayerPipeline(lay, DEV, [p[0] for p in packed], [p[1] for p in packed])
    runs = []
    for _ in range(3):
        outs, lses = pipe.run([q] * L, [k] * L, [v] * L,
                              lse_per_layer=[torch.empty((lay.num_q_heads, lay.padded_tokens),
                                                         dtype=torch.float32, device=DEV) for _ in range(L)])
        runs.append(([o.cpu().numpy() for o in outs], [x.cpu().numpy() for x in lses]))
    torch.cuda.synchronize()
    for r in runs[1:]:
        for layer in range(L):
            assert np.array_equal(r[0][layer], runs[0][0][layer]), f"layer {layer} output differs across runs"
            assert np.array_equal(r[1][layer], runs[0][1][layer]), f"layer {layer} LSE differs across runs"
