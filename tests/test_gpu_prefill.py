"""GPU sparse prefill vs the fp64 oracle (max-abs 1e-2, mean-abs 1e-3) and exact properties."""
import dataclasses

import numpy as np
import pytest

import oracle
from bit_vector_block_amd import workloads as W
import bit_vector_block_amd as sift
from gpu_common import (LSE_ABS, assert_close, assert_full_parity, config, gpu_decode, gpu_prefill,
                        oracle_full, valid_tokens)

pytestmark = pytest.mark.gpu


def _full_check(case):
    out, lse = gpu_prefill(case)
    ref, ref_lse = oracle.attention(case)
    valid = valid_tokens(case)
    mx, mean = assert_close(out[valid], ref[valid], case.name)
    assert np.all(out[~valid] == 0.0), "padded query rows must be exactly 0"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0.0) <= LSE_ABS
    return mx, mean


def _row_raises(case, rp, ci, h, g, lazy_log2=8.0):
    """How often the running tile max of row (h, g) rises by more than lazy_log2 (log2 units)
    along its list: a property of the input, used to show that a case exercises the rescale."""
    q = W.bf16_bits_to_f32(case.q[g * 64:(g + 1) * 64, h]).astype(np.float64)
    kvh = h // (case.num_q_heads // case.num_kv_heads)
    row = h * ((len(rp) - 1) // case.num_q_heads) + g
    m, raises = None, 0
    for t in ci[rp[row]:rp[row + 1]]:
        k = W.bf16_bits_to_f32(case.k[t * 64:(t + 1) * 64, kvh]).astype(np.float64)
        top = float(np.max(q @ k.T)) * case.scale / np.log(2.0)
        if m is None:
            m = top
        elif top > m + lazy_log2:
            m, raises = top, raises + 1
    return raises


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_growing_scores_exercise_the_lazy_rescale(d):
    """Keys scaled up along the sequence (x1 to x13), so the running max of a row rises by more
    than the lazy threshold many times and O and l are rescaled mid-row.  With N(0, 1) inputs
    that never happens after a row's first tile, so the other cases leave this path unexercised."""
    case = W.make_case(f"growing-{d}", 70 + d, [4], [300, 256, 400, 200], [100], 4, 2, d,
                       np.full((1, 4), 0.6), np.full((1, 4), 0.6))
    n = case.k.shape[0]
    grow = (1.0 + 12.0 * np.arange(n) / n).astype(np.float32)
    k = W.bf16_bits_to_f32(case.k) * grow[:, None, None]
    case = dataclasses.replace(case, k=W.f32_to_bf16_bits(k))
    rp, ci = oracle.decode(case)
    G = (len(rp) - 1) // case.num_q_heads
    raises = [_row_raises(case, rp, ci, h, g) for h in range(case.num_q_heads) for g in range(G)]
    assert sum(raises) >= 20 and max(raises) >= 2, f"the case must raise the max mid-row: {raises}"
    _full_check(case)


def test_prefill_tiny_config_fp32_inputs():
    """Config 1: fp32 Q/K/V, rounded to bf16 on the device, vs the oracle on the same rounding."""
    case = config(1)
    mx, mean = _full_check(case)
    print(f"tiny: max_abs {mx:.3e} mean_abs {mean:.3e}")
    # informational: distance to the oracle on the unrounded fp32 inputs
    out, _ = gpu_prefill(case, want_lse=False)
    exact, _ = oracle.attention(case, exact_fp32=True)
    valid = valid_tokens(case)
    print(f"tiny vs unrounded fp32 oracle: max_abs {np.abs(out[valid] - exact[valid]).max():.3e}")


@pytest.mark.parametrize("seed", range(10))
def test_prefill_random_small(seed):
    d = 64 if seed % 2 else 128
    hq, hkv = [(1, 1), (4, 2), (4, 1), (8, 2), (2, 2)][seed % 5]
    case = W.random_small_case(seed, max_requests=3, max_docs=4, max_tiles=5, hq=hq, hkv=hkv, d=d)
    _full_check(case)


# KV-head counts that exercise each way rows are split over the 8 XCD work queues: Hkv dividing 8
# (heads shared by 8 / Hkv queues, interleaved), 8 dividing Hkv (heads dealt to queues in turn)
# and neither (contiguous eighths of the row order); the small cases also leave queues empty,
# so workgroups drain other queues.
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 16, 64), (6, 3, 128), (12, 6, 64), (5, 5, 128)])
def test_prefill_queue_modes(hq, hkv, d):
    case = W.random_small_case(100 + hq + hkv, max_requests=2, max_docs=3, max_tiles=6, hq=hq, hkv=hkv, d=d)
    _full_check(case)


@pytest.mark.parametrize("seed,layer", [(300, 2), (301, 1), (301, 3)])
def test_prefill_repeat_calls_are_bit_identical(seed, layer):
    """Which workgroup takes a row varies from call to call; the result must not.  (These cases
    once differed between calls in a few queries of a diagonal, partial tile: the max of the
    scores was read from the MFMA result registers too early.)"""
    base = W.random_small_case(seed, max_requests=2, max_docs=3, max_tiles=5, hq=4, hkv=2, d=128)
    case = W.with_bits(base, *W.layer_bits(base, layer, 0.4, 0.3))
    first, first_lse = gpu_prefill(case)
    for _ in range(7):
        again, again_lse = gpu_prefill(case)
        assert np.array_equal(again, first) and np.array_equal(again_lse, first_lse)


def test_prefill_many_rows_per_workgroup():
    """More rows than the 512 persistent workgroups hold at once (every workgroup takes several
    rows, prefetching the next row's tiles during the current row's merge), with 64-entry list
    chunks crossed (rows longer than 64 tiles)."""
    case = W.make_case("many-rows", 1200, [6], [64 * 30] * 6, [200], 8, 2, 64,
                       np.full((1, 8), 0.6), np.full((1, 8), 0.5))
    out, lse = gpu_prefill(case)
    valid = valid_tokens(case)
    rng = np.random.default_rng(5)
    heads, toks = _sample_pairs(case, rng, 800)
    ref, ref_lse = oracle.attention(case, heads=heads, tokens=toks)
    keep = valid[toks]
    assert_close(out[toks, heads][keep], ref[keep], "many rows")
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(lse[heads, toks][fin] - ref_lse[fin]), initial=0.0) <= LSE_ABS
    rp, _ = oracle.decode(case)
    assert (np.diff(rp) > 64).any(), "some row must span more than one 64-entry list chunk"


@pytest.mark.parametrize("seed", range(3))
def test_prefill_all_ones_is_dense_causal(seed):
    case = W.random_small_case(50 + seed, hq=4, hkv=2, d=128, max_tiles=6)
    case = W.with_bits(case, *W.all_ones_bits(case))
    _full_check(case)


def _sample_pairs(case, rng, n_random):
    """(head, token) pairs: random valid tokens, the first and last tiles, a strided sweep."""
    valid = np.where(valid_tokens(case))[0]
    toks = [rng.choice(valid, size=n_random)]
    n = case.q.shape[0]
    # first and last 64 tokens of the sequence, plus a strided sweep
    toks.append(np.arange(0, min(64, n)))
    toks.append(np.arange(max(0, n - 64), n))
    toks.append(np.arange(0, n, 997))
    toks = np.concatenate(toks)
    heads = rng.integers(0, case.num_q_heads, size=toks.size)
    return heads.astype(np.int32), toks.astype(np.int64)


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_prefill_configs_every_element(cid):
    """Workloads 2-4 at full size: every valid (token, head) output and every LSE against the
    fp64 oracle; padded query rows exactly 0."""
    case = config(cid)
    print(f"prefill config {cid}: N={case.q.shape[0]} Hq={case.num_q_heads}", flush=True)
    out, lse = gpu_prefill(case)
    ref, ref_lse = oracle_full(cid)
    assert_full_parity(case, out, lse, ref, ref_lse, f"config {cid}")


def _stratified_rows(case, rp, frac, rng):
    """CSR rows (h, g) of workload 5: in every head, a fraction `frac` of the rows drawn in each
    tenth of the head's row-length order (so short, medium and long rows all appear), plus the
    last question tile of every request in every head (the longest rows)."""
    hq = case.num_q_heads
    G = (len(rp) - 1) // hq
    lengths = np.diff(rp).reshape(hq, G)
    from oracle import encoder as E  # segment tables only
    tile_req, tile_doc, _, _, _, _ = E._segments(case)
    last_q = [g for g in range(G) if tile_doc[g] < 0 and (g + 1 == G or tile_req[g + 1] != tile_req[g])]
    rows = set()
    for h in range(hq):
        order = np.argsort(lengths[h], kind="stable")
        for part in np.array_split(order, 10):
            k = max(1, int(np.ceil(frac * part.size)))
            rows.update((h, int(g)) for g in rng.choice(part, size=k, replace=False))
        rows.update((h, g) for g in last_q)
    return sorted(rows), lengths


def test_prefill_config5_stratified_whole_rows():
    """The ragged batch (4 requests, Beta(2, 8) per-head densities): whole CSR rows (all 64
    queries of a (head, query tile)) for at least 5 % of the rows of every head, stratified by row
    length, and the longest question rows of every request and head."""
    case = config(5)
    print(f"prefill config 5: N={case.q.shape[0]} Hq={case.num_q_heads}", flush=True)
    out, lse = gpu_prefill(case)
    valid = valid_tokens(case)
    assert np.all(np.isfinite(out)), "non-finite output"
    assert np.all(out[~valid] == 0.0), "padded query rows must be exactly 0"
    rp, _ = oracle.decode(case)
    rows, lengths = _stratified_rows(case, rp, 0.05, np.random.default_rng(55))
    assert len(rows) >= 0.05 * lengths.size
    heads = np.repeat(np.array([h for h, _ in rows], np.int32), 64)
    toks = (np.array([g for _, g in rows], np.int64)[:, None] * 64 + np.arange(64)).ravel()
    picked = np.array([lengths[h, g] for h, g in rows])
    print(f"config 5: {len(rows)} of {lengths.size} rows, lengths {picked.min()}..{picked.max()} "
          f"(all rows {lengths.min()}..{lengths.max()})", flush=True)
    assert picked.max() == lengths.max()
    ref, ref_lse = oracle.attention(case, heads=heads, tokens=toks)
    keep = valid[toks]
    mx, mean = assert_close(out[toks, heads][keep], ref[keep], "config 5 rows")
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse[heads, toks]))
    assert np.max(np.abs(lse[heads, toks][fin] - ref_lse[fin]), initial=0.0) <= LSE_ABS
    print(f"config 5: {int(keep.sum())} (token, head) outputs, max_abs {mx:.3e} mean_abs {mean:.3e}")


def test_prefill_config5_sampled_pairs():
    """Extra check of workload 5 on random (head, token) pairs all over the batch."""
    case = config(5)
    out, lse = gpu_prefill(case)
    valid = valid_tokens(case)
    rng = np.random.default_rng(5)
    heads, toks = _sample_pairs(case, rng, 600)
    ref, ref_lse = oracle.attention(case, heads=heads, tokens=toks)
    keep = valid[toks]
    assert_close(out[toks, heads][keep], ref[keep], "config 5 pairs")
    fin = np.isfinite(ref_lse)
    assert np.max(np.abs(lse[heads, toks][fin] - ref_lse[fin]), initial=0.0) <= LSE_ABS


def test_prefill_full_recompute_config2_every_element():
    """Full recompute (every LA and CA bit set, i.e. dense causal attention per request) at the
    10 x 1k-token, 32/8-head, d=128 size, through the same decode and prefill launches: every
    valid output against the oracle."""
    case = config(2)
    case = W.with_bits(case, *W.all_ones_bits(case))
    rp, ci = gpu_decode(case)
    lay = sift.Layout.from_case(case)
    assert rp[-1] == lay.csr_max_nnz, "all-ones bits must give the dense causal tile count"
    out, lse = gpu_prefill(case)
    print("oracle: full recompute of workload 2", flush=True)
    ref, ref_lse = oracle.attention(case)
    assert_full_parity(case, out, lse, ref, ref_lse, "full recompute, config 2")


def test_prefill_single_key_is_exact():
    """P7 on the GPU: the first token of doc 0 sees only itself, so O = v_0 exactly."""
    case = W.make_case("p7", 700, [2], [100, 70], [30], 2, 1, 128, [[0.3, 0.3]], [[0.5, 0.5]])
    out, lse = gpu_prefill(case)
    v0 = W.bf16_bits_to_f32(case.v[0, 0])
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)


def test_prefill_locality_poisoned_tiles():
    """P8: NaN in K/V of every tile a row does not list, NaN in padded K slots and +-1e4 in
    padded V slots leave that row's output finite and bit-identical."""
    case = W.make_case("p8", 800, [3], [150, 64, 100], [40], 2, 1, 128,
                       np.full((1, 2), 0.4), np.full((1, 2), 0.4))
    out0, _ = gpu_prefill(case, want_lse=False)
    rp, ci = oracle.decode(case)
    G = case.q.shape[0] // 64
    valid = valid_tokens(case)
    nan16 = np.uint16(0x7FC0)
    big = W.f32_to_bf16_bits(np.array([1e4], np.float32))[0]
    for h in range(case.num_q_heads):
        for g in range(G):
            listed = set(ci[rp[h * G + g]: rp[h * G + g + 1]].tolist())
            k, v = case.k.copy(), case.v.copy()
            for t in range(G):
                if t not in listed:
                    k[64 * t: 64 * t + 64] = nan16
                    v[64 * t: 64 * t + 64] = nan16
            pad = ~valid
            k[pad] = nan16
            v[pad] = big
            out, _ = gpu_prefill(case, k=k, v=v, want_lse=False)
            sl = slice(64 * g, 64 * g + 64)
            assert np.array_equal(out[sl, h], out0[sl, h]), f"row (h={h}, g={g}) changed"


def test_prefill_empty_rows():
    """Rows with no listed tiles give O = 0 and LSE = -inf."""
    case = W.make_case("empty-rows", 900, [2], [200, 64], [0], 2, 1, 64, np.zeros((1, 2)), np.zeros((1, 2)))
    la = [np.zeros_like(x) for x in case.la_bool]
    ca = [np.zeros_like(x) for x in case.ca_bool]
    case = W.with_bits(case, la, ca)
    out, lse = gpu_prefill(case)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def test_prefill_nan_in_padded_queries():
    """NaN in the Q of padded query slots stays in those slots: a query's softmax state lives in
    its own lanes, so every valid query's output and LSE are bit-identical to a run with finite
    padding, and padded query rows are still exactly 0 with LSE -inf (question and documents
    not tile-aligned, GQA)."""
    case = W.make_case("pad-q", 810, [2], [150, 90], [40], 4, 2, 128,
                       np.full((1, 4), 0.5), np.full((1, 4), 0.5))
    out0, lse0 = gpu_prefill(case)
    valid = valid_tokens(case)
    assert (~valid).any()
    q = case.q.copy()
    q[~valid] = np.uint16(0x7FC0)  # bf16 quiet NaN
    out1, lse1 = gpu_prefill(case, q=q)
    assert np.array_equal(out1[valid], out0[valid])
    assert np.array_equal(lse1[:, valid], lse0[:, valid])
    assert np.all(out1[~valid] == 0.0)
    assert np.all(np.isneginf(lse1[:, ~valid]))
