"""The C ABI on the host (no GPU calls): exports, sizing helpers and validation."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import bit_vector_block_amd as sift
from bit_vector_block_amd import _binding as B
from bit_vector_block_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sift.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sift_[a-z0-9_]+)\s*\(", text)))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises: there is no CPU fallback."""
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libsift.so"))
    monkeypatch.setattr(B, "_LIB", None)
    with pytest.raises(RuntimeError, match="not built"):
        B._lib()
    lay = sift.Layout(req_num_docs=[1], doc_len=[64], question_len=[0], num_q_heads=1,
                      num_kv_heads=1, head_dim=64)
    with pytest.raises(RuntimeError, match="not built"):
        lay.workspace_bytes()


def test_library_exports_every_declared_symbol():
    lib = sift.library()
    declared = _declared_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTED) == declared
    assert lib.sift_abi_version() >> 16 == 3


@pytest.mark.parametrize("cid", [1, 2])
def test_sizing_helpers_match_the_generator(cid):
    case = W.config_case(cid)
    lay = sift.Layout.from_case(case)
    assert lay.padded_tokens == case.q.shape[0]
    assert lay.num_tiles * 64 == case.q.shape[0]
    assert lay.num_rows == lay.num_tiles * case.num_q_heads
    assert lay.la_words == case.la_words.size
    assert lay.ca_words == case.ca_words.size


@pytest.mark.parametrize("cid,G,la_words,ca_words", [
    (3, 516, 32 * 32 * 5, 32 * 32), (4, 644, 20 * 64 * 17, 20 * 64)])
def test_sizing_of_large_workloads(cid, G, la_words, ca_words):
    r, dl, ql, hq, hkv, d = W.config_layout(cid)
    lay = sift.Layout(r, dl, ql, hq, hkv, d)
    assert lay.num_tiles == G and lay.la_words == la_words and lay.ca_words == ca_words


def test_ragged_layout_matches_the_case_draw():
    r, dl, ql, hq, hkv, d = W.config_layout(5)
    lay = sift.Layout(r, dl, ql, hq, hkv, d)
    assert lay.padded_tokens == W.padded_total(r, dl, ql)
    assert lay.padded_tokens > 100_000


@pytest.mark.parametrize("seed", range(6))
def test_max_nnz_is_the_all_ones_count(seed):
    case = W.random_small_case(seed, max_requests=3, max_docs=4, hq=3, hkv=1, d=64)
    ones = W.with_bits(case, *W.all_ones_bits(case))
    lay = sift.Layout.from_case(case)
    assert lay.csr_max_nnz == int(oracle.row_counts(ones).sum())
    assert lay.csr_max_nnz >= int(oracle.row_counts(case).sum())
    assert lay.la_words == case.la_words.size and lay.ca_words == case.ca_words.size


def _status(lay, **kw):
    lib = sift.library()
    args = dict(plan=1, la=1, ca=1, row_ptr=1, col_idx=1, ws=1, ws_bytes=lay.workspace_bytes())
    args.update(kw)
    if "cap" not in args:
        args["cap"] = lay.csr_max_nnz
    vp = ctypes.c_void_p
    return lib.sift_decode_bits(lay.ref, vp(args["plan"]), vp(args["la"]), vp(args["ca"]),
                                vp(args["row_ptr"]), vp(args["col_idx"]), args["cap"], vp(args["ws"]),
                                args["ws_bytes"], vp(0))


def test_decode_validation_rejects_before_any_launch():
    case = W.random_small_case(3, d=64)
    lay = sift.Layout.from_case(case)
    assert _status(lay, plan=0) == B.SIFT_ERR_INVALID
    assert _status(lay, row_ptr=0) == B.SIFT_ERR_INVALID
    assert _status(lay, la=0) == B.SIFT_ERR_INVALID
    assert _status(lay, cap=lay.csr_max_nnz - 1) == B.SIFT_ERR_CAPACITY
    assert _status(lay, ws_bytes=0) == B.SIFT_ERR_CAPACITY
    assert _status(lay, ws=0) == B.SIFT_ERR_CAPACITY


def test_prefill_validation_rejects_before_any_launch():
    case = W.random_small_case(4, d=64)
    lay = sift.Layout.from_case(case)
    lib = sift.library()
    vp = ctypes.c_void_p
    st = lib.sift_sparse_prefill(lay.ref, vp(1), vp(0), vp(1), vp(1), B.SIFT_BF16, vp(1), vp(1), 10,
                                 ctypes.c_float(0.0), vp(1), vp(0), vp(0), 0, vp(0))
    assert st == B.SIFT_ERR_INVALID
    st = lib.sift_sparse_prefill(lay.ref, vp(1), vp(1), vp(1), vp(1), 7, vp(1), vp(1), 10,
                                 ctypes.c_float(0.0), vp(1), vp(0), vp(0), 0, vp(0))
    assert st == B.SIFT_ERR_INVALID
    # Q/K/V/O must be 16-byte aligned (fake, never dereferenced, addresses)
    a = vp(4096)
    st = lib.sift_sparse_prefill(lay.ref, a, vp(4096 + 8), a, a, B.SIFT_BF16, a, a, 10,
                                 ctypes.c_float(0.0), a, vp(0), a, 1 << 30, vp(0))
    assert st == B.SIFT_ERR_INVALID
    # col_entries: not negative, and col_idx may be null only when it is 0
    st = lib.sift_sparse_prefill(lay.ref, a, a, a, a, B.SIFT_BF16, a, a, -1,
                                 ctypes.c_float(0.0), a, vp(0), a, 1 << 30, vp(0))
    assert st == B.SIFT_ERR_INVALID
    st = lib.sift_sparse_prefill(lay.ref, a, a, a, a, B.SIFT_BF16, a, vp(0), 5,
                                 ctypes.c_float(0.0), a, vp(0), a, 1 << 30, vp(0))
    assert st == B.SIFT_ERR_INVALID
    # the workspace holds the header and V^T (bf16), plus the bf16 copies of Q and K for fp32 inputs
    for dt in (B.SIFT_BF16, B.SIFT_FP32):
        st = lib.sift_sparse_prefill(lay.ref, a, a, a, a, dt, a, a, 10,
                                     ctypes.c_float(0.0), a, vp(0), vp(0), 0, vp(0))
        assert st == B.SIFT_ERR_CAPACITY
    vt = 256 + 2 * lay.padded_tokens * lay.num_kv_heads * lay.head_dim
    assert lay.workspace_bytes(B.SIFT_BF16) >= vt
    assert lay.workspace_bytes(B.SIFT_FP32) >= vt + 2 * lay.padded_tokens * (lay.num_q_heads + lay.num_kv_heads) * lay.head_dim


@pytest.mark.parametrize("kw,expect", [
    (dict(num_q_heads=3, num_kv_heads=2), B.SIFT_ERR_INVALID),
    (dict(head_dim=96), B.SIFT_ERR_UNSUPPORTED),
    (dict(tile=32), B.SIFT_ERR_UNSUPPORTED),
    (dict(doc_len=[100, 0]), B.SIFT_ERR_INVALID),
    (dict(question_len=[-1]), B.SIFT_ERR_INVALID),
])
def test_invalid_layouts(kw, expect):
    base = dict(req_num_docs=[2], doc_len=[100, 70], question_len=[10], num_q_heads=4,
                num_kv_heads=2, head_dim=64, tile=64)
    base.update(kw)
    lay = sift.Layout(**base)
    assert sift.library().sift_num_tiles(lay.ref) == -1
    assert lay.plan_bytes == 0
    assert _status(lay, cap=0) == expect


def test_int32_overflow_is_unsupported():
    # one request of 4M tokens: the dense-causal CSR bound passes 2^31 entries
    lay = sift.Layout([1], [4_000_000], [0], 32, 8, 128)
    assert sift.library().sift_num_tiles(lay.ref) == -1
    assert _status(lay, cap=0) == B.SIFT_ERR_UNSUPPORTED


def test_empty_layout_sizes():
    lay = sift.Layout([0], [], [0], 2, 1, 64)
    assert lay.num_tiles == 0 and lay.num_rows == 0 and lay.csr_max_nnz == 0
    assert lay.plan_bytes > 0 and lay.workspace_bytes() > 0

def test_prefill_bits_validation():
    case = W.random_small_case(4, d=64)
    lay = sift.Layout.from_case(case)
    lib = sift.library()
    vp = ctypes.c_void_p
    a = vp(4096)
    # null Q
    st = lib.sift_sparse_prefill_bits(lay.ref, a, a, a, vp(0), a, a, B.SIFT_BF16, ctypes.c_float(0.0),
                                      a, vp(0), a, 1 << 30, vp(0))
    assert st == B.SIFT_ERR_INVALID
    # workspace too small
    st = lib.sift_sparse_prefill_bits(lay.ref, a, a, a, a, a, a, B.SIFT_BF16, ctypes.c_float(0.0),
                                      a, vp(0), a, 16, vp(0))
    assert st == B.SIFT_ERR_CAPACITY
    # the fused call's workspace holds the CSR its decode writes (max_nnz entries) on top of the
    # prefill's V^T; layouts past the single-launch decode also hold that decode's scratch
    for lay2 in (lay, sift.Layout([1], [1985 * 64], [0], 1, 1, 64)):
        fused = lib.sift_workspace_bytes(lay2.ref, B.SIFT_BF16)
        assert fused >= 256 + 2 * lay2.padded_tokens * 1 * 64 + 4 * (lay2.num_rows + 1) + 4 * lay2.csr_max_nnz


def test_encoder_validation():
    case = W.random_small_case(4, d=64)
    lay = sift.Layout.from_case(case)
    lib = sift.library()
    vp, f, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    a = vp(4096)
    need = lib.sift_encode_masses_bytes(lay.ref)
    tiles = [-(-int(n) // 64) for n in case.doc_len]
    rt, d0 = 0, 0
    for b, k in enumerate(case.req_num_docs):
        rt = max(rt, sum(tiles[d0:d0 + k]) + -(-int(case.question_len[b]) // 64))
        d0 += k
    assert need == 4 * lay.num_q_heads * lay.num_tiles * rt
    # the workspace: a 256-byte header, then one slot per persistent workgroup (2 hpw wavefronts,
    # 4096 wavefronts in all, never more than the work items) of rt tiles x hpw heads x 64 queries
    group = lay.num_q_heads // lay.num_kv_heads
    hpw = 4 if group % 4 == 0 else (2 if group % 2 == 0 else 1)
    slots = min(lay.num_kv_heads * (group // hpw) * lay.num_tiles, 4096 // (2 * hpw))
    wneed = lib.sift_encode_workspace_bytes(lay.ref)
    assert wneed == 256 + slots * rt * hpw * 64 * 4
    z = sz(wneed)
    tm = lib.sift_tile_masses
    assert tm(lay.ref, a, vp(0), a, f(0.0), a, need, a, z, vp(0), vp(0)) == B.SIFT_ERR_INVALID
    assert tm(lay.ref, a, vp(4104), a, f(0.0), a, need, a, z, vp(0), vp(0)) == B.SIFT_ERR_INVALID
    assert tm(lay.ref, a, a, a, f(0.0), a, need, vp(4100), z, vp(0), vp(0)) == B.SIFT_ERR_INVALID
    assert tm(lay.ref, a, a, a, f(0.0), a, need - 4, a, z, vp(0), vp(0)) == B.SIFT_ERR_CAPACITY
    assert tm(lay.ref, a, a, a, f(0.0), a, need, a, sz(wneed - 4), vp(0), vp(0)) == B.SIFT_ERR_CAPACITY
    assert tm(lay.ref, a, a, a, f(0.0), a, need, vp(0), z, vp(0), vp(0)) == B.SIFT_ERR_CAPACITY
    for p_la, p_ca in ((0.0, 0.5), (0.5, 1.5), (float("nan"), 0.5)):
        assert lib.sift_select_bits(lay.ref, a, a, need, f(p_la), f(p_ca), a, a, vp(0), vp(0)) == B.SIFT_ERR_INVALID
    assert lib.sift_select_bits(lay.ref, a, a, need - 4, f(0.9), f(0.9), a, a, vp(0), vp(0)) == B.SIFT_ERR_CAPACITY
    big = sift.Layout([1], [65 * 64], [0], 1, 1, 64)
    nb = lib.sift_encode_masses_bytes(big.ref)
    assert lib.sift_select_bits(big.ref, a, a, nb, f(0.9), f(0.9), a, a, vp(0), vp(0)) == B.SIFT_ERR_UNSUPPORTED


def test_device_status_validation():
    lib = sift.library()
    vp = ctypes.c_void_p
    flags = ctypes.c_int32(-1)
    assert lib.sift_device_status(vp(0), 4096, ctypes.addressof(flags), vp(0)) == B.SIFT_ERR_INVALID
    assert lib.sift_device_status(vp(4096), 4096, vp(0), vp(0)) == B.SIFT_ERR_INVALID
    assert lib.sift_device_status(vp(4096), 255, ctypes.addressof(flags), vp(0)) == B.SIFT_ERR_CAPACITY
    assert flags.value == -1  # nothing enqueued


def _cpu_inputs(case, torch):
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16)
    k = torch.from_numpy(case.k.view(np.int16)).view(torch.bfloat16)
    v = torch.from_numpy(case.v.view(np.int16)).view(torch.bfloat16)
    return q, k, v


def test_binding_rejects_bad_output_and_csr_tensors():
    """The binding checks every caller-supplied tensor (shape, dtype, device, contiguity) before
    the C call: the C ABI cannot know their sizes, and a short buffer would be an out-of-bounds
    device write.  (CPU tensors here: the checks raise before any device work.)"""
    import torch
    case = W.random_small_case(6, d=64, hq=2, hkv=1)
    lay = sift.Layout.from_case(case)
    q, k, v = _cpu_inputs(case, torch)
    n, hq, d = lay.padded_tokens, lay.num_q_heads, lay.head_dim
    rp = torch.zeros(lay.num_rows + 1, dtype=torch.int32)
    ci = torch.zeros(max(lay.csr_max_nnz, 1), dtype=torch.int32)
    good_out = torch.empty((n, hq, d), dtype=torch.float32)
    bad = [
        dict(out=torch.empty((n, hq, d), dtype=torch.bfloat16)),
        dict(out=torch.empty((n - 1, hq, d), dtype=torch.float32)),
        dict(out=torch.empty((n, d, hq), dtype=torch.float32).transpose(1, 2)),
        dict(out=good_out, want_lse=True, lse=torch.empty((n, hq), dtype=torch.float32)),
        dict(out=good_out, want_lse=True, lse=torch.empty((hq, n), dtype=torch.float64)),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            sift.sparse_prefill(lay, q, k, v, rp, ci, **kw)
    with pytest.raises(ValueError):
        sift.sparse_prefill(lay, q, k, v, rp[:-1], ci, out=good_out)
    with pytest.raises(ValueError):
        sift.sparse_prefill(lay, q, k, v, rp.to(torch.int64), ci, out=good_out)
    with pytest.raises(ValueError):
        sift.sparse_prefill(lay, q, k, v, rp, ci.to(torch.int64), out=good_out)
    with pytest.raises(ValueError):
        sift.sparse_prefill(lay, q, k, v, rp, ci[::2], out=good_out)
    la = torch.from_numpy(case.la_words.view(np.int32))
    ca = torch.from_numpy(case.ca_words.view(np.int32))
    with pytest.raises(ValueError):
        sift.decode_bits(lay, la, ca, row_ptr=torch.zeros(lay.num_rows, dtype=torch.int32))
    with pytest.raises(ValueError):
        sift.decode_bits(lay, la, ca, row_ptr=rp, col_idx=torch.zeros(lay.csr_max_nnz - 1, dtype=torch.int32))
    with pytest.raises(ValueError):
        sift.sparse_prefill_bits(lay, la, ca, q, k, v, out=torch.empty((n, hq, d - 1), dtype=torch.float32))
    with pytest.raises(ValueError):
        sift.tile_masses(lay, q, k, masses=torch.empty(3, dtype=torch.float32))
    with pytest.raises(ValueError):
        sift.tile_masses(lay, q, k, status=torch.empty(1, dtype=torch.int64))
    with pytest.raises(ValueError):
        sift.tile_masses(lay, q, k, workspace=torch.empty(8, dtype=torch.uint8))


def test_noalloc_decode_rejects_a_layout_beyond_its_scratch():
    """The allocation-free decode's scratch is a fixed array per GPU: a layout whose decode
    scratch is larger (200 requests x 100 tiles, 64 q heads: about 10 MiB) is rejected on the
    host, before any HIP call (fake, never dereferenced, pointers)."""
    lib = sift.library()
    lay = sift.Layout([1] * 200, [6400] * 200, [0] * 200, 64, 8, 128)
    scratch = 256 + 4 * 64 * 200 + 2 * 4 * 64 * lay.num_tiles
    assert lay.num_tiles == 20000 and scratch > B.DECODE_NOALLOC_MAX_BYTES
    a = ctypes.c_void_p(4096)
    st = lib.sift_decode_bits_noalloc(lay.ref, a, a, a, a, a, lay.csr_max_nnz, ctypes.c_void_p(0))
    assert st == B.SIFT_ERR_CAPACITY
    small = sift.Layout([1], [640], [0], 2, 1, 64)
    assert lib.sift_decode_bits_noalloc(small.ref, a, a, a, a, a, small.csr_max_nnz - 1,
                                        ctypes.c_void_p(0)) == B.SIFT_ERR_CAPACITY
    assert lib.sift_decode_bits_noalloc(small.ref, ctypes.c_void_p(0), a, a, a, a, small.csr_max_nnz,
                                        ctypes.c_void_p(0)) == B.SIFT_ERR_INVALID
