"""GPU: what only the device can see is reported in a status word, never by a silent no-op or
an out-of-bounds access.  A plan uploaded for another layout makes every call compute nothing
(the decode writes an empty CSR; the attention, the fused call and the encoder leave their
outputs untouched) and raise SIFT_DEVICE_PLAN_MISMATCH; a listed tile outside [0, G) is skipped
(SIFT_DEVICE_TILE_RANGE); a CSR row outside the given col_idx is taken as empty
(SIFT_DEVICE_ROW_RANGE).  The next good call on the same workspace clears the word.  Every
kernel exits normally: the conditions are set up on the host and checked by the kernels' own
bounds checks."""
import numpy as np
import pytest
import torch

import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W
from gpu_common import DEV, valid_tokens, values_tensor, words_tensor

pytestmark = pytest.mark.gpu

SENTINEL = 123.25


def _case(seed=900, lens=(200, 130, 64), q=90, hq=4, hkv=2, d=128):
    return W.make_case(f"status-{seed}", seed, [len(lens)], list(lens), [q], hq, hkv, d,
                       np.full((1, hq), 0.5), np.full((1, hq), 0.5))


def _other_layouts(case):
    """A layout with the same tile count but other document lengths (another fingerprint), and
    one with another tile count."""
    same_g = sift.Layout(case.req_num_docs, [int(x) - 1 for x in case.doc_len], case.question_len,
                         case.num_q_heads, case.num_kv_heads, case.head_dim)
    other_g = sift.Layout([1], [64], [10], case.num_q_heads, case.num_kv_heads, case.head_dim)
    return {"same_tiles": same_g, "other_tiles": other_g}


@pytest.mark.parametrize("which", ["same_tiles", "other_tiles"])
def test_decode_with_a_plan_of_another_layout(which):
    case = _case()
    lay = sift.Layout.from_case(case)
    other = _other_layouts(case)[which]
    assert which != "same_tiles" or other.num_tiles == lay.num_tiles
    print(f"status: decode, plan of another layout ({which})", flush=True)
    bad_plan = sift.plan_upload(other, DEV)
    ws = sift.workspace(lay, device=DEV)
    la, ca = words_tensor(case.la_words), words_tensor(case.ca_words)
    row_ptr = torch.full((lay.num_rows + 1,), 77, dtype=torch.int32, device=DEV)
    col_idx = torch.full((lay.csr_max_nnz,), -7, dtype=torch.int32, device=DEV)
    sift.decode_bits(lay, la, ca, plan=bad_plan, workspace=ws, row_ptr=row_ptr, col_idx=col_idx)
    assert sift.device_status(ws) == sift.SIFT_DEVICE_PLAN_MISMATCH
    assert torch.all(row_ptr == 0), "a mismatched plan gives an empty CSR"
    assert torch.all(col_idx == -7), "col_idx untouched"
    # the right plan on the same workspace: status cleared, a real CSR
    sift.decode_bits(lay, la, ca, plan=sift.plan_upload(lay, DEV), workspace=ws, row_ptr=row_ptr, col_idx=col_idx)
    assert sift.device_status(ws) == sift.SIFT_DEVICE_OK
    assert int(row_ptr[-1]) > 0


@pytest.mark.parametrize("which", ["same_tiles", "other_tiles"])
@pytest.mark.parametrize("fused", [False, True])
def test_prefill_with_a_plan_of_another_layout(which, fused):
    case = _case()
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    bad_plan = sift.plan_upload(_other_layouts(case)[which], DEV)
    print(f"status: prefill fused={fused}, plan of another layout ({which})", flush=True)
    la, ca = words_tensor(case.la_words), words_tensor(case.ca_words)
    q, k, v = (values_tensor(case, x) for x in (case.q, case.k, case.v))
    row_ptr, col_idx = sift.decode_bits(lay, la, ca, plan=plan)
    ws = sift.workspace(lay, device=DEV)
    n, hq, d = lay.padded_tokens, lay.num_q_heads, lay.head_dim
    out = torch.full((n, hq, d), SENTINEL, dtype=torch.float32, device=DEV)
    lse = torch.full((hq, n), SENTINEL, dtype=torch.float32, device=DEV)
    call = (lambda p: sift.sparse_prefill_bits(lay, la, ca, q, k, v, plan=p, workspace=ws, out=out, lse=lse,
                                               want_lse=True)) if fused else \
        (lambda p: sift.sparse_prefill(lay, q, k, v, row_ptr, col_idx, plan=p, workspace=ws, out=out, lse=lse,
                                       want_lse=True))
    call(bad_plan)
    assert sift.device_status(ws) == sift.SIFT_DEVICE_PLAN_MISMATCH
    assert torch.all(out == SENTINEL) and torch.all(lse == SENTINEL), "outputs untouched"
    call(plan)
    assert sift.device_status(ws) == sift.SIFT_DEVICE_OK
    valid = torch.from_numpy(valid_tokens(case)).to(DEV)
    assert torch.all(torch.isfinite(out)) and not torch.any(out[valid] == SENTINEL)


def _csr(case):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    rp, ci = sift.decode_bits(lay, words_tensor(case.la_words), words_tensor(case.ca_words), plan=plan)
    torch.cuda.synchronize()
    nnz = int(rp[-1])
    return lay, plan, rp.cpu().numpy(), ci[:nnz].cpu().numpy()


def _prefill_csr(case, lay, plan, rp, ci, ws):
    q, k, v = (values_tensor(case, x) for x in (case.q, case.k, case.v))
    rp_t = torch.from_numpy(np.ascontiguousarray(rp, np.int32)).to(DEV)
    ci_t = torch.from_numpy(np.ascontiguousarray(ci, np.int32)).to(DEV)
    out, lse = sift.sparse_prefill(lay, q, k, v, rp_t, ci_t, plan=plan, workspace=ws, want_lse=True)
    flags = sift.device_status(ws)
    return out.cpu().numpy(), lse.cpu().numpy(), flags


def test_listed_tiles_out_of_range_are_skipped_and_flagged():
    """Ids G, G + 5, -1 and -2^31 + 1 inserted into three rows: those entries are skipped, so each
    output is bit-identical to the CSR without them, and the status says so."""
    case = _case(seed=901)
    lay, plan, rp, ci = _csr(case)
    ws = sift.workspace(lay, device=DEV)
    base_out, base_lse, flags = _prefill_csr(case, lay, plan, rp, ci, ws)
    assert flags == sift.SIFT_DEVICE_OK
    G = lay.num_tiles
    rows = {3: [G], 2 * G + 4: [-1, G + 5], lay.num_rows - 1: [-(2 ** 31) + 1]}
    new_ci, new_rp = [], [0]
    for r in range(lay.num_rows):
        seg = list(ci[rp[r]:rp[r + 1]])
        for j, bad in enumerate(rows.get(r, [])):
            seg.insert(min(len(seg), 1 + j), bad)
        new_ci.extend(seg)
        new_rp.append(len(new_ci))
    out, lse, flags = _prefill_csr(case, lay, plan, np.array(new_rp), np.array(new_ci), ws)
    assert flags == sift.SIFT_DEVICE_TILE_RANGE
    assert np.array_equal(out, base_out) and np.array_equal(lse, base_lse)


def test_csr_rows_outside_col_idx_are_empty_and_flagged():
    """col_idx one entry short of the last row's range, and one row whose range runs backwards:
    those rows are read as empty (O = 0, LSE = -inf), every other row is unchanged, no read leaves
    col_idx, and the status says so."""
    case = _case(seed=902)
    lay, plan, rp, ci = _csr(case)
    ws = sift.workspace(lay, device=DEV)
    base_out, base_lse, _ = _prefill_csr(case, lay, plan, rp, ci, ws)
    G = lay.num_tiles
    rp2 = rp.copy()
    r_back = G + 2  # row (h = 1, g = 2): start after its end
    rp2[r_back] = rp2[r_back + 1] + 1
    out, lse, flags = _prefill_csr(case, lay, plan, rp2, ci[:-1], ws)
    assert flags == sift.SIFT_DEVICE_ROW_RANGE
    bad_rows = {r for r in range(lay.num_rows) if not (0 <= rp2[r] <= rp2[r + 1] <= ci.size - 1)}
    assert bad_rows == {lay.num_rows - 1, r_back}
    valid = valid_tokens(case)
    for r in range(lay.num_rows):
        if r == r_back - 1:
            continue  # a valid range that now runs into r_back's entries: another list
        h, g = divmod(r, G)
        sl = slice(64 * g, 64 * g + 64)
        if r in bad_rows:
            assert np.all(out[sl, h] == 0.0) and np.all(np.isneginf(lse[h, sl][valid[sl]]))
        else:
            assert np.array_equal(out[sl, h], base_out[sl, h]), f"row {r} changed"


@pytest.mark.parametrize("which", ["same_tiles", "other_tiles"])
def test_encoder_with_a_plan_of_another_layout(which):
    case = _case(seed=903, d=64)
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    bad_plan = sift.plan_upload(_other_layouts(case)[which], DEV)
    print(f"status: encoder, plan of another layout ({which})", flush=True)
    q, k = values_tensor(case, case.q), values_tensor(case, case.k)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    rt = sift.encode_masses_bytes(lay) // (4 * lay.num_q_heads * lay.num_tiles)
    masses = torch.full((lay.num_q_heads, lay.num_tiles, rt), SENTINEL, dtype=torch.float32, device=DEV)
    sift.tile_masses(lay, q, k, plan=bad_plan, masses=masses, status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == sift.SIFT_DEVICE_PLAN_MISMATCH and torch.all(masses == SENTINEL)
    sift.tile_masses(lay, q, k, plan=plan, masses=masses, status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == sift.SIFT_DEVICE_OK
    la = torch.full((lay.la_words,), 5, dtype=torch.int32, device=DEV)
    ca = torch.full((lay.ca_words,), 5, dtype=torch.int32, device=DEV)
    sift.select_bits(lay, masses, 0.9, 0.9, plan=bad_plan, la=la, ca=ca, status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == sift.SIFT_DEVICE_PLAN_MISMATCH
    assert torch.all(la == 5) and torch.all(ca == 5)
    sift.select_bits(lay, masses, 0.9, 0.9, plan=plan, la=la, ca=ca, status=status)
    torch.cuda.synchronize()
    assert int(status[0]) == sift.SIFT_DEVICE_OK
