"""Shared helpers of the GPU parity tests (they call the library through the C ABI)."""
import functools

import numpy as np
import torch

import bit_vector_block_amd as sift
from bit_vector_block_amd import workloads as W

DEV = "cuda:0"

MAX_ABS = 1e-2   # tolerance on fp32 output vs the fp64 oracle (max-abs, mean-abs)
MEAN_ABS = 1e-3
# LSE = m + ln(l) where l sums the bf16-rounded P (relative rounding <= 2^-9 per term, so
# |d ln l| <= 2^-9 ~ 1.95e-3) plus fp32 accumulation over up to ~3e4 keys per lane
# (<= 2e-3 worst case): 4e-3 absolute.
LSE_ABS = 4e-3


@functools.lru_cache(maxsize=3)
def config(cid):
    return W.config_case(cid)


@functools.lru_cache(maxsize=1)
def oracle_full(cid):
    """The fp64 oracle's whole output (O [N, Hq, D], LSE [Hq, N]) of a workload, kept for the
    next test that asks for the same workload."""
    import oracle
    print(f"oracle: workload {cid}, every (token, head)", flush=True)
    return oracle.attention(config(cid))


def words_tensor(words):
    w = np.ascontiguousarray(words, dtype=np.uint32)
    if w.size == 0:
        w = np.zeros(1, np.uint32)
    return torch.from_numpy(w.view(np.int32)).to(DEV)


def values_tensor(case, x):
    if case.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def gpu_decode(case, la_words=None, ca_words=None):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    la = words_tensor(case.la_words if la_words is None else la_words)
    ca = words_tensor(case.ca_words if ca_words is None else ca_words)
    row_ptr, col_idx = sift.decode_bits(lay, la, ca, plan=plan)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()[: rp[-1]]
    return rp, ci


def gpu_prefill(case, q=None, k=None, v=None, want_lse=True, la_words=None, ca_words=None):
    lay = sift.Layout.from_case(case)
    plan = sift.plan_upload(lay, DEV)
    la = words_tensor(case.la_words if la_words is None else la_words)
    ca = words_tensor(case.ca_words if ca_words is None else ca_words)
    row_ptr, col_idx = sift.decode_bits(lay, la, ca, plan=plan)
    qt, kt, vt = (values_tensor(case, x) for x in (case.q if q is None else q,
                                                   case.k if k is None else k,
                                                   case.v if v is None else v))
    out, lse = sift.sparse_prefill(lay, qt, kt, vt, row_ptr, col_idx, plan=plan, want_lse=want_lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def valid_tokens(case):
    """Boolean [N]: token lies inside its segment's true length."""
    valid = []
    d = 0
    for b, k in enumerate(case.req_num_docs):
        for _ in range(int(k)):
            n = int(case.doc_len[d])
            t = -(-n // 64)
            valid.extend([x < n for x in range(64 * t)])
            d += 1
        m = int(case.question_len[b])
        t = -(-m // 64)
        valid.extend([x < m for x in range(64 * t)])
    return np.array(valid, dtype=bool)


def assert_full_parity(case, out, lse, ref, ref_lse, what):
    """Every valid (token, head) output and LSE against the oracle; padded query rows exactly 0
    with LSE -inf."""
    valid = valid_tokens(case)
    mx, mean = assert_close(out[valid], ref[valid], what)
    assert np.all(out[~valid] == 0.0), f"{what}: padded query rows must be exactly 0"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: LSE finiteness differs"
    lmx = float(np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0.0))
    assert lmx <= LSE_ABS, f"{what}: LSE max_abs {lmx:.3e}"
    print(f"{what}: {int(valid.sum()) * case.num_q_heads} (token, head) outputs, max_abs {mx:.3e} "
          f"mean_abs {mean:.3e}, LSE max_abs {lmx:.3e}", flush=True)
    return mx, mean


def assert_close(got, ref, what=""):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max_abs {mx:.3e} mean_abs {mean:.3e}"
    return mx, mean
