"""CPU oracle for bit-vector sparse RAG prefill (SIFT) -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path never does; it shares no code,
header, table or helper with the GPU library.

The arithmetic lives in ``sift_oracle.c`` (plain C, fp64, OpenMP over output
rows).  What it follows is stated in that file's header: SIFT technical
summary, section 2 "Metodologia" ("Design del Sistema": LA and CA bit vectors
per document, layer and head; "Dettagli di Implementazione": decode to explicit
tile indices, then attention over those indices only).

Every function here is pinned by the tests against brute force, closed forms
and library routines (no page prints a worked example); none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsift_oracle.so")
SRC_PATH = os.path.join(_HERE, "sift_oracle.c")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", LIB_PATH + ".tmp",
           SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    f64p = ctypes.POINTER(ctypes.c_double)
    lay = [ctypes.c_int32, i32p, i32p, i32p]
    lib.sift_oracle_num_tiles.argtypes = lay
    lib.sift_oracle_num_tiles.restype = ctypes.c_int64
    lib.sift_oracle_row_counts.argtypes = lay + [ctypes.c_int32, u32p, u32p, i64p]
    lib.sift_oracle_row_counts.restype = ctypes.c_int64
    lib.sift_oracle_decode.argtypes = lay + [ctypes.c_int32, u32p, u32p, i64p, i32p, ctypes.c_int64]
    lib.sift_oracle_decode.restype = ctypes.c_int64
    lib.sift_oracle_attention.argtypes = lay + [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, u32p, u32p, ctypes.c_double,
        ctypes.c_int64, i32p, i64p, f64p, f64p, ctypes.c_int32]
    lib.sift_oracle_attention.restype = ctypes.c_int
    lib.sift_oracle_max_threads.argtypes = []
    lib.sift_oracle_max_threads.restype = ctypes.c_int32
    _lib = lib
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _layout_args(case):
    rnd = np.ascontiguousarray(case.req_num_docs, dtype=np.int32)
    dl = np.ascontiguousarray(case.doc_len, dtype=np.int32)
    if dl.size == 0:
        dl = np.zeros(1, np.int32)
    ql = np.ascontiguousarray(case.question_len, dtype=np.int32)
    keep = (rnd, dl, ql)
    return keep, [ctypes.c_int32(len(rnd)), _ptr(rnd, ctypes.c_int32), _ptr(dl, ctypes.c_int32),
                  _ptr(ql, ctypes.c_int32)]


def _words(w):
    w = np.ascontiguousarray(w, dtype=np.uint32)
    return w if w.size else np.zeros(1, np.uint32)


def num_tiles(case) -> int:
    keep, la = _layout_args(case)
    return int(_load().sift_oracle_num_tiles(*la))


def row_counts(case, la_words=None, ca_words=None) -> np.ndarray:
    """Per-row tile counts, rows ordered h*G + g."""
    lib = _load()
    keep, lay = _layout_args(case)
    la = _words(case.la_words if la_words is None else la_words)
    ca = _words(case.ca_words if ca_words is None else ca_words)
    g = num_tiles(case)
    counts = np.zeros(case.num_q_heads * g, dtype=np.int64)
    nnz = lib.sift_oracle_row_counts(*lay, case.num_q_heads, _ptr(la, ctypes.c_uint32),
                                     _ptr(ca, ctypes.c_uint32), _ptr(counts, ctypes.c_int64))
    if nnz < 0:
        raise ValueError("oracle: bad layout")
    return counts


def decode(case, la_words=None, ca_words=None):
    """Oracle CSR: (row_ptr int64 [Hq*G+1], col_idx int32 [nnz])."""
    lib = _load()
    keep, lay = _layout_args(case)
    la = _words(case.la_words if la_words is None else la_words)
    ca = _words(case.ca_words if ca_words is None else ca_words)
    counts = row_counts(case, la, ca)
    nnz = int(counts.sum())
    row_ptr = np.zeros(counts.size + 1, dtype=np.int64)
    col_idx = np.zeros(max(nnz, 1), dtype=np.int32)
    got = lib.sift_oracle_decode(*lay, case.num_q_heads, _ptr(la, ctypes.c_uint32),
                                 _ptr(ca, ctypes.c_uint32), _ptr(row_ptr, ctypes.c_int64),
                                 _ptr(col_idx, ctypes.c_int32), ctypes.c_int64(col_idx.size))
    if got != nnz:
        raise RuntimeError(f"oracle decode failed ({got})")
    return row_ptr, col_idx[:nnz]


_DTYPE_CODE = {"bf16": 0, "fp32_round": 1, "fp32_exact": 2}


def attention(case, heads=None, tokens=None, exact_fp32=False, num_threads=0,
              la_words=None, ca_words=None, q=None, k=None, v=None):
    """fp64 attention for (head, padded token) pairs.

    With heads/tokens None, every (h, token) pair is computed and the result is
    shaped [N, Hq, D] (and lse [Hq, N]); otherwise out is [npairs, D], lse [npairs].
    fp32 inputs are rounded to bf16 first unless exact_fp32 (the unrounded reading).
    """
    lib = _load()
    keep, lay = _layout_args(case)
    la = _words(case.la_words if la_words is None else la_words)
    ca = _words(case.ca_words if ca_words is None else ca_words)
    q = case.q if q is None else q
    k = case.k if k is None else k
    v = case.v if v is None else v
    if case.dtype == "bf16":
        code = 0
        q, k, v = (np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v))
    else:
        code = 2 if exact_fp32 else 1
        q, k, v = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v))
    n = q.shape[0]
    full = heads is None
    if full:
        hh, tt = np.meshgrid(np.arange(case.num_q_heads, dtype=np.int32),
                             np.arange(n, dtype=np.int64), indexing="ij")
        heads, tokens = hh.ravel(), tt.ravel()
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    npairs = heads.size
    out = np.zeros((max(npairs, 1), case.head_dim), dtype=np.float64)
    lse = np.zeros(max(npairs, 1), dtype=np.float64)
    rc = lib.sift_oracle_attention(
        *lay, case.num_q_heads, case.num_kv_heads, case.head_dim, code,
        q.ctypes.data_as(ctypes.c_void_p), k.ctypes.data_as(ctypes.c_void_p),
        v.ctypes.data_as(ctypes.c_void_p), _ptr(la, ctypes.c_uint32), _ptr(ca, ctypes.c_uint32),
        ctypes.c_double(case.scale), ctypes.c_int64(npairs), _ptr(heads, ctypes.c_int32),
        _ptr(tokens, ctypes.c_int64), _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
        ctypes.c_int32(num_threads))
    if rc != 0:
        raise RuntimeError("oracle attention failed")
    out, lse = out[:npairs], lse[:npairs]
    if full:
        out = out.reshape(case.num_q_heads, n, case.head_dim).transpose(1, 0, 2).copy()
        lse = lse.reshape(case.num_q_heads, n)
    return out, lse


def max_threads() -> int:
    return int(_load().sift_oracle_max_threads())
