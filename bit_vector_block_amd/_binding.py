"""ctypes binding of libsift.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; torch provides device
memory and the current stream.  The names follow include/sift.h.  If the
library is not built this module raises on first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsift.so")

SIFT_OK, SIFT_ERR_INVALID, SIFT_ERR_CAPACITY, SIFT_ERR_UNSUPPORTED, SIFT_ERR_HIP = range(5)
SIFT_BF16, SIFT_FP32 = 0, 1
# bits of a device status word (sift_device_flag)
SIFT_DEVICE_OK, SIFT_DEVICE_PLAN_MISMATCH, SIFT_DEVICE_TILE_RANGE, SIFT_DEVICE_ROW_RANGE = 0, 1, 2, 4
# scratch array of sift_decode_bits_noalloc, per GPU (SIFT_DECODE_NOALLOC_MAX_BYTES)
DECODE_NOALLOC_MAX_BYTES = 8 << 20

EXPORTED = (
    "sift_num_tiles", "sift_padded_tokens", "sift_num_rows", "sift_la_words", "sift_ca_words",
    "sift_csr_max_nnz", "sift_plan_bytes", "sift_workspace_bytes", "sift_plan_upload",
    "sift_decode_bits", "sift_sparse_prefill", "sift_sparse_prefill_bits", "sift_status_string",
    "sift_abi_version", "sift_encode_masses_bytes", "sift_tile_masses", "sift_select_bits",
    "sift_device_status", "sift_decode_bits_noalloc", "sift_encode_workspace_bytes",
)


class SiftError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().sift_status_string(status).decode()}")


class _CLayout(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("req_num_docs", ctypes.POINTER(ctypes.c_int32)),
        ("doc_len", ctypes.POINTER(ctypes.c_int32)),
        ("question_len", ctypes.POINTER(ctypes.c_int32)),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tile", ctypes.c_int32),
    ]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libsift.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    L = ctypes.POINTER(_CLayout)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    for name in ("sift_num_tiles", "sift_padded_tokens", "sift_num_rows", "sift_la_words",
                 "sift_ca_words", "sift_csr_max_nnz"):
        getattr(lib, name).argtypes = [L]
        getattr(lib, name).restype = i64
    lib.sift_plan_bytes.argtypes = [L]
    lib.sift_plan_bytes.restype = sz
    lib.sift_workspace_bytes.argtypes = [L, ctypes.c_int]
    lib.sift_workspace_bytes.restype = sz
    lib.sift_plan_upload.argtypes = [L, vp, sz, vp]
    lib.sift_plan_upload.restype = ctypes.c_int
    lib.sift_decode_bits.argtypes = [L, vp, vp, vp, vp, vp, i64, vp, sz, vp]
    lib.sift_decode_bits.restype = ctypes.c_int
    lib.sift_sparse_prefill.argtypes = [L, vp, vp, vp, vp, ctypes.c_int, vp, vp, i64, ctypes.c_float,
                                        vp, vp, vp, sz, vp]
    lib.sift_sparse_prefill.restype = ctypes.c_int
    lib.sift_sparse_prefill_bits.argtypes = [L, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_float,
                                             vp, vp, vp, sz, vp]
    lib.sift_sparse_prefill_bits.restype = ctypes.c_int
    lib.sift_encode_masses_bytes.argtypes = [L]
    lib.sift_encode_masses_bytes.restype = sz
    lib.sift_encode_workspace_bytes.argtypes = [L]
    lib.sift_encode_workspace_bytes.restype = sz
    lib.sift_tile_masses.argtypes = [L, vp, vp, vp, ctypes.c_float, vp, sz, vp, sz, vp, vp]
    lib.sift_tile_masses.restype = ctypes.c_int
    lib.sift_select_bits.argtypes = [L, vp, vp, sz, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp]
    lib.sift_select_bits.restype = ctypes.c_int
    lib.sift_device_status.argtypes = [vp, sz, vp, vp]
    lib.sift_device_status.restype = ctypes.c_int
    lib.sift_decode_bits_noalloc.argtypes = [L, vp, vp, vp, vp, vp, i64, vp]
    lib.sift_decode_bits_noalloc.restype = ctypes.c_int
    lib.sift_status_string.argtypes = [ctypes.c_int]
    lib.sift_status_string.restype = ctypes.c_char_p
    lib.sift_abi_version.argtypes = []
    lib.sift_abi_version.restype = ctypes.c_int32
    _LIB = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


class Layout:
    """Host description of one batch (see sift_layout in include/sift.h)."""

    def __init__(self, req_num_docs: Sequence[int], doc_len: Sequence[int],
                 question_len: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                 tile: int = 64):
        self.req_num_docs = np.ascontiguousarray(req_num_docs, dtype=np.int32)
        self.doc_len = np.ascontiguousarray(doc_len, dtype=np.int32)
        self.question_len = np.ascontiguousarray(question_len, dtype=np.int32)
        self.num_q_heads, self.num_kv_heads, self.head_dim, self.tile = (
            int(num_q_heads), int(num_kv_heads), int(head_dim), int(tile))
        p32 = ctypes.POINTER(ctypes.c_int32)
        dl = self.doc_len if self.doc_len.size else np.zeros(1, np.int32)
        self._keep = dl
        self._c = _CLayout(len(self.req_num_docs), self.req_num_docs.ctypes.data_as(p32),
                           dl.ctypes.data_as(p32), self.question_len.ctypes.data_as(p32),
                           self.num_q_heads, self.num_kv_heads, self.head_dim, self.tile)

    @classmethod
    def from_case(cls, case) -> "Layout":
        return cls(case.req_num_docs, case.doc_len, case.question_len, case.num_q_heads,
                   case.num_kv_heads, case.head_dim, case.tile)

    @property
    def ref(self):
        return ctypes.byref(self._c)

    def _i64(self, name):
        v = getattr(_lib(), name)(self.ref)
        if v < 0:
            raise SiftError(SIFT_ERR_INVALID, name)
        return int(v)

    num_tiles = property(lambda self: self._i64("sift_num_tiles"))
    padded_tokens = property(lambda self: self._i64("sift_padded_tokens"))
    num_rows = property(lambda self: self._i64("sift_num_rows"))
    la_words = property(lambda self: self._i64("sift_la_words"))
    ca_words = property(lambda self: self._i64("sift_ca_words"))
    csr_max_nnz = property(lambda self: self._i64("sift_csr_max_nnz"))

    @property
    def plan_bytes(self) -> int:
        return int(_lib().sift_plan_bytes(self.ref))

    def workspace_bytes(self, dtype: int = SIFT_BF16) -> int:
        return int(_lib().sift_workspace_bytes(self.ref, dtype))


def _stream_handle(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status: int, what: str):
    if status != SIFT_OK:
        raise SiftError(status, what)


def plan_upload(layout: Layout, device=None):
    """Device plan tensor (uint8) for `layout`, uploaded on the current stream."""
    import torch
    device = torch.device("cuda") if device is None else torch.device(device)
    nbytes = layout.plan_bytes
    if nbytes == 0:
        raise SiftError(SIFT_ERR_INVALID, "sift_plan_bytes")
    plan = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(_lib().sift_plan_upload(layout.ref, ctypes.c_void_p(plan.data_ptr()), nbytes,
                                   _stream_handle(torch, device)), "sift_plan_upload")
    plan._sift_layout = layout  # keep the layout alive alongside the plan
    return plan


def _workspace(torch, layout, dtype, device, workspace):
    need = layout.workspace_bytes(dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    else:
        _need_tensor("workspace", workspace, None, device)
    return workspace, workspace.numel() * workspace.element_size()


def workspace(layout: Layout, dtype: int = SIFT_BF16, device=None):
    """A workspace tensor (uint8) large enough for every call on `layout` with `dtype`; pass it to
    the calls to reuse it and to read its device status word (device_status)."""
    import torch
    device = torch.device("cuda") if device is None else torch.device(device)
    return torch.empty(max(layout.workspace_bytes(dtype), 256), dtype=torch.uint8, device=device)


def device_status(workspace) -> int:
    """The sift_device_flag bits of the last call that used `workspace` (waits for the current
    stream to reach this point)."""
    import torch
    flags = torch.zeros(1, dtype=torch.int32).pin_memory()
    stream = torch.cuda.current_stream(workspace.device)
    _check(_lib().sift_device_status(ctypes.c_void_p(workspace.data_ptr()),
                                     workspace.numel() * workspace.element_size(),
                                     ctypes.c_void_p(flags.data_ptr()), ctypes.c_void_p(stream.cuda_stream)),
           "sift_device_status")
    stream.synchronize()
    return int(flags[0])


def _need_tensor(name, t, dtype, device, shape=None, min_numel=None):
    """Raise ValueError unless t is a contiguous tensor of dtype (None: any) on device, with the
    given shape or at least min_numel elements."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: need a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: need dtype {dtype}, got {t.dtype}")
    if t.device != torch.device(device):
        raise ValueError(f"{name}: need a tensor on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: need shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: need at least {min_numel} elements, got {t.numel()}")


def decode_bits(layout: Layout, la, ca, plan=None, workspace=None, row_ptr=None, col_idx=None):
    """Expand LA/CA words (device uint32 tensors, or int32 views) into the CSR.

    Returns (row_ptr int32 [Hq*G+1], col_idx int32 [csr_max_nnz]); nnz = row_ptr[-1].
    """
    import torch
    device = la.device
    for name, t, n in (("la", la, layout.la_words), ("ca", ca, layout.ca_words)):
        if t.device != device or not t.is_contiguous() or t.element_size() != 4 or t.numel() < n:
            raise ValueError(f"{name}: need a contiguous 32-bit device tensor of >= {n} words")
    rows = layout.num_rows
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=device)
    _need_tensor("row_ptr", row_ptr, torch.int32, device, shape=(rows + 1,))
    if col_idx is None:
        col_idx = torch.empty(max(layout.csr_max_nnz, 1), dtype=torch.int32, device=device)
    _need_tensor("col_idx", col_idx, torch.int32, device, min_numel=layout.csr_max_nnz)
    if plan is None:
        plan = plan_upload(layout, device)
    ws, ws_bytes = _workspace(torch, layout, SIFT_BF16, device, workspace)
    _check(_lib().sift_decode_bits(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(la.data_ptr()),
        ctypes.c_void_p(ca.data_ptr()), ctypes.c_void_p(row_ptr.data_ptr()),
        ctypes.c_void_p(col_idx.data_ptr()), col_idx.numel(), ctypes.c_void_p(ws.data_ptr()),
        ws_bytes, _stream_handle(torch, device)), "sift_decode_bits")
    return row_ptr, col_idx


def decode_bits_noalloc(layout: Layout, la, ca, plan, row_ptr, col_idx):
    """decode_bits without a workspace: the library's own per-GPU scratch array (see
    sift_decode_bits_noalloc).  The caller passes every buffer (plan, row_ptr int32 [Hq*G+1],
    col_idx int32 [>= csr_max_nnz]); nothing is allocated.  Calls on one GPU must not overlap."""
    import torch
    device = la.device
    for name, t, n in (("la", la, layout.la_words), ("ca", ca, layout.ca_words)):
        if t.device != device or not t.is_contiguous() or t.element_size() != 4 or t.numel() < n:
            raise ValueError(f"{name}: need a contiguous 32-bit device tensor of >= {n} words")
    _need_tensor("row_ptr", row_ptr, torch.int32, device, shape=(layout.num_rows + 1,))
    _need_tensor("col_idx", col_idx, torch.int32, device, min_numel=layout.csr_max_nnz)
    _need_tensor("plan", plan, torch.uint8, device, min_numel=layout.plan_bytes)
    _check(_lib().sift_decode_bits_noalloc(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(la.data_ptr()),
        ctypes.c_void_p(ca.data_ptr()), ctypes.c_void_p(row_ptr.data_ptr()),
        ctypes.c_void_p(col_idx.data_ptr()), col_idx.numel(), _stream_handle(torch, device)),
        "sift_decode_bits_noalloc")
    return row_ptr, col_idx


def _qkv_dtype(torch, layout, q, k, v):
    n, hq, hkv, d = layout.padded_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    if q.dtype == torch.bfloat16:
        dt = SIFT_BF16
    elif q.dtype == torch.float32:
        dt = SIFT_FP32
    else:
        raise ValueError("q/k/v must be bfloat16 or float32")
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d)), ("v", v, (n, hkv, d))):
        _need_tensor(name, t, q.dtype, q.device, shape=shape)
    return dt


def _outputs(torch, layout, device, want_lse, out, lse):
    n, hq, d = layout.padded_tokens, layout.num_q_heads, layout.head_dim
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=device)
    _need_tensor("out", out, torch.float32, device, shape=(n, hq, d))
    if not want_lse:
        lse = None  # never written, whatever was passed
    elif lse is None:
        lse = torch.empty((hq, n), dtype=torch.float32, device=device)
    if lse is not None:
        _need_tensor("lse", lse, torch.float32, device, shape=(hq, n))
    return out, lse


def sparse_prefill(layout: Layout, q, k, v, row_ptr, col_idx, plan=None, scale: Optional[float] = None,
                   want_lse: bool = False, workspace=None, out=None, lse=None):
    """Block-sparse attention over the CSR.  q [N,Hq,D], k/v [N,Hkv,D] bf16 or fp32.

    Returns (out fp32 [N,Hq,D], lse fp32 [Hq,N] or None).
    """
    import torch
    device = q.device
    dt = _qkv_dtype(torch, layout, q, k, v)
    _need_tensor("row_ptr", row_ptr, torch.int32, device, shape=(layout.num_rows + 1,))
    _need_tensor("col_idx", col_idx, torch.int32, device)
    out, lse = _outputs(torch, layout, device, want_lse, out, lse)
    if plan is None:
        plan = plan_upload(layout, device)
    ws, ws_bytes = _workspace(torch, layout, dt, device, workspace)
    sc = 0.0 if scale is None else float(scale)
    _check(_lib().sift_sparse_prefill(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(q.data_ptr()),
        ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), dt,
        ctypes.c_void_p(row_ptr.data_ptr()), ctypes.c_void_p(col_idx.data_ptr()), col_idx.numel(),
        ctypes.c_float(sc), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
        ctypes.c_void_p(ws.data_ptr()), ws_bytes, _stream_handle(torch, device)),
        "sift_sparse_prefill")
    return out, lse


def sparse_prefill_bits(layout: Layout, la, ca, q, k, v, plan=None, scale: Optional[float] = None,
                        want_lse: bool = False, workspace=None, out=None, lse=None):
    """The same attention with the decode fused in (no CSR): la / ca are the layer's bit words
    (int32 tensors on the device, as for decode_bits).  Returns (out, lse or None)."""
    import torch
    device = q.device
    dt = _qkv_dtype(torch, layout, q, k, v)
    for name, t, words in (("la", la, layout.la_words), ("ca", ca, layout.ca_words)):
        _need_tensor(name, t, torch.int32, device, min_numel=max(words, 1))
    out, lse = _outputs(torch, layout, device, want_lse, out, lse)
    if plan is None:
        plan = plan_upload(layout, device)
    ws, ws_bytes = _workspace(torch, layout, dt, device, workspace)
    sc = 0.0 if scale is None else float(scale)
    _check(_lib().sift_sparse_prefill_bits(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(la.data_ptr()),
        ctypes.c_void_p(ca.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), dt, ctypes.c_float(sc), ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(lse.data_ptr() if lse is not None else 0), ctypes.c_void_p(ws.data_ptr()), ws_bytes,
        _stream_handle(torch, device)), "sift_sparse_prefill_bits")
    return out, lse


def encode_masses_bytes(layout: Layout) -> int:
    return int(_lib().sift_encode_masses_bytes(layout.ref))


def encode_workspace_bytes(layout: Layout) -> int:
    return int(_lib().sift_encode_workspace_bytes(layout.ref))


def tile_masses(layout: Layout, q, k, plan=None, scale: Optional[float] = None, masses=None, status=None,
                workspace=None):
    """Per-tile softmax mass of the dense causal attention (offline encoder, first step).

    q [N,Hq,D], k [N,Hkv,D] bfloat16.  Returns fp32 masses [Hq, G, RT] (RT = the largest
    request's tile count); entry (h, g, c - first tile of g's request) for the causal c <= g.
    status: optional int32 device tensor of one element for the call's sift_device_flag bits.
    workspace: optional uint8 device tensor of at least encode_workspace_bytes(layout) bytes
    (allocated per call when omitted).
    """
    import torch
    device = q.device
    n, hq, hkv, d = layout.padded_tokens, layout.num_q_heads, layout.num_kv_heads, layout.head_dim
    for name, t, shape in (("q", q, (n, hq, d)), ("k", k, (n, hkv, d))):
        _need_tensor(name, t, torch.bfloat16, device, shape=shape)
    nbytes = encode_masses_bytes(layout)
    if masses is None:
        rt = max(nbytes // (4 * max(hq * layout.num_tiles, 1)), 1)
        masses = torch.empty((hq, layout.num_tiles, rt), dtype=torch.float32, device=device)
    _need_tensor("masses", masses, torch.float32, device, min_numel=nbytes // 4)
    if status is not None:
        _need_tensor("status", status, torch.int32, device, min_numel=1)
    wbytes = encode_workspace_bytes(layout)
    if workspace is None:
        workspace = torch.empty(max(wbytes, 256), dtype=torch.uint8, device=device)
    _need_tensor("workspace", workspace, torch.uint8, device, min_numel=wbytes)
    if plan is None:
        plan = plan_upload(layout, device)
    sc = 0.0 if scale is None else float(scale)
    _check(_lib().sift_tile_masses(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_float(sc), ctypes.c_void_p(masses.data_ptr()), masses.numel() * masses.element_size(),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
        ctypes.c_void_p(status.data_ptr() if status is not None else 0), _stream_handle(torch, device)),
        "sift_tile_masses")
    return masses


def select_bits(layout: Layout, masses, p_la: float = 0.9, p_ca: float = 0.9, plan=None, la=None, ca=None,
                status=None):
    """LA / CA words (int32 device tensors, layout as for decode_bits) from tile masses by top-p.
    status: optional int32 device tensor of one element for the call's sift_device_flag bits."""
    import torch
    device = masses.device
    _need_tensor("masses", masses, torch.float32, device, min_numel=encode_masses_bytes(layout) // 4)
    if la is None:
        la = torch.empty(max(layout.la_words, 1), dtype=torch.int32, device=device)
    if ca is None:
        ca = torch.empty(max(layout.ca_words, 1), dtype=torch.int32, device=device)
    for name, t, words in (("la", la, layout.la_words), ("ca", ca, layout.ca_words)):
        _need_tensor(name, t, torch.int32, device, min_numel=max(words, 1))
    if status is not None:
        _need_tensor("status", status, torch.int32, device, min_numel=1)
    if plan is None:
        plan = plan_upload(layout, device)
    _check(_lib().sift_select_bits(
        layout.ref, ctypes.c_void_p(plan.data_ptr()), ctypes.c_void_p(masses.data_ptr()),
        masses.numel() * masses.element_size(), ctypes.c_float(p_la), ctypes.c_float(p_ca),
        ctypes.c_void_p(la.data_ptr()), ctypes.c_void_p(ca.data_ptr()),
        ctypes.c_void_p(status.data_ptr() if status is not None else 0), _stream_handle(torch, device)),
        "sift_select_bits")
    return la, ca


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
