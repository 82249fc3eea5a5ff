"""Multi-layer prefill pipeline over the C ABI.

SIFT technical summary, section 2 "Metodologia" ("Design del Sistema"): the LA and CA bit
vectors are computed offline per document, per layer and per head, kept in CPU DRAM and handed
to the GPU at prefill time, where each layer decodes its bits and runs the sparse attention.

This module is host orchestration only (streams, events, pinned buffers); every step of the
path runs in the library's kernels.  Per layer l:

  copy stream:    H2D of layer l's LA/CA words (pinned host -> one of two device slots)
  compute stream: wait for that copy; sift_decode_bits -> CSR; sift_sparse_prefill -> O_l

The copy of layer l + 1 is issued before layer l's kernels are enqueued, so it runs under layer
l's attention.  The device bit slots are double buffered: layer l + 2's copy waits until layer l's
decode, the last reader of that slot, has run.  The plan is uploaded once (it depends on the
layout only) and the CSR and workspace buffers are reused by every layer (their users are all on
the compute stream, so they are ordered).
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import _binding as B


class LayerPipeline:
    """Decode + sparse prefill for a stack of layers sharing one batch layout."""

    def __init__(self, layout: B.Layout, device, la_words_per_layer: Sequence[np.ndarray],
                 ca_words_per_layer: Sequence[np.ndarray], dtype: int = B.SIFT_BF16):
        import torch

        if len(la_words_per_layer) != len(ca_words_per_layer):
            raise ValueError("one LA and one CA word array per layer")
        self.torch = torch
        self.layout = layout
        self.device = torch.device(device)
        self.dtype = dtype
        self.num_layers = len(la_words_per_layer)
        la_n, ca_n = max(layout.la_words, 1), max(layout.ca_words, 1)
        # pinned host copies of every layer's bits (the "CPU DRAM" store), int32 views of uint32 words
        self.la_host, self.ca_host = [], []
        for la, ca in zip(la_words_per_layer, ca_words_per_layer):
            la = np.ascontiguousarray(la, dtype=np.uint32)
            ca = np.ascontiguousarray(ca, dtype=np.uint32)
            if la.size != layout.la_words or ca.size != layout.ca_words:
                raise ValueError("bit arrays do not match the layout's word counts")
            hla = torch.zeros(la_n, dtype=torch.int32, pin_memory=True)
            hca = torch.zeros(ca_n, dtype=torch.int32, pin_memory=True)
            if la.size:
                hla.numpy()[:] = la.view(np.int32)
            if ca.size:
                hca.numpy()[:] = ca.view(np.int32)
            self.la_host.append(hla)
            self.ca_host.append(hca)
        self.la_dev = [torch.empty(la_n, dtype=torch.int32, device=self.device) for _ in range(2)]
        self.ca_dev = [torch.empty(ca_n, dtype=torch.int32, device=self.device) for _ in range(2)]
        self.plan = B.plan_upload(layout, self.device)
        self.row_ptr = torch.empty(layout.num_rows + 1, dtype=torch.int32, device=self.device)
        self.col_idx = torch.empty(max(layout.csr_max_nnz, 1), dtype=torch.int32, device=self.device)
        self.workspace = torch.empty(max(layout.workspace_bytes(dtype), layout.workspace_bytes(B.SIFT_BF16), 1),
                                     dtype=torch.uint8, device=self.device)
        self.copy_stream = torch.cuda.Stream(device=self.device)  # default priority

    def run(self, q_per_layer: Sequence, k_per_layer: Sequence, v_per_layer: Sequence,
            out_per_layer: Optional[List] = None, lse_per_layer: Optional[List] = None):
        """Enqueue every layer on the current stream (the copies on the side stream); returns the
        per-layer outputs.  Nothing here synchronises the device."""
        torch = self.torch
        L = self.num_layers
        if not (len(q_per_layer) == len(k_per_layer) == len(v_per_layer) == L):
            raise ValueError("one Q, K and V per layer")
        compute = torch.cuda.current_stream(self.device)
        copied = [torch.cuda.Event() for _ in range(L)]
        slot_free = [torch.cuda.Event() for _ in range(L)]
        outs = out_per_layer if out_per_layer is not None else [None] * L
        lses = lse_per_layer if lse_per_layer is not None else [None] * L

        def issue_copy(l):
            s = l % 2
            with torch.cuda.stream(self.copy_stream):
                if l >= 2:
                    self.copy_stream.wait_event(slot_free[l - 2])
                self.la_dev[s].copy_(self.la_host[l], non_blocking=True)
                self.ca_dev[s].copy_(self.ca_host[l], non_blocking=True)
                copied[l].record(self.copy_stream)

        issue_copy(0)
        for l in range(L):
            if l + 1 < L:
                issue_copy(l + 1)
            s = l % 2
            compute.wait_event(copied[l])
            B.decode_bits(self.layout, self.la_dev[s], self.ca_dev[s], plan=self.plan,
                          workspace=self.workspace, row_ptr=self.row_ptr, col_idx=self.col_idx)
            slot_free[l].record(compute)
            o, lse = B.sparse_prefill(self.layout, q_per_layer[l], k_per_layer[l], v_per_layer[l],
                                      self.row_ptr, self.col_idx, plan=self.plan, workspace=self.workspace,
                                      out=outs[l], lse=lses[l], want_lse=lses[l] is not None)
            outs[l] = o
            lses[l] = lse
        return outs, lses
