"""Multi-layer prefill pipeline over the C ABI.

SIFT technical summary, section 2 "Metodologia" ("Design del Sistema"): the LA and CA bit
vectors are computed offline per document, per layer and per head, kept in CPU DRAM and handed
to the GPU at prefill time, where each layer decodes its bits and runs the sparse attention.

This module is host orchestration only (streams, events, pinned buffers); every step of the
path runs in the library's kernels.  Per layer l, on three streams (all at the default priority):

  copy stream:    H2D of layer l's LA/CA words (pinned host -> bit slot l % 2)
  decode stream:  wait for that copy; sift_decode_bits -> CSR slot l % 2
  compute stream: wait for that decode; sift_sparse_prefill -> O_l

Layer l + 1's decode is enqueued right after layer l's attention, and layer l + 2's copy after
that, so both run while layer l's attention does.  The attention kernel holds every CU while its
queues last, and the decode kernels take the CUs its workgroups leave when they run dry.  The
bit and CSR slots are double buffered.  Layer l + 2's copy waits until decode(l), the last reader
of its bit slot, has run.  Decode(l + 2) waits until prefill(l), the last reader of its CSR slot,
has run.  The decode stream has a workspace of its own, since the prefill's workspace is in use
meanwhile.  The plan is uploaded once: it depends on the layout only.
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
        self.row_ptr = [torch.empty(layout.num_rows + 1, dtype=torch.int32, device=self.device) for _ in range(2)]
        self.col_idx = [torch.empty(max(layout.csr_max_nnz, 1), dtype=torch.int32, device=self.device)
                        for _ in range(2)]
        self.workspace = torch.empty(max(layout.workspace_bytes(dtype), layout.workspace_bytes(B.SIFT_BF16), 1),
                                     dtype=torch.uint8, device=self.device)
        self.decode_workspace = torch.empty(max(layout.workspace_bytes(B.SIFT_BF16), 1), dtype=torch.uint8,
                                            device=self.device)
        self.copy_stream = torch.cuda.Stream(device=self.device)    # default priority
        self.decode_stream = torch.cuda.Stream(device=self.device)  # default priority

    def run(self, q_per_layer: Sequence, k_per_layer: Sequence, v_per_layer: Sequence,
            out_per_layer: Optional[List] = None, lse_per_layer: Optional[List] = None):
        """Enqueue every layer: the attention on the current stream, the copies and decodes on the
        side streams; returns the per-layer outputs.  Nothing here synchronises the device."""
        torch = self.torch
        L = self.num_layers
        if not (len(q_per_layer) == len(k_per_layer) == len(v_per_layer) == L):
            raise ValueError("one Q, K and V per layer")
        compute = torch.cuda.current_stream(self.device)
        copied = [torch.cuda.Event() for _ in range(L)]
        decoded = [torch.cuda.Event() for _ in range(L)]    # CSR slot l % 2 holds layer l; bit slot free
        attended = [torch.cuda.Event() for _ in range(L)]   # prefill(l) done with CSR slot l % 2
        outs = out_per_layer if out_per_layer is not None else [None] * L
        lses = lse_per_layer if lse_per_layer is not None else [None] * L
        # the caller's inputs (produced on the compute stream) and the plan must be ready before
        # the side streams start
        start = torch.cuda.Event()
        start.record(compute)

        def issue_copy(l):
            s = l % 2
            with torch.cuda.stream(self.copy_stream):
                self.copy_stream.wait_event(start)
                if l >= 2:
                    self.copy_stream.wait_event(decoded[l - 2])
                self.la_dev[s].copy_(self.la_host[l], non_blocking=True)
                self.ca_dev[s].copy_(self.ca_host[l], non_blocking=True)
                copied[l].record(self.copy_stream)

        def issue_decode(l):
            s = l % 2
            with torch.cuda.stream(self.decode_stream):
                self.decode_stream.wait_event(start)
                self.decode_stream.wait_event(copied[l])
                if l >= 2:
                    self.decode_stream.wait_event(attended[l - 2])
                B.decode_bits(self.layout, self.la_dev[s], self.ca_dev[s], plan=self.plan,
                              workspace=self.decode_workspace, row_ptr=self.row_ptr[s], col_idx=self.col_idx[s])
                decoded[l].record(self.decode_stream)

        issue_copy(0)
        issue_decode(0)
        if L > 1:
            issue_copy(1)
        for l in range(L):
            s = l % 2
            compute.wait_event(decoded[l])
            o, lse = B.sparse_prefill(self.layout, q_per_layer[l], k_per_layer[l], v_per_layer[l],
                                      self.row_ptr[s], self.col_idx[s], plan=self.plan, workspace=self.workspace,
                                      out=outs[l], lse=lses[l], want_lse=lses[l] is not None)
            attended[l].record(compute)
            outs[l] = o
            lses[l] = lse
            if l + 1 < L:
                issue_decode(l + 1)
            if l + 2 < L:
                issue_copy(l + 2)
        # the caller's stream is the last to touch every buffer: later work on it (or a reuse of
        # this pipeline) is ordered after the side streams
        compute.wait_event(decoded[L - 1])
        return outs, lses
