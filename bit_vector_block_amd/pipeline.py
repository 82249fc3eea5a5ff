"""Multi-layer prefill pipeline over the C ABI.

SIFT technical summary, section 2 "Metodologia" ("Design del Sistema"): the LA and CA bit
vectors are computed offline per document, per layer and per head, kept in CPU DRAM and handed
to the GPU at prefill time, where each layer decodes its bits and runs the sparse attention.

This module is host orchestration only (streams, events, pinned buffers); every step of the
path runs in the library's kernels.  Two streams, both at the default priority:

  copy stream:     H2D of the layers' LA/CA words (pinned host -> device), in groups of 1, 2,
                   4, 8, ... layers, each group with an event;
  compute stream:  per group, one wait for its copy; per layer, sift_sparse_prefill_bits (its
                   decode and V^T in one launch, then the attention) -> O_l.

The copies are small and run ahead of the compute stream, so the H2D traffic never sits on the
critical path after the first layer's words, and every layer has a slot of its own, so the
compute stream records no event.  Each wait between two kernels of the compute stream costs it
about 9 us, hence the doubling groups: log2(layers) waits instead of one per layer.  A layer's
decode is not overlapped with the previous layer's attention on another stream: the attention
kernel is persistent and holds every CU while its row queues last, and kernels of a second
stream that take CUs from it (or events between them) cost more than the overlap saves
(measured: decode or decode + V^T on a side stream, two or three slots or one per layer, all
2.4-7 % slower per layer than the calls in sequence on one stream).  The plan is uploaded once:
it depends on the layout only.
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
        # pinned host copies of every layer's bits (the "CPU DRAM" store), int32 views of uint32
        # words, layer after layer; and a device slot for every layer
        L = self.num_layers
        self.la_n, self.ca_n = la_n, ca_n
        self.la_host = torch.zeros(L * la_n, dtype=torch.int32, pin_memory=True)
        self.ca_host = torch.zeros(L * ca_n, dtype=torch.int32, pin_memory=True)
        for l, (la, ca) in enumerate(zip(la_words_per_layer, ca_words_per_layer)):
            la = np.ascontiguousarray(la, dtype=np.uint32)
            ca = np.ascontiguousarray(ca, dtype=np.uint32)
            if la.size != layout.la_words or ca.size != layout.ca_words:
                raise ValueError("bit arrays do not match the layout's word counts")
            if la.size:
                self.la_host.numpy()[l * la_n:l * la_n + la.size] = la.view(np.int32)
            if ca.size:
                self.ca_host.numpy()[l * ca_n:l * ca_n + ca.size] = ca.view(np.int32)
        self.la_dev = torch.empty(L * la_n, dtype=torch.int32, device=self.device)
        self.ca_dev = torch.empty(L * ca_n, dtype=torch.int32, device=self.device)
        self.plan = B.plan_upload(layout, self.device)
        self.workspace = torch.empty(max(layout.workspace_bytes(dtype), 1), dtype=torch.uint8, device=self.device)
        self.copy_stream = torch.cuda.Stream(device=self.device)  # default priority

    def run(self, q_per_layer: Sequence, k_per_layer: Sequence, v_per_layer: Sequence,
            out_per_layer: Optional[List] = None, lse_per_layer: Optional[List] = None):
        """Enqueue every layer: the copies on the side stream, the layers on the current stream;
        returns the per-layer outputs.  Nothing here synchronises the device."""
        torch = self.torch
        L = self.num_layers
        if not (len(q_per_layer) == len(k_per_layer) == len(v_per_layer) == L):
            raise ValueError("one Q, K and V per layer")
        compute = torch.cuda.current_stream(self.device)
        outs = out_per_layer if out_per_layer is not None else [None] * L
        lses = lse_per_layer if lse_per_layer is not None else [None] * L
        # a previous run's layers on the compute stream may still read the slots: this run's copies
        # start after them
        start = torch.cuda.Event()
        start.record(compute)
        groups = []  # (first layer, end, event)
        with torch.cuda.stream(self.copy_stream):
            self.copy_stream.wait_event(start)
            first, size = 0, 1
            while first < L:
                end = min(L, first + size)
                self.la_dev[first * self.la_n:end * self.la_n].copy_(self.la_host[first * self.la_n:end * self.la_n],
                                                                    non_blocking=True)
                self.ca_dev[first * self.ca_n:end * self.ca_n].copy_(self.ca_host[first * self.ca_n:end * self.ca_n],
                                                                    non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(self.copy_stream)
                groups.append((first, end, ev))
                first, size = end, 2 * size
        for first, end, ev in groups:
            compute.wait_event(ev)
            for l in range(first, end):
                la = self.la_dev[l * self.la_n:(l + 1) * self.la_n]
                ca = self.ca_dev[l * self.ca_n:(l + 1) * self.ca_n]
                o, lse = B.sparse_prefill_bits(self.layout, la, ca, q_per_layer[l], k_per_layer[l], v_per_layer[l],
                                               plan=self.plan, workspace=self.workspace, out=outs[l], lse=lses[l],
                                               want_lse=lses[l] is not None)
                outs[l] = o
                lses[l] = lse
        # the last layer waited for the last copy, so later work on the caller's stream (or a
        # reuse of this pipeline) is ordered after every copy
        return outs, lses
