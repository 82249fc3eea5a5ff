"""bit_vector_block_amd: SIFT bit-vector sparse RAG prefill on MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of include/sift.h:
  * ``decode_bits``    -- LA/CA bit vectors -> per-(head, query tile) CSR of KV tiles;
  * ``sparse_prefill`` -- block-sparse causal GQA attention over that CSR
                          (bf16 MFMA, online softmax, fp32 output);
  * ``sparse_prefill_bits`` -- the same attention with the decode fused in (reads the bits);
  * ``tile_masses`` / ``select_bits`` -- the offline encoder: per-tile softmax mass of the dense
                          attention, then top-p selection into LA/CA bits.
What only the device can see (a plan of another layout, tile ids or CSR rows out of range) is
reported in a device status word: ``device_status(workspace)``.
This package is the ctypes binding (argument marshalling), the seeded synthetic
workloads in ``workloads`` and the multi-layer stream orchestration in ``pipeline``.
"""
from ._binding import (SIFT_BF16, SIFT_DEVICE_OK, SIFT_DEVICE_PLAN_MISMATCH, SIFT_DEVICE_ROW_RANGE,
                       SIFT_DEVICE_TILE_RANGE, SIFT_FP32, Layout, SiftError, decode_bits, decode_bits_noalloc,
                       default_scale, device_status, encode_masses_bytes, encode_workspace_bytes, library,
                       plan_upload, select_bits, sparse_prefill, sparse_prefill_bits, tile_masses, workspace)

__all__ = ["Layout", "SiftError", "decode_bits", "decode_bits_noalloc", "sparse_prefill", "sparse_prefill_bits",
           "plan_upload", "tile_masses", "select_bits", "encode_masses_bytes", "encode_workspace_bytes", "library",
           "default_scale", "workspace", "device_status", "SIFT_BF16", "SIFT_FP32", "SIFT_DEVICE_OK", "SIFT_DEVICE_PLAN_MISMATCH",
           "SIFT_DEVICE_TILE_RANGE", "SIFT_DEVICE_ROW_RANGE"]
