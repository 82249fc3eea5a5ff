/*
 * sift.h -- C ABI of libsift.so: bit-vector sparse RAG prefill on MI355X (gfx950).
 *
 * SIFT (Selective-Index For Fast Compute of RAG Prefill by Exploiting Attention
 * Invariance), technical summary, section 2 "Metodologia":
 *   - "Design del Sistema": for every retrieved document, and per layer and
 *     head, two compact bit vectors are stored.  Local-Attention (LA) bits mark
 *     the high-score tiles of the document's own self-attention matrix;
 *     Cross-Attention (CA) bits mark the document's KV pages (columns) that
 *     draw attention from other documents.  At prefill time a sparse attention
 *     kernel reads the bits and evaluates scores only on the marked tiles/pages.
 *   - "Dettagli di Implementazione": a decode kernel turns the bit vectors into
 *     explicit tile indices, and a FlashAttention-style kernel iterates over
 *     those indices only.
 *
 * Readings fixed here where the pages are silent: tile = KV page = 64 tokens;
 * CA pages of document i are visited by every query tile of every later
 * document of the same request; question tokens attend densely and causally to
 * every earlier token of their request; causality is per token.
 *
 * Data formats
 * ------------
 * Token layout: requests in order; in each request its documents in order and
 * then its question; each segment is padded up to a multiple of 64 tokens.
 * G = total tiles, N = 64 * G padded tokens.  Global tile g covers tokens
 * [64 g, 64 g + 64).
 *
 * Q is [N][Hq][D], K and V are [N][Hkv][D], row-major, bf16 (or fp32, see
 * sift_dtype), post-RoPE.  Padded slots may hold any finite values (padded
 * K slots may even hold NaN); they are never attended.  Query head h reads
 * KV head h / (Hq / Hkv).
 *
 * Bits (one layer): LA(d,h; r,c) for 0 <= c <= r < T_d is bit r(r+1)/2 + c of
 * the (doc d, q head h) vector; CA(d,h; c) for 0 <= c < T_d is bit c.  Bit k
 * is in uint32 word k >> 5 at position k & 31 (LSB first).  Every vector starts
 * on a word boundary; vectors are stored [global doc][q head][words] with no
 * gaps.  Bits beyond a vector's length are ignored.  The CA vector of the
 * last document of a request is read by nobody.
 *
 * CSR: rows are ordered h * G + g.  Row (h, g) for tile r of document d lists,
 * ascending, the global tiles of the CA-marked pages of documents 0..d-1 of
 * the same request, then the tiles t0_d + c (c <= r) with LA(d,h; r,c) set.
 * A question tile g lists every tile of its request from the first up to g.
 * row_ptr is int32 [Hq*G + 1] with row_ptr[0] = 0 and row_ptr[Hq*G] = nnz;
 * col_idx is int32 [nnz].
 *
 * Output: O is fp32 [N][Hq][D]; LSE (optional) is fp32 [Hq][N], natural log.
 * Padded query tokens and queries with an empty key set get O = 0 and
 * LSE = -inf.
 *
 * Conventions of every call
 * -------------------------
 * Ownership: the caller allocates and frees every device buffer (plan,
 * workspace, inputs, outputs); the library allocates no device memory and keeps
 * no device state.  Layout arrays are host memory read during the call only.
 * Asynchrony: work is enqueued on `stream` and the call returns without waiting
 * for it; results are ready when the stream reaches that point.  The library
 * never synchronises the device.
 * Workspace: a call's workspace is its scratch (row-queue counters, V^T tiles,
 * decode intermediates) until its stream has passed the call.  Calls that can
 * run at the same time, e.g. on different streams, need separate workspaces;
 * calls in order on one stream may share one.  Its first 256 bytes are a
 * header that holds, among others, the device status word of the last call
 * that used the workspace (sift_device_status).
 * Errors: every call validates its host-side arguments first and launches
 * nothing on error; that is the sift_status it returns.  What only the device
 * can see -- a plan uploaded for another layout, a listed tile id outside
 * [0, G), a CSR row outside the given col_idx -- the kernels report as
 * sift_device_flag bits in a device status word, which a call clears when it
 * starts; they never read or write out of bounds for it.  Nothing throws
 * across the ABI.
 */
#ifndef SIFT_H
#define SIFT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SIFT_OK = 0,
    SIFT_ERR_INVALID = 1,     /* bad argument: null pointer, inconsistent layout, bad sizes */
    SIFT_ERR_CAPACITY = 2,    /* a caller buffer is smaller than the size helper requires */
    SIFT_ERR_UNSUPPORTED = 3, /* valid but unsupported: head_dim not 64/128, tile not 64, int32 overflow */
    SIFT_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} sift_status;

/* Bytes of the per-GPU scratch array of sift_decode_bits_noalloc. */
#define SIFT_DECODE_NOALLOC_MAX_BYTES ((size_t)8 << 20)

/* Bits of a device status word (see sift_device_status): what the kernels found that the host
 * could not check.  0 = SIFT_DEVICE_OK. */
typedef enum {
    SIFT_DEVICE_OK = 0,
    SIFT_DEVICE_PLAN_MISMATCH = 1, /* d_plan holds another layout's plan: the call computed nothing
                                      (sift_decode_bits writes an empty CSR, row_ptr all 0; the
                                      other calls leave their outputs untouched) */
    SIFT_DEVICE_TILE_RANGE = 2,    /* a listed tile id outside [0, G): the entry was skipped */
    SIFT_DEVICE_ROW_RANGE = 4      /* a CSR row whose [row_ptr[r], row_ptr[r+1]) is not inside
                                      [0, col_entries]: the row was taken as empty */
} sift_device_flag;

typedef enum {
    SIFT_BF16 = 0, /* Q/K/V are bf16 */
    SIFT_FP32 = 1  /* Q/K/V are fp32; rounded to bf16 (nearest even) on the device first */
} sift_dtype;

/* One batch of RAG prompts.  All pointers are host memory. */
typedef struct {
    int32_t num_requests;          /* >= 1 */
    const int32_t *req_num_docs;   /* [num_requests], >= 0 */
    const int32_t *doc_len;        /* [sum req_num_docs], unpadded tokens, >= 1 */
    const int32_t *question_len;   /* [num_requests], unpadded tokens, >= 0 */
    int32_t num_q_heads;           /* Hq >= 1 */
    int32_t num_kv_heads;          /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t head_dim;              /* D: 64 or 128 */
    int32_t tile;                  /* must be 64 */
} sift_layout;

/* ---- sizing helpers: return -1 (or 0 for size_t) if the layout is invalid ---- */

int64_t sift_num_tiles(const sift_layout *layout);     /* G */
int64_t sift_padded_tokens(const sift_layout *layout); /* N = 64 G */
int64_t sift_num_rows(const sift_layout *layout);      /* Hq * G */
int64_t sift_la_words(const sift_layout *layout);      /* uint32 words of all LA vectors */
int64_t sift_ca_words(const sift_layout *layout);      /* uint32 words of all CA vectors */
/* Upper bound of nnz: the count with every bit set (dense causal tiles). */
int64_t sift_csr_max_nnz(const sift_layout *layout);
/* Bytes of the device plan written by sift_plan_upload. */
size_t sift_plan_bytes(const sift_layout *layout);
/* Bytes of device scratch that sift_decode_bits / sift_sparse_prefill / sift_sparse_prefill_bits need. */
size_t sift_workspace_bytes(const sift_layout *layout, sift_dtype dtype);

/*
 * sift_plan_upload: write the layout's device tables (per-tile segment data,
 * per-document bit offsets, per-request first tiles, and the same facts gathered
 * into one record per tile and per document) into d_plan, a caller buffer of at
 * least sift_plan_bytes() bytes, with one hipMemcpyAsync on `stream` from a host
 * staging copy.  A plan depends on the layout only, so one upload serves every
 * layer of a batch.  The plan carries a fingerprint of the layout and its format
 * version; a kernel launched with a plan of another layout (or of another version
 * of this library) computes nothing and
 * raises SIFT_DEVICE_PLAN_MISMATCH in the call's device status word (the host
 * cannot see the plan's contents without a synchronisation).
 * Errors: SIFT_ERR_INVALID (layout, null), SIFT_ERR_CAPACITY (plan_bytes),
 * SIFT_ERR_HIP.
 */
sift_status sift_plan_upload(const sift_layout *layout, void *d_plan, size_t plan_bytes,
                             hipStream_t stream);

/*
 * sift_decode_bits: the decode kernel of the technical summary's
 * "Dettagli di Implementazione" -- expand one layer's LA and CA bit vectors
 * (device, sift_la_words / sift_ca_words uint32 words) into the CSR described
 * above: d_row_ptr int32 [Hq*G + 1] and d_col_idx int32 [col_capacity].
 * col_capacity must be >= sift_csr_max_nnz(), which makes the fill safe
 * without a host read-back of nnz (nnz is row_ptr[Hq*G] on the device).
 * d_workspace: >= sift_workspace_bytes(layout, SIFT_BF16) bytes of scratch; its
 * status word gets SIFT_DEVICE_OK, or SIFT_DEVICE_PLAN_MISMATCH (and the CSR is
 * then empty: row_ptr all 0).
 * Errors: SIFT_ERR_INVALID, SIFT_ERR_CAPACITY (col_capacity, workspace),
 * SIFT_ERR_UNSUPPORTED (nnz bound >= 2^31), SIFT_ERR_HIP.
 */
sift_status sift_decode_bits(const sift_layout *layout, const void *d_plan,
                             const uint32_t *d_la, const uint32_t *d_ca,
                             int32_t *d_row_ptr, int32_t *d_col_idx, int64_t col_capacity,
                             void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sift_decode_bits_noalloc: sift_decode_bits for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument and no allocation.  The decode's scratch is an array of the library's own,
 * one per GPU, of SIFT_DECODE_NOALLOC_MAX_BYTES bytes (8 MiB), held until the process ends;
 * layouts whose decode scratch is larger (sift_workspace_bytes, about 8 Hq G bytes plus
 * 4 Hq ndocs) get SIFT_ERR_CAPACITY.  `stream` must belong to the current device.  Same
 * arguments, output and errors as sift_decode_bits otherwise; a plan of another layout gives an
 * empty CSR (row_ptr all 0).  Every call on a GPU shares that GPU's array: calls that can run at
 * the same time on one GPU (other streams, other threads) race and must not overlap.
 */
sift_status sift_decode_bits_noalloc(const sift_layout *layout, const void *d_plan,
                                     const uint32_t *d_la, const uint32_t *d_ca,
                                     int32_t *d_row_ptr, int32_t *d_col_idx, int64_t col_capacity,
                                     hipStream_t stream);

/*
 * sift_sparse_prefill: the sparse attention kernel of "Dettagli di
 * Implementazione" -- block-sparse causal GQA attention with online softmax
 * that, for each row (h, g), visits only the KV tiles listed in the CSR.
 * scores = scale * q.k (scale <= 0 selects 1/sqrt(head_dim)), bf16 MFMA with
 * fp32 accumulation, fp32 softmax, fp32 output d_out [N][Hq][D]; d_lse
 * [Hq][N] may be NULL.  d_col_idx holds col_entries readable int32 entries; a row
 * whose range [row_ptr[r], row_ptr[r+1]) is not inside [0, col_entries] is taken
 * as empty (SIFT_DEVICE_ROW_RANGE), and a listed tile outside [0, G) is skipped
 * (SIFT_DEVICE_TILE_RANGE): no read leaves the given buffers.
 * d_q, d_k, d_v, d_out and d_workspace must be 16-byte aligned (SIFT_ERR_INVALID otherwise).
 * d_workspace: >= sift_workspace_bytes(layout, dtype) bytes of scratch; it holds
 * the header (status word), V transposed to bf16, tile by tile [Hkv][G][D][64]
 * (written by the call, in a token order internal to the library) and, for
 * SIFT_FP32 inputs, the bf16 copies of Q and K.
 * Errors: SIFT_ERR_INVALID, SIFT_ERR_CAPACITY (workspace),
 * SIFT_ERR_UNSUPPORTED (head_dim, tile), SIFT_ERR_HIP.
 */
sift_status sift_sparse_prefill(const sift_layout *layout, const void *d_plan,
                                const void *d_q, const void *d_k, const void *d_v, sift_dtype dtype,
                                const int32_t *d_row_ptr, const int32_t *d_col_idx, int64_t col_entries,
                                float scale, float *d_out, float *d_lse,
                                void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sift_sparse_prefill_bits: the same attention, with the decode folded into the call: the caller
 * passes the bits and gets the attention output, no CSR.  The SIFT technical summary's "Design
 * del Sistema" has the attention read the bit vectors; here one launch decodes them into a CSR
 * in the workspace (each workgroup counts its q head's rows in closed form and lists its share of
 * them) while its other workgroups write V^T, and the attention kernel then reads that CSR.
 * Layouts past the single-launch decode's bounds (more than 2048 tiles, 512 documents or 64 tiles
 * in a document; more than 8192 LA words or 2048 CA words in all, or 4096 LA words in one q
 * head's vectors) run the V^T transpose and the two-launch decode first instead.
 * d_la, d_ca: the layer's bits as for sift_decode_bits.  Other arguments, the output and the
 * 16-byte alignment rule as for sift_sparse_prefill; the result is bit-identical to
 * sift_decode_bits followed by sift_sparse_prefill on the same bits.
 * d_workspace: >= sift_workspace_bytes(layout, dtype) bytes (it also holds the CSR: 4 (Hq G + 1)
 * + 4 sift_csr_max_nnz() bytes more than sift_sparse_prefill needs); status word as for
 * sift_sparse_prefill.
 * Errors: SIFT_ERR_INVALID, SIFT_ERR_CAPACITY (workspace), SIFT_ERR_UNSUPPORTED (head_dim, tile,
 * nnz bound >= 2^31), SIFT_ERR_HIP.
 */
sift_status sift_sparse_prefill_bits(const sift_layout *layout, const void *d_plan,
                                     const uint32_t *d_la, const uint32_t *d_ca,
                                     const void *d_q, const void *d_k, const void *d_v, sift_dtype dtype,
                                     float scale, float *d_out, float *d_lse,
                                     void *d_workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Offline encoder.  The SIFT technical summary's "Design del Sistema" computes the bits offline
 * from a dense prefill of each document, keeping the positions with high attention scores; the
 * pages leave the selection rule open.  This encoder reads it as a top-p rule on tile masses:
 *
 * sift_tile_masses: mass(h, g, c) = sum, over the valid queries of query tile g and the keys of
 * key tile c, of the softmax probability of the dense causal attention of the request (bf16
 * Q [N][Hq][D] and K [N][Hkv][D], 16-byte aligned; scale <= 0 selects 1/sqrt(head_dim)).
 * d_masses: fp32 [Hq][G][RT], RT = the largest request's tile count; entry (h, g, c - first)
 * with first = the first tile of g's request, written for first <= c <= g only.  masses_bytes >=
 * sift_encode_masses_bytes(layout).  The scores are computed once: each query's per-tile sums of
 * exp2 go to d_workspace (>= sift_encode_workspace_bytes(layout) bytes, 16-byte aligned; about
 * 512 KiB per tile of the largest request: a slot per resident workgroup, not per work item),
 * and are weighted by the query's 1 / (row sum) once its row is done.  Calls that run at the
 * same time need separate workspaces.
 *
 * sift_select_bits: LA row r of document d keeps its candidate tiles c <= r by decreasing mass
 * (ties: smaller c) up to the first prefix whose mass reaches p_la of their total, plus tiles r
 * and 0; CA page c of d gets the mass that the request's later documents' query tiles put on it
 * (summed in increasing tile order) and the pages are kept the same way with p_ca, plus page 0.
 * The threshold test sums in float32 in a fixed order (an inclusive Hillis-Steele scan of the
 * sorted masses).  Writes every word of d_la / d_ca (layout as for sift_decode_bits).
 * Errors: SIFT_ERR_INVALID (p outside (0, 1], nulls, misaligned pointers), SIFT_ERR_CAPACITY
 * (masses_bytes, workspace), SIFT_ERR_UNSUPPORTED (sift_select_bits: a document of more than 64
 * tiles), SIFT_ERR_HIP.
 *
 * d_status (both calls, may be NULL): one device int32 that the call sets to SIFT_DEVICE_OK, or to
 * SIFT_DEVICE_PLAN_MISMATCH when d_plan holds another layout's plan (the outputs are then left
 * untouched).  A call with nothing to do (no tiles, no documents) leaves it as it is.
 */
size_t sift_encode_masses_bytes(const sift_layout *layout);
size_t sift_encode_workspace_bytes(const sift_layout *layout);
sift_status sift_tile_masses(const sift_layout *layout, const void *d_plan, const void *d_q, const void *d_k,
                             float scale, float *d_masses, size_t masses_bytes, void *d_workspace,
                             size_t workspace_bytes, int32_t *d_status, hipStream_t stream);
sift_status sift_select_bits(const sift_layout *layout, const void *d_plan, const float *d_masses,
                             size_t masses_bytes, float p_la, float p_ca, uint32_t *d_la, uint32_t *d_ca,
                             int32_t *d_status, hipStream_t stream);

/*
 * sift_device_status: enqueue on `stream` a copy of the device status word of the workspace
 * d_workspace (>= 256 bytes) into *h_flags (host memory; a sift_device_flag bit set).  The value
 * is that of the last call on the workspace that launched work, and is valid once the stream has
 * passed this point (e.g. after hipStreamSynchronize).  A call with no tiles launches nothing
 * and leaves the word as it was.
 * Errors: SIFT_ERR_INVALID (null), SIFT_ERR_CAPACITY (workspace_bytes < 256), SIFT_ERR_HIP.
 */
sift_status sift_device_status(const void *d_workspace, size_t workspace_bytes, int32_t *h_flags,
                               hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *sift_status_string(sift_status status);

/* Version of this ABI: (major << 16) | minor. */
int32_t sift_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SIFT_H */
