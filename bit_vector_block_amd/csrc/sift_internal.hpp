// Internal declarations shared by the libsift.so translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "sift.h"

namespace sift {

constexpr int kTile = 64;
constexpr int kPrefillQueues = 8;  // row-queue counters (one per XCD) at the start of the workspace
constexpr uint32_t kPlanMagic = 0x54464953u;  // "SIFT"
constexpr int kHeaderWords = 16;
constexpr int32_t kPlanVersion = 2;  // header word 1: the plan image's format

// Every workspace starts with a 256-byte header: int32 words 0..7 are the attention kernel's
// row-queue counters, word kStatusWord holds the sift_device_flag bits of the last call that
// used the workspace (read with sift_device_status).
constexpr size_t kWorkspaceHeader = 256;
constexpr int kStatusWord = 32;

// Device view of an uploaded plan.  Every array lives inside the plan buffer.
struct PlanView {
    const int32_t *header;      // [16]: magic, version, fp_lo, fp_hi, R, Ndocs, G, Hq, ...
    const int32_t *tile_doc;    // [G]: global doc of a document tile, -(request+1) for a question tile
    const int32_t *tile_local;  // [G]: tile index inside its segment
    const int32_t *tile_valid;  // [G]: valid tokens in the tile (1..64)
    const int32_t *doc_first;   // [Ndocs]: global first tile
    const int32_t *doc_tiles;   // [Ndocs]: T_d
    const int32_t *doc_la_off;  // [Ndocs]: word offset of the (d, head 0) LA vector
    const int32_t *doc_ca_off;  // [Ndocs]
    const int32_t *doc_la_w;    // [Ndocs]: words per (d, h) LA vector
    const int32_t *doc_ca_w;    // [Ndocs]
    const int32_t *doc_req;     // [Ndocs]: request of the document
    const int32_t *req_first;   // [R]: global first tile of the request
    const int32_t *req_first_doc;  // [R]: global index of the request's first document
    const int32_t *req_ndocs;   // [R]
    // The same facts gathered per tile and per document (kRecWords int32 each), so that a
    // kernel gets all of a row's or a document's fields in one round trip to memory:
    const int32_t *tile_rec;    // [G][8]: TileRec fields
    const int32_t *doc_rec;     // [Ndocs][8]: DocRec fields
    uint32_t fp_lo, fp_hi;      // fingerprint the host expects
    int32_t num_requests, num_docs, num_tiles, num_q_heads;
};

constexpr int kRecWords = 8;
// tile_rec[g]: the segment of tile g and where its row's bits and list parts live.
enum TileRec {
    kTrDoc = 0,    // global document, or -(b + 1) for a question tile of request b
    kTrLocal = 1,  // r: index of the tile in its segment
    kTrFirst = 2,  // first tile of the document (of the request, for a question tile)
    kTrReq = 3,    // first tile of the request
    kTrLaOff = 4,  // word offset of the document's (head 0) LA vector (0 for a question tile)
    kTrLaW = 5,    // words per (document, head) LA vector (0 for a question tile)
    kTrLo = 6,     // first LA bit of the row: r (r + 1) / 2 (0 for a question tile)
};
// doc_rec[d]
enum DocRec {
    kDrCaOff = 0,  // word offset of the document's (head 0) CA vector
    kDrCaW = 1,    // words per (document, head) CA vector
    kDrTiles = 2,  // T_d
    kDrReqDoc = 3, // first document of the request
    kDrFirst = 4,  // first tile of the document
    kDrReq = 5,    // first tile of the request
    kDrLaOff = 6,  // word offset of the document's (head 0) LA vector
    kDrAfter = 7,  // tiles of the later documents of the request
};

// Device check that an uploaded plan belongs to the layout the host validated: the plan header's
// magic, format, fingerprint and tile count against the host's values carried in `pv`.
__device__ inline bool plan_ok(const PlanView &pv) {
    return pv.header[0] == static_cast<int32_t>(kPlanMagic) && pv.header[1] == kPlanVersion &&
           static_cast<uint32_t>(pv.header[2]) == pv.fp_lo &&
           static_cast<uint32_t>(pv.header[3]) == pv.fp_hi && pv.header[6] == pv.num_tiles;
}

// Host-side summary of a validated layout.
struct HostLayout {
    int32_t R = 0, ndocs = 0, G = 0, Hq = 0, Hkv = 0, D = 0;
    int64_t la_words = 0, ca_words = 0, max_nnz = 0;
    int64_t max_doc_tiles = 0;
    int64_t max_req_tiles = 0;
    int64_t question_nnz = 0;  // list entries of one head's question rows (the same for every head)
    uint64_t fingerprint = 0;
    std::vector<int32_t> plan;  // the full plan image (header + arrays)
};

// Validates `layout` and fills `out` (plan image included).  Returns SIFT_OK,
// SIFT_ERR_INVALID or SIFT_ERR_UNSUPPORTED.
sift_status build_layout(const sift_layout *layout, HostLayout *out);

// Pointers into a device plan buffer laid out like HostLayout::plan.
PlanView plan_view(const HostLayout &hl, const void *d_plan);

size_t decode_workspace_bytes(const HostLayout &hl);

// Launchers (return hipSuccess or the launch error).
// Decode: `scratch` is the decode's scratch (past the workspace header), `status` the status word.
hipError_t launch_decode(const HostLayout &hl, const PlanView &pv, const uint32_t *la,
                         const uint32_t *ca, int32_t *row_ptr, int32_t *col_idx, void *scratch,
                         int32_t *status, hipStream_t stream);
// Fused path: the single-launch decode into a CSR of the workspace beside the V^T transpose, in
// one launch, for layouts that decode_transpose_fits (the others run launch_transpose_v, then
// launch_decode).  The decode writes the status word; the transpose clears the row-queue counters.
bool decode_transpose_fits(const HostLayout &hl);
hipError_t launch_decode_transpose(const HostLayout &hl, const PlanView &pv, const uint32_t *la, const uint32_t *ca,
                                   int32_t *row_ptr, int32_t *col_idx, int32_t *status, const void *v, bool fp32,
                                   uint16_t *vt, int *header, hipStream_t stream);
// Offline encoder (tile masses of dense attention, then top-p selection into LA/CA words).
// `status` (may be null): the caller's device word for the sift_device_flag bits.
// The tile-mass kernel is persistent: each workgroup claims work items from its XCD's queue
// (the first kMassQueues ints of the workspace, cleared by the launch) and keeps its queries'
// per-tile sums in its own slot of the workspace (past the 256-byte header).
constexpr int kMassQueues = 8;    // one work queue per XCD
constexpr int kMassWaves = 4096;  // wavefronts the persistent grid is sized for: 256 CUs x 16
int64_t mass_slots(const HostLayout &hl);
size_t mass_workspace_bytes(const HostLayout &hl);
hipError_t launch_tile_masses(const HostLayout &hl, const PlanView &pv, const uint16_t *q, const uint16_t *k,
                              float scale, float *masses, int RT, void *workspace, int32_t *status,
                              hipStream_t stream);
hipError_t launch_select_bits(const HostLayout &hl, const PlanView &pv, const float *masses, int RT, float p_la,
                              float p_ca, uint32_t *la_out, uint32_t *ca_out, int32_t *status, hipStream_t stream);
hipError_t launch_cast_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream);
// V [N][Hkv][D] (bf16, or fp32 when fp32 is set) -> bf16 V^T tiles [Hkv][G][D][64] in the prefill layout;
// also zeroes the workspace header (the 8 row-queue counters the attention kernel claims rows
// from, and the status word); `header` is the workspace start.
hipError_t launch_transpose_v(const HostLayout &hl, const void *v, bool fp32, uint16_t *vt, int *header,
                              hipStream_t stream);
// Attention over the CSR (col_entries readable col_idx entries).  `header`: the workspace start
// (row-queue counters, status word).
hipError_t launch_prefill(const HostLayout &hl, const PlanView &pv, const uint16_t *q,
                          const uint16_t *k, const uint16_t *vt, const int32_t *row_ptr,
                          const int32_t *col_idx, int64_t col_entries, float scale, float *out, float *lse,
                          int *header, hipStream_t stream);

}  // namespace sift
