// Host side of libsift.so: layout validation, sizing, the device plan, and the
// extern "C" entry points declared in include/sift.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sift_internal.hpp"

namespace sift {

namespace {

constexpr int64_t kInt32Max = 2147483647LL;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

uint64_t fnv1a(uint64_t h, const void *data, size_t n) {
    const unsigned char *p = static_cast<const unsigned char *>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 1099511628211ULL;
    }
    return h;
}

}  // namespace

sift_status build_layout(const sift_layout *layout, HostLayout *out) {
    if (!layout || !out) return SIFT_ERR_INVALID;
    const sift_layout &L = *layout;
    if (L.num_requests < 1 || !L.req_num_docs || !L.question_len) return SIFT_ERR_INVALID;
    if (L.num_q_heads < 1 || L.num_kv_heads < 1 || L.num_q_heads % L.num_kv_heads != 0)
        return SIFT_ERR_INVALID;
    int64_t ndocs = 0;
    for (int32_t b = 0; b < L.num_requests; ++b) {
        if (L.req_num_docs[b] < 0 || L.question_len[b] < 0) return SIFT_ERR_INVALID;
        ndocs += L.req_num_docs[b];
    }
    if (ndocs > 0 && !L.doc_len) return SIFT_ERR_INVALID;
    if (L.tile != kTile) return SIFT_ERR_UNSUPPORTED;
    if (L.head_dim != 64 && L.head_dim != 128) return SIFT_ERR_UNSUPPORTED;
    if (ndocs > kInt32Max) return SIFT_ERR_UNSUPPORTED;

    HostLayout hl;
    hl.R = L.num_requests;
    hl.ndocs = static_cast<int32_t>(ndocs);
    hl.Hq = L.num_q_heads;
    hl.Hkv = L.num_kv_heads;
    hl.D = L.head_dim;

    int64_t G = 0, la_words = 0, ca_words = 0, max_nnz = 0;
    for (int64_t d = 0; d < ndocs; ++d)
        if (L.doc_len[d] < 1) return SIFT_ERR_INVALID;
    {
        int64_t d = 0;
        for (int32_t b = 0; b < L.num_requests; ++b) {
            int64_t tb = 0;
            for (int32_t i = 0; i < L.req_num_docs[b]; ++i, ++d) {
                const int64_t T = ceil_div(L.doc_len[d], kTile);
                if (T > hl.max_doc_tiles) hl.max_doc_tiles = T;
                tb += T;
                la_words += static_cast<int64_t>(L.num_q_heads) * ceil_div(T * (T + 1) / 2, 32);
                ca_words += static_cast<int64_t>(L.num_q_heads) * ceil_div(T, 32);
            }
            tb += ceil_div(L.question_len[b], kTile);
            if (tb > hl.max_req_tiles) hl.max_req_tiles = tb;
            G += tb;
            max_nnz += tb * (tb + 1) / 2;
        }
    }
    max_nnz *= L.num_q_heads;
    // Token indices, CSR entries and word offsets are int32 on the device; a lane's offset into
    // V^T (row d of D, 2 N bytes per row) is uint32.
    if (G * kTile > kInt32Max || G * L.num_q_heads >= kInt32Max || max_nnz >= kInt32Max ||
        la_words > kInt32Max || ca_words > kInt32Max ||
        G * kTile * 2 * static_cast<int64_t>(L.head_dim) > 2 * kInt32Max)
        return SIFT_ERR_UNSUPPORTED;
    hl.G = static_cast<int32_t>(G);
    hl.la_words = la_words;
    hl.ca_words = ca_words;
    hl.max_nnz = max_nnz;

    uint64_t fp = 1469598103934665603ULL;
    const int32_t dims[4] = {L.num_requests, L.num_q_heads, L.num_kv_heads, L.head_dim};
    fp = fnv1a(fp, dims, sizeof(dims));
    fp = fnv1a(fp, L.req_num_docs, sizeof(int32_t) * L.num_requests);
    fp = fnv1a(fp, L.question_len, sizeof(int32_t) * L.num_requests);
    if (ndocs) fp = fnv1a(fp, L.doc_len, sizeof(int32_t) * ndocs);
    hl.fingerprint = fp;

    // plan image
    const int64_t nd = ndocs, R = L.num_requests;
    std::vector<int32_t> &p = hl.plan;
    p.assign(kHeaderWords + 3 * G + 7 * nd + 3 * R + kRecWords * (G + nd), 0);
    int32_t *hdr = p.data();
    hdr[0] = static_cast<int32_t>(kPlanMagic);
    hdr[1] = kPlanVersion;
    hdr[2] = static_cast<int32_t>(fp & 0xffffffffu);
    hdr[3] = static_cast<int32_t>(fp >> 32);
    hdr[4] = L.num_requests;
    hdr[5] = hl.ndocs;
    hdr[6] = hl.G;
    hdr[7] = hl.Hq;
    int32_t *tile_doc = hdr + kHeaderWords;
    int32_t *tile_local = tile_doc + G;
    int32_t *tile_valid = tile_local + G;
    int32_t *doc_first = tile_valid + G;
    int32_t *doc_tiles = doc_first + nd;
    int32_t *doc_la_off = doc_tiles + nd;
    int32_t *doc_ca_off = doc_la_off + nd;
    int32_t *doc_la_w = doc_ca_off + nd;
    int32_t *doc_ca_w = doc_la_w + nd;
    int32_t *doc_req = doc_ca_w + nd;
    int32_t *req_first = doc_req + nd;
    int32_t *req_first_doc = req_first + R;
    int32_t *req_ndocs = req_first_doc + R;
    int32_t *tile_rec = req_ndocs + R;
    int32_t *doc_rec = tile_rec + kRecWords * G;
    int64_t g = 0, d = 0, la_acc = 0, ca_acc = 0;
    for (int32_t b = 0; b < L.num_requests; ++b) {
        req_first[b] = static_cast<int32_t>(g);
        req_first_doc[b] = static_cast<int32_t>(d);
        req_ndocs[b] = L.req_num_docs[b];
        for (int32_t i = 0; i < L.req_num_docs[b]; ++i, ++d) {
            const int64_t n = L.doc_len[d];
            const int64_t T = ceil_div(n, kTile);
            doc_first[d] = static_cast<int32_t>(g);
            doc_req[d] = b;
            doc_tiles[d] = static_cast<int32_t>(T);
            doc_la_w[d] = static_cast<int32_t>(ceil_div(T * (T + 1) / 2, 32));
            doc_ca_w[d] = static_cast<int32_t>(ceil_div(T, 32));
            doc_la_off[d] = static_cast<int32_t>(la_acc);
            doc_ca_off[d] = static_cast<int32_t>(ca_acc);
            la_acc += static_cast<int64_t>(L.num_q_heads) * doc_la_w[d];
            ca_acc += static_cast<int64_t>(L.num_q_heads) * doc_ca_w[d];
            int32_t *dr = doc_rec + kRecWords * d;
            dr[kDrCaOff] = doc_ca_off[d];
            dr[kDrCaW] = doc_ca_w[d];
            dr[kDrTiles] = doc_tiles[d];
            dr[kDrReqDoc] = req_first_doc[b];
            dr[kDrFirst] = doc_first[d];
            dr[kDrReq] = req_first[b];
            dr[kDrLaOff] = doc_la_off[d];
            for (int64_t r = 0; r < T; ++r, ++g) {
                tile_doc[g] = static_cast<int32_t>(d);
                tile_local[g] = static_cast<int32_t>(r);
                tile_valid[g] = static_cast<int32_t>(std::min<int64_t>(kTile, n - r * kTile));
                int32_t *tr = tile_rec + kRecWords * g;
                tr[kTrDoc] = static_cast<int32_t>(d);
                tr[kTrLocal] = static_cast<int32_t>(r);
                tr[kTrFirst] = doc_first[d];
                tr[kTrReq] = req_first[b];
                tr[kTrLaOff] = doc_la_off[d];
                tr[kTrLaW] = doc_la_w[d];
                tr[kTrLo] = static_cast<int32_t>(r * (r + 1) / 2);
            }
        }
        for (int64_t e = req_first_doc[b]; e < d; ++e)  // g is now the request's first question tile
            doc_rec[kRecWords * e + kDrAfter] = static_cast<int32_t>(g - (doc_first[e] + doc_tiles[e]));
        const int64_t m = L.question_len[b];
        const int64_t TQ = ceil_div(m, kTile);
        for (int64_t r = 0; r < TQ; ++r, ++g) {
            hl.question_nnz += g - req_first[b] + 1;
            tile_doc[g] = -(b + 1);
            tile_local[g] = static_cast<int32_t>(r);
            tile_valid[g] = static_cast<int32_t>(std::min<int64_t>(kTile, m - r * kTile));
            int32_t *tr = tile_rec + kRecWords * g;
            tr[kTrDoc] = -(b + 1);
            tr[kTrLocal] = static_cast<int32_t>(r);
            tr[kTrFirst] = req_first[b];
            tr[kTrReq] = req_first[b];
        }
    }
    *out = std::move(hl);
    return SIFT_OK;
}

PlanView plan_view(const HostLayout &hl, const void *d_plan) {
    const int32_t *base = static_cast<const int32_t *>(d_plan);
    const int64_t G = hl.G, nd = hl.ndocs, R = hl.R;
    PlanView v;
    v.header = base;
    v.tile_doc = base + kHeaderWords;
    v.tile_local = v.tile_doc + G;
    v.tile_valid = v.tile_local + G;
    v.doc_first = v.tile_valid + G;
    v.doc_tiles = v.doc_first + nd;
    v.doc_la_off = v.doc_tiles + nd;
    v.doc_ca_off = v.doc_la_off + nd;
    v.doc_la_w = v.doc_ca_off + nd;
    v.doc_ca_w = v.doc_la_w + nd;
    v.doc_req = v.doc_ca_w + nd;
    v.req_first = v.doc_req + nd;
    v.req_first_doc = v.req_first + R;
    v.req_ndocs = v.req_first_doc + R;
    v.tile_rec = v.req_ndocs + R;
    v.doc_rec = v.tile_rec + kRecWords * G;
    v.fp_lo = static_cast<uint32_t>(hl.fingerprint & 0xffffffffu);
    v.fp_hi = static_cast<uint32_t>(hl.fingerprint >> 32);
    v.num_requests = hl.R;
    v.num_docs = hl.ndocs;
    v.num_tiles = hl.G;
    v.num_q_heads = hl.Hq;
    return v;
}

// Decode workspace: the header, then ca_prefix [Hq][ndocs], row offsets [Hq][G], head totals
// [Hq], CA page lists [Hq][G] (int32).
size_t decode_workspace_bytes(const HostLayout &hl) {
    return kWorkspaceHeader + align256(sizeof(int32_t) * size_t(hl.Hq) * size_t(std::max(hl.ndocs, 1))) +
           align256(sizeof(int32_t) * size_t(hl.Hq) * size_t(std::max(hl.G, 1))) +
           align256(sizeof(int32_t) * size_t(hl.Hq)) +
           align256(sizeof(int32_t) * size_t(hl.Hq) * size_t(std::max(hl.G, 1)));
}

// Prefill workspace: the header (row-queue counters, status word), V^T (bf16 tiles
// [Hkv][G][D][64]); for SIFT_FP32 inputs the bf16 copies of Q and K follow.
static size_t prefill_workspace_bytes(const HostLayout &hl, sift_dtype dtype) {
    const size_t N = size_t(hl.G) * kTile;
    const size_t vt = kWorkspaceHeader + align256(2 * N * hl.Hkv * hl.D);
    if (dtype != SIFT_FP32) return vt;
    return vt + align256(2 * N * hl.Hq * hl.D) + align256(2 * N * hl.Hkv * hl.D);
}
// The fused path's tables past the prefill workspace: the CSR its decode writes (row_ptr [Hq G + 1],
// col_idx [max_nnz]) and, for layouts beyond the single-launch decode, that decode's scratch.
static size_t fused_tables_bytes(const HostLayout &hl) {
    const size_t csr = align256(4 * (size_t(hl.Hq) * size_t(hl.G) + 1)) +
                       align256(4 * size_t(hl.max_nnz > 0 ? hl.max_nnz : 1));
    return csr + (decode_transpose_fits(hl) ? 0 : decode_workspace_bytes(hl) - kWorkspaceHeader);
}

// Scratch of the allocation-free decode (sift_decode_bits_noalloc): one array per GPU, in the
// library's code object, held until the process ends.  Host code never passes its name to a
// kernel -- that would be a host-side stand-in -- but the per-device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = SIFT_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream`, which must be the current device.
sift_status noalloc_scratch(hipStream_t stream, char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SIFT_ERR_HIP;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SIFT_ERR_HIP;
        if (sdev != dev) return SIFT_ERR_INVALID;
    }
    if (dev < 0 || dev >= kMaxDevices) return SIFT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SIFT_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return SIFT_OK;
}
}  // namespace

}  // namespace sift

using namespace sift;

extern "C" {

int32_t sift_abi_version(void) { return (3 << 16) | 0; }

const char *sift_status_string(sift_status s) {
    switch (s) {
        case SIFT_OK: return "SIFT_OK";
        case SIFT_ERR_INVALID: return "SIFT_ERR_INVALID: invalid argument or layout";
        case SIFT_ERR_CAPACITY: return "SIFT_ERR_CAPACITY: a caller buffer is too small";
        case SIFT_ERR_UNSUPPORTED: return "SIFT_ERR_UNSUPPORTED: head_dim/tile unsupported or int32 overflow";
        case SIFT_ERR_HIP: return "SIFT_ERR_HIP: HIP runtime or launch failure";
    }
    return "unknown sift_status";
}

int64_t sift_num_tiles(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? hl.G : -1;
}

int64_t sift_padded_tokens(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? int64_t(hl.G) * kTile : -1;
}

int64_t sift_num_rows(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? int64_t(hl.G) * hl.Hq : -1;
}

int64_t sift_la_words(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? hl.la_words : -1;
}

int64_t sift_ca_words(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? hl.ca_words : -1;
}

int64_t sift_csr_max_nnz(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? hl.max_nnz : -1;
}

size_t sift_plan_bytes(const sift_layout *layout) {
    HostLayout hl;
    return build_layout(layout, &hl) == SIFT_OK ? hl.plan.size() * sizeof(int32_t) : 0;
}

size_t sift_workspace_bytes(const sift_layout *layout, sift_dtype dtype) {
    HostLayout hl;
    if (build_layout(layout, &hl) != SIFT_OK) return 0;
    if (dtype != SIFT_BF16 && dtype != SIFT_FP32) return 0;
    return std::max(decode_workspace_bytes(hl), prefill_workspace_bytes(hl, dtype) + fused_tables_bytes(hl));
}

sift_status sift_plan_upload(const sift_layout *layout, void *d_plan, size_t plan_bytes,
                             hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (!d_plan) return SIFT_ERR_INVALID;
    const size_t need = hl.plan.size() * sizeof(int32_t);
    if (plan_bytes < need) return SIFT_ERR_CAPACITY;
    // Pageable source: the runtime stages it before returning, so the host
    // vector may die right after the call.
    if (hipMemcpyAsync(d_plan, hl.plan.data(), need, hipMemcpyHostToDevice, stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

sift_status sift_decode_bits(const sift_layout *layout, const void *d_plan, const uint32_t *d_la,
                             const uint32_t *d_ca, int32_t *d_row_ptr, int32_t *d_col_idx,
                             int64_t col_capacity, void *d_workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (!d_plan || !d_row_ptr) return SIFT_ERR_INVALID;
    if ((hl.la_words > 0 && !d_la) || (hl.ca_words > 0 && !d_ca)) return SIFT_ERR_INVALID;
    if (hl.max_nnz > 0 && !d_col_idx) return SIFT_ERR_INVALID;
    if (col_capacity < hl.max_nnz) return SIFT_ERR_CAPACITY;
    if (!d_workspace || workspace_bytes < decode_workspace_bytes(hl)) return SIFT_ERR_CAPACITY;
    const PlanView pv = plan_view(hl, d_plan);
    char *ws = static_cast<char *>(d_workspace);
    if (launch_decode(hl, pv, d_la, d_ca, d_row_ptr, d_col_idx, ws + kWorkspaceHeader,
                      reinterpret_cast<int32_t *>(ws) + kStatusWord, stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

sift_status sift_decode_bits_noalloc(const sift_layout *layout, const void *d_plan, const uint32_t *d_la,
                                     const uint32_t *d_ca, int32_t *d_row_ptr, int32_t *d_col_idx,
                                     int64_t col_capacity, hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (!d_plan || !d_row_ptr) return SIFT_ERR_INVALID;
    if ((hl.la_words > 0 && !d_la) || (hl.ca_words > 0 && !d_ca)) return SIFT_ERR_INVALID;
    if (hl.max_nnz > 0 && !d_col_idx) return SIFT_ERR_INVALID;
    if (col_capacity < hl.max_nnz) return SIFT_ERR_CAPACITY;
    if (decode_workspace_bytes(hl) > kNoAllocScratchBytes) return SIFT_ERR_CAPACITY;
    char *ws = nullptr;
    st = noalloc_scratch(stream, &ws);
    if (st != SIFT_OK) return st;
    const PlanView pv = plan_view(hl, d_plan);
    if (launch_decode(hl, pv, d_la, d_ca, d_row_ptr, d_col_idx, ws + kWorkspaceHeader,
                      reinterpret_cast<int32_t *>(ws) + kStatusWord, stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

sift_status sift_sparse_prefill(const sift_layout *layout, const void *d_plan, const void *d_q,
                                const void *d_k, const void *d_v, sift_dtype dtype,
                                const int32_t *d_row_ptr, const int32_t *d_col_idx, int64_t col_entries,
                                float scale, float *d_out, float *d_lse, void *d_workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (dtype != SIFT_BF16 && dtype != SIFT_FP32) return SIFT_ERR_INVALID;
    if (hl.G == 0) return SIFT_OK;
    if (!d_plan || !d_q || !d_k || !d_v || !d_row_ptr || !d_out || col_entries < 0 ||
        (col_entries > 0 && !d_col_idx))
        return SIFT_ERR_INVALID;
    // Q/K/V are read and O written in 16-byte vectors
    auto aligned16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_out) ||
        (d_workspace && !aligned16(d_workspace)))
        return SIFT_ERR_INVALID;
    if (!(scale > 0.0f)) scale = 1.0f / sqrtf(float(hl.D));
    if (!isfinite(scale)) return SIFT_ERR_INVALID;
    const size_t need = prefill_workspace_bytes(hl, dtype);
    if (!d_workspace || workspace_bytes < need) return SIFT_ERR_CAPACITY;
    const PlanView pv = plan_view(hl, d_plan);
    const uint16_t *q = static_cast<const uint16_t *>(d_q);
    const uint16_t *k = static_cast<const uint16_t *>(d_k);
    const int64_t N = int64_t(hl.G) * kTile;
    const int64_t nq = N * hl.Hq * hl.D, nkv = N * hl.Hkv * hl.D;
    char *ws = static_cast<char *>(d_workspace);
    int *header = reinterpret_cast<int *>(ws);
    uint16_t *vt = reinterpret_cast<uint16_t *>(ws + kWorkspaceHeader);
    if (dtype == SIFT_FP32) {
        char *ws2 = ws + kWorkspaceHeader + align256(2 * size_t(nkv));
        uint16_t *qb = reinterpret_cast<uint16_t *>(ws2);
        uint16_t *kb = reinterpret_cast<uint16_t *>(ws2 + align256(2 * size_t(nq)));
        if (launch_cast_bf16(static_cast<const float *>(d_q), qb, nq, stream) != hipSuccess ||
            launch_cast_bf16(static_cast<const float *>(d_k), kb, nkv, stream) != hipSuccess)
            return SIFT_ERR_HIP;
        q = qb;
        k = kb;
    }
    if (launch_transpose_v(hl, d_v, dtype == SIFT_FP32, vt, header, stream) != hipSuccess ||
        launch_prefill(hl, pv, q, k, vt, d_row_ptr, d_col_idx, col_entries, scale, d_out, d_lse, header,
                       stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

// The fused path in two steps.  prepare: fp32 inputs cast, the bits decoded into the workspace
// CSR and V^T written (one launch where the layout allows, see launch_decode_transpose); attend:
// the attention kernel over them.  Both take a validated call.
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static sift_status check_bits_call(const HostLayout &hl, sift_dtype dtype, const void *d_plan, size_t workspace_bytes,
                                   const void *d_workspace) {
    if (dtype != SIFT_BF16 && dtype != SIFT_FP32) return SIFT_ERR_INVALID;
    if (hl.G == 0) return SIFT_OK;
    if (!d_plan || (d_workspace && !aligned16(d_workspace))) return SIFT_ERR_INVALID;
    if (!d_workspace || workspace_bytes < prefill_workspace_bytes(hl, dtype) + fused_tables_bytes(hl))
        return SIFT_ERR_CAPACITY;
    return SIFT_OK;
}

struct BitsWorkspace {
    int *header;
    uint16_t *vt, *qb, *kb;  // V^T; the bf16 copies of fp32 Q and K
    int32_t *row_ptr, *col_idx;
    void *decode_scratch;    // the two-launch decode's scratch (layouts past the single launch)
};
static BitsWorkspace bits_workspace(const HostLayout &hl, sift_dtype dtype, void *d_workspace) {
    const int64_t N = int64_t(hl.G) * kTile;
    const int64_t nq = N * hl.Hq * hl.D, nkv = N * hl.Hkv * hl.D;
    char *ws = static_cast<char *>(d_workspace);
    BitsWorkspace w;
    w.header = reinterpret_cast<int *>(ws);
    w.vt = reinterpret_cast<uint16_t *>(ws + kWorkspaceHeader);
    char *ws2 = ws + kWorkspaceHeader + align256(2 * size_t(nkv));
    w.qb = reinterpret_cast<uint16_t *>(ws2);
    w.kb = reinterpret_cast<uint16_t *>(ws2 + align256(2 * size_t(nq)));
    char *tb = ws + prefill_workspace_bytes(hl, dtype);
    w.row_ptr = reinterpret_cast<int32_t *>(tb);
    w.col_idx = reinterpret_cast<int32_t *>(tb + align256(4 * (size_t(hl.Hq) * size_t(hl.G) + 1)));
    w.decode_scratch = reinterpret_cast<char *>(w.col_idx) + align256(4 * size_t(hl.max_nnz > 0 ? hl.max_nnz : 1));
    return w;
}

static sift_status prepare_bits(const HostLayout &hl, const PlanView &pv, const uint32_t *d_la, const uint32_t *d_ca,
                                const void *d_q, const void *d_k, const void *d_v, sift_dtype dtype,
                                void *d_workspace, hipStream_t stream) {
    const BitsWorkspace w = bits_workspace(hl, dtype, d_workspace);
    const int64_t N = int64_t(hl.G) * kTile;
    if (dtype == SIFT_FP32 &&
        (launch_cast_bf16(static_cast<const float *>(d_q), w.qb, N * hl.Hq * hl.D, stream) != hipSuccess ||
         launch_cast_bf16(static_cast<const float *>(d_k), w.kb, N * hl.Hkv * hl.D, stream) != hipSuccess))
        return SIFT_ERR_HIP;
    int32_t *status = w.header + kStatusWord;
    if (decode_transpose_fits(hl)) {
        if (launch_decode_transpose(hl, pv, d_la, d_ca, w.row_ptr, w.col_idx, status, d_v, dtype == SIFT_FP32, w.vt,
                                    w.header, stream) != hipSuccess)
            return SIFT_ERR_HIP;
    } else {  // the transpose clears the header, then the decode sets the status word
        if (launch_transpose_v(hl, d_v, dtype == SIFT_FP32, w.vt, w.header, stream) != hipSuccess ||
            launch_decode(hl, pv, d_la, d_ca, w.row_ptr, w.col_idx, w.decode_scratch, status, stream) != hipSuccess)
            return SIFT_ERR_HIP;
    }
    return SIFT_OK;
}

static sift_status attend_prepared(const HostLayout &hl, const PlanView &pv, const void *d_q, const void *d_k,
                                   sift_dtype dtype, float scale, float *d_out, float *d_lse, void *d_workspace,
                                   hipStream_t stream) {
    const BitsWorkspace w = bits_workspace(hl, dtype, d_workspace);
    const uint16_t *q = dtype == SIFT_FP32 ? w.qb : static_cast<const uint16_t *>(d_q);
    const uint16_t *k = dtype == SIFT_FP32 ? w.kb : static_cast<const uint16_t *>(d_k);
    if (launch_prefill(hl, pv, q, k, w.vt, w.row_ptr, w.col_idx, hl.max_nnz, scale, d_out, d_lse, w.header, stream) !=
        hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

// scale <= 0 (or NaN) takes 1 / sqrt(D); a non-finite result is invalid
static bool resolve_scale(const HostLayout &hl, float &scale) {
    if (!(scale > 0.0f)) scale = 1.0f / sqrtf(float(hl.D));
    return isfinite(scale);
}

sift_status sift_sparse_prefill_bits(const sift_layout *layout, const void *d_plan, const uint32_t *d_la,
                                     const uint32_t *d_ca, const void *d_q, const void *d_k, const void *d_v,
                                     sift_dtype dtype, float scale, float *d_out, float *d_lse,
                                     void *d_workspace, size_t workspace_bytes, hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (dtype != SIFT_BF16 && dtype != SIFT_FP32) return SIFT_ERR_INVALID;
    if (hl.G == 0) return SIFT_OK;
    if (!d_q || !d_k || !d_v || !d_out) return SIFT_ERR_INVALID;
    if ((hl.la_words > 0 && !d_la) || (hl.ca_words > 0 && !d_ca)) return SIFT_ERR_INVALID;
    if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_out)) return SIFT_ERR_INVALID;
    if (!resolve_scale(hl, scale)) return SIFT_ERR_INVALID;
    if ((st = check_bits_call(hl, dtype, d_plan, workspace_bytes, d_workspace)) != SIFT_OK) return st;
    const PlanView pv = plan_view(hl, d_plan);
    if ((st = prepare_bits(hl, pv, d_la, d_ca, d_q, d_k, d_v, dtype, d_workspace, stream)) != SIFT_OK) return st;
    return attend_prepared(hl, pv, d_q, d_k, dtype, scale, d_out, d_lse, d_workspace, stream);
}

size_t sift_encode_masses_bytes(const sift_layout *layout) {
    HostLayout hl;
    if (build_layout(layout, &hl) != SIFT_OK) return 0;
    return sizeof(float) * size_t(hl.Hq) * size_t(hl.G) * size_t(hl.max_req_tiles > 0 ? hl.max_req_tiles : 1);
}

size_t sift_encode_workspace_bytes(const sift_layout *layout) {
    HostLayout hl;
    if (build_layout(layout, &hl) != SIFT_OK) return 0;
    return mass_workspace_bytes(hl);
}

sift_status sift_tile_masses(const sift_layout *layout, const void *d_plan, const void *d_q, const void *d_k,
                             float scale, float *d_masses, size_t masses_bytes, void *d_workspace,
                             size_t workspace_bytes, int32_t *d_status, hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (hl.G == 0) return SIFT_OK;
    if (!d_plan || !d_q || !d_k || !d_masses) return SIFT_ERR_INVALID;
    auto aligned16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!aligned16(d_q) || !aligned16(d_k) || (d_workspace && !aligned16(d_workspace))) return SIFT_ERR_INVALID;
    if (!(scale > 0.0f)) scale = 1.0f / sqrtf(float(hl.D));
    if (!isfinite(scale)) return SIFT_ERR_INVALID;
    if (masses_bytes < sift_encode_masses_bytes(layout)) return SIFT_ERR_CAPACITY;
    if (!d_workspace || workspace_bytes < mass_workspace_bytes(hl)) return SIFT_ERR_CAPACITY;
    const PlanView pv = plan_view(hl, d_plan);
    if (launch_tile_masses(hl, pv, static_cast<const uint16_t *>(d_q), static_cast<const uint16_t *>(d_k), scale,
                           d_masses, static_cast<int>(hl.max_req_tiles), d_workspace, d_status, stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

sift_status sift_select_bits(const sift_layout *layout, const void *d_plan, const float *d_masses,
                             size_t masses_bytes, float p_la, float p_ca, uint32_t *d_la, uint32_t *d_ca,
                             int32_t *d_status, hipStream_t stream) {
    HostLayout hl;
    sift_status st = build_layout(layout, &hl);
    if (st != SIFT_OK) return st;
    if (hl.ndocs == 0) return SIFT_OK;
    if (!d_plan || !d_masses || (hl.la_words > 0 && !d_la) || (hl.ca_words > 0 && !d_ca)) return SIFT_ERR_INVALID;
    if (!(p_la > 0.0f && p_la <= 1.0f) || !(p_ca > 0.0f && p_ca <= 1.0f)) return SIFT_ERR_INVALID;
    if (hl.max_doc_tiles > 64) return SIFT_ERR_UNSUPPORTED;  // one lane per candidate tile
    if (masses_bytes < sift_encode_masses_bytes(layout)) return SIFT_ERR_CAPACITY;
    const PlanView pv = plan_view(hl, d_plan);
    if (launch_select_bits(hl, pv, d_masses, static_cast<int>(hl.max_req_tiles), p_la, p_ca, d_la, d_ca, d_status,
                           stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

sift_status sift_device_status(const void *d_workspace, size_t workspace_bytes, int32_t *h_flags,
                               hipStream_t stream) {
    if (!d_workspace || !h_flags) return SIFT_ERR_INVALID;
    if (workspace_bytes < kWorkspaceHeader) return SIFT_ERR_CAPACITY;
    const int32_t *word = static_cast<const int32_t *>(d_workspace) + kStatusWord;
    if (hipMemcpyAsync(h_flags, word, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return SIFT_ERR_HIP;
    return SIFT_OK;
}

}  // extern "C"
