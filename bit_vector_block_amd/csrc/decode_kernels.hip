// Decode kernel: LA/CA bit vectors -> per-(head, query tile) CSR of KV-tile ids.
//
// SIFT technical summary, section 2, "Dettagli di Implementazione": a custom
// kernel expands the bit vectors into explicit tile indices before the sparse
// attention runs.  CSR convention (rows h*G + g, ascending tiles): CA pages of
// the earlier documents of the request, then the LA tiles c <= r of the row's
// own document; question tiles list every tile of their request up to
// themselves.
//
// Two launches, both stream-ordered, no host read-back:
//   decode_count  (one workgroup per q head): per-document CA popcounts and
//                 their per-request exclusive prefix (block scans), the
//                 head's CA page list of every request (document order), the
//                 per-row counts in closed form, block scans over the head's
//                 G rows -> row offsets relative to the head, and the head's
//                 total;
//   decode_fill   (one wavefront per row): adds the totals of earlier heads,
//                 writes row_ptr, copies the row's CA part (a leading slice
//                 of its request's page list) and expands its LA bits with
//                 one lane per bit: ballot gives the set mask, mbcnt the
//                 lane's rank among the set bits, so the 64 lanes write their
//                 tile ids in order with no atomics.
#include "bits_common.hpp"
#include "sift_internal.hpp"

namespace sift {

namespace {

using namespace bits;

constexpr int kFillWaves = 4;


__device__ inline int row_count(const PlanView &pv, const uint32_t *la, const int32_t *ca_prefix_h,
                                int h, int g) {
    const int d = pv.tile_doc[g];
    if (d < 0) return g - pv.req_first[-d - 1] + 1;
    const int r = pv.tile_local[g];
    const uint32_t *vec = la + pv.doc_la_off[d] + h * pv.doc_la_w[d];
    const int lo = r * (r + 1) / 2;
    return ca_prefix_h[d] + popcount_range(vec, lo, lo + r);
}

__global__ __launch_bounds__(kCountThreads) void decode_count_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca,
    int32_t *__restrict__ ca_prefix, int32_t *__restrict__ ca_list, int32_t *__restrict__ row_local,
    int32_t *__restrict__ head_total, int32_t *__restrict__ status) {
    const bool ok = plan_ok(pv);
    // the call's status word: written once, by this thread alone
    if (blockIdx.x == 0 && threadIdx.x == 0) *status = ok ? SIFT_DEVICE_OK : SIFT_DEVICE_PLAN_MISMATCH;
    if (!ok) return;
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int ndocs = pv.num_docs, G = pv.num_tiles;
    int32_t *pref = ca_prefix + static_cast<int64_t>(h) * ndocs;
    int32_t *loc = row_local + static_cast<int64_t>(h) * G;
    __shared__ int sh[kCountThreads / 64];
    // 1. Per document: CA entries of the earlier documents of its request (bits past T ignored);
    //    the head's row offsets (G >= ndocs entries) serve as the scratch.
    head_ca_prefix(pv, ca, h, pref, loc, sh);
    // 2. The head's CA page list per request (the fill copies each row's CA part from it).
    head_ca_list(pv, ca, h, pref, ca_list + static_cast<int64_t>(h) * G);
    // 3. Row counts in closed form, scanned kCountThreads rows at a time -> offsets in the head.
    int carry = 0;
    for (int base = 0; base < G; base += kCountThreads) {
        const int g = base + tid;
        const int c = g < G ? row_count(pv, la, pref, h, g) : 0;
        int total;
        const int ex = block_excl_scan(c, sh, total);
        if (g < G) loc[g] = carry + ex;
        carry += total;
    }
    if (tid == 0) head_total[h] = carry;
}

// A batch without tiles: row_ptr = {0}, and the status word cleared.
__global__ void empty_decode_kernel(int32_t *row_ptr, int32_t *status) {
    if (threadIdx.x == 0) {
        row_ptr[0] = 0;
        *status = SIFT_DEVICE_OK;
    }
}

__device__ inline int wave_sum(int x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__global__ __launch_bounds__(64 * kFillWaves) void decode_fill_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const int32_t *__restrict__ ca_prefix,
    const int32_t *__restrict__ ca_list, const int32_t *__restrict__ row_local,
    const int32_t *__restrict__ head_total, int32_t *__restrict__ row_ptr,
    int32_t *__restrict__ col_idx) {
    const int lane = threadIdx.x & 63;
    const int G = pv.num_tiles, Hq = pv.num_q_heads;  // the host's layout, not read from the plan
    const int64_t nrows = static_cast<int64_t>(Hq) * G;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kFillWaves + (threadIdx.x >> 6);
    if (row >= nrows) return;  // whole wavefront leaves together
    if (!plan_ok(pv)) {  // a plan of another layout: an empty CSR (the count kernel set the status)
        if (lane == 0) {
            row_ptr[row] = 0;
            if (row == nrows - 1) row_ptr[nrows] = 0;
        }
        return;
    }
    const int h = static_cast<int>(row / G), g = static_cast<int>(row % G);

    int partial = 0;
    for (int j = lane; j < h; j += 64) partial += head_total[j];
    const int head_base = wave_sum(partial);
    const int local = row_local[row];
    const int next = (g + 1 < G) ? row_local[row + 1] : head_total[h];
    const int start = head_base + local;
    if (lane == 0) {
        row_ptr[row] = start;
        if (row == nrows - 1) row_ptr[nrows] = head_base + next;
    }

    const int d = pv.tile_doc[g];
    if (d < 0) {  // question tile: every tile of the request up to g
        const int first = pv.req_first[-d - 1];
        const int cnt = next - local;
        for (int c = lane; c < cnt; c += 64) col_idx[start + c] = first + c;
        return;
    }
    // CA pages of the earlier documents of the same request: the leading slice of the request's
    // CA page list
    const int nca = ca_prefix[static_cast<int64_t>(h) * pv.num_docs + d];
    const int32_t *src = ca_list + static_cast<int64_t>(h) * G + pv.req_first[pv.doc_req[d]];
    for (int c = lane; c < nca; c += 64) col_idx[start + c] = src[c];
    int pos = start + nca;
    // LA tiles c <= r of the row's own document
    const int r = pv.tile_local[g];
    const uint32_t *vec = la + pv.doc_la_off[d] + h * pv.doc_la_w[d];
    const int lo = r * (r + 1) / 2, t0 = pv.doc_first[d];
    for (int c0 = 0; c0 <= r; c0 += 64) {
        const int c = c0 + lane;
        const int k = lo + c;
        const bool bit = c <= r && ((vec[k >> 5] >> (k & 31)) & 1u);
        const uint64_t mask = __ballot(bit);
        if (bit) col_idx[pos + lane_rank(mask)] = t0 + c;
        pos += __popcll(mask);
    }
}

}  // namespace

hipError_t launch_decode(const HostLayout &hl, const PlanView &pv, const uint32_t *la,
                         const uint32_t *ca, int32_t *row_ptr, int32_t *col_idx, void *scratch,
                         int32_t *status, hipStream_t stream) {
    const size_t a0 = (sizeof(int32_t) * size_t(hl.Hq) * size_t(hl.ndocs > 0 ? hl.ndocs : 1) + 255) & ~size_t(255);
    const size_t a1 = (sizeof(int32_t) * size_t(hl.Hq) * size_t(hl.G > 0 ? hl.G : 1) + 255) & ~size_t(255);
    char *ws = static_cast<char *>(scratch);
    int32_t *ca_prefix = reinterpret_cast<int32_t *>(ws);
    int32_t *row_local = reinterpret_cast<int32_t *>(ws + a0);
    int32_t *head_total = reinterpret_cast<int32_t *>(ws + a0 + a1);
    int32_t *ca_list = reinterpret_cast<int32_t *>(ws + a0 + a1 + ((sizeof(int32_t) * size_t(hl.Hq) + 255) & ~size_t(255)));
    if (hl.G == 0) {  // no rows: row_ptr[0] = 0
        empty_decode_kernel<<<1, 64, 0, stream>>>(row_ptr, status);
        return hipGetLastError();
    }
    decode_count_kernel<<<hl.Hq, kCountThreads, 0, stream>>>(pv, la, ca, ca_prefix, ca_list, row_local,
                                                              head_total, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nrows = int64_t(hl.Hq) * hl.G;
    const int64_t blocks = (nrows + kFillWaves - 1) / kFillWaves;
    decode_fill_kernel<<<static_cast<unsigned>(blocks), 64 * kFillWaves, 0, stream>>>(
        pv, la, ca_prefix, ca_list, row_local, head_total, row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace sift
