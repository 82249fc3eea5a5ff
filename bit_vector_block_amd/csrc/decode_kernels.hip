// Decode kernel: LA/CA bit vectors -> per-(head, query tile) CSR of KV-tile ids.
//
// SIFT technical summary, section 2, "Dettagli di Implementazione": a custom
// kernel expands the bit vectors into explicit tile indices before the sparse
// attention runs.  CSR convention (rows h*G + g, ascending tiles): CA pages of
// the earlier documents of the request, then the LA tiles c <= r of the row's
// own document; question tiles list every tile of their request up to
// themselves.
//
// Stream-ordered, no host read-back.  Layouts whose per-head tables fit in LDS (up to 2048 rows
// per head, 1024 documents of up to 64 tiles, 8192 LA words in all) take one launch:
//   decode_one    (about 256 workgroups, a few per q head): each workgroup counts its whole
//                 head in LDS (CA prefixes, CA page lists, row counts in closed form, their
//                 scan) and the list entries of the earlier heads in closed form (CA entries x
//                 the tiles of the later documents of their request, plus all LA entries), then
//                 fills its share of the head's rows.
// Larger layouts take two:
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
#include "decode_one.hpp"
#include "sift_internal.hpp"

namespace sift {

namespace {

using namespace bits;

constexpr int kFillWaves = 4;

// One workgroup per q head h:
//   documents, kCountThreads at a time: CA popcounts (bits past T ignored), their batch-wide
//   exclusive scan, and per document the CA entries of the earlier documents of its request
//   (ca_prefix), then its CA pages written into the request's page list;
//   rows, kCountThreads at a time: the counts in closed form, scanned -> row offsets in the head.
// The first row chunk's records and LA words are loaded ahead of the document pass, so that
// every load of the common case (at most kCountThreads documents and rows) lands in two round
// trips after the plan check.
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
    int32_t *lst = ca_list + static_cast<int64_t>(h) * G;
    __shared__ int sh[kCountThreads / 64];
    __shared__ int s_ex[kCountThreads];
    __shared__ int s_pref[kCountThreads];  // ca_prefix of the documents of the first chunk

    const RowFacts f0 = tid < G ? row_facts(pv, la, h, tid) : RowFacts{};
    // CA prefixes and page lists (the head's row offsets, G >= ndocs entries, as the scratch)
    head_ca_pass(pv, ca, h, pref, lst, loc, sh, s_ex, s_pref);

    int rcarry = 0;
    for (int base = 0; base < G; base += kCountThreads) {
        const int g = base + tid;
        const RowFacts f = base == 0 ? f0 : (g < G ? row_facts(pv, la, h, g) : RowFacts{});
        int c = 0;
        if (g < G) {
            if (f.d < 0) c = g - f.req + 1;  // question row: every tile of its request up to g
            else c = (ndocs <= kCountThreads ? s_pref[f.d] : pref[f.d]) + f.la_cnt;
        }
        int total;
        const int ex = block_excl_scan(c, sh, total);
        if (g < G) loc[g] = rcarry + ex;
        rcarry += total;
    }
    if (tid == 0) head_total[h] = rcarry;
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

// One wavefront per row (h, g).  Its loads go out in two waves: the row's record, its offsets and
// the earlier heads' totals; then (document row) its CA prefix, the first 64 entries of its
// request's CA page list and the LA words of its first 64 candidate tiles.
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

    const int32_t *tr = pv.tile_rec + static_cast<int64_t>(g) * kRecWords;
    const int d = tr[kTrDoc], r = tr[kTrLocal], t0 = tr[kTrFirst], req = tr[kTrReq];
    const int la_off = tr[kTrLaOff], la_w = tr[kTrLaW], lo = tr[kTrLo];
    int partial = 0;
    for (int j = lane; j < h; j += 64) partial += head_total[j];
    const int local = row_local[row];
    const int next = (g + 1 < G) ? row_local[row + 1] : head_total[h];

    int nca = 0, ca0 = 0;
    uint32_t law = 0u;
    const int32_t *src = ca_list + static_cast<int64_t>(h) * G + req;
    const uint32_t *vec = la + la_off + h * la_w;
    if (d >= 0) {
        nca = ca_prefix[static_cast<int64_t>(h) * pv.num_docs + d];
        if (req + lane < G) ca0 = src[lane];  // inside the head's page-list area
        if (lane <= r) law = vec[(lo + lane) >> 5];
    }
    const int head_base = wave_sum(partial);
    const int start = head_base + local;
    if (lane == 0) {
        row_ptr[row] = start;
        if (row == nrows - 1) row_ptr[nrows] = head_base + next;
    }
    if (d < 0) {  // question tile: every tile of the request up to g
        const int cnt = next - local;
        for (int c = lane; c < cnt; c += 64) col_idx[start + c] = t0 + c;
        return;
    }
    // CA pages of the earlier documents of the same request: the leading slice of the request's
    // CA page list
    if (lane < nca) col_idx[start + lane] = ca0;
    for (int c = 64 + lane; c < nca; c += 64) col_idx[start + c] = src[c];
    int pos = start + nca;
    // LA tiles c <= r of the row's own document: one lane per candidate, ballot + rank
    for (int c0 = 0; c0 <= r; c0 += 64) {
        const int c = c0 + lane;
        const int k = lo + c;
        const uint32_t word = c0 == 0 ? law : (c <= r ? vec[k >> 5] : 0u);
        const bool bit = c <= r && ((word >> (k & 31)) & 1u);
        const uint64_t mask = __ballot(bit);
        if (bit) col_idx[pos + lane_rank(mask)] = t0 + c;
        pos += __popcll(mask);
    }
}

__global__ __launch_bounds__(kOneThreads) void decode_one_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca, int la_words, int ca_words,
    int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx, int32_t *__restrict__ status, int splits,
    int question_nnz) {
    __shared__ DecodeOneLds lds;
    decode_one_block(pv, la, ca, la_words, ca_words, row_ptr, col_idx, status, splits, question_nnz, lds,
                     blockIdx.x);
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
    if (decode_one_fits(hl)) {
        const int splits = decode_one_splits(hl, kDecodeOneTarget);
        decode_one_kernel<<<static_cast<unsigned>(hl.Hq * splits), kOneThreads, 0, stream>>>(
            pv, la, ca, static_cast<int>(hl.la_words), static_cast<int>(hl.ca_words), row_ptr, col_idx, status,
            splits, static_cast<int>(hl.question_nnz));
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
