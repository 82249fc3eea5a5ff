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
#include "sift_internal.hpp"

namespace sift {

namespace {

using namespace bits;

constexpr int kFillWaves = 4;

// Set bits among bits [lo, lo + n) of a word array.  Up to 64 bits (three words at most) the
// loads are independent of each other, so they arrive in one round trip; longer ranges loop.
__device__ inline int popcount_bits(const uint32_t *vec, int lo, int n) {
    if (n <= 0) return 0;
    if (n > 64) return popcount_range(vec, lo, lo + n - 1);
    const int hi = lo + n - 1, w0 = lo >> 5, w1 = hi >> 5;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int w = w0 + j;
        if (w > w1) break;
        uint32_t x = vec[w];
        if (w == w0) x &= ~0u << (lo & 31);
        if (w == w1 && (hi & 31) != 31) x &= (2u << (hi & 31)) - 1u;
        cnt += __popc(x);
    }
    return cnt;
}

// A row's plan record (tile_rec) and its LA count for q head h; question rows need no bits.
struct RowFacts {
    int d, r, first, req;
    int la_cnt;
};
__device__ inline RowFacts row_facts(const PlanView &pv, const uint32_t *__restrict__ la, int h, int g) {
    const int32_t *tr = pv.tile_rec + static_cast<int64_t>(g) * kRecWords;
    RowFacts f;
    f.d = tr[kTrDoc];
    f.r = tr[kTrLocal];
    f.first = tr[kTrFirst];
    f.req = tr[kTrReq];
    const int la_off = tr[kTrLaOff], la_w = tr[kTrLaW], lo = tr[kTrLo];
    f.la_cnt = f.d >= 0 ? popcount_bits(la + la_off + h * la_w, lo, f.r + 1) : 0;
    return f;
}

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
    __shared__ int s_ex[kCountThreads];    // the current document chunk's batch-wide CA prefixes
    __shared__ int s_pref[kCountThreads];  // ca_prefix of the documents of the first chunk

    const RowFacts f0 = tid < G ? row_facts(pv, la, h, tid) : RowFacts{};

    int carry = 0;
    for (int base = 0; base < ndocs; base += kCountThreads) {
        const int d = base + tid;
        const int32_t *dr = pv.doc_rec + static_cast<int64_t>(d < ndocs ? d : 0) * kRecWords;
        const int ca_off = dr[kDrCaOff], ca_w = dr[kDrCaW], T = dr[kDrTiles];
        const int req_doc = dr[kDrReqDoc], first = dr[kDrFirst], req = dr[kDrReq];
        const uint32_t *vec = ca + ca_off + h * ca_w;
        const int c = d < ndocs ? popcount_bits(vec, 0, T) : 0;
        int total;
        const int gex = carry + block_excl_scan(c, sh, total);
        s_ex[tid] = gex;
        if (d < ndocs) loc[d] = gex;  // for later chunks (the head's row offsets, G >= ndocs, as scratch)
        __syncthreads();
        if (d < ndocs) {
            const int p = gex - (req_doc >= base ? s_ex[req_doc - base] : loc[req_doc]);
            pref[d] = p;
            if (base == 0) s_pref[tid] = p;
            // this document's CA pages, in order, at their place in the request's page list
            int pos = req + p;
            for (int w = 0; 32 * w < T; ++w) {
                uint32_t bits = vec[w];
                if (T - 32 * w < 32) bits &= (1u << (T - 32 * w)) - 1u;  // bits past T are ignored
                while (bits != 0u) {
                    lst[pos++] = first + 32 * w + __builtin_ctz(bits);
                    bits &= bits - 1u;
                }
            }
        }
        carry += total;
        __syncthreads();  // s_ex and loc free again
    }

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

// Single-launch decode for layouts whose per-head tables fit in LDS (the common case; larger
// layouts take decode_count + decode_fill).  Workgroup (h, part) recomputes all of q head h's
// counts in LDS -- CA prefixes, CA page lists, LA words, row offsets -- and the list entries of
// the earlier heads in closed form, then fills rows [part * rows_per, ...) of head h.  No scratch
// in global memory and no second launch: after the plan check, every load is in one of two
// rounds (the plan records, then the bit words).
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kOneMaxG = 2048;       // rows per head (two per thread)
constexpr int kOneMaxDocs = 1024;    // documents in the batch (one per thread)
constexpr int kOneMaxLaW = 4096;     // LA words per head
constexpr int kOneMaxDocTiles = 64;  // tiles per document: one lane per LA candidate of a row
constexpr int kOneUnroll = 4;        // independent word loads in flight per thread
constexpr int64_t kOneMaxBatchLaW = 8 * kOneThreads;  // LA words of all heads

__device__ inline int la_words_of(int T) { return (T * (T + 1) / 2 + 31) >> 5; }

// The document whose LA words hold head-local word x: the last d with s_laloc[d] <= x
// (s_laloc ascends strictly from 0: every document has at least one word).
__device__ inline int doc_of_word(const int *s_laloc, int ndocs, int x) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_laloc[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kOneThreads) void decode_one_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca, int32_t *__restrict__ row_ptr,
    int32_t *__restrict__ col_idx, int32_t *__restrict__ status, int splits, int question_nnz, int law_head) {
    __shared__ int sh[kOneWaves];
    __shared__ int s_ex[kOneMaxDocs];        // batch-wide exclusive CA prefix of each document
    __shared__ int s_pref[kOneMaxDocs];      // CA entries of the earlier documents of its request
    __shared__ int s_laloc[kOneMaxDocs];     // first word of the document's LA vector in s_la
    __shared__ int s_laoff[kOneMaxDocs];     // word offset of its (head 0) LA vector in la
    __shared__ int s_caoff[kOneMaxDocs];     // word offset of its (head 0) CA vector in ca
    __shared__ int s_T[kOneMaxDocs];         // its tiles
    __shared__ int s_after[kOneMaxDocs];     // tiles of the later documents of its request
    __shared__ int s_loc[kOneMaxG + 1];      // row offsets in the head; [G] = the head's total
    __shared__ int s_lst[kOneMaxG];          // the head's CA page list of every request
    __shared__ uint32_t s_la[kOneMaxLaW];    // the head's LA words, documents in order
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = pv.num_tiles, Hq = pv.num_q_heads, ndocs = pv.num_docs;
    const int64_t nrows = static_cast<int64_t>(Hq) * G;
    const int h = blockIdx.x / splits, part = blockIdx.x % splits;
    const int rows_per = (G + splits - 1) / splits;
    const int g_lo = part * rows_per, g_hi = min(G, g_lo + rows_per);
    const bool ok = plan_ok(pv);
    // the call's status word: written once, by this thread alone
    if (blockIdx.x == 0 && tid == 0) *status = ok ? SIFT_DEVICE_OK : SIFT_DEVICE_PLAN_MISMATCH;
    if (!ok) {  // a plan of another layout: an empty CSR
        for (int g = g_lo + tid; g < g_hi; g += kOneThreads) row_ptr[static_cast<int64_t>(h) * G + g] = 0;
        if (tid == 0 && h == Hq - 1 && g_lo <= G - 1 && G - 1 < g_hi) row_ptr[nrows] = 0;
        return;
    }

    // 1. Plan records: this thread's document and rows (tid, tid + kOneThreads), and the rows this
    //    wavefront fills (lane j: its j-th row, g_lo + wave + j kOneWaves).
    int d_rfd = 0, d_first = 0, d_req = 0, d_T = 0;
    uint32_t d_caw[2] = {0u, 0u};
    if (tid < ndocs) {
        const int32_t *dr = pv.doc_rec + static_cast<int64_t>(tid) * kRecWords;
        d_T = dr[kDrTiles];
        d_rfd = dr[kDrReqDoc];
        d_first = dr[kDrFirst];
        d_req = dr[kDrReq];
        const int ca_off = dr[kDrCaOff], la_off = dr[kDrLaOff];
        s_laloc[tid] = la_off / Hq;  // the (d, head 0) offset counts Hq vectors per earlier document
        s_laoff[tid] = la_off;
        s_caoff[tid] = ca_off;
        s_T[tid] = d_T;
        s_after[tid] = dr[kDrAfter];
        const int ca_w = (d_T + 31) >> 5;
        d_caw[0] = ca[ca_off + h * ca_w];
        if (ca_w > 1) d_caw[1] = ca[ca_off + h * ca_w + 1];
    }
    int r_d[2] = {0, 0}, r_r[2] = {0, 0}, r_req[2] = {0, 0}, r_lo[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int g = tid + k * kOneThreads;
        if (g < G) {
            const int32_t *tr = pv.tile_rec + static_cast<int64_t>(g) * kRecWords;
            r_d[k] = tr[kTrDoc];
            r_r[k] = tr[kTrLocal];
            r_req[k] = tr[kTrReq];
            r_lo[k] = tr[kTrLo];
        }
    }
    const int nmine = g_hi > g_lo + wave ? (g_hi - g_lo - wave + kOneWaves - 1) / kOneWaves : 0;  // <= 64
    int f_d = 0, f_r = 0, f_first = 0, f_req = 0, f_lo = 0;
    if (lane < nmine) {
        const int32_t *tr = pv.tile_rec + static_cast<int64_t>(g_lo + wave + kOneWaves * lane) * kRecWords;
        f_d = tr[kTrDoc];
        f_r = tr[kTrLocal];
        f_first = tr[kTrFirst];
        f_req = tr[kTrReq];
        f_lo = tr[kTrLo];
    }
    __syncthreads();

    // 2. Bit words, one per thread and slot: head h's LA words into s_la; the earlier heads' LA
    //    entries (the (d, h') vectors of heads h' < h are contiguous for each document) and CA
    //    entries times the tiles of the later documents of the request (each CA entry of a
    //    document is listed by every row of those documents).
    for (int i = tid; i < law_head; i += kOneThreads) {
        const int d = doc_of_word(s_laloc, ndocs, i), law = la_words_of(s_T[d]);
        s_la[i] = la[s_laoff[d] + h * law + (i - s_laloc[d])];
    }
    int64_t earlier = 0;  // list entries of heads 0 .. h - 1, this thread's share
    const int n_la = h * law_head;
    for (int i0 = tid; i0 < n_la; i0 += kOneThreads * kOneUnroll) {
        uint32_t word[kOneUnroll];
        int keep[kOneUnroll];
#pragma unroll
        for (int u = 0; u < kOneUnroll; ++u) {
            const int i = i0 + u * kOneThreads;
            word[u] = 0u;
            keep[u] = 32;
            if (i < n_la) {
                const int d = doc_of_word(s_laloc, ndocs, i / h);
                const int T = s_T[d], law = la_words_of(T), j = i - h * s_laloc[d];
                word[u] = la[s_laoff[d] + j];
                if (j % law == law - 1) keep[u] = T * (T + 1) / 2 - 32 * (law - 1);  // bits past the triangle
            }
        }
#pragma unroll
        for (int u = 0; u < kOneUnroll; ++u)
            earlier += __popc(keep[u] == 32 ? word[u] : (word[u] & ((1u << keep[u]) - 1u)));
    }
    for (int p = tid; p < h * ndocs; p += kOneThreads) {
        const int hp = p / ndocs, d = p % ndocs;
        const int T = s_T[d], ca_w = (T + 31) >> 5;
        earlier += static_cast<int64_t>(popcount_bits(ca + s_caoff[d] + hp * ca_w, 0, T)) * s_after[d];
    }

    // 3. CA prefixes (documents scanned batch-wide, less the value at the request's first
    //    document), the head's CA page lists, and the list entries of the earlier heads.
    int c_doc = 0;
    if (tid < ndocs) {
        d_caw[0] &= d_T >= 32 ? ~0u : ((1u << d_T) - 1u);  // bits past T are ignored
        d_caw[1] &= d_T >= 64 ? ~0u : (d_T > 32 ? ((1u << (d_T - 32)) - 1u) : 0u);
        c_doc = __popc(d_caw[0]) + __popc(d_caw[1]);
    }
    int tot;
    const int ex = block_excl_scan<kOneThreads>(c_doc, sh, tot);
    if (tid < ndocs) s_ex[tid] = ex;
    int base_h;  // (the barriers of this scan also publish s_ex)
    block_excl_scan<kOneThreads>(static_cast<int>(earlier), sh, base_h);  // a share of the CSR: < 2^31
    base_h += h * question_nnz;
    if (tid < ndocs) {
        const int p = ex - s_ex[d_rfd];
        s_pref[tid] = p;
        int pos = d_req + p;
        for (int w = 0; w < 2; ++w) {
            uint32_t bits = d_caw[w];
            while (bits != 0u) {
                s_lst[pos++] = d_first + 32 * w + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
    }
    __syncthreads();

    // 4. Row counts in closed form, scanned -> s_loc.
    int carry = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (k * kOneThreads >= G) break;
        const int g = tid + k * kOneThreads;
        int c = 0;
        if (g < G) {
            if (r_d[k] < 0) c = g - r_req[k] + 1;  // question row: every tile of its request up to g
            else c = s_pref[r_d[k]] + popcount_bits(s_la + s_laloc[r_d[k]], r_lo[k], r_r[k] + 1);
        }
        int total;
        const int e = block_excl_scan<kOneThreads>(c, sh, total);
        if (g < G) s_loc[g] = carry + e;
        carry += total;
    }
    if (tid == 0) s_loc[G] = carry;
    __syncthreads();

    // 5. Fill rows g_lo .. g_hi - 1, one wavefront per row.
    for (int j = 0; j < nmine; ++j) {
        const int g = g_lo + wave + kOneWaves * j;
        const int d = __builtin_amdgcn_readlane(f_d, j), r = __builtin_amdgcn_readlane(f_r, j);
        const int first = __builtin_amdgcn_readlane(f_first, j), req = __builtin_amdgcn_readlane(f_req, j);
        const int lo = __builtin_amdgcn_readlane(f_lo, j);
        const int start = base_h + s_loc[g];
        if (lane == 0) {
            row_ptr[static_cast<int64_t>(h) * G + g] = start;
            if (h == Hq - 1 && g == G - 1) row_ptr[nrows] = base_h + s_loc[G];
        }
        if (d < 0) {  // question tile: every tile of the request up to g
            const int cnt = g - req + 1;
            for (int c = lane; c < cnt; c += 64) col_idx[start + c] = first + c;
            continue;
        }
        // CA pages of the earlier documents of the request: the leading slice of its page list
        const int nca = s_pref[d];
        for (int c = lane; c < nca; c += 64) col_idx[start + c] = s_lst[req + c];
        // LA tiles c <= r of the row's own document (r < kOneMaxDocTiles: one lane each)
        const int k = lo + min(lane, r);  // lanes past r read a word of the row, unused
        const bool bit = lane <= r && ((s_la[s_laloc[d] + (k >> 5)] >> (k & 31)) & 1u);
        const uint64_t mask = __ballot(bit);
        if (bit) col_idx[start + nca + lane_rank(mask)] = first + lane;
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
    // The single launch re-reads the bits of the earlier heads in every workgroup: worth it while
    // they are a few words per thread.
    if (hl.G <= kOneMaxG && hl.ndocs <= kOneMaxDocs && hl.la_words / hl.Hq <= kOneMaxLaW &&
        hl.max_doc_tiles <= kOneMaxDocTiles && hl.la_words <= kOneMaxBatchLaW) {
        // about 256 workgroups in all; each fills at most 1024 rows of its head (64 per wavefront)
        // and, where the head has enough, at least 16
        const int64_t most = std::max<int64_t>(1, (hl.G + 15) / 16), least = (hl.G + 1023) / 1024;
        const int splits = static_cast<int>(
            std::max<int64_t>(least, std::min<int64_t>(most, (256 + hl.Hq - 1) / hl.Hq)));
        decode_one_kernel<<<static_cast<unsigned>(hl.Hq * splits), kOneThreads, 0, stream>>>(
            pv, la, ca, row_ptr, col_idx, status, splits, static_cast<int>(hl.question_nnz),
            static_cast<int>(hl.la_words / hl.Hq));
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
