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
//                 their per-request exclusive prefix, per-row counts in closed
//                 form, a block scan over the head's G rows -> row offsets
//                 relative to the head, and the head's total;
//   decode_fill   (one wavefront per row): adds the totals of earlier heads,
//                 writes row_ptr, and expands the row's candidate bits with
//                 one lane per bit: ballot gives the set mask, mbcnt the
//                 lane's rank among the set bits, so the 64 lanes write their
//                 tile ids in order with no atomics.
#include "sift_internal.hpp"

namespace sift {

namespace {

constexpr int kCountThreads = 256;
constexpr int kFillWaves = 4;

__device__ inline bool plan_ok(const PlanView &pv) {
    return pv.header[0] == static_cast<int32_t>(kPlanMagic) &&
           static_cast<uint32_t>(pv.header[2]) == pv.fp_lo &&
           static_cast<uint32_t>(pv.header[3]) == pv.fp_hi && pv.header[6] == pv.num_tiles;
}

// Number of set bits among bits [lo, hi] (inclusive) of a word array.
__device__ inline int popcount_range(const uint32_t *vec, int lo, int hi) {
    int cnt = 0;
    for (int w = lo >> 5; w <= (hi >> 5); ++w) {
        const int b0 = max(lo, w << 5) - (w << 5);
        const int b1 = min(hi, (w << 5) + 31) - (w << 5);
        const uint32_t upper = (b1 == 31) ? 0xffffffffu : ((1u << (b1 + 1)) - 1u);
        const uint32_t mask = upper & ~((1u << b0) - 1u);
        cnt += __popc(vec[w] & mask);
    }
    return cnt;
}

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
    int32_t *__restrict__ ca_prefix, int32_t *__restrict__ row_local,
    int32_t *__restrict__ head_total) {
    if (!plan_ok(pv)) return;
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int ndocs = pv.num_docs, G = pv.num_tiles;
    int32_t *pref = ca_prefix + static_cast<int64_t>(h) * ndocs;

    // 1. CA popcount of every (doc, h) vector (bits past T are ignored).
    for (int d = tid; d < ndocs; d += kCountThreads) {
        const uint32_t *vec = ca + pv.doc_ca_off[d] + h * pv.doc_ca_w[d];
        pref[d] = popcount_range(vec, 0, pv.doc_tiles[d] - 1);
    }
    __syncthreads();
    // 2. Exclusive prefix over the documents of each request (serial per request).
    for (int b = tid; b < pv.num_requests; b += kCountThreads) {
        int acc = 0;
        const int d0 = pv.req_first_doc[b], d1 = d0 + pv.req_ndocs[b];
        for (int d = d0; d < d1; ++d) {
            const int c = pref[d];
            pref[d] = acc;
            acc += c;
        }
    }
    __syncthreads();
    // 3. Row counts: each thread owns a contiguous run of tiles; block scan of the run sums.
    __shared__ int run_sum[kCountThreads];
    const int per = (G + kCountThreads - 1) / kCountThreads;
    const int g0 = min(G, tid * per), g1 = min(G, g0 + per);
    int s = 0;
    for (int g = g0; g < g1; ++g) s += row_count(pv, la, pref, h, g);
    run_sum[tid] = s;
    __syncthreads();
    for (int off = 1; off < kCountThreads; off <<= 1) {
        const int add = tid >= off ? run_sum[tid - off] : 0;
        __syncthreads();
        run_sum[tid] += add;
        __syncthreads();
    }
    int base = run_sum[tid] - s;  // exclusive
    int32_t *loc = row_local + static_cast<int64_t>(h) * G;
    for (int g = g0; g < g1; ++g) {
        loc[g] = base;
        base += row_count(pv, la, pref, h, g);
    }
    if (tid == kCountThreads - 1) head_total[h] = run_sum[tid];
}

__global__ void zero_kernel(int32_t *p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__device__ inline int lane_rank(uint64_t mask) {
    // number of set bits of `mask` below this lane
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ inline int wave_sum(int x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__global__ __launch_bounds__(64 * kFillWaves) void decode_fill_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca,
    const int32_t *__restrict__ ca_prefix, const int32_t *__restrict__ row_local,
    const int32_t *__restrict__ head_total, int32_t *__restrict__ row_ptr,
    int32_t *__restrict__ col_idx) {
    if (!plan_ok(pv)) return;
    const int lane = threadIdx.x & 63;
    const int G = pv.num_tiles, Hq = pv.num_q_heads;
    const int64_t nrows = static_cast<int64_t>(Hq) * G;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kFillWaves + (threadIdx.x >> 6);
    if (row >= nrows) return;  // whole wavefront leaves together
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
    int pos = start;
    // CA pages of the earlier documents of the same request
    const int first_doc = pv.req_first_doc[pv.doc_req[d]];
    for (int i = first_doc; i < d; ++i) {
        const uint32_t *vec = ca + pv.doc_ca_off[i] + h * pv.doc_ca_w[i];
        const int T = pv.doc_tiles[i], t0 = pv.doc_first[i];
        for (int c0 = 0; c0 < T; c0 += 64) {
            const int c = c0 + lane;
            const bool bit = c < T && ((vec[c >> 5] >> (c & 31)) & 1u);
            const uint64_t mask = __ballot(bit);
            if (bit) col_idx[pos + lane_rank(mask)] = t0 + c;
            pos += __popcll(mask);
        }
    }
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

// Pre-pass of the fused path (no CSR): one workgroup per q head h.
//   ca_prefix[h][d] : CA entries of the earlier documents of d's request (request-local);
//   ca_list[h][req_first[b] + k] : the k-th CA-marked page of request b, in document order --
//                      the CA part of every document row of the request is a leading slice of it;
//   rowinfo[h][g]   : what the attention kernel needs to build row (h, g)'s list itself:
//                      {n, ca_n (-1: question row, dense range), ca_base, la_word, la_lo, t0, r, 0}.
__global__ __launch_bounds__(kCountThreads) void bits_prepass_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca,
    int32_t *__restrict__ ca_prefix, int32_t *__restrict__ ca_list, int32_t *__restrict__ rowinfo) {
    if (!plan_ok(pv)) return;
    const int h = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ndocs = pv.num_docs, G = pv.num_tiles;
    int32_t *pref = ca_prefix + static_cast<int64_t>(h) * ndocs;
    for (int d = tid; d < ndocs; d += kCountThreads) {
        const uint32_t *vec = ca + pv.doc_ca_off[d] + h * pv.doc_ca_w[d];
        pref[d] = popcount_range(vec, 0, pv.doc_tiles[d] - 1);
    }
    __syncthreads();
    for (int b = tid; b < pv.num_requests; b += kCountThreads) {
        int acc = 0;
        const int d0 = pv.req_first_doc[b], d1 = d0 + pv.req_ndocs[b];
        for (int d = d0; d < d1; ++d) {
            const int c = pref[d];
            pref[d] = acc;
            acc += c;
        }
    }
    __syncthreads();
    // CA pages of each document, one wavefront per document: ballot and lane rank place them
    int32_t *lst = ca_list + static_cast<int64_t>(h) * G;
    for (int d = wave; d < ndocs; d += kCountThreads / 64) {
        const uint32_t *vec = ca + pv.doc_ca_off[d] + h * pv.doc_ca_w[d];
        const int T = pv.doc_tiles[d], t0 = pv.doc_first[d];
        int pos = pv.req_first[pv.doc_req[d]] + pref[d];
        for (int c0 = 0; c0 < T; c0 += 64) {
            const int c = c0 + lane;
            const bool bit = c < T && ((vec[c >> 5] >> (c & 31)) & 1u);
            const uint64_t mask = __ballot(bit);
            if (bit) lst[pos + lane_rank(mask)] = t0 + c;
            pos += __popcll(mask);
        }
    }
    // per-row records
    for (int g = tid; g < G; g += kCountThreads) {
        int32_t *ri = rowinfo + (static_cast<int64_t>(h) * G + g) * 8;
        const int d = pv.tile_doc[g];
        if (d < 0) {
            const int first = pv.req_first[-d - 1];
            ri[0] = g - first + 1;
            ri[1] = -1;
            ri[2] = 0;
            ri[3] = 0;
            ri[4] = 0;
            ri[5] = first;
            ri[6] = 0;
        } else {
            const int r = pv.tile_local[g];
            const int lo = r * (r + 1) / 2;
            const int la_word = pv.doc_la_off[d] + h * pv.doc_la_w[d];
            const int la_n = popcount_range(la + la_word, lo, lo + r);
            ri[0] = pref[d] + la_n;
            ri[1] = pref[d];
            ri[2] = h * G + pv.req_first[pv.doc_req[d]];
            ri[3] = la_word;
            ri[4] = lo;
            ri[5] = pv.doc_first[d];
            ri[6] = r;
        }
        ri[7] = 0;
    }
}

}  // namespace

hipError_t launch_bits_prepass(const HostLayout &hl, const PlanView &pv, const uint32_t *la, const uint32_t *ca,
                               int32_t *ca_prefix, int32_t *ca_list, int32_t *rowinfo, hipStream_t stream) {
    if (hl.G == 0) return hipSuccess;
    bits_prepass_kernel<<<hl.Hq, kCountThreads, 0, stream>>>(pv, la, ca, ca_prefix, ca_list, rowinfo);
    return hipGetLastError();
}

hipError_t launch_decode(const HostLayout &hl, const PlanView &pv, const uint32_t *la,
                         const uint32_t *ca, int32_t *row_ptr, int32_t *col_idx, void *workspace,
                         hipStream_t stream) {
    const size_t a0 = (sizeof(int32_t) * size_t(hl.Hq) * size_t(hl.ndocs > 0 ? hl.ndocs : 1) + 255) & ~size_t(255);
    const size_t a1 = (sizeof(int32_t) * size_t(hl.Hq) * size_t(hl.G > 0 ? hl.G : 1) + 255) & ~size_t(255);
    char *ws = static_cast<char *>(workspace);
    int32_t *ca_prefix = reinterpret_cast<int32_t *>(ws);
    int32_t *row_local = reinterpret_cast<int32_t *>(ws + a0);
    int32_t *head_total = reinterpret_cast<int32_t *>(ws + a0 + a1);
    if (hl.G == 0) {  // no rows: row_ptr[0] = 0
        zero_kernel<<<1, 64, 0, stream>>>(row_ptr, 1);
        return hipGetLastError();
    }
    decode_count_kernel<<<hl.Hq, kCountThreads, 0, stream>>>(pv, la, ca, ca_prefix, row_local,
                                                              head_total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nrows = int64_t(hl.Hq) * hl.G;
    const int64_t blocks = (nrows + kFillWaves - 1) / kFillWaves;
    decode_fill_kernel<<<static_cast<unsigned>(blocks), 64 * kFillWaves, 0, stream>>>(
        pv, la, ca, ca_prefix, row_local, head_total, row_ptr, col_idx);
    return hipGetLastError();
}

}  // namespace sift
