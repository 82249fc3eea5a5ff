// Bit-vector helpers of the decode kernels (device code).
#pragma once

#include "sift_internal.hpp"

namespace sift {
namespace bits {

constexpr int kCountThreads = 256;

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

// Inclusive scan over the 64 lanes of a wavefront with DPP moves (no LDS traffic): shifts by 1, 2,
// 4 and 8 inside each row of 16 lanes, then the last lane of row 0 (row 2) added to row 1 (row 3),
// and lane 31 added to rows 2 and 3.  Lanes a move has no source for add the `old` operand, 0.
__device__ inline int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

// Exclusive scan of one int per thread over a workgroup of NT threads (wave scans, then the wave
// totals through sh[NT / 64]); total gets the workgroup's sum.  Every thread of the workgroup
// calls it.
template <int NT = kCountThreads>
__device__ inline int block_excl_scan(int x, int *sh, int &total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int incl = wave_incl_scan(x);
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    int below = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int v = sh[w];
        below += w < wave ? v : 0;
        all += v;
    }
    __syncthreads();  // sh is free again
    total = all;
    return below + incl - x;
}

// block_excl_scan of x, and the workgroup's sum of y, with one pair of barriers (sh: 2 NT / 64 ints).
template <int NT>
__device__ inline int block_excl_scan_sum(int x, int y, int *sh, int &total_x, int &total_y) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int incl = wave_incl_scan(x), ysum = wave_incl_scan(y);
    if (lane == 63) {
        sh[wave] = incl;
        sh[NT / 64 + wave] = ysum;
    }
    __syncthreads();
    int below = 0, all = 0, ally = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int v = sh[w];
        below += w < wave ? v : 0;
        all += v;
        ally += sh[NT / 64 + w];
    }
    __syncthreads();  // sh is free again
    total_x = all;
    total_y = ally;
    return below + incl - x;
}

__device__ inline int lane_rank(uint64_t mask) {
    // number of set bits of `mask` below this lane
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

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
    int d, r, first, req, la_word, lo;
    int la_cnt;
};
__device__ inline RowFacts row_facts(const PlanView &pv, const uint32_t *__restrict__ la, int h, int g) {
    const int32_t *tr = pv.tile_rec + static_cast<int64_t>(g) * kRecWords;
    RowFacts f;
    f.d = tr[kTrDoc];
    f.r = tr[kTrLocal];
    f.first = tr[kTrFirst];
    f.req = tr[kTrReq];
    f.la_word = tr[kTrLaOff] + h * tr[kTrLaW];
    f.lo = tr[kTrLo];
    f.la_cnt = f.d >= 0 ? popcount_bits(la + f.la_word, f.lo, f.r + 1) : 0;
    return f;
}

// The CA pass over the documents of the batch for q head h, kCountThreads documents at a time:
// CA popcounts (bits past T ignored), their batch-wide exclusive scan, and per document
//   pref[d]                 CA entries of the earlier documents of its request;
//   lst[req_first + k]      the k-th CA-marked page of each request, in document order (the CA part
//                           of every document row of the request is a leading slice of it).
// s_pref[d] also gets pref[d] for the documents of the first chunk (all of them when ndocs <=
// kCountThreads).  tmp: >= ndocs ints of global scratch; s_ex: kCountThreads ints of LDS.  Every
// thread of the workgroup calls it.
__device__ inline void head_ca_pass(const PlanView &pv, const uint32_t *__restrict__ ca, int h, int32_t *pref,
                                    int32_t *lst, int32_t *tmp, int *sh, int *s_ex, int *s_pref) {
    const int tid = threadIdx.x, ndocs = pv.num_docs;
    int carry = 0;
    for (int base = 0; base < ndocs; base += kCountThreads) {
        const int d = base + tid;
        const int32_t *dr = pv.doc_rec + static_cast<int64_t>(d < ndocs ? d : 0) * kRecWords;
        const int T = dr[kDrTiles], req_doc = dr[kDrReqDoc], first = dr[kDrFirst], req = dr[kDrReq];
        const uint32_t *vec = ca + dr[kDrCaOff] + h * ((T + 31) >> 5);
        const int c = d < ndocs ? popcount_bits(vec, 0, T) : 0;
        int total;
        const int gex = carry + block_excl_scan(c, sh, total);
        s_ex[tid] = gex;
        if (d < ndocs) tmp[d] = gex;  // for later chunks
        __syncthreads();
        if (d < ndocs) {
            const int p = gex - (req_doc >= base ? s_ex[req_doc - base] : tmp[req_doc]);
            pref[d] = p;
            if (base == 0) s_pref[tid] = p;
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
        __syncthreads();  // s_ex and tmp free again
    }
}

}  // namespace bits
}  // namespace sift
