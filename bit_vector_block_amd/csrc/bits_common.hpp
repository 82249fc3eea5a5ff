// Bit-vector helpers shared by the decode and the fused path's pre-pass (device code).
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

// Exclusive scan of one int per thread over a workgroup of NT threads (wave scans, then the wave
// totals through sh[NT / 64]); total gets the workgroup's sum.  Every thread of the workgroup
// calls it.
template <int NT = kCountThreads>
__device__ inline int block_excl_scan(int x, int *sh, int &total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
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

// pref[d] = CA entries of the earlier documents of d's request, for q head h: the CA popcounts of
// all documents scanned in chunks of kCountThreads, then each document's value less that of its
// request's first document.  tmp: >= ndocs ints of scratch in global memory.
__device__ inline void head_ca_prefix(const PlanView &pv, const uint32_t *__restrict__ ca, int h, int32_t *pref,
                                      int32_t *tmp, int *sh) {
    const int tid = threadIdx.x, ndocs = pv.num_docs;
    int carry = 0;
    for (int base = 0; base < ndocs; base += kCountThreads) {
        const int d = base + tid;
        const int c = d < ndocs ? popcount_range(ca + pv.doc_ca_off[d] + h * pv.doc_ca_w[d], 0, pv.doc_tiles[d] - 1)
                                : 0;
        int total;
        const int ex = block_excl_scan(c, sh, total);
        if (d < ndocs) tmp[d] = carry + ex;  // CA entries of every earlier document of the batch
        carry += total;
    }
    __syncthreads();
    for (int d = tid; d < ndocs; d += kCountThreads) pref[d] = tmp[d] - tmp[pv.req_first_doc[pv.doc_req[d]]];
    __syncthreads();
}

__device__ inline int lane_rank(uint64_t mask) {
    // number of set bits of `mask` below this lane
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// lst[req_first[b] + k] = the k-th CA-marked page of request b for q head h, in document order (the
// CA part of every document row of the request is a leading slice of it).  One thread per
// document walks its set bits in order, so all documents proceed at once.  pref from
// head_ca_prefix.
__device__ inline void head_ca_list(const PlanView &pv, const uint32_t *__restrict__ ca, int h,
                                    const int32_t *pref, int32_t *lst) {
    for (int d = threadIdx.x; d < pv.num_docs; d += kCountThreads) {
        const uint32_t *vec = ca + pv.doc_ca_off[d] + h * pv.doc_ca_w[d];
        const int T = pv.doc_tiles[d], t0 = pv.doc_first[d];
        int pos = pv.req_first[pv.doc_req[d]] + pref[d];
        for (int w = 0; 32 * w < T; ++w) {
            uint32_t bits = vec[w];
            if (T - 32 * w < 32) bits &= (1u << (T - 32 * w)) - 1u;  // bits past T are ignored
            while (bits != 0u) {
                lst[pos++] = t0 + 32 * w + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
    }
}

}  // namespace bits
}  // namespace sift
