// Single-launch decode (device code): LA/CA bit vectors -> per-(head, query tile) CSR, for
// layouts whose per-head tables fit in LDS.  Used by decode_one_kernel (sift_decode_bits) and by
// the fused path's preparation launch, which runs it beside the V^T transpose.
#pragma once

#include "bits_common.hpp"

namespace sift {
namespace bits {

// Single-launch decode for layouts whose per-head tables fit in LDS (the common case; larger
// layouts take decode_count + decode_fill).  Workgroup (h, part) recomputes all of q head h's
// counts in LDS -- CA prefixes, CA page lists, LA words, row offsets -- and the list entries of
// the earlier heads in closed form, then fills rows [part * rows_per, ...) of head h.  No scratch
// in global memory and no second launch: after the plan check, every load is in one of two
// rounds (the plan records, then the bit words).
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kOneMaxG = 2048;       // rows per head (two per thread)
constexpr int kOneMaxDocs = 512;     // documents in the batch
constexpr int kOneMaxLaW = 4096;     // LA words per head
constexpr int kOneMaxDocTiles = 64;  // tiles per document: one lane per LA candidate of a row
constexpr int kOneLaK = 8;           // LA words of the batch per thread, at most
constexpr int kOneCaK = 2;           // CA words of the batch per thread, at most

__device__ inline int la_words_of(int T) { return (T * (T + 1) / 2 + 31) >> 5; }

// The last document d with key[d] <= x (key ascends strictly from key[0] = 0).
__device__ inline int doc_of(const int *key, int ndocs, int x) {
    int lo = 0, hi = ndocs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (key[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The LDS one workgroup of decode_one uses.
struct DecodeOneLds {
    int sh[2 * kOneWaves];
    uint32_t s_rcp[kOneMaxDocs];  // ceil(2^32 / lw), lw = la_words_of(T) > 1: floor(j / lw) = umulhi(j, s_rcp)
    int s_ex[kOneMaxDocs];        // batch-wide exclusive CA prefix of each document
    int s_pref[kOneMaxDocs];      // CA entries of the earlier documents of its request
    int s_laloc[kOneMaxDocs];     // first word of the document's LA vector in s_la
    int s_laoff[kOneMaxDocs];     // word offset of its (head 0) LA vector in la
    int s_caoff[kOneMaxDocs];     // word offset of its (head 0) CA vector in ca
    int s_T[kOneMaxDocs];         // its tiles
    int s_after[kOneMaxDocs];     // tiles of the later documents of its request
    uint32_t s_caw[2 * kOneMaxDocs];  // the head's CA words (two per document, bits past T cleared)
    int s_loc[kOneMaxG + 1];      // row offsets in the head; [G] = the head's total
    int s_lst[kOneMaxG];          // the head's CA page list of every request
    uint32_t s_la[kOneMaxLaW];    // the head's LA words, documents in order
};

// Whether a layout takes the single launch: its per-head tables fit in LDS, and every workgroup can
// read all bits of the batch (kOneLaK + kOneCaK words per thread).
inline bool decode_one_fits(const HostLayout &hl) {
    return hl.G > 0 && hl.G <= kOneMaxG && hl.ndocs <= kOneMaxDocs && hl.la_words / hl.Hq <= kOneMaxLaW &&
           hl.max_doc_tiles <= kOneMaxDocTiles && hl.la_words <= int64_t(kOneLaK) * kOneThreads &&
           hl.ca_words <= int64_t(kOneCaK) * kOneThreads;
}

// Workgroups per q head of the single launch, for about `target` workgroups in all; each fills at
// most 1024 rows of its head (64 per wavefront) and, where the head has enough, at least 16.
inline int decode_one_splits(const HostLayout &hl, int target) {
    const int64_t most = std::max<int64_t>(1, (hl.G + 15) / 16), least = (hl.G + 1023) / 1024;
    return static_cast<int>(std::max<int64_t>(least, std::min<int64_t>(most, (target + hl.Hq - 1) / hl.Hq)));
}
// Alone, the decode is fastest spread over about 256 workgroups; beside the V^T transpose in the
// fused path's launch, over about 64, which leaves more of the chip to the transpose (config 2:
// 345.8 against 349.6 us per fused call, one process).
constexpr int kDecodeOneTarget = 256;
constexpr int kDecodeTransposeTarget = 64;

// Workgroup `bid` (of Hq * splits, kOneThreads threads) of the single-launch decode; L: its LDS.
// After the plan check, all of its loads go out in one round: the plan records it needs and every
// LA and CA word of the batch (by flat index, so no address waits on a record).
__device__ inline void decode_one_block(const PlanView &pv, const uint32_t *__restrict__ la,
                                        const uint32_t *__restrict__ ca, int la_words, int ca_words,
                                        int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx,
                                        int32_t *__restrict__ status, int splits, int question_nnz,
                                        DecodeOneLds &L, int bid) {
    int *const sh = L.sh, *const s_ex = L.s_ex, *const s_pref = L.s_pref, *const s_laloc = L.s_laloc;
    int *const s_laoff = L.s_laoff, *const s_caoff = L.s_caoff, *const s_T = L.s_T, *const s_after = L.s_after;
    int *const s_loc = L.s_loc, *const s_lst = L.s_lst;
    uint32_t *const s_la = L.s_la, *const s_caw = L.s_caw, *const s_rcp = L.s_rcp;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = pv.num_tiles, Hq = pv.num_q_heads, ndocs = pv.num_docs;
    const int64_t nrows = static_cast<int64_t>(Hq) * G;
    const int h = bid / splits, part = bid % splits;
    const int rows_per = (G + splits - 1) / splits;
    const int g_lo = part * rows_per, g_hi = min(G, g_lo + rows_per);
    const bool ok = plan_ok(pv);
    // the call's status word: written once, by this thread alone
    if (bid == 0 && tid == 0) *status = ok ? SIFT_DEVICE_OK : SIFT_DEVICE_PLAN_MISMATCH;
    if (!ok) {  // a plan of another layout: an empty CSR
        for (int g = g_lo + tid; g < g_hi; g += kOneThreads) row_ptr[static_cast<int64_t>(h) * G + g] = 0;
        if (tid == 0 && h == Hq - 1 && g_lo <= G - 1 && G - 1 < g_hi) row_ptr[nrows] = 0;
        return;
    }

    // 1. One round of loads: this thread's document and rows (tid, tid + kOneThreads), the rows
    //    this wavefront fills (lane j: its j-th row, g_lo + wave + j kOneWaves), and words
    //    tid + k kOneThreads of the LA and CA arrays.
    int d_rfd = 0, d_first = 0, d_req = 0, d_T = 0;
    if (tid < ndocs) {
        const int32_t *dr = pv.doc_rec + static_cast<int64_t>(tid) * kRecWords;
        d_T = dr[kDrTiles];
        d_rfd = dr[kDrReqDoc];
        d_first = dr[kDrFirst];
        d_req = dr[kDrReq];
        const int la_off = dr[kDrLaOff];
        s_laloc[tid] = la_off / Hq;  // the (d, head 0) offset counts Hq vectors per earlier document
        s_laoff[tid] = la_off;
        s_caoff[tid] = dr[kDrCaOff];
        s_T[tid] = d_T;
        const uint64_t lw = la_words_of(d_T);
        s_rcp[tid] = static_cast<uint32_t>((0x100000000ull + lw - 1) / lw);  // (unused for lw = 1)
        s_after[tid] = dr[kDrAfter];
        s_caw[2 * tid] = 0u;
        s_caw[2 * tid + 1] = 0u;
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
    uint32_t law[kOneLaK], caw[kOneCaK];
#pragma unroll
    for (int k = 0; k < kOneLaK; ++k) {
        const int i = tid + k * kOneThreads;
        law[k] = i < la_words ? la[i] : 0u;
    }
#pragma unroll
    for (int k = 0; k < kOneCaK; ++k) {
        const int i = tid + k * kOneThreads;
        caw[k] = i < ca_words ? ca[i] : 0u;
    }
    __syncthreads();

    // 2. Each word's (document, head, word): head h's go to LDS; the earlier heads' are counted --
    //    all their LA entries, and each CA entry times the tiles of the later documents of its
    //    request (every row of those documents lists it).
    int64_t earlier = 0;  // list entries of heads 0 .. h - 1, this thread's share
#pragma unroll
    for (int k = 0; k < kOneLaK; ++k) {
        const int i = tid + k * kOneThreads;
        if (i < la_words) {
            const int d = doc_of(s_laoff, ndocs, i);
            // j < 2^13 and lw <= 65, so the rounded-up reciprocal gives floor(j / lw) exactly
            const int T = s_T[d], lw = la_words_of(T), j = i - s_laoff[d];
            const int hp = lw == 1 ? j : static_cast<int>(__umulhi(static_cast<uint32_t>(j), s_rcp[d]));
            const int w = j - hp * lw;
            if (hp == h) {
                s_la[s_laloc[d] + w] = law[k];
            } else if (hp < h) {
                const int keep = w == lw - 1 ? T * (T + 1) / 2 - 32 * w : 32;  // bits past the triangle
                earlier += __popc(keep == 32 ? law[k] : (law[k] & ((1u << keep) - 1u)));
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kOneCaK; ++k) {
        const int i = tid + k * kOneThreads;
        if (i < ca_words) {
            const int d = doc_of(s_caoff, ndocs, i);
            const int T = s_T[d], cw = (T + 31) >> 5, j = i - s_caoff[d];  // cw is 1 or 2
            const int hp = j >> (cw - 1), w = j - hp * cw;
            const int keep = T - 32 * w;  // bits past T are ignored
            const uint32_t x = keep >= 32 ? caw[k] : (caw[k] & ((1u << keep) - 1u));
            if (hp == h) s_caw[2 * d + w] = x;
            else if (hp < h) earlier += static_cast<int64_t>(__popc(x)) * s_after[d];
        }
    }
    __syncthreads();

    // 3. CA prefixes (documents scanned batch-wide, less the value at the request's first
    //    document), the head's CA page lists, and the list entries of the earlier heads.
    const uint32_t cw0 = tid < ndocs ? s_caw[2 * tid] : 0u, cw1 = tid < ndocs ? s_caw[2 * tid + 1] : 0u;
    const int c_doc = __popc(cw0) + __popc(cw1);
    int tot, base_h;  // earlier: a share of the CSR, < 2^31
    const int ex = block_excl_scan_sum<kOneThreads>(c_doc, static_cast<int>(earlier), sh, tot, base_h);
    if (tid < ndocs) s_ex[tid] = ex;
    base_h += h * question_nnz;
    __syncthreads();
    if (tid < ndocs) {
        const int p = ex - s_ex[d_rfd];
        s_pref[tid] = p;
        int pos = d_req + p;
        const uint32_t cws[2] = {cw0, cw1};
        for (int w = 0; w < 2; ++w) {
            uint32_t bits = cws[w];
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

}  // namespace bits
}  // namespace sift
