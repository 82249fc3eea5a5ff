// Work that prepares the attention kernel's inputs (gfx950):
//   transpose_v_kernel  V [N][Hkv][D] -> V^T tiles in the attention's layout (CSR path), and the
//                       workspace header (row-queue counters, status word) cleared;
//   fused_prep_kernel   the fused path's bits pre-pass (per q head: CA prefixes, CA page lists,
//                       per-row list records) and the same transpose in one launch;
//   cast_bf16_kernel    fp32 inputs rounded to bf16.
#include <algorithm>

#include "bits_common.hpp"
#include "sift_internal.hpp"

namespace sift {

namespace {

using namespace bits;

// position of token n inside V^T: bits 2 and 3 of n swapped, so that within every 16-token
// group the 8 tokens {0..3, 8..11} come first and {4..7, 12..15} second -- the 8 keys that
// lane half 0 and lane half 1 feed into one PV K-step
__host__ __device__ inline int64_t vt_pos(int64_t n) { return (n & ~int64_t(12)) | ((n & 4) << 1) | ((n & 8) >> 1); }

// Pre-pass of the fused path (no CSR), one workgroup of kCountThreads threads per q head h:
//   ca_prefix[h][d] : CA entries of the earlier documents of d's request (request-local);
//   ca_list[h][req_first[b] + k] : the k-th CA-marked page of request b, in document order --
//                      the CA part of every document row of the request is a leading slice of it;
//   rowinfo[h][g]   : what the attention kernel needs to build row (h, g)'s list itself:
//                      {n, ca_n (-1: question row, dense range), ca_base, la_word, la_lo, t0, r, 0}.
__device__ inline void prepass_head(const PlanView &pv, const uint32_t *__restrict__ la,
                                    const uint32_t *__restrict__ ca, int32_t *__restrict__ ca_prefix,
                                    int32_t *__restrict__ ca_list, int32_t *__restrict__ rowinfo, int h) {
    const int tid = threadIdx.x;
    const int ndocs = pv.num_docs, G = pv.num_tiles;
    int32_t *pref = ca_prefix + static_cast<int64_t>(h) * ndocs;
    int32_t *lst = ca_list + static_cast<int64_t>(h) * G;
    __shared__ int sh[kCountThreads / 64];
    head_ca_prefix(pv, ca, h, pref, lst, sh);  // the head's page list (G >= ndocs) as scratch
    head_ca_list(pv, ca, h, pref, lst);
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

// V [N][Hkv][D] (bf16 or fp32, rounded to bf16) -> V^T tiles [Hkv][G][D][64] (each 64-token tile's
// D rows of 128 bytes contiguous, so that the attention's tile loads cover one 16 KB block) with
// the tokens of every 16-token group at vt_pos.  One workgroup of 256 threads per (64-token tile t,
// kv head): the tile goes through LDS so that both the 2D-byte row reads and the 128-byte V^T row
// writes are whole rows.
template <int D, typename T>
__device__ inline void transpose_tile(const T *__restrict__ v, uint16_t *__restrict__ vt, int Hkv, int64_t N, int t,
                                      int kvh) {
    constexpr int LD = D + 2;  // padded LDS row (bf16 elements): column reads hit distinct banks
    constexpr int CH = D / 8;  // 8-element chunks per token row
    __shared__ uint16_t tile[64 * LD];
    const int tid = threadIdx.x;
    const int64_t tok0 = static_cast<int64_t>(t) * kTile;
    // read: 8 consecutive elements (16 or 32 bytes) of one token row per thread and pass
    for (int x = tid; x < 64 * CH; x += 256) {
        const int r = x / CH, c = x % CH;
        const T *src = v + ((tok0 + r) * Hkv + kvh) * D + 8 * c;
        uint16_t *dst = tile + r * LD + 8 * c;
        if constexpr (sizeof(T) == 2) {
            const uint4 w = *reinterpret_cast<const uint4 *>(src);
            const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dst[2 * j] = static_cast<uint16_t>(p[j] & 0xFFFFu);
                dst[2 * j + 1] = static_cast<uint16_t>(p[j] >> 16);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4 *>(src);
            const float4 b = *reinterpret_cast<const float4 *>(src + 4);
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f[j]));
        }
    }
    __syncthreads();
    // V^T row d of this tile: 64 stored positions; thread writes 8 consecutive positions
    for (int x = tid; x < D * 8; x += 256) {
        const int d = x / 8, c = x % 8;
        uint16_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = tile[static_cast<int>(vt_pos(8 * c + j)) * LD + d];
        uint4 pk;
        pk.x = w[0] | (uint32_t(w[1]) << 16);
        pk.y = w[2] | (uint32_t(w[3]) << 16);
        pk.z = w[4] | (uint32_t(w[5]) << 16);
        pk.w = w[6] | (uint32_t(w[7]) << 16);
        *reinterpret_cast<uint4 *>(vt + ((static_cast<int64_t>(kvh) * (N / kTile) + t) * D + d) * kTile + 8 * c) = pk;
    }
}

// The attention kernel claims rows from the header's counters and raises flags in its status
// word: both start at zero for every call.
__device__ inline void clear_prefill_header(int *__restrict__ header) {
    if (threadIdx.x < kPrefillQueues) header[threadIdx.x] = 0;
    if (threadIdx.x == 64) header[kStatusWord] = 0;
}

// CSR path: the V^T transpose, one workgroup per (tile, kv head); block (0, 0) clears the header.
template <int D, typename T>
__global__ __launch_bounds__(256) void transpose_v_kernel(const T *__restrict__ v, uint16_t *__restrict__ vt,
                                                          int Hkv, int64_t N, int *__restrict__ header) {
    if (blockIdx.x == 0 && blockIdx.y == 0) clear_prefill_header(header);
    transpose_tile<D, T>(v, vt, Hkv, N, blockIdx.x, blockIdx.y);
}

// Fused path: the bits pre-pass and the V^T transpose are independent, so they share one launch:
// blocks 0 .. Hq-1 run the pre-pass of one q head each (short, latency-bound: they come first), the
// other blocks transpose one (tile, kv head) each (bandwidth-bound) and the first of them clears
// the header.  A plan of another layout skips the pre-pass (the attention kernel flags it).
template <int D, typename T>
__global__ __launch_bounds__(256) void fused_prep_kernel(PlanView pv, const uint32_t *__restrict__ la,
                                                         const uint32_t *__restrict__ ca,
                                                         int32_t *__restrict__ ca_prefix,
                                                         int32_t *__restrict__ ca_list, int32_t *__restrict__ rowinfo,
                                                         const T *__restrict__ v, uint16_t *__restrict__ vt, int Hq,
                                                         int Hkv, int G, int *__restrict__ header) {
    const int b = blockIdx.x;
    if (b < Hq) {
        if (plan_ok(pv)) prepass_head(pv, la, ca, ca_prefix, ca_list, rowinfo, b);
        return;
    }
    const int x = b - Hq;
    if (x == 0) clear_prefill_header(header);
    transpose_tile<D, T>(v, vt, Hkv, static_cast<int64_t>(G) * kTile, x % G, x / G);
}

__global__ void cast_bf16_kernel(const float *__restrict__ src, __bf16 *__restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = static_cast<__bf16>(src[i]);  // round to nearest even
}

}  // namespace

hipError_t launch_cast_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    cast_bf16_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        src, reinterpret_cast<__bf16 *>(dst), n);
    return hipGetLastError();
}

hipError_t launch_transpose_v(const HostLayout &hl, const void *v, bool fp32, uint16_t *vt, int *header,
                              hipStream_t stream) {
    if (hl.G == 0) return hipSuccess;
    const int64_t N = int64_t(hl.G) * kTile;
    const dim3 grid(static_cast<unsigned>(hl.G), static_cast<unsigned>(hl.Hkv));
    if (hl.D == 128) {
        if (fp32) transpose_v_kernel<128, float><<<grid, 256, 0, stream>>>(static_cast<const float *>(v), vt, hl.Hkv, N, header);
        else transpose_v_kernel<128, __bf16><<<grid, 256, 0, stream>>>(static_cast<const __bf16 *>(v), vt, hl.Hkv, N, header);
    } else {
        if (fp32) transpose_v_kernel<64, float><<<grid, 256, 0, stream>>>(static_cast<const float *>(v), vt, hl.Hkv, N, header);
        else transpose_v_kernel<64, __bf16><<<grid, 256, 0, stream>>>(static_cast<const __bf16 *>(v), vt, hl.Hkv, N, header);
    }
    return hipGetLastError();
}

hipError_t launch_fused_prep(const HostLayout &hl, const PlanView &pv, const uint32_t *la, const uint32_t *ca,
                             int32_t *ca_prefix, int32_t *ca_list, int32_t *rowinfo, const void *v, bool fp32,
                             uint16_t *vt, int *header, hipStream_t stream) {
    if (hl.G == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(hl.Hq + int64_t(hl.G) * hl.Hkv);
#define SIFT_FUSED_PREP(DD, TT)                                                                                  \
    fused_prep_kernel<DD, TT><<<grid, 256, 0, stream>>>(pv, la, ca, ca_prefix, ca_list, rowinfo,               \
                                                        static_cast<const TT *>(v), vt, hl.Hq, hl.Hkv, hl.G, header)
    if (hl.D == 128) {
        if (fp32) SIFT_FUSED_PREP(128, float);
        else SIFT_FUSED_PREP(128, __bf16);
    } else {
        if (fp32) SIFT_FUSED_PREP(64, float);
        else SIFT_FUSED_PREP(64, __bf16);
    }
#undef SIFT_FUSED_PREP
    return hipGetLastError();
}

}  // namespace sift
