// Work that prepares the attention kernel's inputs (gfx950):
//   transpose_v_kernel       V [N][Hkv][D] -> V^T tiles in the attention's layout, and the
//                            workspace header (row-queue counters, status word) cleared;
//   decode_transpose_kernel  the fused path's launch: the single-launch decode of the layer's
//                            bits into a CSR of the workspace, beside the same transpose;
//   cast_bf16_kernel         fp32 inputs rounded to bf16.
#include <algorithm>

#include "bits_common.hpp"
#include "decode_one.hpp"
#include "sift_internal.hpp"

namespace sift {

namespace {

using namespace bits;

// position of token n inside V^T: bits 2 and 3 of n swapped, so that within every 16-token
// group the 8 tokens {0..3, 8..11} come first and {4..7, 12..15} second -- the 8 keys that
// lane half 0 and lane half 1 feed into one PV K-step
__host__ __device__ inline int64_t vt_pos(int64_t n) { return (n & ~int64_t(12)) | ((n & 4) << 1) | ((n & 8) >> 1); }

// V [N][Hkv][D] (bf16 or fp32, rounded to bf16) -> V^T tiles [Hkv][G][D][64] (each 64-token tile's
// D rows of 128 bytes contiguous, so that the attention's tile loads cover one 16 KB block) with
// the tokens of every 16-token group at vt_pos.  One workgroup of 256 threads per (64-token tile t,
// kv head): the tile goes through LDS so that both the 2D-byte row reads and the 128-byte V^T row
// writes are whole rows.
template <int D>
constexpr int kTransposeLd = D + 2;  // padded LDS row (bf16 elements): column reads hit distinct banks

template <int D, typename T, int NT>
__device__ inline void transpose_tile(const T *__restrict__ v, uint16_t *__restrict__ vt, int Hkv, int64_t N, int t,
                                      int kvh, uint16_t *tile) {
    constexpr int LD = kTransposeLd<D>;
    constexpr int CH = D / 8;  // 8-element chunks per token row
    const int tid = threadIdx.x;
    const int64_t tok0 = static_cast<int64_t>(t) * kTile;
    // read: 8 consecutive elements (16 or 32 bytes) of one token row per thread and pass
    for (int x = tid; x < 64 * CH; x += NT) {
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
    for (int x = tid; x < D * 8; x += NT) {
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

// Tiles x0 .. x0 + n - 1 (n <= TPB) of the (kv head, tile) order x = kvh G + t, all staged in LDS at
// once: every thread first loads its 16-byte chunks of all n tiles (one round trip to memory for
// the workgroup), then the V^T rows are gathered from LDS and written.  NT threads.
template <int D, typename T, int NT, int TPB>
__device__ inline void transpose_tiles(const T *__restrict__ v, uint16_t *__restrict__ vt, int Hkv, int G, int x0,
                                       int n, uint16_t *lds) {
    constexpr int LD = kTransposeLd<D>;
    constexpr int CH = D / 8;             // 8-element chunks per token row
    constexpr int PER = 64 * CH;          // chunks per tile
    constexpr int K = (TPB * PER + NT - 1) / NT;  // chunks per thread, at most
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    u32x4 got[K];  // 8 bf16 each
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int x = tid + k * NT;
        got[k] = u32x4{0u, 0u, 0u, 0u};
        if (x < n * PER) {
            const int j = x / PER, y = x % PER, r = y / CH, c = y % CH;
            const int tile = x0 + j, t = tile % G, kvh = tile / G;
            const T *src = v + ((static_cast<int64_t>(t) * kTile + r) * Hkv + kvh) * D + 8 * c;
            if constexpr (sizeof(T) == 2) {
                got[k] = *reinterpret_cast<const u32x4 *>(src);
            } else {
                const float4 a = *reinterpret_cast<const float4 *>(src);
                const float4 b = *reinterpret_cast<const float4 *>(src + 4);
                const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f[2 * e])) |
                           (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f[2 * e + 1]))) << 16);
                got[k] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int x = tid + k * NT;
        if (x < n * PER) {
            const int j = x / PER, y = x % PER, r = y / CH, c = y % CH;
            uint32_t *dst = reinterpret_cast<uint32_t *>(lds + (j * 64 + r) * LD + 8 * c);  // 4-byte aligned
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = got[k][e];
        }
    }
    __syncthreads();
    for (int x = tid; x < n * D * 8; x += NT) {
        const int j = x / (D * 8), y = x % (D * 8), d = y / 8, c = y % 8;
        const int tile = x0 + j, t = tile % G, kvh = tile / G;
        const uint16_t *tl = lds + j * 64 * LD;
        uint16_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = tl[static_cast<int>(vt_pos(8 * c + e)) * LD + d];
        uint4 pk;
        pk.x = w[0] | (uint32_t(w[1]) << 16);
        pk.y = w[2] | (uint32_t(w[3]) << 16);
        pk.z = w[4] | (uint32_t(w[5]) << 16);
        pk.w = w[6] | (uint32_t(w[7]) << 16);
        *reinterpret_cast<uint4 *>(vt + ((static_cast<int64_t>(kvh) * G + t) * D + d) * kTile + 8 * c) = pk;
    }
}

// V^T tiles one workgroup of the decode-transpose launch stages together.
template <int D>
constexpr int kTransposeTpb = static_cast<int>(sizeof(DecodeOneLds) / (sizeof(uint16_t) * 64 * kTransposeLd<D>));

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
    __shared__ uint16_t tile[64 * kTransposeLd<D>];
    if (blockIdx.x == 0 && blockIdx.y == 0) clear_prefill_header(header);
    transpose_tile<D, T, 256>(v, vt, Hkv, N, blockIdx.x, blockIdx.y, tile);
}

// Fused path, one launch: the single-launch decode of the layer's bits into the workspace CSR
// (workgroups 0 .. ndec - 1, dispatched first: they are latency-bound) beside the V^T transpose,
// one tile per workgroup, whose first workgroup clears the attention's row-queue counters (the
// status word is the decode's).
template <int D, typename T>
__global__ __launch_bounds__(kOneThreads) void decode_transpose_kernel(
    PlanView pv, const uint32_t *__restrict__ la, const uint32_t *__restrict__ ca, int la_words, int ca_words,
    int32_t *__restrict__ row_ptr, int32_t *__restrict__ col_idx, int32_t *__restrict__ status, int splits,
    int question_nnz, const T *__restrict__ v, uint16_t *__restrict__ vt, int Hkv, int G, int *__restrict__ header) {
    __shared__ DecodeOneLds lds;  // a transpose workgroup stages its kTransposeTpb<D> tiles here
    constexpr int TPB = kTransposeTpb<D>;
    static_assert(TPB >= 1, "a tile fits");
    const int b = blockIdx.x, ndec = pv.num_q_heads * splits;
    if (b < ndec) {
        decode_one_block(pv, la, ca, la_words, ca_words, row_ptr, col_idx, status, splits, question_nnz, lds, b);
        return;
    }
    const int x0 = (b - ndec) * TPB;
    if (x0 == 0 && threadIdx.x < kPrefillQueues) header[threadIdx.x] = 0;
    transpose_tiles<D, T, kOneThreads, TPB>(v, vt, Hkv, G, x0, min(TPB, G * Hkv - x0),
                                            reinterpret_cast<uint16_t *>(&lds));
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

bool decode_transpose_fits(const HostLayout &hl) { return decode_one_fits(hl); }

hipError_t launch_decode_transpose(const HostLayout &hl, const PlanView &pv, const uint32_t *la, const uint32_t *ca,
                                   int32_t *row_ptr, int32_t *col_idx, int32_t *status, const void *v, bool fp32,
                                   uint16_t *vt, int *header, hipStream_t stream) {
    if (!decode_one_fits(hl)) return hipErrorInvalidValue;
    const int splits = decode_one_splits(hl, kDecodeTransposeTarget);
    const int64_t tiles = int64_t(hl.G) * hl.Hkv, tpb = hl.D == 128 ? kTransposeTpb<128> : kTransposeTpb<64>;
    const unsigned grid = static_cast<unsigned>(int64_t(hl.Hq) * splits + (tiles + tpb - 1) / tpb);
    const int qn = static_cast<int>(hl.question_nnz);
    const int law = static_cast<int>(hl.la_words), caw = static_cast<int>(hl.ca_words);
#define SIFT_DT(DD, TT)                                                                                 \
    decode_transpose_kernel<DD, TT><<<grid, kOneThreads, 0, stream>>>(pv, la, ca, law, caw, row_ptr, col_idx, \
                                                                      status, splits, qn,                \
                                                                      static_cast<const TT *>(v), vt,    \
                                                                      hl.Hkv, hl.G, header)
    if (hl.D == 128) {
        if (fp32) SIFT_DT(128, float);
        else SIFT_DT(128, __bf16);
    } else {
        if (fp32) SIFT_DT(64, float);
        else SIFT_DT(64, __bf16);
    }
#undef SIFT_DT
    return hipGetLastError();
}

}  // namespace sift
