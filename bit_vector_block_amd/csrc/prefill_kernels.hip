// Block-sparse causal GQA attention over decoded CSR rows (gfx950).
//
// SIFT technical summary, section 2, "Dettagli di Implementazione": the sparse
// attention kernel extends a FlashAttention-style kernel so that it iterates
// only over the tile indices decoded from the bit vectors.  This is an
// MI355X-native design, not the FlashAttention-3 (Hopper) kernel the pages
// build on:
//
//  * one workgroup = one CSR row (q head h, query tile g) = 64 queries, two
//    wavefronts of 32 queries each;
//  * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    lane l of a wave then holds 16 keys of query (l % 32) per 32-key block, so
//    the online-softmax state (running max, running sum) of a query lives in
//    one lane (plus its partner lane l ^ 32 for the other half of the keys);
//  * the output is accumulated transposed too, O^T += V^T P^T: the MFMA's B
//    operand is exactly the lane's own P values (no cross-lane shuffles) once
//    the 16 keys of a K-step are permuted consistently in A and B;
//  * K is staged in LDS row-major (padded rows), V is staged transposed (d-major,
//    padded) so that the A operand of V^T reads two 8-byte runs per lane;
//  * exp2 with log2(e) folded into the scale; masking (causal on the diagonal
//    tile, padded keys) is a select, so NaN in padded K slots never leaks;
//  * P is rounded to bf16 for the PV product and the row sum l is accumulated
//    from the same rounded values;
//  * the fp32 output tile is staged through LDS and written as full rows.
#include <math.h>

#include <algorithm>

#include "sift_internal.hpp"

namespace sift {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 128;  // two wavefronts

__device__ inline bool plan_ok(const PlanView &pv) {
    return pv.header[0] == static_cast<int32_t>(kPlanMagic) &&
           static_cast<uint32_t>(pv.header[2]) == pv.fp_lo &&
           static_cast<uint32_t>(pv.header[3]) == pv.fp_hi && pv.header[6] == pv.num_tiles;
}

template <int D>
struct Smem {
    static constexpr int KS = D + 8;   // K row stride (bf16): 16-byte pad per row
    static constexpr int VS = 64 + 4;  // V^T row stride (bf16): 8-byte pad per row
    static constexpr int OS = D + 4;   // output staging row stride (fp32)
    static constexpr int kBytes = 2 * 64 * KS + 2 * D * VS;
    static constexpr int oBytes = 4 * 64 * OS;
    static constexpr int bytes = kBytes > oBytes ? kBytes : oBytes;
};

template <int D>
__global__ __launch_bounds__(kThreads) void sparse_prefill_kernel(
    PlanView pv, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, float scale, float scale_log2, float *__restrict__ out,
    float *__restrict__ lse, int Hq, int Hkv) {
    using S = Smem<D>;
    constexpr int KS = S::KS, VS = S::VS, OS = S::OS;
    constexpr int DC = D / 16;  // 16-wide d chunks (QK^T K-steps)
    constexpr int DB = D / 32;  // 32-wide d blocks of O^T
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::bytes];
    uint16_t *Ks = reinterpret_cast<uint16_t *>(smem);
    uint16_t *Vt = Ks + 64 * KS;
    float *Os = reinterpret_cast<float *>(smem);

    if (!plan_ok(pv)) return;
    const int G = pv.num_tiles;
    const int64_t N = static_cast<int64_t>(G) * kTile;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

    // Longest rows first: later tiles of a request carry longer rows.
    const int bid = blockIdx.x;
    const int h = bid % Hq;
    const int g = G - 1 - bid / Hq;
    const int64_t row = static_cast<int64_t>(h) * G + g;
    const int kvh = h / (Hq / Hkv);
    const int q_valid = pv.tile_valid[g];
    const int64_t tok0 = static_cast<int64_t>(g) * kTile;
    const int qi = wave * 32 + l32;  // this lane's query inside the tile

    // Q fragments (MFMA B operand): Q[qi][16 dc + 8 hi .. +7]
    bf16x8 qf[DC];
    {
        const uint16_t *qrow = q + ((tok0 + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * dc);
    }

    f32x16 acc_o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db] = f32x16{};
    float m_run = -INFINITY;  // running max of raw q.k (unscaled)
    float l_run = 0.0f;       // this lane's partial row sum

    const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
    for (int e = e0; e < e1; ++e) {
        const int t = col_idx[e];
        if (t < 0 || t >= G) continue;
        const int kv_valid = pv.tile_valid[t];
        const int64_t ktok0 = static_cast<int64_t>(t) * kTile;
        __syncthreads();  // the previous tile's LDS reads are done
        // K tile -> Ks[key][d]; 16-byte chunks, each row read contiguously
        {
            constexpr int CPR = D / 8;          // chunks per row
            constexpr int RPP = kThreads / CPR;  // rows per pass
            const int c = tid % CPR;
#pragma unroll
            for (int p = 0; p < 64 / RPP; ++p) {
                const int r = p * RPP + tid / CPR;
                const uint4 val = *reinterpret_cast<const uint4 *>(
                    k + ((ktok0 + r) * Hkv + kvh) * D + 8 * c);
                *reinterpret_cast<uint4 *>(Ks + r * KS + 8 * c) = val;
            }
        }
        // V tile -> Vt[d][key]; a thread moves 4 keys x D/8 dims
        {
            constexpr int DPT = D / 8;  // dims per thread
            const int kq = tid & 15, dg = tid >> 4;
            uint32_t w[4][DPT / 2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint16_t *src = v + ((ktok0 + 4 * kq + j) * Hkv + kvh) * D + dg * DPT;
#pragma unroll
                for (int x = 0; x < DPT / 8; ++x) {
                    const uint4 val = *reinterpret_cast<const uint4 *>(src + 8 * x);
                    w[j][4 * x + 0] = val.x;
                    w[j][4 * x + 1] = val.y;
                    w[j][4 * x + 2] = val.z;
                    w[j][4 * x + 3] = val.w;
                }
            }
#pragma unroll
            for (int dd = 0; dd < DPT; ++dd) {
                const int sh = (dd & 1) * 16;
                const uint32_t a0 = (w[0][dd >> 1] >> sh) & 0xffffu, a1 = (w[1][dd >> 1] >> sh) & 0xffffu;
                const uint32_t a2 = (w[2][dd >> 1] >> sh) & 0xffffu, a3 = (w[3][dd >> 1] >> sh) & 0xffffu;
                uint2 pk;
                pk.x = a0 | (a1 << 16);
                pk.y = a2 | (a3 << 16);
                *reinterpret_cast<uint2 *>(Vt + (dg * DPT + dd) * VS + 4 * kq) = pk;
            }
        }
        __syncthreads();

        // S^T = K Q^T: block kb covers keys 32 kb .. 32 kb + 31
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Ks + (32 * kb + l32) * KS + 16 * dc + 8 * hi);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[kb], 0, 0, 0);
            }
        }
        // masks: register i of block kb is key 32 kb + 8 (i / 4) + 4 hi + i % 4
        if (kv_valid < kTile || t >= g) {
            const int shift = (t - g) * kTile;  // key token - query token offset of the tiles
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
                    const bool ok = key < kv_valid && shift + key <= qi;
                    s[kb][i] = ok ? s[kb][i] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * scale_log2);
        const float nbias = -m_use * scale_log2;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
        // P (bf16) as the MFMA B operand: half j of block kb = registers 8 j .. 8 j + 7
        bf16x8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], scale_log2, nbias));
                const __bf16 pr = static_cast<__bf16>(p);
                l_run += static_cast<float>(pr);
                pb[kb][i >> 3][i & 7] = pr;
            }
        // O^T += V^T P^T over four 16-key steps
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint16_t *vrow = Vt + (32 * db + l32) * VS + 4 * hi;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int k0 = 32 * kb + 16 * j;
                    const bf16x4 lo4 = *reinterpret_cast<const bf16x4 *>(vrow + k0);
                    const bf16x4 hi4 = *reinterpret_cast<const bf16x4 *>(vrow + k0 + 8);
                    const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][j], acc_o[db], 0, 0, 0);
                }
        }
    }

    // epilogue: O = acc / l, staged through LDS, written as whole rows
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    __syncthreads();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 o4;
            o4[0] = acc_o[db][4 * i4 + 0] * inv;
            o4[1] = acc_o[db][4 * i4 + 1] * inv;
            o4[2] = acc_o[db][4 * i4 + 2] * inv;
            o4[3] = acc_o[db][4 * i4 + 3] * inv;
            *reinterpret_cast<f32x4 *>(Os + qi * OS + 32 * db + 8 * i4 + 4 * hi) = o4;
        }
    if (lse != nullptr && hi == 0) {
        const bool live = qi < q_valid && l_tot > 0.0f;
        lse[static_cast<int64_t>(h) * N + tok0 + qi] = live ? m_run * scale + logf(l_tot) : -INFINITY;
    }
    __syncthreads();
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < 64 * C4; idx += kThreads) {
        const int r = idx / C4, c4 = idx % C4;
        f32x4 val = *reinterpret_cast<const f32x4 *>(Os + r * OS + 4 * c4);
        if (r >= q_valid) val = f32x4{};
        *reinterpret_cast<f32x4 *>(out + ((tok0 + r) * Hq + h) * D + 4 * c4) = val;
    }
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

hipError_t launch_prefill(const HostLayout &hl, const PlanView &pv, const uint16_t *q,
                          const uint16_t *k, const uint16_t *v, const int32_t *row_ptr,
                          const int32_t *col_idx, float scale, float *out, float *lse,
                          hipStream_t stream) {
    const int64_t rows = int64_t(hl.Hq) * hl.G;
    if (rows == 0) return hipSuccess;
    const float scale_log2 = scale * 1.4426950408889634f;
    if (hl.D == 128)
        sparse_prefill_kernel<128><<<static_cast<unsigned>(rows), kThreads, 0, stream>>>(
            pv, q, k, v, row_ptr, col_idx, scale, scale_log2, out, lse, hl.Hq, hl.Hkv);
    else
        sparse_prefill_kernel<64><<<static_cast<unsigned>(rows), kThreads, 0, stream>>>(
            pv, q, k, v, row_ptr, col_idx, scale, scale_log2, out, lse, hl.Hq, hl.Hkv);
    return hipGetLastError();
}

}  // namespace sift
