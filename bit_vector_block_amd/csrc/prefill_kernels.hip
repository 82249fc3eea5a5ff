// Block-sparse causal GQA attention over decoded CSR rows (gfx950).
//
// SIFT technical summary, section 2, "Dettagli di Implementazione": the sparse
// attention kernel extends a FlashAttention-style kernel so that it iterates
// only over the tile indices decoded from the bit vectors.  This is an
// MI355X-native design, not the FlashAttention-3 (Hopper) kernel the pages
// build on:
//
//  * one workgroup = one CSR row (q head h, query tile g) = 64 queries, four
//    wavefronts: wave w takes queries 32 (w & 1) .. +31 and, of every listed
//    KV tile, keys 32 (w >> 1) .. +31.  Each wave keeps its own online-softmax
//    state; the two key halves are merged once at the end;
//  * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
//    register staging), double buffered so the next listed tile streams in
//    while the current one is multiplied.  16-byte chunks are XOR-swizzled per
//    row so that the MFMA operand reads below are free of bank conflicts;
//  * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    lane l then holds 16 keys of query (l % 32); the online-softmax state of
//    a query lives in lanes l and l ^ 32;
//  * the output is accumulated transposed, O^T += V^T P^T: the B operand is the
//    lane's own P values, and the V^T operand comes from ds_read_b64_tr_b16
//    (a 16-lane transposing LDS read) on the row-major V tile;
//  * exp2 with log2(e) folded into the scale; the running maximum is raised
//    (and O, l rescaled) only when a tile's maximum exceeds it by more than
//    kLazyLog2 in log2 units, which bounds P by 2^kLazyLog2 and leaves
//    O = sum P V / sum P unchanged; masking is a select, so NaN in padded K
//    never leaks;
//  * P is rounded to bf16 for the PV product and l sums the same rounded
//    values (v_dot2_f32_bf16 against ones);
//  * rows are assigned to workgroups KV-head-major, one contiguous share per
//    XCD, longest rows (latest query tiles) first.
#include <math.h>

#include <algorithm>

#include "sift_internal.hpp"

namespace sift {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef const __attribute__((address_space(4))) int32_t const_i32;

// Uniform read of a table the kernel never writes, through the constant address
// space so it becomes a scalar load (a vector load here would make the wait on it
// also wait for the in-flight K/V prefetch).
__device__ inline int32_t uniform_read(const int32_t *p, int64_t i) {
    return reinterpret_cast<const_i32 *>(reinterpret_cast<uintptr_t>(p))[i];
}

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazyLog2 = 8.0f;
constexpr int kXcds = 8;

__device__ inline bool plan_ok(const PlanView &pv) {
    return pv.header[0] == static_cast<int32_t>(kPlanMagic) &&
           static_cast<uint32_t>(pv.header[2]) == pv.fp_lo &&
           static_cast<uint32_t>(pv.header[3]) == pv.fp_hi && pv.header[6] == pv.num_tiles;
}

template <int D>
struct Cfg {
    static constexpr int CPR = D / 8;                        // 16-byte chunks per K/V row
    static constexpr int TILE = 64 * D;                      // bf16 elements per K or V tile
    static constexpr int RPL = 64 / CPR;                     // rows per 64-lane load
    static constexpr int LOADS = 64 * CPR / (64 * kWaves);   // loads per wave per matrix per tile
    static constexpr int BUF = 2 * TILE;                     // K then V
    static_assert(64 * D * 4 <= BUF * 2, "output staging must fit one buffer");
    static_assert((D / 2) * 2 * 64 * 4 <= BUF * 2, "merge scratch must fit one buffer");
};

// slot of 16-byte chunk c in K row r / V row r
template <int D>
__device__ inline int k_slot(int r, int c) { return c ^ (r & (Cfg<D>::CPR - 1)); }
template <int D>
__device__ inline int v_slot(int r, int c) { return c ^ ((2 * r) & (Cfg<D>::CPR - 1)); }

__device__ inline void wait_vmcnt_le(int n) {
    // s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima)
    if (n >= 8) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8) | ((8 >> 4) << 14));
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// Issue the direct-to-LDS loads of K and V tile t (rows ktok0 .. +63) into buffer `buf`.
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                 int64_t ktok0, int Hkv, int kvh, uint16_t *buf, int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check this builtin
    using C = Cfg<D>;
    const int64_t row_stride = static_cast<int64_t>(Hkv) * D;
    const uint16_t *kg = k + (ktok0 * Hkv + kvh) * D;
    const uint16_t *vg = v + (ktok0 * Hkv + kvh) * D;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
        const int I = wave * C::LOADS + j;  // this load fills LDS elements [512 I, 512 I + 512)
        const int r = I * C::RPL + lane / C::CPR;
        const int s = lane % C::CPR;
        __builtin_amdgcn_global_load_lds(kg + r * row_stride + 8 * k_slot<D>(r, s),
                                         (lds_void *)(buf + 512 * I), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vg + r * row_stride + 8 * v_slot<D>(r, s),
                                         (lds_void *)(buf + C::TILE + 512 * I), 16, 0, 0);
    }
#endif
}

// Online-softmax state of one wavefront (32 queries x one 32-key half of each tile).
template <int D>
struct WaveState {
    bf16x8 qf[D / 16];
    f32x16 acc_o[D / 32];
    float m_run, l_run;
};

// One listed KV tile: wait for its loads, prefetch the next tile into the
// other buffer, then QK^T -> online softmax -> PV from this buffer.
template <int D>
__device__ __forceinline__ void tile_step(WaveState<D> &st, uint16_t *__restrict__ cur,
                                          uint16_t *__restrict__ nxt, int t, int t_next,
                                          bool has_next, const PlanView &pv, const uint16_t *k,
                                          const uint16_t *v, int Hkv, int kvh, int g, int qi,
                                          float scale_log2, float lazy_raw, int wave, int lane) {
    using C = Cfg<D>;
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    const int l32 = lane & 31, hi = lane >> 5, kh = wave >> 1;
    if (has_next) {
        load_tile<D>(k, v, static_cast<int64_t>(t_next < 0 ? 0 : t_next) * kTile, Hkv, kvh, nxt, wave, lane);
        wait_vmcnt_le(2 * C::LOADS);
    } else {
        wait_vmcnt_le(0);
    }
    __builtin_amdgcn_s_barrier();  // tile t is in LDS for every wave

    const int kv_valid = t < 0 ? 0 : uniform_read(pv.tile_valid, t);
    const uint16_t *Kt = cur;
    const uint16_t *Vt = cur + C::TILE;

    // S^T for keys 32 kh .. 32 kh + 31: register i is key 32 kh + 8 (i / 4) + 4 hi + i % 4
    f32x16 s = f32x16{};
    {
        const int R = 32 * kh + l32;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kt + R * D + 8 * k_slot<D>(R, 2 * dc + hi));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qf[dc], s, 0, 0, 0);
        }
    }
    if (kv_valid < kTile || t >= g) {
        const int shift = (t - g) * kTile;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * kh + 8 * (i >> 2) + 4 * hi + (i & 3);
            const bool ok = key < kv_valid && shift + key <= qi;
            s[i] = ok ? s[i] : -INFINITY;
        }
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__ballot(mt > st.m_run + lazy_raw)) {  // wave-uniform: raise the reference max
        const float m_new = fmaxf(st.m_run, mt);
        const float alpha = (st.m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((st.m_run - m_new) * scale_log2);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) st.acc_o[db] *= alpha;
    }
    const float nbias = (st.m_run == -INFINITY) ? 0.0f : -st.m_run * scale_log2;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, nbias));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], scale_log2, nbias));
        const bf16x2 pr = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
        st.l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, st.l_run, false);
        pb[i >> 3][i & 7] = pr[0];
        pb[i >> 3][(i & 7) + 1] = pr[1];
    }
    // O^T += V^T P^T; K-step j covers keys 32 kh + 16 j + {0..3, 8..11} + 4 hi
    {
        const int s16 = lane & 15;
        const int dsub = 16 * ((lane >> 4) & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = 32 * db + dsub + 4 * (s16 & 3);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r0 = 32 * kh + 16 * j + 4 * hi + (s16 >> 2);
                const int r1 = r0 + 8;
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(Vt + r0 * D + 8 * v_slot<D>(r0, col >> 3) + (col & 7)));
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(Vt + r1 * D + 8 * v_slot<D>(r1, col >> 3) + (col & 7)));
                const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, v0),
                                                         __builtin_bit_cast(bf16x4, v1), 0, 1, 2, 3, 4, 5, 6, 7);
                st.acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[j], st.acc_o[db], 0, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_barrier();  // every wave is done with `cur` before it is refilled
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_prefill_kernel(
    PlanView pv, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, float scale, float scale_log2, float lazy_raw,
    float *__restrict__ out, float *__restrict__ lse, int Hq, int Hkv, int rows_per_xcd) {
    using C = Cfg<D>;
    constexpr int DC = D / 16;
    constexpr int DB = D / 32;
    // two separate buffers, so that each LDS read has one known underlying object
    __shared__ __attribute__((aligned(16))) uint16_t buf0[C::BUF];
    __shared__ __attribute__((aligned(16))) uint16_t buf1[C::BUF];

    if (!plan_ok(pv)) return;
    const int G = pv.num_tiles;
    const int nrows = Hq * G;
    // workgroup -> row: XCD x (= blockIdx % 8) owns a contiguous share of the
    // KV-head-major, latest-tile-first row order
    const int idx = (blockIdx.x % kXcds) * rows_per_xcd + blockIdx.x / kXcds;
    if (idx >= nrows) return;
    const int group = Hq / Hkv;
    const int kvh = idx / (G * group);
    const int rem = idx % (G * group);
    const int g = G - 1 - rem / group;
    const int h = kvh * group + rem % group;
    const int64_t row = static_cast<int64_t>(h) * G + g;
    const int64_t N = static_cast<int64_t>(G) * kTile;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int qh = wave & 1, kh = wave >> 1;
    const int qi = 32 * qh + l32;  // this lane's query in the tile
    const int q_valid = uniform_read(pv.tile_valid, g);
    const int64_t tok0 = static_cast<int64_t>(g) * kTile;

    WaveState<D> st;
    {
        const uint16_t *qrow = q + ((tok0 + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) st.qf[dc] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * dc);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc_o[db] = f32x16{};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    const int e0 = uniform_read(row_ptr, row), e1 = uniform_read(row_ptr, row + 1);
    auto tile_at = [&](int e) {
        if (e >= e1) return -1;
        const int t = uniform_read(col_idx, e);
        return (t >= 0 && t < G) ? t : -1;  // -1: loads tile 0 and masks every key
    };
    int t_cur = tile_at(e0);
    if (e0 < e1)
        load_tile<D>(k, v, static_cast<int64_t>(t_cur < 0 ? 0 : t_cur) * kTile, Hkv, kvh, buf0, wave, lane);
    for (int e = e0; e < e1; e += 2) {
        int t_next = tile_at(e + 1);
        tile_step<D>(st, buf0, buf1, t_cur, t_next, e + 1 < e1, pv, k, v, Hkv, kvh, g, qi, scale_log2,
                     lazy_raw, wave, lane);
        if (e + 1 >= e1) break;
        t_cur = t_next;
        t_next = tile_at(e + 2);
        tile_step<D>(st, buf1, buf0, t_cur, t_next, e + 2 < e1, pv, k, v, Hkv, kvh, g, qi, scale_log2,
                     lazy_raw, wave, lane);
        t_cur = t_next;
    }

    // merge the two key halves: waves with kh = 1 publish, waves with kh = 0 combine
    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
    float *X = reinterpret_cast<float *>(buf0);   // [D/2 registers][2 query halves][64 lanes]
    float *ML = reinterpret_cast<float *>(buf1);  // [2 query halves][32 queries][m, l]
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) X[((db * 16 + i) * 2 + qh) * 64 + lane] = st.acc_o[db][i];
        if (hi == 0) {
            ML[(qh * 32 + l32) * 2 + 0] = st.m_run;
            ML[(qh * 32 + l32) * 2 + 1] = l_tot;
        }
    }
    __syncthreads();
    float m_fin = -INFINITY, l_fin = 0.0f;
    if (kh == 0) {
        const float m1 = ML[(qh * 32 + l32) * 2 + 0];
        const float l1 = ML[(qh * 32 + l32) * 2 + 1];
        m_fin = fmaxf(st.m_run, m1);
        const float a0 = (st.m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((st.m_run - m_fin) * scale_log2);
        const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m1 - m_fin) * scale_log2);
        l_fin = l_tot * a0 + l1 * a1;
        const float inv = l_fin > 0.0f ? 1.0f / l_fin : 0.0f;
        const float w0 = a0 * inv, w1 = a1 * inv;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                st.acc_o[db][i] = st.acc_o[db][i] * w0 + X[((db * 16 + i) * 2 + qh) * 64 + lane] * w1;
    }
    __syncthreads();
    // output tile staged in buf0 as [64 rows][D/4 float4 chunks], chunk c of row r at c ^ (r % 32)
    float *Os = reinterpret_cast<float *>(buf0);
    constexpr int C4 = D / 4;
    if (kh == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 o4 = {st.acc_o[db][4 * i4 + 0], st.acc_o[db][4 * i4 + 1],
                                  st.acc_o[db][4 * i4 + 2], st.acc_o[db][4 * i4 + 3]};
                const int c4 = 8 * db + 2 * i4 + hi;
                *reinterpret_cast<f32x4 *>(Os + qi * D + 4 * (c4 ^ (qi & (C4 - 1)))) = o4;
            }
        if (lse != nullptr && hi == 0) {
            const bool live = qi < q_valid && l_fin > 0.0f;
            lse[static_cast<int64_t>(h) * N + tok0 + qi] = live ? m_fin * scale + logf(l_fin) : -INFINITY;
        }
    }
    __syncthreads();
    for (int x = tid; x < 64 * C4; x += kThreads) {
        const int r = x / C4, c4 = x % C4;
        f32x4 val = *reinterpret_cast<const f32x4 *>(Os + r * D + 4 * (c4 ^ (r & (C4 - 1))));
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
    const float lazy_raw = kLazyLog2 / scale_log2;
    const int rows_per_xcd = static_cast<int>((rows + kXcds - 1) / kXcds);
    const unsigned grid = static_cast<unsigned>(rows_per_xcd) * kXcds;
    if (hl.D == 128)
        sparse_prefill_kernel<128><<<grid, kThreads, 0, stream>>>(
            pv, q, k, v, row_ptr, col_idx, scale, scale_log2, lazy_raw, out, lse, hl.Hq, hl.Hkv,
            rows_per_xcd);
    else
        sparse_prefill_kernel<64><<<grid, kThreads, 0, stream>>>(
            pv, q, k, v, row_ptr, col_idx, scale, scale_log2, lazy_raw, out, lse, hl.Hq, hl.Hkv,
            rows_per_xcd);
    return hipGetLastError();
}

}  // namespace sift
