// Block-sparse causal GQA attention over decoded CSR rows (gfx950).
//
// SIFT technical summary, section 2, "Dettagli di Implementazione": the sparse
// attention kernel extends a FlashAttention-style kernel so that it iterates
// only over the tile indices decoded from the bit vectors.  This is an
// MI355X-native design, not the FlashAttention-3 (Hopper) kernel the pages
// build on:
//
//  * a CSR row (q head h, query tile g) = 64 queries is handled by one workgroup
//    of four wavefronts: wave w takes queries 32 (w & 1) .. +31 and, of every
//    listed KV tile, keys 32 (w >> 1) .. +31.  Each wave keeps its own
//    online-softmax state; the two key halves are merged once at the end;
//  * V arrives as V^T ([kv head][D][N], bf16), written by transpose_v_kernel
//    (prepare_kernels.hip) before this kernel, with the tokens of every
//    16-token group stored in the order the PV operands consume them, so
//    that every MFMA operand -- K for the scores, V^T for the output -- is one
//    16-byte LDS read per lane;
//  * K and V^T tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds:
//    the tile's base address in a scalar buffer descriptor, a 32-bit offset per
//    lane, no register staging), double buffered so the next listed tile streams in
//    while the current one is multiplied.  K rows are padded by 16 bytes and
//    V^T 16-byte chunks are XOR-swizzled per row, so the operand reads are free
//    of bank conflicts and K's need a single address register;
//  * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    lane l then holds 16 keys of query (l % 32); the online-softmax state of
//    a query lives in lanes l and l ^ 32; the output is accumulated
//    transposed, O^T += V^T P^T, whose B operand is the lane's own P values;
//  * one pipeline step issues all operand reads of the step first, then the
//    score MFMAs of the next tile interleaved (pinned with scheduling
//    barriers) with the exponentials of the current tile, then the output
//    MFMAs of the current tile interleaved with the max tree of the next; the
//    VALU work left after the last MFMA runs at a raised wave priority;
//  * exp2 with log2(e) folded into the scale; the running maximum is raised
//    (and O, l rescaled) only when a tile's maximum exceeds it by more than
//    kLazyLog2 in log2 units, which bounds P by 2^kLazyLog2 and leaves
//    O = sum P V / sum P unchanged; masking is a select, so NaN in padded K
//    never leaks;
//  * P is rounded to bf16 for the PV product and l sums the same rounded
//    values (v_dot2_f32_bf16 against ones);
//  * the kernel is persistent (two workgroups per CU): each workgroup claims
//    rows with an atomic counter from its XCD's queue over the KV-head-major
//    row order (longest rows, i.e. latest query tiles, first), and helps the
//    other XCDs' queues once its own is exhausted; the next row's claim,
//    metadata, Q and first K/V^T tiles are fetched while the current row runs.
#include <math.h>

#include <algorithm>

#include "sift_internal.hpp"

namespace sift {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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
static_assert(kXcds == kPrefillQueues, "one row queue per XCD");
constexpr int kPersistentPerXcd = 64;  // 2 workgroups on each of the 32 CUs of an XCD


template <int D>
struct Cfg {
    static constexpr int CPR = D / 8;                   // 16-byte chunks per K row
    static constexpr int KROW = 2 * D + 16;             // LDS bytes per K row (16 bytes of padding)
    static constexpr int KBYTES = 64 * KROW;            // LDS bytes per K tile
    static constexpr int KLOADS = KBYTES / 1024;        // 1 KB loads per K tile (17 or 9)
    static constexpr int KLOADS_W = (KLOADS + kWaves - 1) / kWaves;  // per wave, at most
    static constexpr int VBYTES = 128 * D;              // LDS bytes per V^T tile (D rows x 64 tokens)
    static constexpr int VLOADS_W = VBYTES / 1024 / kWaves;  // 1 KB loads per wave per V^T tile
    static constexpr int DC = D / 16;                   // MFMA K-steps of the scores
    static constexpr int DB = D / 32;                   // 32-row blocks of O^T
    static_assert(KBYTES % 1024 == 0 && VBYTES % (1024 * kWaves) == 0, "whole 1 KB loads");
    static_assert(32 * D * 4 <= KBYTES, "32 fp32 output rows fit one K buffer");
};
// slot of 16-byte chunk c in V^T row d (64 tokens = 8 chunks per row): the 16 lanes of one
// LDS cycle read rows d0 .. d0 + 15 at one chunk; (d & 1, (d >> 1) & 7) is distinct over them
__device__ inline int vt_slot(int d, int c) { return c ^ ((d >> 1) & 7); }

__device__ inline void wait_vmcnt_le(int n) {
    // s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima)
    if (n >= 8) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8) | ((8 >> 4) << 14));
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// Per-lane byte offsets of this lane's direct-to-LDS loads inside a K tile and a V^T tile
// (the same for every tile; the tile itself only moves a uniform base pointer).  A load
// writes lane i's 16 bytes at LDS offset 16 i of its 1 KB destination, so the layout is
// applied on the global side: lane i fetches the chunk that belongs at that LDS position.
// Wave w issues K loads w, w + 4, ...; a lane whose position is a K row's padding fetches
// chunk 0 of that row again (never read).
template <int D>
struct LoadOffsets {
    uint32_t k[Cfg<D>::KLOADS_W];
    uint32_t v[2];  // loads j and j + 2 of a V^T tile differ by 2048 bytes
};

template <int D>
__device__ inline LoadOffsets<D> make_load_offsets(int Hkv, int64_t N, int wave, int lane) {
    using C = Cfg<D>;
    LoadOffsets<D> o;
    const uint32_t krow_bytes = static_cast<uint32_t>(Hkv) * D * 2;
    constexpr uint32_t vrow_bytes = kTile * 2;  // V^T rows of one tile are contiguous
#pragma unroll
    for (int j = 0; j < C::KLOADS_W; ++j) {
        const int b = 1024 * (wave + kWaves * j) + 16 * lane;  // LDS byte this lane fills
        const int r = b / C::KROW, c = (b % C::KROW) / 16;
        o.k[j] = r * krow_bytes + 16u * static_cast<uint32_t>(c < C::CPR ? c : 0);
    }
    static_assert(C::VLOADS_W % 2 == 0, "V^T loads come in pairs");
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int I = wave * C::VLOADS_W + j;  // this load fills V^T tile bytes [1024 I, 1024 I + 1024)
        const int d = I * 8 + lane / 8;
        o.v[j] = d * vrow_bytes + 16u * static_cast<uint32_t>(vt_slot(d, lane % 8));
    }
    return o;
}

// The tile loads are buffer loads into LDS: the tile's (uniform) base address sits in the buffer
// descriptor (scalar registers), each lane supplies only its 32-bit offset, so no per-load vector
// address arithmetic is needed.  Word 3 of the descriptor is the gfx9 raw-buffer default.
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check these builtins
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, 0x7FFFFFFF, 0x00020000);
}
#endif

// Direct-to-LDS load of one K tile (base = the tile's first token row of this kv head).
template <int D>
__device__ __forceinline__ void load_k_tile(const uint16_t *base, char *dst, int wave, const uint32_t *off) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg<D>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base);  // uniform
#pragma unroll
    for (int j = 0; j < C::KLOADS_W; ++j)
        if (wave + kWaves * j < C::KLOADS)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + 1024 * (wave + kWaves * j)), 16,
                                                     static_cast<int>(off[j]), 0, 0, 0);
#endif
}

// Direct-to-LDS load of one V^T tile (base = row d = 0 of this kv head at the tile's first token).
// Loads j and j + 2 cover rows 16 apart: same swizzle, 2048 bytes further on both sides, which is
// the instruction's immediate offset (added to the global and to the LDS address alike).
template <int D>
__device__ __forceinline__ void load_vt_tile(const uint16_t *base, char *dst, int wave, const uint32_t *off) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg<D>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(base);  // uniform
    static_assert(C::VLOADS_W == 2 || C::VLOADS_W == 4, "two or four V^T loads per wave");
    char *d0 = dst + 1024 * wave * C::VLOADS_W;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)d0, 16, static_cast<int>(off[0]), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(d0 + 1024), 16, static_cast<int>(off[1]), 0, 0, 0);
    if constexpr (C::VLOADS_W == 4) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)d0, 16, static_cast<int>(off[0]), 0, 2048, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(d0 + 1024), 16, static_cast<int>(off[1]), 0, 2048, 0);
    }
#endif
}

__device__ inline float pair_max(float x) {  // max over lanes l and l ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float pair_sum(float x) {  // sum over lanes l and l ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max of three (v_maximum3_f32).  Plain code, not inline asm: the inputs are MFMA results, and
// only the compiler's hazard tracking inserts the wait states a VALU read of an MFMA result needs.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Online-softmax state of one wavefront (32 queries x one 32-key half of each tile).
template <int D>
struct WaveState {
    bf16x8 qf[D / 16];
    f32x16 acc_o[D / 32];
    float m_run, l_run;
    float thr;  // m_run + the lazy margin (raw score units): a raise is due when a score exceeds it
};

// Per-row constants a pipeline step needs.
struct RowCtx {
    const uint16_t *k, *vt;
    int64_t N;
    int Hkv, kvh, g, qi, wave, lane;
    float scale_log2, lazy_raw;
};

template <int D>
__device__ __forceinline__ const uint16_t *k_tile_base(const RowCtx &c, int t) {
    return c.k + (static_cast<int64_t>(t < 0 ? 0 : t) * kTile * c.Hkv + c.kvh) * D;
}
template <int D>
__device__ __forceinline__ const uint16_t *vt_tile_base(const RowCtx &c, int t) {
    // V^T is stored tile by tile: [Hkv][G][D][64], each tile one contiguous D x 128-byte block
    return c.vt + (static_cast<int64_t>(c.kvh) * (c.N / kTile) + (t < 0 ? 0 : t)) * D * kTile;
}

// Operand reads of one step: K(e+1) rows for the scores, V^T(e) rows for the output.
// Score register i is key 32 kh + 8 (i / 4) + 4 hi + i % 4 of the tile, for query qi.
template <int D>
__device__ __forceinline__ void read_k(bf16x8 (&kf)[D / 16], const char *Kt, const RowCtx &c) {
    const int hi = c.lane >> 5, R = 32 * (c.wave >> 1) + (c.lane & 31);
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
        kf[dc] = *reinterpret_cast<const bf16x8 *>(Kt + R * Cfg<D>::KROW + 16 * (2 * dc + hi));
}
// A operand of PV K-step j of block db: V^T row 32 db + l32, stored tokens 32 kh + 16 j + 8 hi .. +7
template <int D>
__device__ __forceinline__ void read_vt(bf16x8 (&vf)[D / 16], const char *Vt, const RowCtx &c) {
    const int hi = c.lane >> 5, kh = c.wave >> 1, l32 = c.lane & 31;
#pragma unroll
    for (int q = 0; q < D / 16; ++q) {
        const int d = 32 * (q >> 1) + l32, ch = 4 * kh + 2 * (q & 1) + hi;
        vf[q] = *reinterpret_cast<const bf16x8 *>(Vt + d * 128 + 16 * vt_slot(d, ch));
    }
}

__device__ __forceinline__ bool needs_mask(int t, int kv_valid, const RowCtx &c) {
    return kv_valid < kTile || t >= c.g;
}

// Causal mask on the diagonal tile and padding mask on a partial tile (a select,
// so NaN in padded K slots never leaks); t < 0 marks a skipped entry (kv_valid 0).
__device__ __forceinline__ void apply_mask(f32x16 &s, int t, int kv_valid, const RowCtx &c) {
    const int hi = c.lane >> 5, kh = c.wave >> 1;
    const int lim = min(kv_valid, c.qi - (t - c.g) * kTile + 1);  // keys < lim survive
    // key of register i = 32 kh + 4 hi + (8 (i / 4) + i % 4): compare the constant part with the
    // limit less the lane's part
    const int lk = lim - 32 * kh - 4 * hi;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 8 * (i >> 2) + (i & 3) < lk ? s[i] : -INFINITY;
}

// Raise the reference max when a score of the tile exceeds it by more than kLazyLog2 (decided
// wave-uniformly from each lane's own 16 scores: the two lanes of a query share m_run, so some
// lane of the wave exceeds thr exactly when the query's tile max does), rescaling O and l, and
// update the exp2 bias nbias = -m * scale_log2.  Only a raise needs the query's tile max.
template <int D>
__device__ __forceinline__ void lazy_raise(WaveState<D> &st, float lmax, float &nbias, const RowCtx &c) {
    if (__ballot(lmax > st.thr) != 0) {
        const float m_new = fmaxf(st.m_run, pair_max(lmax));
        // m_run = -inf gives exp2(-inf) = 0; both -inf leaves alpha = 1 (O and l are still 0)
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f((st.m_run - m_new) * c.scale_log2);
        st.m_run = m_new;
        st.thr = m_new + c.lazy_raw;
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.acc_o[db] *= alpha;
        nbias = (m_new == -INFINITY) ? 0.0f : -m_new * c.scale_log2;
    }
}

// The row's first tile: the reference max is set from it without a rescale (O and l are still 0).
// Same state as lazy_raise from m = -inf.
template <int D>
__device__ __forceinline__ void first_max(WaveState<D> &st, float lmax, float &nbias, const RowCtx &c) {
    const float m = fmaxf(-INFINITY, pair_max(lmax));  // -inf when the tile is all masked (or NaN)
    st.m_run = m;
    st.thr = m + c.lazy_raw;
    nbias = (m == -INFINITY) ? 0.0f : -m * c.scale_log2;
}

// max of the lane's 16 scores
__device__ __forceinline__ float lane_max(const f32x16 &s) {
    const float a = max3f(s[0], s[1], s[2]), b = max3f(s[3], s[4], s[5]), d = max3f(s[6], s[7], s[8]);
    const float e = max3f(a, s[9], s[10]), f = max3f(b, s[11], s[12]), h = max3f(d, s[13], s[14]);
    return max3f(e, f, max3f(h, s[15], s[15]));
}

// Scores of one K tile (used once per row, for the first listed tile).
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const WaveState<D> &st, const char *Kt, const RowCtx &c) {
    bf16x8 kf[D / 16];
    read_k<D>(kf, Kt, c);
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dc], st.qf[dc], s, 0, 0, 0);
    return s;
}

// P = exp2(s * scale_log2 + nbias) rounded to bf16, l += sum of the rounded P, then
// O += V^T P^T (used once per row, for the last listed tile).
template <int D>
__device__ __forceinline__ void exp_pv_tile(WaveState<D> &st, const f32x16 &s, float nbias, const char *Vt,
                                            const RowCtx &c) {
    bf16x8 vf[D / 16];
    read_vt<D>(vf, Vt, c);
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    bf16x8 pb[2];
    float l = st.l_run;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], c.scale_log2, nbias));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c.scale_log2, nbias));
        const bf16x2 pr = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
        l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        pb[i >> 3][i & 7] = pr[0];
        pb[i >> 3][(i & 7) + 1] = pr[1];
    }
    st.l_run = l;
#pragma unroll
    for (int q = 0; q < D / 16; ++q)
        st.acc_o[q >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[q], pb[q & 1], st.acc_o[q >> 1], 0, 0, 0);
}

// The V^T operands of one parity of PV K-steps, q = PAR, PAR + 2, ... (A operand of block q / 2,
// K-step q % 2), in the layout of read_vt
template <int D, int PAR>
__device__ __forceinline__ void read_vt_parity(bf16x8 (&vf)[D / 16], const char *Vt, const RowCtx &c) {
    const int hi = c.lane >> 5, kh = c.wave >> 1, l32 = c.lane & 31;
#pragma unroll
    for (int q = PAR; q < D / 16; q += 2) {
        const int d = 32 * (q >> 1) + l32, ch = 4 * kh + 2 * (q & 1) + hi;
        vf[q] = *reinterpret_cast<const bf16x8 *>(Vt + d * 128 + 16 * vt_slot(d, ch));
    }
}

// The compute of one pipeline step for listed tile e, whose scores s_cur are formed, masked and
// prepped (nbias): reads K(e+1) and V^T(e), forms S(e+1) -> s_nxt (masked), computes
// P(e) = exp2(...) and O += V^T(e) P(e)^T, and runs the lazy raise for S(e+1) (updates nbias).
// Only a wave's own VALU work overlaps its MFMAs (the MFMAs of one wave and the VALU work of
// another on the same SIMD do not co-execute), so the VALU work is spread over all MFMAs:
//   score MFMAs of S(e+1)      <- exponentials of P(e) pairs 0..3, V^T operand reads;
//   PV MFMAs of P pairs 0..3   <- exponentials of pairs 4..7;
//   PV MFMAs of P pairs 4..7   <- max tree of S(e+1).
// A pair's fma and exponentials are issued one slot ahead of its rounding, so no VALU op waits on
// the one before it.
template <int D>
__device__ __forceinline__ void step_compute(WaveState<D> &st, const f32x16 &s_cur, f32x16 &s_nxt, float &nbias,
                                             const char *Kt, const char *Vt, int t_next, int v_next,
                                             const RowCtx &c) {
    constexpr int DC = D / 16;
    constexpr int SPP = DC / 4;  // score MFMAs ahead of each of pairs 0..3
    bf16x8 kf[DC], vf[DC];
    read_k<D>(kf, Kt, c);
    __builtin_amdgcn_sched_barrier(0);
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    f32x16 s = f32x16{};
    bf16x8 pb[2];
    float l = st.l_run;
    float x0 = fmaf(s_cur[0], c.scale_log2, nbias), x1 = fmaf(s_cur[1], c.scale_log2, nbias);
    auto round_pair = [&](int k, float a, float b) {
        const bf16x2 pr = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
        l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
        pb[k >> 2][(2 * k) & 7] = pr[0];
        pb[k >> 2][((2 * k) & 7) + 1] = pr[1];
    };
    // l += the rounded pair k (the l sums run in pair order, so l is the same sum whatever the
    // MFMA placement)
    auto sum_pair = [&](int k) {
        const bf16x2 pr = {pb[k >> 2][(2 * k) & 7], pb[k >> 2][((2 * k) & 7) + 1]};
        l = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l, false);
    };
    float p0 = 0.0f, p1 = 0.0f;  // exponentials of the last pair computed, not yet rounded
    // exponentials of pair k, the fma of pair k + 1, and pair k - 1 rounded into pb; pair 3 is
    // rounded on its own, ahead of the PV MFMAs that read it, so pair 4 does not round it again
    auto next_pair = [&](int k) {
        const float n0 = __builtin_amdgcn_exp2f(x0), n1 = __builtin_amdgcn_exp2f(x1);
        if (k < 7) {
            x0 = fmaf(s_cur[2 * k + 2], c.scale_log2, nbias);
            x1 = fmaf(s_cur[2 * k + 3], c.scale_log2, nbias);
        }
        if (k > 0 && k != 4) round_pair(k - 1, p0, p1);
        p0 = n0;
        p1 = n1;
    };
    // score region: S(e+1), with pairs 0..3 of P(e) and the V^T operand reads behind it
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int m = 0; m < SPP; ++m) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k * SPP + m], st.qf[k * SPP + m], s, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        next_pair(k);
        // V^T operands into the registers the consumed K operands free
        if (k == 1) read_vt_parity<D, 0>(vf, Vt, c);
        if (k == 2) read_vt_parity<D, 1>(vf, Vt, c);
        __builtin_amdgcn_sched_barrier(0);
    }
    round_pair(3, p0, p1);  // pb[0] complete
    __builtin_amdgcn_sched_barrier(0);
    // PV of pairs 0..3 (pb[0]: the even K-steps), with the exponentials of pairs 4..7 behind it
#pragma unroll
    for (int k = 4; k < 8; ++k) {
        const int qi = (k - 4) * (DC / 2) / 4;  // the even-q MFMA issued at this slot, if any
        if (((k - 4) * (DC / 2)) % 4 == 0) {
            st.acc_o[qi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * qi], pb[0], st.acc_o[qi], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        next_pair(k);
        __builtin_amdgcn_sched_barrier(0);
    }
    round_pair(7, p0, p1);  // pb[1] complete
    __builtin_amdgcn_sched_barrier(0);
    // PV of pairs 4..7 (pb[1]: the odd K-steps), with the l sums of all eight pairs and the max
    // tree of S(e+1) behind it (no branch inside this region: a branch would let the
    // exponentials above sink past the barriers)
    float m0 = 0.0f, m1 = 0.0f, m2 = 0.0f;
#pragma unroll
    for (int j = 0; j < DC / 2; ++j) {
        st.acc_o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * j + 1], pb[1], st.acc_o[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 6; ++x) {
            if ((x * (DC / 2)) / 6 != j) continue;
            if (x == 0) m0 = max3f(s[0], s[1], s[2]);
            if (x == 1) m1 = max3f(s[3], s[4], s[5]);
            if (x == 2) m2 = max3f(s[6], s[7], s[8]);
            if (x == 3) m0 = max3f(m0, s[9], s[10]);
            if (x == 4) m1 = max3f(m1, s[11], s[12]);
            if (x == 5) m2 = max3f(m2, s[13], s[14]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // The rest of the step is VALU work with no MFMA of this wave to hide behind (the l sums the
    // compiler sinks here, the mask and the raise check): it runs at a raised wave priority, so
    // that the other wave's issue does not stretch it (0.5-1.8 % less time on the five workloads)
    __builtin_amdgcn_s_setprio(2);
    float mt = max3f(m0, m1, max3f(m2, s[15], s[15]));
    // both results taken here, ahead of the mask branch: otherwise the compiler sinks the l sums
    // (rebuilding packed words whose registers it reused) and merges this max tree with the
    // masked one, out of the MFMA region
    asm volatile("" : "+v"(mt));
    st.l_run = l;
    if (needs_mask(t_next, v_next, c)) {  // diagonal or partial tile: mask, then max again
        apply_mask(s, t_next, v_next, c);
        mt = lane_max(s);
    }
    lazy_raise<D>(st, mt, nbias, c);
    s_nxt = s;
    asm volatile("" : "+v"(st.l_run));  // the l sums are done before the priority drops
    __builtin_amdgcn_s_setprio(0);
}

// The row's listed tiles, 64 entries per chunk held across the lanes of one register
// (lane j of chunk c: entry 64 c + j packed as tile id | (valid tokens - 1) << 25, or -1
// for a skipped entry), read with v_readlane.  Vector loads keep these reads out of the
// scalar/LDS counter, so no per-tile scalar-load latency sits on the critical path.  Chunk
// c + 1 is fetched as raw tile ids when entry 64 c is reached and packed with its valid
// counts one step later, so neither load is waited for where it is issued.
struct TileList {
    int c0, c1;  // chunks c and c + 1
    int c;
    bool raw1;   // c1 still holds raw ids
};

// Marks a list position past the row's last entry (no CSR value can be it: they are checked
// against [0, G) and G < 2^25).
constexpr int kNoEntry = INT32_MIN;

// raw tile ids of entries [base, base + 64) of a row starting at CSR offset e0 with n entries
// (kNoEntry past the end); no use of the loaded value here, so nothing waits for it
__device__ __forceinline__ int load_ids(int base, int n, int e0, const int32_t *__restrict__ col_idx, int lane) {
    const int j = base + lane;
    return j < n ? col_idx[e0 + j] : kNoEntry;
}

// out-of-range entries (and kNoEntry) are skipped (masked)
__device__ __forceinline__ int valid_id(int x, int G) { return (x >= 0 && x < G) ? x : -1; }

// Raise flag bits in the call's status word, once per wavefront (`raise` is per lane).
__device__ __forceinline__ void flag_status(bool raise, int flags, int *__restrict__ status) {
    const uint64_t m = __ballot(raise);
    if (m != 0 && (threadIdx.x & 63) == __builtin_ctzll(m)) atomicOr(status, flags);
}

// a raw tile id packed with its valid-token count (1..64); a listed id outside [0, G) is skipped
// and flagged in the status word
__device__ __forceinline__ int with_valid(int x, int G, const int32_t *__restrict__ tile_valid, int *status) {
    flag_status(x != kNoEntry && (x < 0 || x >= G), SIFT_DEVICE_TILE_RANGE, status);
    x = valid_id(x, G);
    return x >= 0 ? (x | ((tile_valid[x] - 1) << 25)) : -1;
}

// Entry i (uniform; c <= i / 64 <= c + 1): tile id (-1: skipped) and valid count (0: skipped).
__device__ __forceinline__ void list_entry(const TileList &L, int i, int &t, int &valid) {
    const int p = __builtin_amdgcn_readlane((i >> 6) == L.c ? L.c0 : L.c1, i & 63);
    t = p < 0 ? -1 : (p & 0x1FFFFFF);
    valid = p < 0 ? 0 : (p >> 25) + 1;
}

// A row's list in the CSR: its entries are col_idx[e0 .. e0 + n).
struct RowMeta {
    int n;   // entries
    int e0;  // the row's first entry in col_idx
};

// The word a row's metadata is read from: lanes 0, 1 get row_ptr[row], row_ptr[row + 1].
__device__ __forceinline__ int meta_word(int64_t row, const int32_t *__restrict__ row_ptr, int lane) {
    return row_ptr[row + (lane & 1)];
}

__device__ __forceinline__ RowMeta meta_of(int w) {
    RowMeta m;
    m.e0 = __builtin_amdgcn_readlane(w, 0);
    m.n = __builtin_amdgcn_readlane(w, 1) - m.e0;
    return m;
}

// A row whose [row_ptr[r], row_ptr[r + 1]) is not inside [0, col_entries] is read as empty and
// flagged in the status word, so no entry outside the caller's col_idx is read.
__device__ __forceinline__ int checked_meta(int w, int64_t col_entries, int *status) {
    const int e0 = __builtin_amdgcn_readlane(w, 0), e1 = __builtin_amdgcn_readlane(w, 1);
    const bool ok = e0 >= 0 && e1 >= e0 && static_cast<int64_t>(e1) <= col_entries;  // uniform
    if (!ok && (threadIdx.x & 63) == 0) atomicOr(status, SIFT_DEVICE_ROW_RANGE);
    return ok ? w : 0;
}

__device__ __forceinline__ void advance_chunk(TileList &L, int i, int mw, int G, const int32_t *__restrict__ col_idx,
                                              const int32_t *__restrict__ tile_valid, int lane, int *status) {
    if ((i >> 6) != L.c) {  // entry i entered chunk c + 1: shift, fetch chunk c + 2's ids
        L.c += 1;
        L.c0 = L.c1;
        const RowMeta m = meta_of(mw);
        L.c1 = load_ids(64 * (L.c + 1), m.n, m.e0, col_idx, lane);
        L.raw1 = true;
    } else if (L.raw1) {  // one step later: their valid counts
        L.c1 = with_valid(L.c1, G, tile_valid, status);
        L.raw1 = false;
    }
}

// A zero the compiler cannot see through: per-row values derived from it are recomputed for
// every row instead of being kept live (in registers) across the output merge.
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

// Workgroup barrier that orders LDS accesses only: in-flight global loads and stores stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A CSR row: q head h, query tile g, read KV head kvh; rows are numbered KV-head-major,
// latest query tile first.
struct RowId {
    int kvh, g, h;
};
__device__ __forceinline__ RowId row_of(int idx, int G, int group) {
    const int kvh = idx / (G * group), rem = idx % (G * group);
    return RowId{kvh, G - 1 - rem / group, kvh * group + rem % group};
}

template <int D>
__device__ __forceinline__ void load_q(WaveState<D> &st, const uint16_t *__restrict__ q, const RowId &r, int Hq,
                                       int qi, int hi) {
    const uint16_t *qrow = q + ((static_cast<int64_t>(r.g) * kTile + qi) * Hq + r.h) * D + 8 * hi;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)  // read once: stream it past L2 (keep L2 for K/V tiles)
        st.qf[dc] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(qrow + 16 * dc));
}

// Row queues, one per XCD, over the KV-head-major row order, so that the workgroups of one
// XCD (one L2) work on one KV head at a time:
//   mode 0 (Hkv divides 8): the 8 / Hkv XCDs of a KV head take its rows interleaved;
//   mode 1 (8 divides Hkv): XCD x takes KV heads x, x + 8, ... in turn;
//   mode 2 (otherwise): XCD x takes the x-th contiguous eighth of the order.
// Within a KV head rows run latest query tile first, i.e. longest rows first.
struct Queues {
    int mode, xpk, Rh, rpx, nrows, Hkv;
};

__device__ inline int queue_len(const Queues &Q, int x) {
    if (Q.mode == 0) {
        const int sub = x % Q.xpk;
        return Q.Rh > sub ? (Q.Rh - sub + Q.xpk - 1) / Q.xpk : 0;
    }
    if (Q.mode == 1) return (Q.Hkv / kXcds) * Q.Rh;
    const int b = x * Q.rpx;
    return max(0, min(Q.nrows, b + Q.rpx) - b);
}

__device__ inline int queue_row(const Queues &Q, int x, int pos) {
    if (Q.mode == 0) return (x / Q.xpk) * Q.Rh + x % Q.xpk + pos * Q.xpk;
    if (Q.mode == 1) return (x + kXcds * (pos / Q.Rh)) * Q.Rh + pos % Q.Rh;
    return x * Q.rpx + pos;
}

// Resolve a claimed position of queue q % 8 into a row; when that queue is exhausted, claim
// from the following queues in turn (a workgroup whose own XCD is done helps the others).
// Returns -1 once all eight are exhausted.  One lane runs it.
__device__ inline int resolve_claim(int *__restrict__ counters, const Queues &Q, int &q, int home, int pos) {
    while (true) {
        if (pos < queue_len(Q, q % kXcds)) return queue_row(Q, q % kXcds, pos);
        if (++q >= home + kXcds) return -1;
        pos = atomicAdd(&counters[q % kXcds], 1);
    }
}

// Output merge of the two key halves.  Register i of acc_o[db] holds O^T row (dim)
// 32 db + 8 (i / 4) + 4 hi + i % 4 of query qi: four consecutive dims per register quad.
// publish_half: blocks [B HB, B HB + HB) as float4 quads, lane-contiguous in LDS.
template <int D, int B>
__device__ __forceinline__ void publish_half(const WaveState<D> &st, f32x4 *dst, int lane) {
    constexpr int HB = D / 64;
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x16 &o = st.acc_o[B * HB + j];
            dst[(j * 4 + a) * 64 + lane] = f32x4{o[4 * a], o[4 * a + 1], o[4 * a + 2], o[4 * a + 3]};
        }
}

// finish_half: blocks [B HB, B HB + HB) = own * w0 + partner's * w1, stored to the query's O row
// (zeros for a padded query), 16 bytes per lane.
template <int D, int B>
__device__ __forceinline__ void finish_half(const WaveState<D> &st, const f32x4 *theirs, float *orow, float w0,
                                            float w1, bool live, int lane, int hi) {
    constexpr int HB = D / 64;
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x16 &o = st.acc_o[B * HB + j];
            const f32x4 t = theirs[(j * 4 + a) * 64 + lane];
            f32x4 r = {o[4 * a] * w0 + t[0] * w1, o[4 * a + 1] * w0 + t[1] * w1,
                       o[4 * a + 2] * w0 + t[2] * w1, o[4 * a + 3] * w0 + t[3] * w1};
            if (!live) r = f32x4{};
            *reinterpret_cast<f32x4 *>(orow + 32 * (B * HB + j) + 8 * a + 4 * hi) = r;
        }
}

// Persistent, two workgroups per CU.  Workgroup b runs on XCD b % 8 and claims rows from that
// XCD's queue with an atomic counter (zeroed by the V transpose that precedes this kernel),
// so rows are balanced dynamically, longest first.  Row r + 1 is claimed when row r starts and
// known to every wave by row r's first barrier; its CSR offsets load during row r's first
// tile, its tile ids during the second, its Q during the last, and its first K and V^T tiles
// stream in while row r's two key halves are merged and stored.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_prefill_kernel(
    PlanView pv, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ vt, const int32_t *__restrict__ row_ptr,
    const int32_t *__restrict__ col_idx, int64_t col_entries, float scale,
    float scale_log2, float lazy_raw, float *__restrict__ out, float *__restrict__ lse, int Hq, int Hkv, Queues Qs,
    int *__restrict__ counters) {
    using C = Cfg<D>;
    constexpr int DB = D / 32;
    constexpr int HB = DB / 2;  // output blocks each key half finalises
    // four separate tile buffers, so that each LDS read has one known underlying object
    __shared__ __attribute__((aligned(1024))) char kb0[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char kb1[C::KBYTES];
    __shared__ __attribute__((aligned(1024))) char vb0[C::VBYTES];
    __shared__ __attribute__((aligned(1024))) char vb1[C::VBYTES];
    // the row the claiming lane resolved for the workgroup, in slot (claim number & 1): a slot is
    // written again only after the barrier that follows every wave's read of it
    __shared__ int s_row[2];
    static_assert(HB * 16 * 64 * 4 * 2 <= C::VBYTES && HB * 16 * 64 * 4 * 2 + 1024 <= C::KBYTES,
                  "merge exchange fits kb1 | vb1");
    int *status = counters + kStatusWord;  // cleared by the V transpose before this kernel

    if (!plan_ok(pv)) {  // a plan of another layout: nothing is computed or written but the flag
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(status, SIFT_DEVICE_PLAN_MISMATCH);
        return;
    }
    const int G = pv.num_tiles;
    const int group = Hq / Hkv;
    const int64_t N = static_cast<int64_t>(G) * kTile;
    const int home = blockIdx.x % kXcds;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wavefront
    __builtin_assume(wave >= 0 && wave < kWaves);
    const int qh = wave & 1, kh = wave >> 1;
    int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    int qi = 32 * qh + l32;  // this lane's query in the tile
    const bool claimer = tid == 0;
    int cq = home;  // claimer: the queue it draws from

    int pending = 0;  // claimer: a claim kept in flight one row ahead of its use
    if (claimer) {
        s_row[0] = resolve_claim(counters, Qs, cq, home, atomicAdd(&counters[home], 1));
        pending = atomicAdd(&counters[cq % kXcds], 1);
    }
    lds_barrier();
    int row_idx = s_row[0];
    int claim_no = 1;  // claims resolved so far (uniform)
    if (row_idx < 0) return;

    // the first row's Q, list metadata and first tile ids
    RowId rid = row_of(row_idx, G, group);
    WaveState<D> st;
    load_q<D>(st, q, rid, Hq, qi, hi);
    int mw = checked_meta(meta_word(static_cast<int64_t>(rid.h) * G + rid.g, row_ptr, lane), col_entries, status);
    int n = meta_of(mw).n;
    // raw tile ids of the row's entries 0..63
    int ids0 = load_ids(0, n, meta_of(mw).e0, col_idx, lane);
    bool first_issued = false;  // K(0) -> kb0 and V(0) -> vb0 already in flight

    while (true) {
        lane = (tid & 63) + opaque_zero();
        l32 = lane & 31;
        hi = lane >> 5;
        qi = 32 * qh + l32;
        const LoadOffsets<D> off = make_load_offsets<D>(Hkv, N, wave, lane);
        const int g = rid.g, h = rid.h;
        const int64_t tok0 = static_cast<int64_t>(g) * kTile;
        const int q_valid = uniform_read(pv.tile_valid, g);
        const RowCtx ctx{k, vt, N, Hkv, rid.kvh, g, qi, wave, lane, scale_log2, lazy_raw};
#pragma unroll
        for (int db = 0; db < DB; ++db) st.acc_o[db] = f32x16{};
        st.m_run = -INFINITY;
        st.l_run = 0.0f;
        st.thr = -INFINITY;

        // the next row: its claim went out one row ago and resolves at this row's first barrier,
        // when the claim for the row after it goes out
        int next_idx = -1;
        int nmw = 0;      // the next row's metadata word
        int nids = -1;    // raw tile ids of the next row's entries 0..63, once fetched
        bool nfetched = false;
        auto resolve_next = [&]() {  // every wave; includes a workgroup barrier
            const int slot = claim_no & 1;
            if (claimer) {
                const int r = resolve_claim(counters, Qs, cq, home, pending);
                s_row[slot] = r;
                if (r >= 0) pending = atomicAdd(&counters[cq % kXcds], 1);
            }
            lds_barrier();
            next_idx = s_row[slot];
            ++claim_no;
            if (next_idx >= 0) {
                const RowId nid = row_of(next_idx, G, group);
                nmw = meta_word(static_cast<int64_t>(nid.h) * G + nid.g, row_ptr, lane);
            }
        };
        // the next row's metadata landed -> its tile ids
        auto fetch_next_ids = [&]() {
            if (next_idx < 0 || nfetched) return;
            nmw = checked_meta(nmw, col_entries, status);  // before any col_idx read of the row
            const RowMeta nm = meta_of(nmw);
            nids = load_ids(0, nm.n, nm.e0, col_idx, lane);
            nfetched = true;
        };

        int i = 0;
        f32x16 sa, sb;  // S(e) and S(e + 1), formed before use
        float nbias = 0.0f;
        if (n > 0) {
            // prologue: K(0), V(0) (unless already in flight), K(1); then the list's valid counts;
            // S(0) formed, masked, prepped
            if (!first_issued) {
                const int i0 = valid_id(__builtin_amdgcn_readlane(ids0, 0), G);
                load_k_tile<D>(k_tile_base<D>(ctx, i0), kb0, wave, off.k);
                load_vt_tile<D>(vt_tile_base<D>(ctx, i0), vb0, wave, off.v);
            }
            if (n > 1) load_k_tile<D>(k_tile_base<D>(ctx, valid_id(__builtin_amdgcn_readlane(ids0, 1), G)), kb1, wave, off.k);
            TileList L;
            L.c = 0;
            L.c0 = with_valid(ids0, G, pv.tile_valid, status);
            L.c1 = n > 64 ? load_ids(64, n, meta_of(mw).e0, col_idx, lane) : -1;
            L.raw1 = n > 64;
            int t0, v0, t1, v1;
            list_entry(L, 0, t0, v0);
            list_entry(L, 1, t1, v1);  // entry n: t = -1 when past the end
            wait_vmcnt_le(0);
            resolve_next();  // the prologue barrier
            sa = qk_tile<D>(st, kb0, ctx);
            if (needs_mask(t0, v0, ctx)) apply_mask(sa, t0, v0, ctx);
            first_max<D>(st, lane_max(sa), nbias, ctx);
            // steady state, unrolled by two so that every buffer and score register has a fixed
            // role: step e: wait + barrier; K(e+2) -> free K buffer, V(e+1) -> free V buffer; compute
            int t_a = t1, v_a = v1;  // entry i + 1
            while (i + 1 < n) {
                advance_chunk(L, i, mw, G, col_idx, pv.tile_valid, lane, status);
                int t_b, v_b;
                list_entry(L, i + 2, t_b, v_b);
                wait_vmcnt_le(0);
                __builtin_amdgcn_s_barrier();  // K(e+1), V(e) landed; everyone left step e-1
                if (i + 2 < n) load_k_tile<D>(k_tile_base<D>(ctx, t_b), kb0, wave, off.k);
                load_vt_tile<D>(vt_tile_base<D>(ctx, t_a), vb1, wave, off.v);
                if (i == 0) fetch_next_ids();  // the next row's metadata landed with the wait above
                __builtin_amdgcn_sched_barrier(0);
                step_compute<D>(st, sa, sb, nbias, kb1, vb0, t_a, v_a, ctx);
                ++i;
                t_a = t_b;
                v_a = v_b;
                if (i + 1 >= n) break;
                advance_chunk(L, i, mw, G, col_idx, pv.tile_valid, lane, status);
                list_entry(L, i + 2, t_b, v_b);
                wait_vmcnt_le(0);
                __builtin_amdgcn_s_barrier();
                if (i + 2 < n) load_k_tile<D>(k_tile_base<D>(ctx, t_b), kb1, wave, off.k);
                load_vt_tile<D>(vt_tile_base<D>(ctx, t_a), vb0, wave, off.v);
                __builtin_amdgcn_sched_barrier(0);
                step_compute<D>(st, sb, sa, nbias, kb0, vb1, t_a, v_a, ctx);
                ++i;
                t_a = t_b;
                v_a = v_b;
            }
            // last listed tile: softmax + PV only (its scores in sa for even i, its V^T in vb[i % 2]);
            // Q is no longer needed, so the next row's Q starts loading now
            wait_vmcnt_le(0);
            __builtin_amdgcn_s_barrier();
        } else {
            resolve_next();
        }
        fetch_next_ids();
        if (next_idx >= 0) load_q<D>(st, q, row_of(next_idx, G, group), Hq, qi, hi);
        if (n > 0) {
            if ((i & 1) == 0) exp_pv_tile<D>(st, sa, nbias, vb0, ctx);
            else exp_pv_tile<D>(st, sb, nbias, vb1, ctx);
        }

        // merge the two key halves: wave (qh, kh) finalises output blocks [kh HB, kh HB + HB) and
        // publishes the other HB blocks, and its (m, l), for its partner (qh, 1 - kh)
        const float l_tot = pair_sum(st.l_run);
        char *xq = qh ? vb1 : kb1;  // [2 publishers kh][HB blocks][4 quads][64 lanes] float4
        float *ML = reinterpret_cast<float *>(kb1 + 2 * HB * 16 * 64 * 4);  // [qh][kh][32 queries][m, l]
        lds_barrier();  // every wave is done with the last tile's buffers
        {
            f32x4 *mine = reinterpret_cast<f32x4 *>(xq) + kh * HB * 4 * 64;
            // register arrays take compile-time indices only: one branch per key half
            if (kh == 0) publish_half<D, 1>(st, mine, lane);
            else publish_half<D, 0>(st, mine, lane);
            if (hi == 0) {
                ML[((qh * 2 + kh) * 32 + l32) * 2 + 0] = st.m_run;
                ML[((qh * 2 + kh) * 32 + l32) * 2 + 1] = l_tot;
            }
        }
        // the next row's first K and V^T tiles stream in during the merge
        const bool has_next = next_idx >= 0;
        int nn = 0;
        if (has_next) {
            nn = meta_of(nmw).n;
            if (nn > 0) {
                const RowId nid = row_of(next_idx, G, group);
                const int i0 = valid_id(__builtin_amdgcn_readlane(nids, 0), G);
                const RowCtx nctx{k, vt, N, Hkv, nid.kvh, nid.g, qi, wave, lane, scale_log2, lazy_raw};
                load_k_tile<D>(k_tile_base<D>(nctx, i0), kb0, wave, off.k);
                load_vt_tile<D>(vt_tile_base<D>(nctx, i0), vb0, wave, off.v);
            }
        }
        lds_barrier();
        {
            const f32x4 *theirs = reinterpret_cast<const f32x4 *>(xq) + (1 - kh) * HB * 4 * 64;
            const float m1 = ML[((qh * 2 + (1 - kh)) * 32 + l32) * 2 + 0];
            const float l1 = ML[((qh * 2 + (1 - kh)) * 32 + l32) * 2 + 1];
            const float m_fin = fmaxf(st.m_run, m1);
            const float a0 = (st.m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((st.m_run - m_fin) * scale_log2);
            const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m1 - m_fin) * scale_log2);
            const float l_fin = l_tot * a0 + l1 * a1;
            const float inv = l_fin > 0.0f ? 1.0f / l_fin : 0.0f;
            const float w0 = a0 * inv, w1 = a1 * inv;
            const bool live = qi < q_valid;
            float *orow = out + ((tok0 + qi) * Hq + h) * D;
            if (kh == 0) finish_half<D, 0>(st, theirs, orow, w0, w1, live, lane, hi);
            else finish_half<D, 1>(st, theirs, orow, w0, w1, live, lane, hi);
            if (lse != nullptr && kh == 0 && hi == 0)
                lse[static_cast<int64_t>(h) * N + tok0 + qi] =
                    (live && l_fin > 0.0f) ? m_fin * scale + logf(l_fin) : -INFINITY;
        }
        if (!has_next) break;
        lds_barrier();  // every wave has read the exchange before the next row's K(1) lands in kb1
        rid = row_of(next_idx, G, group);
        mw = nmw;
        n = nn;
        ids0 = nids;
        first_issued = nn > 0;
    }
}

}  // namespace

hipError_t launch_prefill(const HostLayout &hl, const PlanView &pv, const uint16_t *q,
                          const uint16_t *k, const uint16_t *vt, const int32_t *row_ptr,
                          const int32_t *col_idx, int64_t col_entries, float scale, float *out, float *lse,
                          int *header, hipStream_t stream) {
    const int64_t rows = int64_t(hl.Hq) * hl.G;
    if (rows == 0) return hipSuccess;
    const float scale_log2 = scale * 1.4426950408889634f;
    const float lazy_raw = kLazyLog2 / scale_log2;
    Queues Qs{};
    Qs.nrows = static_cast<int>(rows);
    Qs.Hkv = hl.Hkv;
    Qs.Rh = static_cast<int>(rows / hl.Hkv);
    Qs.rpx = static_cast<int>((rows + kXcds - 1) / kXcds);
    if (kXcds % hl.Hkv == 0) {
        Qs.mode = 0;
        Qs.xpk = kXcds / hl.Hkv;
    } else if (hl.Hkv % kXcds == 0) {
        Qs.mode = 1;
    } else {
        Qs.mode = 2;
    }
    // persistent: two workgroups per CU (256 CUs), never more workgroups than rows
    const int per_xcd = static_cast<int>(std::min<int64_t>((rows + kXcds - 1) / kXcds, kPersistentPerXcd));
    const unsigned grid = static_cast<unsigned>(per_xcd) * kXcds;
    if (hl.D == 128)
        sparse_prefill_kernel<128><<<grid, kThreads, 0, stream>>>(pv, q, k, vt, row_ptr, col_idx, col_entries, scale,
                                                                  scale_log2, lazy_raw, out, lse, hl.Hq, hl.Hkv, Qs,
                                                                  header);
    else
        sparse_prefill_kernel<64><<<grid, kThreads, 0, stream>>>(pv, q, k, vt, row_ptr, col_idx, col_entries, scale,
                                                                 scale_log2, lazy_raw, out, lse, hl.Hq, hl.Hkv, Qs,
                                                                 header);
    return hipGetLastError();
}

}  // namespace sift
