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
    static_assert(32 * D * 4 == TILE * 2, "32 fp32 output rows fill one tile buffer");
};

// slot of 16-byte chunk c in K row r / V row r
template <int D>
__device__ inline int k_slot(int r, int c) { return c ^ (r & (Cfg<D>::CPR - 1)); }
// V rows: the transposing reads of one K-step touch 4 consecutive rows x 2 (16 lanes) or
// 4 (32 lanes) consecutive chunks; XOR masks {0, 6, 12, 10} keep those 8 (or 16) chunks
// on distinct banks for 128-byte and 256-byte LDS cycles alike.
template <int D>
__device__ inline int v_slot(int r, int c) { return c ^ ((0xAC60 >> (4 * (r & 3))) & 15 & (Cfg<D>::CPR - 1)); }

__device__ inline void wait_vmcnt_le(int n) {
    // s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima)
    if (n >= 8) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8) | ((8 >> 4) << 14));
    else if (n >= 4) __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// Per-lane byte offsets of this lane's direct-to-LDS loads inside a K or V tile
// (the same for every tile; the tile itself only moves a uniform base pointer).
template <int D>
struct LoadOffsets {
    uint32_t k[Cfg<D>::LOADS];
    uint32_t v[Cfg<D>::LOADS];
};

template <int D>
__device__ inline LoadOffsets<D> make_load_offsets(int Hkv, int wave, int lane) {
    using C = Cfg<D>;
    LoadOffsets<D> o;
    const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
        const int I = wave * C::LOADS + j;  // this load fills LDS elements [512 I, 512 I + 512)
        const int r = I * C::RPL + lane / C::CPR;
        const int sl = lane % C::CPR;       // LDS slot written by this lane
        o.k[j] = r * row_bytes + 16u * static_cast<uint32_t>(k_slot<D>(r, sl));
        o.v[j] = r * row_bytes + 16u * static_cast<uint32_t>(v_slot<D>(r, sl));
    }
    return o;
}

// Direct-to-LDS load of one K (or V) tile starting at token ktok0 into `dst`.
template <int D>
__device__ __forceinline__ void load_half(const uint16_t *__restrict__ src, int64_t ktok0, int Hkv,
                                          int kvh, uint16_t *dst, int wave, const uint32_t *off) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check this builtin
    using C = Cfg<D>;
    const char *g = reinterpret_cast<const char *>(src + (ktok0 * Hkv + kvh) * D);  // uniform
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
        __builtin_amdgcn_global_load_lds(g + off[j], (lds_void *)(dst + 512 * (wave * C::LOADS + j)), 16, 0, 0);
#endif
}

__device__ inline float pair_max(float x) {  // max over lanes l and l ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float pair_sum(float x) {  // sum over lanes l and l ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online-softmax state of one wavefront (32 queries x one 32-key half of each tile).
template <int D>
struct WaveState {
    bf16x8 qf[D / 16];
    f32x16 acc_o[D / 32];
    float m_run, l_run;
};

// Per-row constants a pipeline step needs.
struct RowCtx {
    const uint16_t *k, *v;
    const int32_t *tile_valid;
    int Hkv, kvh, g, qi, wave, lane;
    float scale_log2, lazy_raw;
};

// S^T for keys 32 kh .. 32 kh + 31 of the K tile in LDS: register i is key
// 32 kh + 8 (i / 4) + 4 hi + i % 4 of the tile, for query qi.
template <int D>
__device__ __forceinline__ f32x16 qk_tile(const WaveState<D> &st, const uint16_t *Kt, const RowCtx &c) {
    const int l32 = c.lane & 31, hi = c.lane >> 5, kh = c.wave >> 1;
    const int R = 32 * kh + l32;
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kt + R * D + 8 * k_slot<D>(R, 2 * dc + hi));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qf[dc], s, 0, 0, 0);
    }
    return s;
}

// Causal mask on the diagonal tile and padding mask on a partial tile (a select,
// so NaN in padded K slots never leaks); t < 0 marks a skipped entry.
__device__ __forceinline__ void mask_tile(f32x16 &s, int t, int kv_valid, const RowCtx &c) {
    if (kv_valid < kTile || t >= c.g) {
        const int hi = c.lane >> 5, kh = c.wave >> 1;
        const int lim = min(kv_valid, c.qi - (t - c.g) * kTile + 1);  // keys < lim survive
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * kh + 8 * (i >> 2) + 4 * hi + (i & 3);
            s[i] = key < lim ? s[i] : -INFINITY;
        }
    }
}

// Online softmax, part 1, run as soon as a tile's (masked) scores exist: tile max,
// the new reference max -- raised only when the tile exceeds the current one by
// more than kLazyLog2 in log2 units, decided wave-uniformly -- and, when it moves,
// the rescale of O and l.  Returns the exp2 bias -m * scale_log2 for part 2.
template <int D>
__device__ __forceinline__ float softmax_prep(WaveState<D> &st, const f32x16 &s, const RowCtx &c) {
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])), fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    mt = pair_max(mt);
    if (__ballot(mt > st.m_run + c.lazy_raw) != 0) {
        const float m_new = fmaxf(st.m_run, mt);
        // m_run = -inf gives exp2(-inf) = 0; both -inf leaves alpha = 1 (O and l are still 0)
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f((st.m_run - m_new) * c.scale_log2);
        st.m_run = m_new;
        st.l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) st.acc_o[db] *= alpha;
    }
    return (st.m_run == -INFINITY) ? 0.0f : -st.m_run * c.scale_log2;
}

// Part 2 (branch-free): P = exp2(s * scale_log2 + nbias) rounded to bf16 (the MFMA
// B operand, two 8-key halves) and l += the sum of the rounded P.
template <int D>
__device__ __forceinline__ void softmax_exp(WaveState<D> &st, const f32x16 &s, bf16x8 (&pb)[2],
                                            float nbias, const RowCtx &c) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
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
}

// O^T += V^T P^T for this wave's 32 keys of the V tile in LDS; K-step j covers
// keys 32 kh + 16 j + {0..3, 8..11} + 4 hi, read with ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ void pv_tile(WaveState<D> &st, const bf16x8 (&pb)[2], const uint16_t *Vt,
                                        const RowCtx &c) {
    const int kh = c.wave >> 1, hi = c.lane >> 5;
    const int s16 = c.lane & 15;
    const int dsub = 16 * ((c.lane >> 4) & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
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

__device__ inline int64_t tile_token(int t) { return static_cast<int64_t>(t < 0 ? 0 : t) * kTile; }

// The row's listed tiles, 64 entries per chunk held across the lanes of two
// registers (lane j of chunk c: entry 64 c + j, its tile id or -1, and that
// tile's valid-token count), read with v_readlane.  Vector loads keep these
// reads out of the scalar/LDS counter, so no per-tile scalar-load latency sits
// on the critical path; chunk c + 1 is fetched 64 tiles ahead of use.
struct TileList {
    int t0, v0;  // chunk c
    int t1, v1;  // chunk c + 1
    int c;
};

__device__ __forceinline__ void fetch_chunk(int &t, int &valid, int base, int n, int e0, int G,
                                            const int32_t *__restrict__ col_idx,
                                            const int32_t *__restrict__ tile_valid, int lane) {
    const int j = base + lane;
    int x = j < n ? col_idx[e0 + j] : -1;
    x = (x >= 0 && x < G) ? x : -1;  // out-of-range entries are skipped (masked)
    t = x;
    valid = x >= 0 ? tile_valid[x] : 0;
}

// Entry i (uniform; c <= i / 64 <= c + 1): tile id and valid count.
__device__ __forceinline__ void list_entry(const TileList &L, int i, int &t, int &valid) {
    const bool first = (i >> 6) == L.c;
    t = __builtin_amdgcn_readlane(first ? L.t0 : L.t1, i & 63);
    valid = __builtin_amdgcn_readlane(first ? L.v0 : L.v1, i & 63);
}

// One pipeline step for listed tile e (scores s_cur formed, masked and prepped):
//   wait + barrier; start K(e+2) -> k_free and V(e+1) -> v_free;
//   S(e+1) = K(e+1) Q^T from k_next interleaved with P(e) = exp2(...) of S(e);
//   O += V(e) P(e) from v_cur; mask and prep S(e+1).
template <int D>
__device__ __forceinline__ void pipe_step(WaveState<D> &st, f32x16 &s_cur, float &nbias,
                                          const uint16_t *k_next, const uint16_t *v_cur,
                                          uint16_t *k_free, uint16_t *v_free, int t_next, int v_next,
                                          int t_next2, bool has_next2, const LoadOffsets<D> &off,
                                          const RowCtx &c) {
    wait_vmcnt_le(0);
    __builtin_amdgcn_s_barrier();  // K(e+1), V(e) landed; everyone left step e-1
    if (has_next2) load_half<D>(c.k, tile_token(t_next2), c.Hkv, c.kvh, k_free, c.wave, off.k);
    load_half<D>(c.v, tile_token(t_next), c.Hkv, c.kvh, v_free, c.wave, off.v);
    // one scheduling region: the MFMA chain of S(e+1) interleaved with P(e)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s_nxt = qk_tile<D>(st, k_next, c);
    bf16x8 pb[2];
    softmax_exp<D>(st, s_cur, pb, nbias, c);
#pragma unroll
    for (int x = 0; x < D / 16; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);  // then VALU + transcendental work
    }
    __builtin_amdgcn_sched_barrier(0);
    pv_tile<D>(st, pb, v_cur, c);
    mask_tile(s_nxt, t_next, v_next, c);
    nbias = softmax_prep<D>(st, s_nxt, c);
    s_cur = s_nxt;
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
    // four separate tile buffers, so that each LDS read has one known underlying object
    __shared__ __attribute__((aligned(16))) uint16_t kb0[C::TILE];
    __shared__ __attribute__((aligned(16))) uint16_t kb1[C::TILE];
    __shared__ __attribute__((aligned(16))) uint16_t vb0[C::TILE];
    __shared__ __attribute__((aligned(16))) uint16_t vb1[C::TILE];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wavefront
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int qh = wave & 1, kh = wave >> 1;
    const int qi = 32 * qh + l32;  // this lane's query in the tile
    const int q_valid = uniform_read(pv.tile_valid, g);
    const int64_t tok0 = static_cast<int64_t>(g) * kTile;
    const LoadOffsets<D> off = make_load_offsets<D>(Hkv, wave, lane);
    const RowCtx ctx{k, v, pv.tile_valid, Hkv, kvh, g, qi, wave, lane, scale_log2, lazy_raw};

    WaveState<D> st;
    {
        const uint16_t *qrow = q + ((tok0 + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)  // read once: stream it past L2 (keep L2 for K/V tiles)
            st.qf[dc] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(qrow + 16 * dc));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) st.acc_o[db] = f32x16{};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    const int e0 = uniform_read(row_ptr, row), e1 = uniform_read(row_ptr, row + 1);
    const int n = e1 - e0;
    if (n > 0) {
        TileList L;
        L.c = 0;
        fetch_chunk(L.t0, L.v0, 0, n, e0, G, col_idx, pv.tile_valid, lane);
        fetch_chunk(L.t1, L.v1, 64, n, e0, G, col_idx, pv.tile_valid, lane);
        int t0, v0, t1, v1;
        list_entry(L, 0, t0, v0);
        list_entry(L, 1, t1, v1);  // entry n: t = -1 when past the end
        // prologue: K(0), V(0), K(1) in flight; S(0) formed, masked, prepped
        load_half<D>(k, tile_token(t0), Hkv, kvh, kb0, wave, off.k);
        load_half<D>(v, tile_token(t0), Hkv, kvh, vb0, wave, off.v);
        if (n > 1) load_half<D>(k, tile_token(t1), Hkv, kvh, kb1, wave, off.k);
        wait_vmcnt_le(0);
        __builtin_amdgcn_s_barrier();
        f32x16 s_cur = qk_tile<D>(st, kb0, ctx);
        mask_tile(s_cur, t0, v0, ctx);
        float nbias = softmax_prep<D>(st, s_cur, ctx);
        // steady state, unrolled by two so every buffer has a fixed role
        int i = 0;
        int t_a = t1, v_a = v1;  // entry i + 1
        while (i + 1 < n) {
            if ((i >> 6) != L.c) {  // entry i entered chunk c + 1: shift, fetch chunk c + 2
                L.c += 1;
                L.t0 = L.t1;
                L.v0 = L.v1;
                fetch_chunk(L.t1, L.v1, 64 * (L.c + 1), n, e0, G, col_idx, pv.tile_valid, lane);
            }
            int t_b, v_b;
            list_entry(L, i + 2, t_b, v_b);
            pipe_step<D>(st, s_cur, nbias, kb1, vb0, kb0, vb1, t_a, v_a, t_b, i + 2 < n, off, ctx);
            ++i;
            if (i + 1 >= n) break;
            if ((i >> 6) != L.c) {
                L.c += 1;
                L.t0 = L.t1;
                L.v0 = L.v1;
                fetch_chunk(L.t1, L.v1, 64 * (L.c + 1), n, e0, G, col_idx, pv.tile_valid, lane);
            }
            t_a = t_b;
            v_a = v_b;
            list_entry(L, i + 2, t_b, v_b);
            pipe_step<D>(st, s_cur, nbias, kb0, vb1, kb1, vb0, t_a, v_a, t_b, i + 2 < n, off, ctx);
            ++i;
            t_a = t_b;
            v_a = v_b;
        }
        // last listed tile: softmax + PV only (its V is in vb[i % 2])
        wait_vmcnt_le(0);
        __builtin_amdgcn_s_barrier();
        bf16x8 pb[2];
        softmax_exp<D>(st, s_cur, pb, nbias, ctx);
        if ((i & 1) == 0) pv_tile<D>(st, pb, vb0, ctx);
        else pv_tile<D>(st, pb, vb1, ctx);
    }

    // merge the two key halves: waves with kh = 1 publish, waves with kh = 0 combine
    const float l_tot = pair_sum(st.l_run);
    float *X = reinterpret_cast<float *>(kb0);  // [D/2 registers][2 query halves][64 lanes] (kb0 + kb1)
    float *ML = reinterpret_cast<float *>(vb0);  // [2 query halves][32 queries][m, l]
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = db * 16 + i;  // first D/4 registers in kb0, the rest in kb1
                float *dst = r < D / 4 ? X : reinterpret_cast<float *>(kb1);
                dst[(((r % (D / 4)) * 2) + qh) * 64 + lane] = st.acc_o[db][i];
            }
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
            for (int i = 0; i < 16; ++i) {
                const int r = db * 16 + i;
                const float *src = r < D / 4 ? X : reinterpret_cast<const float *>(kb1);
                st.acc_o[db][i] = st.acc_o[db][i] * w0 + src[(((r % (D / 4)) * 2) + qh) * 64 + lane] * w1;
            }
    }
    __syncthreads();
    // output tile staged in kb0|kb1 as [64 rows][D/4 float4 chunks], chunk c of row r at c ^ (r % 32);
    // rows 0..31 in kb0, rows 32..63 in kb1
    constexpr int C4 = D / 4;
    auto orow = [&](int r) -> float * {
        return reinterpret_cast<float *>(r < 32 ? kb0 : kb1) + (r & 31) * D;
    };
    if (kh == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 o4 = {st.acc_o[db][4 * i4 + 0], st.acc_o[db][4 * i4 + 1],
                                  st.acc_o[db][4 * i4 + 2], st.acc_o[db][4 * i4 + 3]};
                const int c4 = 8 * db + 2 * i4 + hi;
                *reinterpret_cast<f32x4 *>(orow(qi) + 4 * (c4 ^ (qi & (C4 - 1)))) = o4;
            }
        if (lse != nullptr && hi == 0) {
            const bool live = qi < q_valid && l_fin > 0.0f;
            lse[static_cast<int64_t>(h) * N + tok0 + qi] = live ? m_fin * scale + logf(l_fin) : -INFINITY;
        }
    }
    __syncthreads();
    for (int x = tid; x < 64 * C4; x += kThreads) {
        const int r = x / C4, c4 = x % C4;
        f32x4 val = *reinterpret_cast<const f32x4 *>(orow(r) + 4 * (c4 ^ (r & (C4 - 1))));
        if (r >= q_valid) val = f32x4{};
        // written once: non-temporal, so 32 KB of output per row does not evict K/V tiles
        __builtin_nontemporal_store(val, reinterpret_cast<f32x4 *>(out + ((tok0 + r) * Hq + h) * D + 4 * c4));
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
