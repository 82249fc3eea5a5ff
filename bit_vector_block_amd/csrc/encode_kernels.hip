// Offline encoder: LA / CA bit vectors from dense attention (gfx950).
//
// SIFT technical summary, section 2 "Metodologia" ("Design del Sistema", offline stage): every
// document is prefilled densely once and the positions with high attention scores become its
// per-(layer, head) LA and CA bits.  The pages leave the selection rule open; this encoder uses a
// top-p rule on tile masses:
//   mass(h, g, c) = sum over the valid queries of query tile g and the keys of key tile c of the
//                   softmax probability (dense causal attention of the request, GQA);
//   LA row r of document d: its candidate tiles c <= r by decreasing mass (ties: smaller c), the
//                   shortest prefix reaching p_la of their total, plus tiles r and 0;
//   CA pages of document d: page c's mass from the query tiles of the request's later
//                   documents (summed in increasing tile order), the shortest prefix reaching
//                   p_ca of the total, plus page 0.
//
// tile_mass_kernel   one workgroup per (KV head, group of up to four of its q heads, query tile),
//                    two passes over the row's causal key tiles: the row max and sum of every
//                    query, then every tile's mass (bf16 MFMA scores, fp32 softmax,
//                    deterministic reductions); each K tile is loaded once for the group;
// select_bits_kernel one workgroup per (q head, document), a wavefront per LA row: bitonic sort
//                    of the candidates, an inclusive Hillis-Steele scan (the order in which the
//                    threshold test sums), the cut, and the bit packing in LDS.
#include <math.h>

#include "sift_internal.hpp"

namespace sift {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));



__device__ inline int req_of_tile(const PlanView &pv, int g) {
    const int d = pv.tile_doc[g];
    return d >= 0 ? pv.doc_req[d] : -d - 1;
}

// S^T of this wave's 32 keys x 32 queries: K rows (row stride KROW bytes) in LDS, Q in registers.
// Register i is key 32 kh + 8 (i / 4) + 4 hi + i % 4, query 32 qh + l32.
template <int D>
__device__ inline f32x16 scores(const bf16x8 (&qf)[D / 16], const char *Kt, int kh, int l32, int hi) {
    constexpr int KROW = 2 * D + 16;
    const int R = 32 * kh + l32;
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kt + R * KROW + 16 * (2 * dc + hi));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s, 0, 0, 0);
    }
    return s;
}

// The two lanes l and l ^ 32 hold the same query's two key subsets: their sum, and their max, in
// both lanes (one VALU swap of the wavefront's halves; the same order of addition in both lanes)
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum of exp2(score * sl - R) over this lane's 16 keys of key half kh (MASK: keys >= lim count 0)
template <bool MASK>
__device__ __forceinline__ float exp_sum(const f32x16 &s, int kh, float sl, float R, int lim, int hi) {
    const float nr = -R;
    const int lk = lim - 32 * kh - 4 * hi;  // register i holds a key < lim iff 8 (i / 4) + i % 4 < lk
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float e = __builtin_amdgcn_exp2f(fmaf(s[i], sl, nr));
        if (MASK) e = 8 * (i >> 2) + (i & 3) < lk ? e : 0.0f;
        if (i & 1) a1 += e;
        else a0 += e;
    }
    return a0 + a1;
}

// largest score * sl over this lane's keys < lim of key half kh (-inf if none); sl > 0
__device__ __forceinline__ float scaled_max(const f32x16 &s, int kh, float sl, int lim, int hi) {
    const int lk = lim - 32 * kh - 4 * hi;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) < lk) m = fmaxf(m, s[i]);
    return m * sl;
}

constexpr float kRebase = 0x1p64f;  // a tile sum this large moves the reference (entries stay < 2^64)

// K tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds): one load writes lane i's
// 16 bytes at byte 16 i of a 1 KB LDS block, so the row padding of the LDS layout (rows of
// 2 D + 16 bytes) is applied on the global side: lane i fetches the chunk that belongs at its LDS
// position.  A K tile is 64 rows of 2 D + 16 bytes, 17 (D = 128) or 9 (D = 64) such blocks; wave
// w of W issues blocks w, w + W, ...  A lane whose position is a row's padding fetches chunk 0 of
// that row again (never read).
template <int D, int W>
struct KLds {
    static constexpr int KROW = 2 * D + 16, CPR = D / 8;
    static constexpr int BLOCKS = 64 * KROW / 1024;
    static constexpr int PERW = (BLOCKS + W - 1) / W;
    static_assert(64 * KROW % 1024 == 0, "whole 1 KB blocks");
};

template <int D, int W>
__device__ inline void k_lds_offsets(uint32_t *off, int Hkv, int wave, int lane) {  // off: KLds::PERW entries
    using C = KLds<D, W>;
    const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;
#pragma unroll
    for (int j = 0; j < C::PERW; ++j) {
        const int b = 1024 * (wave + W * j) + 16 * lane;  // the LDS byte this lane fills
        const int r = b / C::KROW, c = (b % C::KROW) / 16;
        off[j] = r * row_bytes + 16u * static_cast<uint32_t>(c < C::CPR ? c : 0);
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS load of K tile c of KV head kvh into dst (the tile's base address sits in the
// buffer descriptor, scalar registers; each lane supplies its 32-bit offset).
template <int D, int W>
__device__ __forceinline__ void load_k_lds(const uint16_t *__restrict__ k, int c, int Hkv, int kvh, char *dst, int wave,
                                           const uint32_t *off) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check these builtins
    using C = KLds<D, W>;
    const uint16_t *base = k + (static_cast<int64_t>(c) * kTile * Hkv + kvh) * D;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int j = 0; j < C::PERW; ++j)
        if (wave + W * j < C::BLOCKS)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + 1024 * (wave + W * j)), 16,
                                                     static_cast<int>(off[j]), 0, 0, 0);
#endif
}

__device__ inline void wait_vmcnt0() {  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// One work item = (KV head, group of HPW q heads of it, query tile g), taken by a persistent
// workgroup of 2 HPW wavefronts from its XCD's queue, latest query tiles (the longest rows) first.
// Wave w takes q head (group base + w / 2) and queries 32 (w % 2) .. + 31, against all 64 keys of
// every key tile; the K tile is loaded once for the HPW heads that share it (GQA) and staged one
// tile ahead in registers.  One pass over the row's causal key tiles: each query's sum of exp2
// over a tile's keys, relative to a reference R of that query, goes to the workgroup's scratch
// slot and into the query's running sum l.  R is the largest scaled score seen when it was last
// set; it is set again only when a tile's sum reaches 2^64 (or R is still unset), and then the
// query's earlier entries and l are scaled down to the new R, so every entry shares the final R.
// The masses are then sum over queries of entry * (1 / l), two wavefronts per head.
template <int D, int HPW>
__device__ __forceinline__ void tile_mass_body(const PlanView &pv, const uint16_t *__restrict__ q,
                                               const uint16_t *__restrict__ k, int Hq, int Hkv, float scale_log2,
                                               float *__restrict__ masses, int RT, int *__restrict__ queue,
                                               float *__restrict__ scratch, int32_t *__restrict__ status) {
    constexpr int NT = 128 * HPW, W = 2 * HPW;
    constexpr int KROW = 2 * D + 16;
    constexpr int ESTRIDE = W * 32;        // floats per key tile in a scratch slot
    __shared__ __attribute__((aligned(16))) char Kt[2][64 * KROW];
    __shared__ float part[W][64];
    __shared__ int s_item;
    const bool ok = plan_ok(pv);
    if (status != nullptr && blockIdx.x == 0 && threadIdx.x == 0)  // the call's one writer
        *status = ok ? SIFT_DEVICE_OK : SIFT_DEVICE_PLAN_MISMATCH;
    if (!ok) return;
    const int G = pv.num_tiles;
    const int group = Hq / Hkv, ngroups = group / HPW, per_g = Hkv * ngroups;
    const int items = G * per_g;
    const int nq = min(kMassQueues, static_cast<int>(gridDim.x)), xq = static_cast<int>(blockIdx.x) % nq;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int qi = 32 * (wave & 1) + l32;
    float *const slot = scratch + static_cast<int64_t>(blockIdx.x) * RT * ESTRIDE;
    float *const mine = slot + wave * 32 + l32;  // this query's entry of key tile e: mine[e * ESTRIDE]
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    uint32_t koff[KLds<D, W>::PERW];
    k_lds_offsets<D, W>(koff, Hkv, uwave, lane);
    for (;;) {
        if (tid == 0) s_item = xq + nq * atomicAdd(&queue[xq], 1);
        __syncthreads();
        const int item = s_item;
        if (item >= items) break;
        const int g = G - 1 - item / per_g;
        const int rest = item % per_g;
        const int kvh = rest / ngroups;
        const int h0 = kvh * group + (rest % ngroups) * HPW;  // the item's first q head
        const int h = h0 + (wave >> 1);
        const int first = pv.req_first[req_of_tile(pv, g)];
        const int q_valid = pv.tile_valid[g];
        const int nt = g - first + 1;
        bf16x8 qf[D / 16];
        {
            const uint16_t *qrow = q + ((static_cast<int64_t>(g) * kTile + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
            for (int dc = 0; dc < D / 16; ++dc) qf[dc] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * dc);
        }
        // K(first) now; at the start of every step, a wait for this wave's loads and a barrier
        // (K(e) has landed, every wave has left step e - 1), then K(e + 1) goes into the buffer
        // that step e - 1 used, one step ahead of its use
        load_k_lds<D, W>(k, first, Hkv, kvh, Kt[0], uwave, koff);
        float R = -INFINITY, l = 0.0f;
        // key tile first + e is in Kt[buf]; the scores of one key half at a time are live.  Every
        // score computation runs with the whole wavefront active (an MFMA takes its operands from
        // all 64 lanes, and each lane reads its own share of the K tile from LDS): the branches
        // around them are uniform, and lanes that need no new R ignore what they compute.
        auto step = [&](int e, int buf) {
            const int c = first + e;
            const int tv = pv.tile_valid[c];
            const int lim = c == g ? min(tv, qi + 1) : tv;  // keys < lim count
            float a = kRebase;                              // R is unset in every lane at e = 0
            if (e > 0) {
                if (c != g && tv >= kTile)
                    a = pair_sum(exp_sum<false>(scores<D>(qf, Kt[buf], 0, l32, hi), 0, scale_log2, R, lim, hi) +
                                 exp_sum<false>(scores<D>(qf, Kt[buf], 1, l32, hi), 1, scale_log2, R, lim, hi));
                else
                    a = pair_sum(exp_sum<true>(scores<D>(qf, Kt[buf], 0, l32, hi), 0, scale_log2, R, lim, hi) +
                                 exp_sum<true>(scores<D>(qf, Kt[buf], 1, l32, hi), 1, scale_log2, R, lim, hi));
            }
            // R unset, or this tile's scores exceed it by ~64 (the two lanes of a query agree)
            const bool rebase = !(a < kRebase);
            if (__ballot(rebase) != 0ull) {
                float mt = scaled_max(scores<D>(qf, Kt[buf], 0, l32, hi), 0, scale_log2, lim, hi);
                asm volatile("" ::: "memory");  // the halves are computed anew, not kept
                mt = pair_max(fmaxf(mt, scaled_max(scores<D>(qf, Kt[buf], 1, l32, hi), 1, scale_log2, lim, hi)));
                const float Rn = fmaxf(R, mt);
                if (rebase && Rn > R) {
                    if (R > -INFINITY) {
                        const float f = __builtin_amdgcn_exp2f(R - Rn);
                        l *= f;
                        if (hi == 0)
                            for (int j = 0; j < e; ++j) mine[j * ESTRIDE] *= f;
                    }
                    R = Rn;
                }
                asm volatile("" ::: "memory");
                float a2 = exp_sum<true>(scores<D>(qf, Kt[buf], 0, l32, hi), 0, scale_log2, R, lim, hi);
                asm volatile("" ::: "memory");
                a2 = pair_sum(a2 + exp_sum<true>(scores<D>(qf, Kt[buf], 1, l32, hi), 1, scale_log2, R, lim, hi));
                if (rebase) a = R > -INFINITY ? a2 : 0.0f;
            }
            l += a;
            if (hi == 0) mine[e * ESTRIDE] = a;
        };
        for (int e = 0; e < nt; e += 2) {
            wait_vmcnt0();
            __syncthreads();
            if (e + 1 < nt) load_k_lds<D, W>(k, first + e + 1, Hkv, kvh, Kt[1], uwave, koff);
            step(e, 0);
            if (e + 1 >= nt) break;
            wait_vmcnt0();
            __syncthreads();
            if (e + 2 < nt) load_k_lds<D, W>(k, first + e + 2, Hkv, kvh, Kt[0], uwave, koff);
            step(e + 1, 1);
        }
        // masses: lane (l32, hi) takes key tile e + hi of each pair; padded queries carry no mass
        const float inv = (qi < q_valid && l > 0.0f) ? 1.0f / l : 0.0f;
        for (int cb = 0; cb < nt; cb += 64) {
            const int n = min(64, nt - cb);
            for (int t = 0; t < n; t += 2) {
                const bool have = t + hi < n;
                float v = have ? mine[(cb + t + hi) * ESTRIDE] * inv : 0.0f;
#pragma unroll
                for (int off = 16; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);  // within the half
                if (l32 == 0 && have) part[wave][t + hi] = v;
            }
            __syncthreads();
            for (int x = tid; x < HPW * 64; x += NT) {
                const int hh = x >> 6, t = x & 63;
                if (t < n)
                    masses[(static_cast<int64_t>(h0 + hh) * G + g) * RT + cb + t] = part[2 * hh][t] + part[2 * hh + 1][t];
            }
            __syncthreads();
        }
    }
}

// GQA groups of 2 or 4 q heads per KV head: 4 or 8 wavefronts; four waves per SIMD (the kernel is
// bound by latency: the resident waves hide each other's loads and barriers)
template <int D, int HPW>
__global__ __launch_bounds__(128 * HPW) __attribute__((amdgpu_waves_per_eu(4, 4))) void tile_mass_kernel(
    PlanView pv, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, int Hq, int Hkv, float scale_log2,
    float *__restrict__ masses, int RT, int *__restrict__ queue, float *__restrict__ scratch,
    int32_t *__restrict__ status) {
    tile_mass_body<D, HPW>(pv, q, k, Hq, Hkv, scale_log2, masses, RT, queue, scratch, status);
}

// one q head per workgroup (odd groups): two wavefronts stage a whole tile each, so more registers
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 2))) void tile_mass_kernel_one(
    PlanView pv, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, int Hq, int Hkv, float scale_log2,
    float *__restrict__ masses, int RT, int *__restrict__ queue, float *__restrict__ scratch,
    int32_t *__restrict__ status) {
    tile_mass_body<D, 1>(pv, q, k, Hq, Hkv, scale_log2, masses, RT, queue, scratch, status);
}

__global__ void mass_queue_reset_kernel(int *__restrict__ queue) {
    if (threadIdx.x < kMassQueues) queue[threadIdx.x] = 0;
}

// One wavefront: sort 64 (mass, index) pairs by decreasing mass, ties by increasing index.
__device__ inline void bitonic_sort_desc(float &v, int &ix, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const float ov = __shfl_xor(v, stride, 64);
            const int oi = __shfl_xor(ix, stride, 64);
            const bool lower = (lane & stride) == 0;
            const bool desc = (lane & size) == 0;  // this block sorts descending
            // "a before b": larger mass, or equal mass and smaller index
            const bool other_first = (ov > v) || (ov == v && oi < ix);
            const bool take = lower ? (desc ? other_first : !other_first) : (desc ? !other_first : other_first);
            if (take) {
                v = ov;
                ix = oi;
            }
        }
    }
}

// Top-p over `n` candidates held one per lane (lane c: mass of candidate c; lanes >= n: none):
// returns whether this lane's candidate is kept (before the forced ones are added).
__device__ inline bool top_p_keep(float mass, int n, float p, int lane) {
    float v = lane < n ? mass : -1.0f;  // masses are >= 0: the empty slots sort last
    int ix = lane;
    bitonic_sort_desc(v, ix, lane);
    float s = lane < n ? v : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(s, off, 64);
        if (lane >= off) s += y;
    }
    const float thr = p * __shfl(s, 63, 64);
    const float before = __shfl_up(s, 1, 64);
    const bool keep_slot = lane < n && (lane == 0 || before < thr);
    // hand the decision back to the candidate's own lane
    const unsigned long long km = __ballot(keep_slot);
    bool mine = false;
    for (int slot = 0; slot < n; ++slot) {  // n <= 64, uniform
        const int who = __shfl(ix, slot, 64);
        if (who == lane && ((km >> slot) & 1ull)) mine = true;
    }
    return mine;
}

constexpr int kSelectWaves = 4;

// One workgroup of kSelectWaves wavefronts per (q head, document): the LA rows are spread over
// the wavefronts (each row's top-p cut is a one-wavefront operation), then wavefront 0 selects the
// CA pages.  The bits are packed in LDS and written out whole.
__global__ __launch_bounds__(64 * kSelectWaves) void select_bits_kernel(PlanView pv, const float *__restrict__ masses,
                                                                        int RT, float p_la, float p_ca,
                                                                        uint32_t *__restrict__ la_out,
                                                                        uint32_t *__restrict__ ca_out,
                                                                        int32_t *__restrict__ status) {
    __shared__ uint32_t la_words[72];  // T <= 64: at most 65 words
    __shared__ uint32_t ca_words[4];
    const bool ok = plan_ok(pv);
    if (status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)  // the call's one writer
        *status = ok ? SIFT_DEVICE_OK : SIFT_DEVICE_PLAN_MISMATCH;
    if (!ok) return;
    const int G = pv.num_tiles;
    const int h = blockIdx.x, d = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = pv.doc_tiles[d], t0 = pv.doc_first[d], b = pv.doc_req[d];
    const int first = pv.req_first[b];
    const int dl = pv.req_first_doc[b] + pv.req_ndocs[b] - 1;
    const int doc_end = pv.doc_first[dl] + pv.doc_tiles[dl];  // the request's question starts here
    const int law = pv.doc_la_w[d], caw = pv.doc_ca_w[d];
    for (int w = tid; w < law; w += 64 * kSelectWaves) la_words[w] = 0u;
    for (int w = tid; w < caw; w += 64 * kSelectWaves) ca_words[w] = 0u;
    __syncthreads();
    // LA: triangle rows r = wave, wave + kSelectWaves, ...
    for (int r = wave; r < T; r += kSelectWaves) {
        const int gq = t0 + r;
        const float mass = lane <= r ? masses[(static_cast<int64_t>(h) * G + gq) * RT + (t0 + lane - first)] : 0.0f;
        const bool keep = top_p_keep(mass, r + 1, p_la, lane) || lane == r || lane == 0;
        if (lane <= r && keep) {
            const int bit = r * (r + 1) / 2 + lane;
            atomicOr(&la_words[bit >> 5], 1u << (bit & 31));
        }
    }
    // CA: page masses from the later documents' query tiles, summed in increasing tile order (the
    // loads go out eight at a time, the additions stay in order)
    if (wave == 0) {
        float cm = 0.0f;
        if (lane < T) {
            const float *col = masses + static_cast<int64_t>(h) * G * RT + (t0 + lane - first);
            int gq = t0 + T;
            for (; gq + 8 <= doc_end; gq += 8) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = col[static_cast<int64_t>(gq + j) * RT];
#pragma unroll
                for (int j = 0; j < 8; ++j) cm += v[j];
            }
            for (; gq < doc_end; ++gq) cm += col[static_cast<int64_t>(gq) * RT];
        }
        const bool keep = top_p_keep(cm, T, p_ca, lane) || lane == 0;
        if (lane < T && keep) atomicOr(&ca_words[lane >> 5], 1u << (lane & 31));
    }
    __syncthreads();
    uint32_t *la_vec = la_out + pv.doc_la_off[d] + h * law;
    for (int w = tid; w < law; w += 64 * kSelectWaves) la_vec[w] = la_words[w];
    uint32_t *ca_vec = ca_out + pv.doc_ca_off[d] + h * caw;
    for (int w = tid; w < caw; w += 64 * kSelectWaves) ca_vec[w] = ca_words[w];
}

}  // namespace

int mass_heads_per_wg(const HostLayout &hl) {
    const int group = hl.Hq / hl.Hkv;
    return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

int64_t mass_slots(const HostLayout &hl) {
    const int hpw = mass_heads_per_wg(hl);
    const int64_t items = int64_t(hl.Hkv) * (hl.Hq / hl.Hkv / hpw) * hl.G;
    return std::min<int64_t>(items, kMassWaves / (2 * hpw));
}

size_t mass_workspace_bytes(const HostLayout &hl) {
    const int64_t rt = hl.max_req_tiles > 0 ? hl.max_req_tiles : 1;
    return kWorkspaceHeader + size_t(mass_slots(hl)) * size_t(rt) * size_t(mass_heads_per_wg(hl)) * 64 * sizeof(float);
}

hipError_t launch_tile_masses(const HostLayout &hl, const PlanView &pv, const uint16_t *q, const uint16_t *k,
                              float scale, float *masses, int RT, void *workspace, int32_t *status,
                              hipStream_t stream) {
    if (hl.G == 0) return hipSuccess;
    const int hpw = mass_heads_per_wg(hl);
    const unsigned grid = static_cast<unsigned>(mass_slots(hl));
    int *queue = static_cast<int *>(workspace);
    float *scratch = reinterpret_cast<float *>(static_cast<char *>(workspace) + kWorkspaceHeader);
    const float sl = scale * 1.4426950408889634f;
    mass_queue_reset_kernel<<<1, 64, 0, stream>>>(queue);
#define SIFT_TILE_MASS(DD, HH)                                                                                   \
    tile_mass_kernel<DD, HH><<<grid, 128 * HH, 0, stream>>>(pv, q, k, hl.Hq, hl.Hkv, sl, masses, RT, queue, scratch, \
                                                            status)
#define SIFT_TILE_MASS_ONE(DD) \
    tile_mass_kernel_one<DD><<<grid, 128, 0, stream>>>(pv, q, k, hl.Hq, hl.Hkv, sl, masses, RT, queue, scratch, status)
    if (hl.D == 128) {
        if (hpw == 4) SIFT_TILE_MASS(128, 4);
        else if (hpw == 2) SIFT_TILE_MASS(128, 2);
        else SIFT_TILE_MASS_ONE(128);
    } else {
        if (hpw == 4) SIFT_TILE_MASS(64, 4);
        else if (hpw == 2) SIFT_TILE_MASS(64, 2);
        else SIFT_TILE_MASS_ONE(64);
    }
#undef SIFT_TILE_MASS
#undef SIFT_TILE_MASS_ONE
    return hipGetLastError();
}

hipError_t launch_select_bits(const HostLayout &hl, const PlanView &pv, const float *masses, int RT, float p_la,
                              float p_ca, uint32_t *la_out, uint32_t *ca_out, int32_t *status, hipStream_t stream) {
    if (hl.ndocs == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(hl.Hq), static_cast<unsigned>(hl.ndocs));
    select_bits_kernel<<<grid, 64 * kSelectWaves, 0, stream>>>(pv, masses, RT, p_la, p_ca, la_out, ca_out, status);
    return hipGetLastError();
}

}  // namespace sift
