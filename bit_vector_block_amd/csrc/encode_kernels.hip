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
// tile_mass_kernel   one workgroup per (q head, query tile), two passes over the row's causal
//                    key tiles: the row max and sum of every query, then every tile's mass
//                    (bf16 MFMA scores, fp32 softmax, deterministic reductions);
// select_bits_kernel one wavefront per (q head, document): bitonic sort of the candidates, an
//                    inclusive Hillis-Steele scan (the order in which the threshold test sums),
//                    the cut, and the bit packing in LDS.
#include <math.h>

#include "sift_internal.hpp"

namespace sift {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kEncThreads = 256;

__device__ inline bool plan_ok(const PlanView &pv) {
    return pv.header[0] == static_cast<int32_t>(kPlanMagic) &&
           static_cast<uint32_t>(pv.header[2]) == pv.fp_lo &&
           static_cast<uint32_t>(pv.header[3]) == pv.fp_hi && pv.header[6] == pv.num_tiles;
}

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

template <int D>
__device__ inline void load_k_rows(char *Kt, const uint16_t *__restrict__ k, int64_t tok0, int Hkv, int kvh,
                                   int tid) {
    constexpr int CH = D / 8, KROW = 2 * D + 16;
    for (int x = tid; x < 64 * CH; x += kEncThreads) {
        const int r = x / CH, c = x % CH;
        const uint4 w = *reinterpret_cast<const uint4 *>(k + ((tok0 + r) * Hkv + kvh) * D + 8 * c);
        *reinterpret_cast<uint4 *>(Kt + r * KROW + 16 * c) = w;
    }
}

__device__ inline float wave_sum(float x) {  // fixed butterfly order: deterministic
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(kEncThreads) void tile_mass_kernel(PlanView pv, const uint16_t *__restrict__ q,
                                                                 const uint16_t *__restrict__ k, int Hq, int Hkv,
                                                                 float scale_log2, float *__restrict__ masses,
                                                                 int RT) {
    constexpr int KROW = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) char Kt[64 * KROW];
    __shared__ float ml[2][2][32][2];  // [qh][kh][query][m, l]
    __shared__ float part[4];
    if (!plan_ok(pv)) return;
    const int G = pv.num_tiles;
    const int h = blockIdx.x / G, g = blockIdx.x % G;
    const int kvh = h / (Hq / Hkv);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int qh = wave & 1, kh = wave >> 1, qi = 32 * qh + l32;
    const int first = pv.req_first[req_of_tile(pv, g)];
    const int q_valid = pv.tile_valid[g];
    bf16x8 qf[D / 16];
    {
        const uint16_t *qrow = q + ((static_cast<int64_t>(g) * kTile + qi) * Hq + h) * D + 8 * hi;
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) qf[dc] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * dc);
    }
    auto masked = [&](f32x16 &s, int c) {
        const int kv_valid = pv.tile_valid[c];
        const int lim = min(kv_valid, c == g ? qi + 1 : kTile);  // keys < lim survive
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = 32 * kh + 8 * (i >> 2) + 4 * hi + (i & 3);
            s[i] = key < lim ? s[i] * scale_log2 : -INFINITY;
        }
    };
    // pass 1: running max and sum of exp2 of every query over its causal keys
    float m = -INFINITY, l = 0.0f;
    for (int c = first; c <= g; ++c) {
        __syncthreads();
        load_k_rows<D>(Kt, k, static_cast<int64_t>(c) * kTile, Hkv, kvh, tid);
        __syncthreads();
        f32x16 s = scores<D>(qf, Kt, kh, l32, hi);
        masked(s, c);
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[i]);
        const float mn = fmaxf(m, mt);
        if (mn > -INFINITY) {
            float add = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) add += exp2f(s[i] - mn);
            l = l * exp2f(m - mn) + add;
            m = mn;
        }
    }
    // merge lanes l and l ^ 32 (same query, other keys), then the two key-half waves
    {
        const float m2 = __shfl_xor(m, 32, 64), l2 = __shfl_xor(l, 32, 64);
        const float mn = fmaxf(m, m2);
        l = (mn == -INFINITY) ? 0.0f : l * exp2f(m - mn) + l2 * exp2f(m2 - mn);
        m = mn;
    }
    if (hi == 0) {
        ml[qh][kh][l32][0] = m;
        ml[qh][kh][l32][1] = l;
    }
    __syncthreads();
    {
        const float m0 = ml[qh][0][l32][0], l0 = ml[qh][0][l32][1];
        const float m1 = ml[qh][1][l32][0], l1 = ml[qh][1][l32][1];
        const float mn = fmaxf(m0, m1);
        l = (mn == -INFINITY) ? 0.0f : l0 * exp2f(m0 - mn) + l1 * exp2f(m1 - mn);
        m = mn;
    }
    const float inv = (qi < q_valid && l > 0.0f) ? 1.0f / l : 0.0f;  // padded queries carry no mass
    // pass 2: every key tile's mass
    float *row = masses + (static_cast<int64_t>(h) * G + g) * RT;
    for (int c = first; c <= g; ++c) {
        __syncthreads();
        load_k_rows<D>(Kt, k, static_cast<int64_t>(c) * kTile, Hkv, kvh, tid);
        __syncthreads();
        f32x16 s = scores<D>(qf, Kt, kh, l32, hi);
        masked(s, c);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc += (s[i] == -INFINITY) ? 0.0f : exp2f(s[i] - m);
        acc = wave_sum(acc * inv);
        if (lane == 0) part[wave] = acc;
        __syncthreads();
        if (tid == 0) row[c - first] = (part[0] + part[1]) + (part[2] + part[3]);
    }
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

__global__ __launch_bounds__(64) void select_bits_kernel(PlanView pv, const float *__restrict__ masses, int RT,
                                                         float p_la, float p_ca, uint32_t *__restrict__ la_out,
                                                         uint32_t *__restrict__ ca_out) {
    __shared__ uint32_t words[72];
    if (!plan_ok(pv)) return;
    const int G = pv.num_tiles;
    const int h = blockIdx.x, d = blockIdx.y, lane = threadIdx.x;
    const int T = pv.doc_tiles[d], t0 = pv.doc_first[d], b = pv.doc_req[d];
    const int first = pv.req_first[b];
    const int dl = pv.req_first_doc[b] + pv.req_ndocs[b] - 1;
    const int doc_end = pv.doc_first[dl] + pv.doc_tiles[dl];  // the request's question starts here
    // LA: one triangle row at a time
    const int law = pv.doc_la_w[d];
    for (int w = lane; w < law; w += 64) words[w] = 0u;
    __syncthreads();
    for (int r = 0; r < T; ++r) {
        const int gq = t0 + r;
        const float mass = lane <= r ? masses[(static_cast<int64_t>(h) * G + gq) * RT + (t0 + lane - first)] : 0.0f;
        const bool keep = top_p_keep(mass, r + 1, p_la, lane) || lane == r || lane == 0;
        if (lane <= r && keep) {
            const int bit = r * (r + 1) / 2 + lane;
            atomicOr(&words[bit >> 5], 1u << (bit & 31));
        }
    }
    __syncthreads();
    uint32_t *la_vec = la_out + pv.doc_la_off[d] + h * law;
    for (int w = lane; w < law; w += 64) la_vec[w] = words[w];
    __syncthreads();
    // CA: page masses from the later documents' query tiles
    const int caw = pv.doc_ca_w[d];
    for (int w = lane; w < caw; w += 64) words[w] = 0u;
    __syncthreads();
    float cm = 0.0f;
    if (lane < T)
        for (int gq = t0 + T; gq < doc_end; ++gq)
            cm += masses[(static_cast<int64_t>(h) * G + gq) * RT + (t0 + lane - first)];
    const bool keep = top_p_keep(cm, T, p_ca, lane) || lane == 0;
    if (lane < T && keep) atomicOr(&words[lane >> 5], 1u << (lane & 31));
    __syncthreads();
    uint32_t *ca_vec = ca_out + pv.doc_ca_off[d] + h * caw;
    for (int w = lane; w < caw; w += 64) ca_vec[w] = words[w];
}

}  // namespace

hipError_t launch_tile_masses(const HostLayout &hl, const PlanView &pv, const uint16_t *q, const uint16_t *k,
                              float scale, float *masses, int RT, hipStream_t stream) {
    if (hl.G == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>(int64_t(hl.Hq) * hl.G);
    const float sl = scale * 1.4426950408889634f;
    if (hl.D == 128)
        tile_mass_kernel<128><<<grid, kEncThreads, 0, stream>>>(pv, q, k, hl.Hq, hl.Hkv, sl, masses, RT);
    else
        tile_mass_kernel<64><<<grid, kEncThreads, 0, stream>>>(pv, q, k, hl.Hq, hl.Hkv, sl, masses, RT);
    return hipGetLastError();
}

hipError_t launch_select_bits(const HostLayout &hl, const PlanView &pv, const float *masses, int RT, float p_la,
                              float p_ca, uint32_t *la_out, uint32_t *ca_out, hipStream_t stream) {
    if (hl.ndocs == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(hl.Hq), static_cast<unsigned>(hl.ndocs));
    select_bits_kernel<<<grid, 64, 0, stream>>>(pv, masses, RT, p_la, p_ca, la_out, ca_out);
    return hipGetLastError();
}

}  // namespace sift
