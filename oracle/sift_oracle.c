/*
 * CPU oracle for bit-vector sparse RAG prefill (SIFT).  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code with the GPU path.
 *
 * What it computes (SIFT technical summary, section 2 "Metodologia":
 * "Design del Sistema" and "Dettagli di Implementazione"): the decode kernel
 * turns the per-document, per-head Local-Attention (LA) and Cross-Attention (CA)
 * bit vectors into explicit tile indices, and the sparse attention kernel
 * evaluates scores for the marked tiles and pages alone.  Once the bits are
 * fixed, that result is exactly a masked softmax attention, so this oracle is
 * the plain definition:
 *
 *   1. layout: requests in order; in each, documents then the question, every
 *      segment padded to a multiple of the 64-token tile;
 *   2. decode, in plain nested loops: a row (head h, global tile g) of
 *      document d lists the CA pages of the earlier documents of its request
 *      (CA marks the KV pages of a document that other, later documents attend
 *      to; read as: visited by every later document), then the LA tiles c <= r of its own
 *      row r; a question tile lists every tile of its request up to itself;
 *   3. attention, per (head, valid query token i): the key set is every valid
 *      token j <= i of a listed tile; s_ij = scale * <q_i, k_j> in fp64 from
 *      the exact bf16 values; two passes: M = max s, then
 *      O = sum e^(s-M) v / sum e^(s-M), LSE = M + ln sum e^(s-M).
 *      Empty key sets and padded query tokens give O = 0, LSE = -inf.
 *
 * Bit format: LA(d,h; r,c) is bit r(r+1)/2 + c of the (d,h) vector, CA(d,h; c)
 * is bit c; bit k is in word k>>5 at position k&31; vectors are word aligned
 * and stored [doc][head][words].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_TILE 64

typedef struct {
    int32_t is_question; /* 0: document tile, 1: question tile */
    int32_t doc;         /* global document index (documents only) */
    int32_t local;       /* tile index inside its segment */
    int32_t seg_first;   /* global index of the segment's first tile */
    int32_t seg_tiles;
    int32_t seg_len;     /* unpadded tokens in the segment */
    int32_t req_first;   /* global index of the request's first tile */
    int32_t req_first_doc;
} oracle_tile;

typedef struct {
    int64_t num_tiles;
    int32_t num_docs;
    oracle_tile *tiles;
    int32_t *doc_first_tile; /* [num_docs] */
    int32_t *doc_tiles;      /* [num_docs] */
    int64_t *la_off;         /* [num_docs]: word offset of (doc, head 0) */
    int64_t *ca_off;
    int64_t *la_vec_words;   /* words per (doc, head) LA vector */
    int64_t *ca_vec_words;
} oracle_layout;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void layout_free(oracle_layout *L) {
    free(L->tiles); free(L->doc_first_tile); free(L->doc_tiles);
    free(L->la_off); free(L->ca_off); free(L->la_vec_words); free(L->ca_vec_words);
    memset(L, 0, sizeof(*L));
}

/* Returns 0 on success. */
static int layout_build(oracle_layout *L, int32_t num_requests, const int32_t *req_num_docs,
                        const int32_t *doc_len, const int32_t *question_len, int32_t num_q_heads) {
    memset(L, 0, sizeof(*L));
    int64_t nd = 0, nt = 0;
    for (int32_t b = 0; b < num_requests; ++b) {
        if (req_num_docs[b] < 0 || question_len[b] < 0) return -1;
        for (int32_t i = 0; i < req_num_docs[b]; ++i) {
            if (doc_len[nd] < 1) return -1;
            nt += ceil_div(doc_len[nd], ORACLE_TILE);
            ++nd;
        }
        nt += ceil_div(question_len[b], ORACLE_TILE);
    }
    L->num_tiles = nt;
    L->num_docs = (int32_t)nd;
    L->tiles = (oracle_tile *)calloc((size_t)(nt > 0 ? nt : 1), sizeof(oracle_tile));
    L->doc_first_tile = (int32_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int32_t));
    L->doc_tiles = (int32_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int32_t));
    L->la_off = (int64_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int64_t));
    L->ca_off = (int64_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int64_t));
    L->la_vec_words = (int64_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int64_t));
    L->ca_vec_words = (int64_t *)calloc((size_t)(nd > 0 ? nd : 1), sizeof(int64_t));
    int64_t g = 0, d = 0, la_acc = 0, ca_acc = 0;
    for (int32_t b = 0; b < num_requests; ++b) {
        int32_t req_first = (int32_t)g;
        int32_t first_doc = (int32_t)d;
        for (int32_t i = 0; i < req_num_docs[b]; ++i, ++d) {
            int64_t T = ceil_div(doc_len[d], ORACLE_TILE);
            L->doc_first_tile[d] = (int32_t)g;
            L->doc_tiles[d] = (int32_t)T;
            L->la_vec_words[d] = ceil_div(T * (T + 1) / 2, 32);
            L->ca_vec_words[d] = ceil_div(T, 32);
            L->la_off[d] = la_acc;
            L->ca_off[d] = ca_acc;
            la_acc += (int64_t)num_q_heads * L->la_vec_words[d];
            ca_acc += (int64_t)num_q_heads * L->ca_vec_words[d];
            for (int64_t r = 0; r < T; ++r, ++g) {
                oracle_tile *t = &L->tiles[g];
                t->is_question = 0; t->doc = (int32_t)d; t->local = (int32_t)r;
                t->seg_first = L->doc_first_tile[d]; t->seg_tiles = (int32_t)T;
                t->seg_len = doc_len[d]; t->req_first = req_first; t->req_first_doc = first_doc;
            }
        }
        int64_t TQ = ceil_div(question_len[b], ORACLE_TILE);
        int32_t qfirst = (int32_t)g;
        for (int64_t r = 0; r < TQ; ++r, ++g) {
            oracle_tile *t = &L->tiles[g];
            t->is_question = 1; t->doc = -1; t->local = (int32_t)r;
            t->seg_first = qfirst; t->seg_tiles = (int32_t)TQ;
            t->seg_len = question_len[b]; t->req_first = req_first; t->req_first_doc = first_doc;
        }
    }
    return 0;
}

static int get_bit(const uint32_t *words, int64_t k) {
    return (int)((words[k >> 5] >> (k & 31)) & 1u);
}

static int la_bit(const oracle_layout *L, const uint32_t *la, int32_t d, int32_t h, int64_t r, int64_t c) {
    const uint32_t *vec = la + L->la_off[d] + (int64_t)h * L->la_vec_words[d];
    return get_bit(vec, r * (r + 1) / 2 + c);
}

static int ca_bit(const oracle_layout *L, const uint32_t *ca, int32_t d, int32_t h, int64_t c) {
    const uint32_t *vec = ca + L->ca_off[d] + (int64_t)h * L->ca_vec_words[d];
    return get_bit(vec, c);
}

/* Decode one row (head h, global tile g); writes its tiles to out (if non-NULL), returns count. */
static int64_t decode_row(const oracle_layout *L, const uint32_t *la, const uint32_t *ca,
                          int32_t h, int64_t g, int32_t *out) {
    const oracle_tile *t = &L->tiles[g];
    int64_t n = 0;
    if (t->is_question) {
        for (int64_t c = t->req_first; c <= g; ++c) {
            if (out) out[n] = (int32_t)c;
            ++n;
        }
        return n;
    }
    for (int32_t i = t->req_first_doc; i < t->doc; ++i) {
        for (int64_t c = 0; c < L->doc_tiles[i]; ++c) {
            if (ca_bit(L, ca, i, h, c)) {
                if (out) out[n] = (int32_t)(L->doc_first_tile[i] + c);
                ++n;
            }
        }
    }
    for (int64_t c = 0; c <= t->local; ++c) {
        if (la_bit(L, la, t->doc, h, t->local, c)) {
            if (out) out[n] = (int32_t)(t->seg_first + c);
            ++n;
        }
    }
    return n;
}

/* ---------------------------------------------------------------- exported */

int64_t sift_oracle_num_tiles(int32_t num_requests, const int32_t *req_num_docs,
                              const int32_t *doc_len, const int32_t *question_len) {
    oracle_layout L;
    if (layout_build(&L, num_requests, req_num_docs, doc_len, question_len, 1) != 0) return -1;
    int64_t g = L.num_tiles;
    layout_free(&L);
    return g;
}

/* Row counts only: counts[h*G + g].  Returns nnz or -1. */
int64_t sift_oracle_row_counts(int32_t num_requests, const int32_t *req_num_docs,
                               const int32_t *doc_len, const int32_t *question_len,
                               int32_t num_q_heads, const uint32_t *la, const uint32_t *ca,
                               int64_t *counts) {
    oracle_layout L;
    if (layout_build(&L, num_requests, req_num_docs, doc_len, question_len, num_q_heads) != 0) return -1;
    int64_t G = L.num_tiles, nnz = 0;
    for (int32_t h = 0; h < num_q_heads; ++h)
        for (int64_t g = 0; g < G; ++g) {
            int64_t c = decode_row(&L, la, ca, h, g, NULL);
            counts[h * G + g] = c;
            nnz += c;
        }
    layout_free(&L);
    return nnz;
}

/* Full CSR: row_ptr [Hq*G+1] (int64), col_idx [cap].  Returns nnz, -1 on bad
 * layout, -2 if cap is too small. */
int64_t sift_oracle_decode(int32_t num_requests, const int32_t *req_num_docs,
                           const int32_t *doc_len, const int32_t *question_len,
                           int32_t num_q_heads, const uint32_t *la, const uint32_t *ca,
                           int64_t *row_ptr, int32_t *col_idx, int64_t cap) {
    oracle_layout L;
    if (layout_build(&L, num_requests, req_num_docs, doc_len, question_len, num_q_heads) != 0) return -1;
    int64_t G = L.num_tiles, pos = 0;
    row_ptr[0] = 0;
    for (int32_t h = 0; h < num_q_heads; ++h)
        for (int64_t g = 0; g < G; ++g) {
            int64_t c = decode_row(&L, la, ca, h, g, NULL);
            if (pos + c > cap) { layout_free(&L); return -2; }
            decode_row(&L, la, ca, h, g, col_idx + pos);
            pos += c;
            row_ptr[h * G + g + 1] = pos;
        }
    layout_free(&L);
    return pos;
}

/* fp32 -> bf16, round to nearest even (finite inputs), as the bf16 value widened back. */
static double bf16_round(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    float y;
    memcpy(&y, &u, 4);
    return (double)y;
}

static double bf16_bits_value(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float y;
    memcpy(&y, &u, 4);
    return (double)y;
}

/* dtype: 0 = bf16 bit patterns, 1 = fp32 rounded to bf16 first, 2 = fp32 taken exactly. */
static double load_value(const void *base, int dtype, int64_t idx) {
    if (dtype == 0) return bf16_bits_value(((const uint16_t *)base)[idx]);
    if (dtype == 1) return bf16_round(((const float *)base)[idx]);
    return (double)((const float *)base)[idx];
}

static int token_valid(const oracle_layout *L, int64_t tok) {
    const oracle_tile *t = &L->tiles[tok / ORACLE_TILE];
    return (int64_t)t->local * ORACLE_TILE + (tok % ORACLE_TILE) < t->seg_len;
}

/*
 * Attention for npairs (head, padded token) pairs.  out [npairs][head_dim] and
 * lse [npairs] in fp64 (lse may be NULL).  q [N][Hq][D], k and v [N][Hkv][D].
 * Returns 0, or -1 on a bad layout or pair.
 */
int sift_oracle_attention(int32_t num_requests, const int32_t *req_num_docs,
                          const int32_t *doc_len, const int32_t *question_len,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t dtype, const void *q, const void *k, const void *v,
                          const uint32_t *la, const uint32_t *ca, double scale,
                          int64_t npairs, const int32_t *pair_head, const int64_t *pair_token,
                          double *out, double *lse, int32_t num_threads) {
    oracle_layout L;
    if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads != 0 || head_dim < 1) return -1;
    if (layout_build(&L, num_requests, req_num_docs, doc_len, question_len, num_q_heads) != 0) return -1;
    const int64_t G = L.num_tiles, N = G * ORACLE_TILE;
    const int32_t group = num_q_heads / num_kv_heads;
    for (int64_t p = 0; p < npairs; ++p)
        if (pair_head[p] < 0 || pair_head[p] >= num_q_heads || pair_token[p] < 0 || pair_token[p] >= N) {
            layout_free(&L);
            return -1;
        }
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        int32_t *row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(G > 0 ? G : 1));
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *qi = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!row || !keys || !s || !qi) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t p = 0; p < npairs; ++p) {
                const int32_t h = pair_head[p];
                const int64_t i = pair_token[p];
                double *o = out + p * head_dim;
                for (int32_t x = 0; x < head_dim; ++x) o[x] = 0.0;
                if (lse) lse[p] = -INFINITY;
                if (!token_valid(&L, i)) continue;
                const int32_t hk = h / group;
                const int64_t nrow = decode_row(&L, la, ca, h, i / ORACLE_TILE, row);
                int64_t nk = 0;
                for (int64_t e = 0; e < nrow; ++e)
                    for (int64_t j = (int64_t)row[e] * ORACLE_TILE; j < (int64_t)(row[e] + 1) * ORACLE_TILE; ++j)
                        if (j <= i && token_valid(&L, j)) keys[nk++] = j;
                if (nk == 0) continue;
                for (int32_t x = 0; x < head_dim; ++x)
                    qi[x] = load_value(q, dtype, (i * num_q_heads + h) * head_dim + x);
                double m = -INFINITY;
                for (int64_t e = 0; e < nk; ++e) {
                    const int64_t kb = (keys[e] * num_kv_heads + hk) * head_dim;
                    double dot = 0.0;
                    for (int32_t x = 0; x < head_dim; ++x) dot += qi[x] * load_value(k, dtype, kb + x);
                    s[e] = scale * dot;
                    if (s[e] > m) m = s[e];
                }
                double z = 0.0;
                for (int64_t e = 0; e < nk; ++e) {
                    const double w = exp(s[e] - m);
                    z += w;
                    const int64_t vb = (keys[e] * num_kv_heads + hk) * head_dim;
                    for (int32_t x = 0; x < head_dim; ++x) o[x] += w * load_value(v, dtype, vb + x);
                }
                for (int32_t x = 0; x < head_dim; ++x) o[x] /= z;
                if (lse) lse[p] = m + log(z);
            }
        }
        free(row); free(keys); free(s); free(qi);
    }
    layout_free(&L);
    return failed ? -1 : 0;
}

int32_t sift_oracle_max_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
