"""Seeded synthetic workloads for bit-vector sparse RAG prefill.

SIFT (Selective-Index For Fast Compute of RAG Prefill by Exploiting Attention
Invariance; technical summary, section 2 "Metodologia", "Design del Sistema")
stores, per document, layer and head, two compact bit vectors: Local-Attention
(LA) bits marking high-score tiles of the document's own self-attention matrix,
and Cross-Attention (CA) bits marking KV pages (columns) of the document that
later co-resident documents attend to.  The pages print no data, so every
workload here is synthetic: N(0,1) post-RoPE Q/K/V and Bernoulli bits.

This module only *draws* inputs and writes them in the packed input format.
It holds none of the decode or attention arithmetic, and both the CPU oracle
and the GPU path read what it produces.  It computes array shapes
(tiles per segment = ceil(len / 64)) and packs its own boolean draws into
uint32 words.

Packed bit format (one layer):
  * LA(d, h; r, c), 0 <= c <= r < T_d, is bit r*(r+1)/2 + c of the vector of
    (doc d, q-head h); CA(d, h; c), 0 <= c < T_d, is bit c of its vector.
  * Bit k sits in word k >> 5 at position k & 31 (LSB first).  Each vector
    starts on a word boundary; unused high bits of the last word are 0.
  * Vectors are laid out doc-major: [global doc][q head][words], where global
    docs run over requests in order.

Token layout: request by request, its documents in order and then its
question; every segment is padded up to a multiple of the 64-token tile.
Q is [N, Hq, D], K and V are [N, Hkv, D], token-major, N = 64 * total tiles.
bf16 values are carried as uint16 bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

TILE = 64

CONFIG_NAMES = {
    1: "tiny",
    2: "llama8b-10x1k",
    3: "llama8b-32x1k",
    4: "qwen3-235b-20x2k",
    5: "ragged-4req",
}


@dataclasses.dataclass
class Case:
    """One synthetic layer of a batched RAG prefill."""

    name: str
    seed: Optional[int]
    req_num_docs: np.ndarray  # int32 [R]
    doc_len: np.ndarray  # int32 [sum docs], unpadded tokens
    question_len: np.ndarray  # int32 [R], unpadded tokens
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" (uint16 bit patterns) or "fp32"
    q: np.ndarray  # [N, Hq, D]
    k: np.ndarray  # [N, Hkv, D]
    v: np.ndarray  # [N, Hkv, D]
    la_bool: List[np.ndarray]  # per global doc: bool [Hq, T, T] (upper triangle False)
    ca_bool: List[np.ndarray]  # per global doc: bool [Hq, T]
    la_words: np.ndarray  # uint32, packed as described in the module docstring
    ca_words: np.ndarray  # uint32
    tile: int = TILE

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def num_tokens_padded(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_docs(self) -> int:
        return int(self.doc_len.shape[0])


# --------------------------------------------------------------------------
# shapes and packing of the generator's own draws
# --------------------------------------------------------------------------

def tiles_of(n_tokens: int) -> int:
    return -(-int(n_tokens) // TILE)


def padded_total(req_num_docs, doc_len, question_len) -> int:
    return TILE * (sum(tiles_of(n) for n in doc_len) + sum(tiles_of(m) for m in question_len))


def _pack_bool_bits(bits: np.ndarray) -> np.ndarray:
    """Pack a 1-D bool array LSB-first into uint32 words (zero-filled tail)."""
    nbits = bits.shape[0]
    nwords = -(-nbits // 32)
    padded = np.zeros(nwords * 32, dtype=np.uint8)
    padded[:nbits] = bits
    by = np.packbits(padded, bitorder="little")
    return by.view("<u4").astype(np.uint32)


def pack_bits(la_bool: Sequence[np.ndarray], ca_bool: Sequence[np.ndarray]):
    """Pack per-doc boolean LA [Hq,T,T] and CA [Hq,T] draws into the word format."""
    la_parts, ca_parts = [], []
    for la, ca in zip(la_bool, ca_bool):
        hq, t, _ = la.shape
        rows, cols = np.tril_indices(t)  # row-major lower triangle incl. diagonal
        for h in range(hq):
            la_parts.append(_pack_bool_bits(la[h][rows, cols]))
            ca_parts.append(_pack_bool_bits(ca[h]))
    la_words = np.concatenate(la_parts) if la_parts else np.zeros(0, np.uint32)
    ca_words = np.concatenate(ca_parts) if ca_parts else np.zeros(0, np.uint32)
    return la_words.astype(np.uint32), ca_words.astype(np.uint32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def _draw_values(rng, n_tokens, heads, dim, as_bf16, chunk=4096):
    """N(0,1) fp32 values drawn in token chunks (same stream as one draw of the whole)."""
    out = np.empty((n_tokens, heads, dim), dtype=np.uint16 if as_bf16 else np.float32)
    for s in range(0, n_tokens, chunk):
        e = min(n_tokens, s + chunk)
        x = rng.standard_normal((e - s, heads, dim), dtype=np.float32)
        out[s:e] = f32_to_bf16_bits(x) if as_bf16 else x
    return out


def _draw_la(rng, t, hq, p_per_head):
    """Bernoulli(p_h) over the lower triangle incl. diagonal, then diagonal forced on."""
    la = np.zeros((hq, t, t), dtype=bool)
    rows, cols = np.tril_indices(t)
    for h in range(hq):
        la[h][rows, cols] = rng.random(rows.shape[0]) < p_per_head[h]
        la[h][np.arange(t), np.arange(t)] = True
    return la


def _draw_ca(rng, t, hq, p_per_head):
    """Bernoulli(p_h) over the doc's pages, then page 0 forced on."""
    ca = np.zeros((hq, t), dtype=bool)
    for h in range(hq):
        ca[h] = rng.random(t) < p_per_head[h]
        ca[h][0] = True
    return ca


def make_case(name, seed, req_num_docs, doc_len, question_len, hq, hkv, d,
              la_p, ca_p, dtype="bf16", rng=None) -> Case:
    """Draw Q, K, V, then LA, then CA for a given layout.

    la_p / ca_p: arrays [R, Hq] of per-(request, q head) Bernoulli densities.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    req_num_docs = np.asarray(req_num_docs, dtype=np.int32)
    doc_len = np.asarray(doc_len, dtype=np.int32)
    question_len = np.asarray(question_len, dtype=np.int32)
    n = padded_total(req_num_docs, doc_len, question_len)
    as_bf16 = dtype == "bf16"
    q = _draw_values(rng, n, hq, d, as_bf16)
    k = _draw_values(rng, n, hkv, d, as_bf16)
    v = _draw_values(rng, n, hkv, d, as_bf16)
    doc_req = np.repeat(np.arange(len(req_num_docs)), req_num_docs)
    la_p = np.asarray(la_p, dtype=np.float64).reshape(len(req_num_docs), hq)
    ca_p = np.asarray(ca_p, dtype=np.float64).reshape(len(req_num_docs), hq)
    la_bool = [_draw_la(rng, tiles_of(n_d), hq, la_p[doc_req[i]]) for i, n_d in enumerate(doc_len)]
    ca_bool = [_draw_ca(rng, tiles_of(n_d), hq, ca_p[doc_req[i]]) for i, n_d in enumerate(doc_len)]
    la_words, ca_words = pack_bits(la_bool, ca_bool)
    return Case(name=name, seed=seed, req_num_docs=req_num_docs, doc_len=doc_len,
                question_len=question_len, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                dtype=dtype, q=q, k=k, v=v, la_bool=la_bool, ca_bool=ca_bool,
                la_words=la_words, ca_words=ca_words)


def _uniform_case(cid, ndocs, doc_tokens, q_tokens, hq, hkv, d, la_p, ca_p, dtype="bf16"):
    seed = cid - 1
    return make_case(CONFIG_NAMES[cid], seed, [ndocs], [doc_tokens] * ndocs, [q_tokens],
                     hq, hkv, d, np.full((1, hq), la_p), np.full((1, hq), ca_p), dtype)


def _ragged_case(cid=5, num_requests=4, max_request_tokens=65536):
    """Ragged batch: per request k~U{16..40} docs with lengths U{300..3000},
    question U{64..512}; docs are kept in draw order while the request's padded
    total (docs + question) stays <= max_request_tokens.  Per (request, q head)
    LA and CA densities ~ Beta(2, 8)."""
    seed = cid - 1
    rng = np.random.default_rng(seed)
    hq, hkv, d = 32, 8, 128
    req_num_docs, doc_len, question_len = [], [], []
    for _ in range(num_requests):
        k = int(rng.integers(16, 41))
        m = int(rng.integers(64, 513))
        lens = rng.integers(300, 3001, size=k)
        total = TILE * tiles_of(m)
        kept = []
        for n_d in lens:
            if total + TILE * tiles_of(int(n_d)) > max_request_tokens:
                break
            total += TILE * tiles_of(int(n_d))
            kept.append(int(n_d))
        req_num_docs.append(len(kept))
        doc_len.extend(kept)
        question_len.append(m)
    la_p = rng.beta(2.0, 8.0, size=(num_requests, hq))
    ca_p = rng.beta(2.0, 8.0, size=(num_requests, hq))
    return make_case(CONFIG_NAMES[cid], seed, req_num_docs, doc_len, question_len,
                     hq, hkv, d, la_p, ca_p, "bf16", rng=rng)


def config_layout(cid: int):
    """(req_num_docs, doc_len, question_len, Hq, Hkv, D) of a workload, without drawing values."""
    if cid == 5:
        rng = np.random.default_rng(cid - 1)
        req_num_docs, doc_len, question_len = [], [], []
        for _ in range(4):
            k = int(rng.integers(16, 41))
            m = int(rng.integers(64, 513))
            lens = rng.integers(300, 3001, size=k)
            total = TILE * tiles_of(m)
            kept = []
            for n_d in lens:
                if total + TILE * tiles_of(int(n_d)) > 65536:
                    break
                total += TILE * tiles_of(int(n_d))
                kept.append(int(n_d))
            req_num_docs.append(len(kept))
            doc_len.extend(kept)
            question_len.append(m)
        return req_num_docs, doc_len, question_len, 32, 8, 128
    shapes = {1: (2, 256, 64, 1, 1, 64), 2: (10, 1024, 128, 32, 8, 128),
              3: (32, 1024, 256, 32, 8, 128), 4: (20, 2048, 256, 64, 4, 128)}
    nd, n, m, hq, hkv, d = shapes[cid]
    return [nd], [n] * nd, [m], hq, hkv, d


def config_case(cid: int) -> Case:
    """The five workloads (1 = tiny ... 5 = ragged batch); seed = id - 1."""
    if cid == 1:
        return _uniform_case(1, 2, 256, 64, 1, 1, 64, 0.5, 0.5, dtype="fp32")
    if cid == 2:
        return _uniform_case(2, 10, 1024, 128, 32, 8, 128, 0.25, 0.20)
    if cid == 3:
        return _uniform_case(3, 32, 1024, 256, 32, 8, 128, 0.15, 0.10)
    if cid == 4:
        return _uniform_case(4, 20, 2048, 256, 64, 4, 128, 0.12, 0.08)
    if cid == 5:
        return _ragged_case(5)
    raise ValueError(f"unknown config id {cid}")


def random_small_case(seed, max_requests=2, max_docs=3, max_tiles=4, hq=2, hkv=1, d=16,
                      aligned=False, dtype="bf16", la_p=None, ca_p=None) -> Case:
    """Tiny random layouts for brute-force checks (ragged lengths unless aligned)."""
    rng = np.random.default_rng(10_000 + seed)
    r = int(rng.integers(1, max_requests + 1))
    req_num_docs, doc_len, question_len = [], [], []
    for _ in range(r):
        k = int(rng.integers(1, max_docs + 1))
        req_num_docs.append(k)
        for _ in range(k):
            t = int(rng.integers(1, max_tiles + 1))
            doc_len.append(TILE * t if aligned else int(rng.integers(TILE * (t - 1) + 1, TILE * t + 1)))
        qt = int(rng.integers(0, 3))
        question_len.append(TILE * qt if aligned else (0 if qt == 0 else int(rng.integers(1, TILE * qt + 1))))
    la = rng.random((r, hq)) if la_p is None else np.full((r, hq), la_p)
    ca = rng.random((r, hq)) if ca_p is None else np.full((r, hq), ca_p)
    return make_case(f"small-{seed}", 10_000 + seed, req_num_docs, doc_len, question_len,
                     hq, hkv, d, la, ca, dtype, rng=rng)


def layer_bits(case: Case, layer: int, la_p, ca_p):
    """LA/CA bits of another layer on the same layout: the same draw as make_case (Bernoulli per
    (request, q head) density, diagonal and page 0 forced) from the stream seeded by
    (case seed, layer).  la_p / ca_p: scalars or arrays [R, Hq].  Returns (la_bool, ca_bool)."""
    rng = np.random.default_rng([int(case.seed), 7919, int(layer)])
    R, hq = len(case.req_num_docs), case.num_q_heads
    la_p = np.broadcast_to(np.asarray(la_p, dtype=np.float64), (R, hq))
    ca_p = np.broadcast_to(np.asarray(ca_p, dtype=np.float64), (R, hq))
    doc_req = np.repeat(np.arange(R), case.req_num_docs)
    la = [_draw_la(rng, tiles_of(int(n_d)), hq, la_p[doc_req[i]]) for i, n_d in enumerate(case.doc_len)]
    ca = [_draw_ca(rng, tiles_of(int(n_d)), hq, ca_p[doc_req[i]]) for i, n_d in enumerate(case.doc_len)]
    return la, ca


def with_bits(case: Case, la_bool, ca_bool) -> Case:
    """Same layout and values, other bits (used to build the special cases)."""
    la_words, ca_words = pack_bits(la_bool, ca_bool)
    return dataclasses.replace(case, la_bool=list(la_bool), ca_bool=list(ca_bool),
                               la_words=la_words, ca_words=ca_words)


def all_ones_bits(case: Case):
    la = [np.tril(np.ones_like(x)) for x in case.la_bool]
    ca = [np.ones_like(x) for x in case.ca_bool]
    return la, ca
