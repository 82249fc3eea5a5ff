"""Independent test-side readings of the layout and of the visibility predicate.

Written from the definitions (SIFT technical summary, section 2: LA bits mark
high-score tiles of a document's own self-attention, CA bits mark KV pages of a
document that later documents attend to; the question attends densely and
causally), straight from the generator's boolean draws -- not from packed
words and not from any CSR -- so that they pin the oracle rather than restate it.
"""
from __future__ import annotations

import numpy as np

TILE = 64


class TokenMap:
    """Per padded token: request, segment kind, document, tile, validity."""

    def __init__(self, case):
        req, kind, doc, local_tile, valid, tile_first = [], [], [], [], [], []
        self.doc_first_tile = []
        self.doc_tiles = []
        self.req_first_tile = []
        self.req_docs = []
        g = 0
        d = 0
        for b, ndocs in enumerate(case.req_num_docs):
            self.req_first_tile.append(g)
            docs = []
            for _ in range(int(ndocs)):
                n = int(case.doc_len[d])
                t = -(-n // TILE)
                self.doc_first_tile.append(g)
                self.doc_tiles.append(t)
                docs.append(d)
                for x in range(t * TILE):
                    req.append(b); kind.append(0); doc.append(d); local_tile.append(x // TILE)
                    valid.append(x < n); tile_first.append(g)
                g += t
                d += 1
            self.req_docs.append(docs)
            m = int(case.question_len[b])
            tq = -(-m // TILE)
            for x in range(tq * TILE):
                req.append(b); kind.append(1); doc.append(-1); local_tile.append(x // TILE)
                valid.append(x < m); tile_first.append(g)
            g += tq
        self.num_tiles = g
        self.req = np.array(req, dtype=np.int64)
        self.kind = np.array(kind, dtype=np.int64)
        self.doc = np.array(doc, dtype=np.int64)
        self.local_tile = np.array(local_tile, dtype=np.int64)
        self.valid = np.array(valid, dtype=bool)
        self.n = len(req)

    def tile_of_token(self, i):
        return i // TILE


def visible(case, tm: TokenMap, h: int, i: int, j: int) -> bool:
    """Definition of 'query token i of head h sees key token j'."""
    if not (tm.valid[i] and tm.valid[j]) or j > i or tm.req[i] != tm.req[j]:
        return False
    if tm.kind[i] == 1:  # question: dense causal over its request
        return True
    d, dj = tm.doc[i], tm.doc[j]
    if tm.kind[j] == 1:
        return False
    r, c = tm.local_tile[i], tm.local_tile[j]
    if dj == d:
        return bool(case.la_bool[d][h][r, c])
    if dj < d:
        return bool(case.ca_bool[dj][h][c])
    return False


def tile_visible(case, tm: TokenMap, h: int, a: int, b: int) -> bool:
    """Tile-level predicate: may query tile a of head h look at key tile b (before causal/padding)?"""
    i, j = a * TILE, b * TILE  # first token of each tile carries the tile's segment data
    if b > a or tm.req[i] != tm.req[j]:
        return False
    if tm.kind[i] == 1:
        return True
    if tm.kind[j] == 1:
        return False
    d, dj = tm.doc[i], tm.doc[j]
    r, c = tm.local_tile[i], tm.local_tile[j]
    if dj == d:
        return bool(case.la_bool[d][h][r, c])
    if dj < d:
        return bool(case.ca_bool[dj][h][c])
    return False


def mask_matrix(case, tm: TokenMap, h: int) -> np.ndarray:
    """Full N x N boolean mask from the bit predicates (tiny cases only)."""
    g = tm.num_tiles
    tmask = np.array([[tile_visible(case, tm, h, a, b) for b in range(g)] for a in range(g)],
                     dtype=bool).reshape(g, g)
    n = tm.n
    idx = np.arange(n)
    m = tmask[idx[:, None] // TILE, idx[None, :] // TILE]
    m &= tm.valid[:, None] & tm.valid[None, :] & (idx[None, :] <= idx[:, None])
    return m


def values_f64(case, x):
    if case.dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)


def dense_masked_attention(case, tm: TokenMap, qf, kf, vf, masks):
    """numpy fp64 softmax(scale QK^T masked) V per head; empty/invalid rows give 0."""
    n, hq, d = qf.shape
    group = hq // case.num_kv_heads
    out = np.zeros((n, hq, d))
    lse = np.full((hq, n), -np.inf)
    for h in range(hq):
        s = case.scale * qf[:, h, :] @ kf[:, h // group, :].T
        m = masks[h]
        s = np.where(m, s, -np.inf)
        has = m.any(axis=1)
        mx = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
        w = np.where(m, np.exp(s - mx[:, None]), 0.0)
        z = w.sum(axis=1)
        o = np.zeros((n, d))
        o[has] = (w[has] @ vf[:, h // group, :]) / z[has, None]
        out[:, h, :] = o
        lse[h, has] = mx[has] + np.log(z[has])
    return out, lse


def expected_counts_closed_form(case, tm: TokenMap):
    """Row length = popcount(LA row r) + sum of popcount(CA) of earlier docs; question: g - first + 1."""
    hq, g_total = case.num_q_heads, tm.num_tiles
    counts = np.zeros(hq * g_total, dtype=np.int64)
    for h in range(hq):
        g = 0
        for b, docs in enumerate(tm.req_docs):
            first = tm.req_first_tile[b]
            prefix = 0
            for d in docs:
                for r in range(tm.doc_tiles[d]):
                    counts[h * g_total + g] = prefix + int(case.la_bool[d][h][r, : r + 1].sum())
                    g += 1
                prefix += int(case.ca_bool[d][h].sum())
            tq = -(-int(case.question_len[b]) // TILE)
            for _ in range(tq):
                counts[h * g_total + g] = g - first + 1
                g += 1
    return counts
