"""Oracle of the offline encoder (LA/CA bits from dense attention) -- TEST INFRASTRUCTURE.

SIFT technical summary, section 2 "Metodologia" ("Design del Sistema", the offline stage):
each retrieved document is prefilled densely once; the positions with high attention scores
are recorded as two bit vectors per document, layer and head -- Local-Attention (LA) bits for
the tiles of the document's own attention matrix, Cross-Attention (CA) bits for the document's
KV pages that draw attention from other documents.  The pages do not state the selection rule;
the reading used here is:

  * attention is the dense causal attention of the whole request (documents in order, then the
    question), scale 1/sqrt(D), GQA, padded tokens excluded;
  * the mass of tile pair (query tile g, key tile c) is the sum over the valid queries of g and
    the keys of c of the softmax probability;
  * LA row r of document d keeps the smallest set of its candidate tiles c <= r, taken by
    decreasing mass (ties: smaller c first), whose mass reaches p_la of the row's candidate
    mass; the diagonal tile and tile 0 are always kept;
  * CA page c of document d has the mass that the query tiles of the request's later
    documents put on key tile c (summed over those query tiles, in increasing tile order); the
    document keeps the smallest set of pages reaching p_ca of its total the same way; page 0 is
    always kept.

tile_masses() is fp64 and is pinned by the tests (every query's probabilities sum to one, so a
query tile's masses sum to its valid query count; brute force on tiny inputs).  select_bits()
makes integer decisions from floating-point sums, so it runs in float32 with the kernel's
summation order (a Hillis-Steele inclusive scan over 64 sorted slots, a sequential column sum);
it is pinned by hand-worked cases and invariants (forced bits, reached threshold, minimality).
"""
from __future__ import annotations

import numpy as np

TILE = 64


def _segments(case):
    """Per tile: (request, doc or -1, local index); per request: first tile; per doc: first tile, T."""
    tile_req, tile_doc, tile_loc, req_first, doc_first, doc_T = [], [], [], [], [], []
    g = 0
    d = 0
    for b, k in enumerate(case.req_num_docs):
        req_first.append(g)
        for _ in range(int(k)):
            T = -(-int(case.doc_len[d]) // TILE)
            doc_first.append(g)
            doc_T.append(T)
            for r in range(T):
                tile_req.append(b)
                tile_doc.append(d)
                tile_loc.append(r)
            g += T
            d += 1
        Tq = -(-int(case.question_len[b]) // TILE)
        for r in range(Tq):
            tile_req.append(b)
            tile_doc.append(-1)
            tile_loc.append(r)
        g += Tq
    return (np.array(tile_req), np.array(tile_doc), np.array(tile_loc), np.array(req_first),
            np.array(doc_first), np.array(doc_T))


def valid_tokens(case):
    out = []
    d = 0
    for b, k in enumerate(case.req_num_docs):
        for _ in range(int(k)):
            n = int(case.doc_len[d])
            out.extend(x < n for x in range(TILE * (-(-n // TILE))))
            d += 1
        m = int(case.question_len[b])
        out.extend(x < m for x in range(TILE * (-(-m // TILE))))
    return np.array(out, dtype=bool)


def _values(case, x):
    if case.dtype != "bf16":
        raise ValueError("the encoder oracle takes bf16 cases (the kernel's operands)")
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tile_masses(case, scale=None):
    """fp64 masses M[h, g, c] (zero outside a request's causal tile range)."""
    tile_req, _, _, req_first, _, _ = _segments(case)
    G = len(tile_req)
    N = G * TILE
    hq, hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    q = _values(case, case.q)
    k = _values(case, case.k)
    valid = valid_tokens(case)
    M = np.zeros((hq, G, G))
    group = hq // hkv
    for b in range(len(case.req_num_docs)):
        t0 = req_first[b]
        t1 = t0 + int((tile_req == b).sum())
        s0, s1 = t0 * TILE, t1 * TILE
        tok = np.arange(s0, s1)
        ok = valid[s0:s1]
        causal = tok[None, :] <= tok[:, None]
        allowed = causal & ok[None, :] & ok[:, None]
        for h in range(hq):
            s = (q[s0:s1, h, :] @ k[s0:s1, h // group, :].T) * sc
            s = np.where(allowed, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            mx = np.where(np.isfinite(mx), mx, 0.0)
            p = np.exp(s - mx)
            l = p.sum(axis=1, keepdims=True)
            p = np.divide(p, l, out=np.zeros_like(p), where=l > 0)
            nt = t1 - t0
            M[h, t0:t1, t0:t1] = p.reshape(nt, TILE, nt, TILE).sum(axis=(1, 3))
    return M


def tile_mass_row(case, h, g, scale=None):
    """fp64 masses M[h, g, :] of one query tile: the definition of tile_masses evaluated for the
    64 queries of tile g only (so that full-size workloads can be checked on sampled rows)."""
    tile_req, _, _, req_first, _, _ = _segments(case)
    G = len(tile_req)
    t0 = int(req_first[tile_req[g]])
    kvh = h // (case.num_q_heads // case.num_kv_heads)
    sc = 1.0 / np.sqrt(case.head_dim) if scale is None else scale
    s0, q0, s1 = t0 * TILE, g * TILE, (g + 1) * TILE
    q = _values(case, case.q[q0:s1, h, :])
    k = _values(case, case.k[s0:s1, kvh, :])
    valid = valid_tokens(case)
    q_tok = np.arange(q0, s1)
    k_tok = np.arange(s0, s1)
    allowed = (k_tok[None, :] <= q_tok[:, None]) & valid[s0:s1][None, :] & valid[q0:s1][:, None]
    s = np.where(allowed, (q @ k.T) * sc, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    p = np.exp(s - mx)
    l = p.sum(axis=1, keepdims=True)
    p = np.divide(p, l, out=np.zeros_like(p), where=l > 0)
    out = np.zeros(G)
    out[t0:g + 1] = p.reshape(TILE, g + 1 - t0, TILE).sum(axis=(0, 2))
    return out


def _scan64(v):
    """Inclusive Hillis-Steele scan of 64 float32 values (each round adds the value `off` slots
    back, all slots at once)."""
    s = np.asarray(v, dtype=np.float32).copy()
    off = 1
    while off < 64:
        prev = s.copy()
        s[off:] = (prev[off:] + prev[:-off]).astype(np.float32)
        off *= 2
    return s


def select_top_p(masses, p, forced):
    """Indices kept from `masses` (float32, at most 64): sort by decreasing mass, ties by index;
    keep slot i when the scanned mass before it is below p * total; then add `forced`."""
    m = np.asarray(masses, dtype=np.float32)
    n = m.size
    assert n <= 64
    order = sorted(range(n), key=lambda i: (-float(m[i]), i))
    vals = np.zeros(64, np.float32)
    vals[:n] = m[order]
    s = _scan64(vals)
    thr = np.float32(np.float32(p) * s[63])
    keep = set()
    for i in range(n):
        before = np.float32(0.0) if i == 0 else s[i - 1]
        if i == 0 or before < thr:
            keep.add(order[i])
    keep.update(forced)
    return keep


def ca_column_masses(case, M32):
    """float32 CA masses per (h, doc): [sum over later-document query tiles g, in increasing g,
    of M[h, g, first_d + c]] for c < T_d."""
    tile_req, tile_doc, _, req_first, doc_first, doc_T = _segments(case)
    out = []
    hq = case.num_q_heads
    for d in range(len(doc_T)):
        b = tile_req[doc_first[d]]
        later = [g for g in range(len(tile_req)) if tile_req[g] == b and tile_doc[g] > d]
        cm = np.zeros((hq, doc_T[d]), np.float32)
        for g in later:
            cm = (cm + M32[:, g, doc_first[d]:doc_first[d] + doc_T[d]]).astype(np.float32)
        out.append(cm)
    return out


def select_bits(case, M, p_la=0.9, p_ca=0.9):
    """LA / CA booleans (lists per doc of [Hq, T, T] and [Hq, T]) from masses M (used as float32)."""
    M32 = np.asarray(M, dtype=np.float32)
    _, _, _, _, doc_first, doc_T = _segments(case)
    hq = case.num_q_heads
    cms = ca_column_masses(case, M32)
    la, ca = [], []
    for d in range(len(doc_T)):
        T, t0 = int(doc_T[d]), int(doc_first[d])
        la_d = np.zeros((hq, T, T), bool)
        ca_d = np.zeros((hq, T), bool)
        for h in range(hq):
            for r in range(T):
                keep = select_top_p(M32[h, t0 + r, t0:t0 + r + 1], p_la, {0, r})
                la_d[h, r, sorted(keep)] = True
            keep = select_top_p(cms[d][h], p_ca, {0})
            ca_d[h, sorted(keep)] = True
        la.append(la_d)
        ca.append(ca_d)
    return la, ca
