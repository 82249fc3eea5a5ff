"""Oracle of the offline encoder (LA/CA bits from dense attention) -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this module;
the product path never does, and it shares no code with the GPU library.

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
    documents put on key tile c; the document keeps the smallest set of pages reaching p_ca of
    its total the same way; page 0 is always kept.

Everything here is fp64 and follows that reading literally: tile_masses() evaluates the
softmax of every request and head at once, tile_masses_by_tile() the same definition one
query tile at a time (each query's softmax is independent of the others, so the two agree;
the second is what the full-size checks use), select_top_p() sorts, accumulates the sorted
masses with exactly rounded sums (math.fsum) and cuts at the first prefix that reaches
p x total.  The pins are in the tests (probabilities of every query sum to one, uniform
attention for Q = 0, torch's fp64 SDPA on V = identity, hand-worked selections, minimality).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

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


def tile_masses_by_tile(case, scale=None, threads=None):
    """fp64 masses M[h, g, c] of every row, evaluated one (query tile, KV head) at a time: the
    queries of tile g of the q heads that read one KV head, against the keys of g's request up
    to tile g.  The same definition as tile_masses (a per-query softmax over the valid causal
    keys, probabilities summed over 64 x 64 tile pairs); this form needs memory for one tile's
    scores only, and the tiles run on a thread pool (numpy releases the GIL in its kernels)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    tile_req, _, _, req_first, _, _ = _segments(case)
    G = len(tile_req)
    hq, hkv, D = case.num_q_heads, case.num_kv_heads, case.head_dim
    group = hq // hkv
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    valid = valid_tokens(case)
    k_all = [_values(case, case.k[:, j, :]) for j in range(hkv)]  # [N, D] per KV head
    M = np.zeros((hq, G, G))

    def one(task):
        g, j = task
        t0 = int(req_first[tile_req[g]])
        s0, q0, s1 = t0 * TILE, g * TILE, (g + 1) * TILE
        heads = range(j * group, (j + 1) * group)
        q = np.concatenate([_values(case, case.q[q0:s1, h, :]) for h in heads])  # [group*64, D]
        s = q @ k_all[j][s0:s1].T                                                 # [group*64, L]
        s *= sc
        # keys a query may not see: padded keys anywhere, and later keys of its own tile
        s[:, ~valid[s0:s1]] = -np.inf
        qpos = np.tile(np.arange(TILE), group)
        s[:, q0 - s0:] = np.where(np.arange(TILE)[None, :] <= qpos[:, None], s[:, q0 - s0:], -np.inf)
        mx = s.max(axis=1, keepdims=True)
        mx[~np.isfinite(mx)] = 0.0
        s -= mx
        np.exp(s, out=s)                                       # e^(s - max), 0 for hidden keys
        l = s.sum(axis=1)
        nt = g + 1 - t0
        per_tile = s.reshape(group * TILE, nt, TILE).sum(axis=2)  # [group*64, nt]: sum of e^ per key tile
        q_ok = np.tile(valid[q0:s1], group) & (l > 0)
        per_tile[q_ok] /= l[q_ok, None]                        # probabilities summed per key tile
        per_tile[~q_ok] = 0.0                                  # padded queries carry no mass
        blk = per_tile.reshape(group, TILE, nt).sum(axis=1)    # [group, nt]
        for i, h in enumerate(heads):
            M[h, g, t0:g + 1] = blk[i]

    tasks = [(g, j) for g in range(G) for j in range(hkv)]
    nthreads = threads or max(1, min(16, len(__import__("os").sched_getaffinity(0))))
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            with ThreadPoolExecutor(max_workers=nthreads) as ex:
                list(ex.map(one, tasks))
    else:  # pragma: no cover
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one, tasks))
    return M


def sorted_candidates(masses):
    """Candidate indices by decreasing mass, ties by smaller index."""
    m = np.asarray(masses, dtype=np.float64)
    return sorted(range(m.size), key=lambda i: (-float(m[i]), i))


def top_p_count(masses, p):
    """k*: the length of the shortest prefix of the sorted candidates whose mass (an exactly
    rounded sum) reaches p x total (total exactly rounded too); at least 1 when there is a
    candidate.  Returns (k*, order)."""
    m = np.asarray(masses, dtype=np.float64)
    order = sorted_candidates(m)
    if m.size == 0:
        return 0, order
    thr = float(p) * math.fsum(m.tolist())
    vals = [float(m[i]) for i in order]
    for k in range(1, len(vals) + 1):
        if math.fsum(vals[:k]) >= thr:
            return k, order
    return len(vals), order


def select_top_p(masses, p, forced):
    """Indices kept from `masses`: the shortest prefix of the candidates sorted by decreasing
    mass (ties: smaller index) that reaches p of their total, then `forced` added."""
    k, order = top_p_count(masses, p)
    return set(order[:k]) | set(forced)


def ca_column_masses(case, M):
    """fp64 CA masses per doc, [Hq, T_d]: page c of doc d gets sum over the query tiles g of the
    request's later documents of M[h, g, first_d + c]."""
    tile_req, tile_doc, _, req_first, doc_first, doc_T = _segments(case)
    out = []
    for d in range(len(doc_T)):
        b = tile_req[doc_first[d]]
        later = [g for g in range(len(tile_req)) if tile_req[g] == b and tile_doc[g] > d]
        cols = slice(doc_first[d], doc_first[d] + doc_T[d])
        cm = np.asarray(M, dtype=np.float64)[:, later, cols].sum(axis=1) if later else \
            np.zeros((case.num_q_heads, doc_T[d]))
        out.append(cm)
    return out


def select_bits(case, M, p_la=0.9, p_ca=0.9):
    """LA / CA booleans (lists per doc of [Hq, T, T] and [Hq, T]) from fp64 masses M."""
    M = np.asarray(M, dtype=np.float64)
    _, _, _, _, doc_first, doc_T = _segments(case)
    hq = case.num_q_heads
    cms = ca_column_masses(case, M)
    la, ca = [], []
    for d in range(len(doc_T)):
        T, t0 = int(doc_T[d]), int(doc_first[d])
        la_d = np.zeros((hq, T, T), bool)
        ca_d = np.zeros((hq, T), bool)
        for h in range(hq):
            for r in range(T):
                keep = select_top_p(M[h, t0 + r, t0:t0 + r + 1], p_la, {0, r})
                la_d[h, r, sorted(keep)] = True
            keep = select_top_p(cms[d][h], p_ca, {0})
            ca_d[h, sorted(keep)] = True
        la.append(la_d)
        ca.append(ca_d)
    return la, ca
