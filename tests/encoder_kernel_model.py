"""A model of the selection kernel's float32 arithmetic (a kernel unit test, NOT the oracle).

The selection kernel sorts a row's (at most 64) fp32 masses, scans them with an inclusive
Hillis-Steele scan in fp32, and keeps slot i when i = 0 or the scan before it is below
p x (the scan's last slot); CA column masses are summed in fp32 in increasing query-tile
order.  Given the GPU's own fp32 masses, this model must reproduce the kernel's words bit for
bit.  It checks the kernel's sorting, scan, cut, forced tiles and packing in isolation.  The
oracle (oracle/encoder.py) is what pins the encoder's bits: an fp64 selection on its own fp64
masses, compared with a decision margin (tests/encoder_compare.py).
"""
import numpy as np

from oracle.encoder import _segments


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


def select_top_p_fp32(masses, p, forced):
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


def ca_column_masses_fp32(case, M32):
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


def select_bits_fp32(case, M, p_la=0.9, p_ca=0.9):
    M32 = np.asarray(M, dtype=np.float32)
    _, _, _, _, doc_first, doc_T = _segments(case)
    hq = case.num_q_heads
    cms = ca_column_masses_fp32(case, M32)
    la, ca = [], []
    for d in range(len(doc_T)):
        T, t0 = int(doc_T[d]), int(doc_first[d])
        la_d = np.zeros((hq, T, T), bool)
        ca_d = np.zeros((hq, T), bool)
        for h in range(hq):
            for r in range(T):
                keep = select_top_p_fp32(M32[h, t0 + r, t0:t0 + r + 1], p_la, {0, r})
                la_d[h, r, sorted(keep)] = True
            keep = select_top_p_fp32(cms[d][h], p_ca, {0})
            ca_d[h, sorted(keep)] = True
        la.append(la_d)
        ca.append(ca_d)
    return la, ca
