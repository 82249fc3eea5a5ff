"""Comparison of the GPU encoder's bits with the fp64 oracle's, row by row, with a decision margin.

The GPU selects from its own fp32 masses; the oracle selects from its own fp64 masses.  The
masses tests assert |GPU mass - oracle mass| <= ATOL + RTOL * |oracle mass| for every entry,
and the kernel's threshold test sums fp32 values (a scan over at most 64 sorted slots, then
p x total), which adds at most SLACK_REL x (total) of rounding.  A row is *robust* when every
masses vector inside that box, with any such rounding, gives the oracle's set: then the GPU
must give exactly that set.  A row that is not robust ("fragile") may differ, but only in a
way that is itself a top-p selection within the margin (checked by valid_within_margin).

Robustness, for candidates m (fp64) with bounds eps, sorted order pi and cut k* (the oracle's
shortest prefix reaching p x T, T = sum m, E = sum eps):
  * the kept set is separated from the rest: min over kept (m - eps) > max over the others
    (m + eps), so no perturbation reorders across the cut;
  * the cut cannot move earlier: the largest possible sum of k* - 1 candidates, sum of the
    k* - 1 largest (m + eps), stays below p (T - E) minus the rounding slack;
  * the cut cannot move later: the smallest possible sum of the k* largest, sum of the k*
    largest (m - eps), reaches p (T + E) plus the slack.
The forced tiles are added after the cut, so a row differs only if the final sets differ.
"""
import math

import numpy as np

from oracle import encoder as E

ATOL, RTOL = 2e-5, 1e-4     # the masses tolerance the GPU tests assert
U32 = 2.0 ** -24           # fp32 unit roundoff
SLACK_REL = 8 * U32        # <= 6 scan roundings + the threshold multiply, relative to the total


def robust(m, eps, p, forced):
    m = np.asarray(m, np.float64)
    eps = np.asarray(eps, np.float64)
    n = m.size
    if n == 0:
        return True
    k, order = E.top_p_count(m, p)
    T, Etot = math.fsum(m.tolist()), math.fsum(eps.tolist())
    slack = SLACK_REL * (T + Etot)
    kept, rest = order[:k], order[k:]
    # no perturbation may reorder a kept candidate below a dropped one, unless both are forced
    # (a forced tile leaving the prefix lets a dropped one in, and the reverse)
    forced = set(forced)
    lo_free = min((m[i] - eps[i] for i in kept if i not in forced), default=math.inf)
    lo_forced = min((m[i] - eps[i] for i in kept if i in forced), default=math.inf)
    hi_free = max((m[j] + eps[j] for j in rest if j not in forced), default=-math.inf)
    hi_forced = max((m[j] + eps[j] for j in rest if j in forced), default=-math.inf)
    if not (lo_free > max(hi_free, hi_forced) and lo_forced > hi_free):
        return False
    up = np.sort(m + eps)[::-1]
    dn = np.sort(m - eps)[::-1]
    if k > 1 and not math.fsum(up[:k - 1].tolist()) < p * (T - Etot) - slack:
        return False
    if k < n and not math.fsum(dn[:k].tolist()) >= p * (T + Etot) + slack:
        return False
    return True


def valid_within_margin(m, eps, p, forced, got):
    """`got` (a set) could be the selection of some masses inside the margin: the forced tiles plus
    a top-p prefix P of those masses.  P is `got` less some of its forced tiles (a forced tile
    need not be in the prefix); for some such P all of these hold:
      * P can sort ahead of every other candidate: min over P of (m + eps) >= max over the
        others of (m - eps);
      * P can reach the threshold: sum over P of (m + eps) >= p (T - E) - slack;
      * P without its smallest member can fall short of it: for some j in P that can be the
        smallest (m_j - eps_j <= min over P of (m + eps)), sum over P - {j} of (m - eps) <
        p (T + E) + slack."""
    m = np.asarray(m, np.float64)
    eps = np.asarray(eps, np.float64)
    forced = set(forced)
    if not forced <= got:
        return False
    T, Etot = math.fsum(m.tolist()), math.fsum(eps.tolist())
    slack = SLACK_REL * (T + Etot)
    opt = sorted(forced & got)
    for mask in range(1 << len(opt)):
        P = set(got) - {opt[b] for b in range(len(opt)) if (mask >> b) & 1}
        if not P:
            continue
        others = [i for i in range(m.size) if i not in P]
        top = min(m[i] + eps[i] for i in P)
        if others and not top >= max(m[i] - eps[i] for i in others):
            continue
        if math.fsum([m[i] + eps[i] for i in P]) < p * (T - Etot) - slack:
            continue
        if len(P) == 1:
            return True
        lows = [m[i] - eps[i] for i in P]
        total_low = math.fsum(lows)
        if any(total_low - (m[j] - eps[j]) < p * (T + Etot) + slack for j in P if m[j] - eps[j] <= top):
            return True
    return False


def la_eps(row):
    return ATOL + RTOL * np.abs(row)


def compare(case, M, la_gpu, ca_gpu, p_la, p_ca):
    """Row-by-row comparison.  M: fp64 oracle masses [Hq, G, G]; la_gpu / ca_gpu: per-doc GPU
    booleans ([Hq, T, T], [Hq, T]).  Returns a dict of counts; raises AssertionError on a
    difference in a robust row or an invalid fragile row."""
    tile_req, tile_doc, _, _, doc_first, doc_T = E._segments(case)
    hq = case.num_q_heads
    cms = E.ca_column_masses(case, M)
    rows = fragile = differ = 0
    for d in range(len(doc_T)):
        T, t0 = int(doc_T[d]), int(doc_first[d])
        b = tile_req[t0]
        later = [g for g in range(len(tile_req)) if tile_req[g] == b and tile_doc[g] > d]
        for h in range(hq):
            for r in range(T):
                m = M[h, t0 + r, t0:t0 + r + 1]
                eps = la_eps(m)
                forced = {0, r}
                want = E.select_top_p(m, p_la, forced)
                got = set(np.nonzero(la_gpu[d][h, r, :r + 1])[0].tolist())
                assert not la_gpu[d][h, r, r + 1:].any(), f"LA bits above the diagonal (d={d}, h={h}, r={r})"
                rows += 1
                ok = robust(m, eps, p_la, forced)
                fragile += not ok
                if got != want:
                    differ += 1
                    assert not ok, f"LA row d={d} h={h} r={r}: robust row differs: gpu {sorted(got)} oracle {sorted(want)}"
                    assert valid_within_margin(m, eps, p_la, forced, got), \
                        f"LA row d={d} h={h} r={r}: gpu {sorted(got)} is no top-p selection within the margin"
            cm = cms[d][h]
            # column sums: the entries' bounds add up, plus fp32 rounding of the sequential sum
            eps_c = np.zeros(T)
            if later:
                cols = slice(t0, t0 + T)
                eps_c = (ATOL + RTOL * np.abs(M[h, later, cols])).sum(axis=0) + len(later) * U32 * np.abs(cm)
            want = E.select_top_p(cm, p_ca, {0})
            got = set(np.nonzero(ca_gpu[d][h])[0].tolist())
            rows += 1
            ok = robust(cm, eps_c, p_ca, {0})
            fragile += not ok
            if got != want:
                differ += 1
                assert not ok, f"CA d={d} h={h}: robust row differs: gpu {sorted(got)} oracle {sorted(want)}"
                assert valid_within_margin(cm, eps_c, p_ca, {0}, got), \
                    f"CA d={d} h={h}: gpu {sorted(got)} is no top-p selection within the margin"
    return {"rows": rows, "fragile": fragile, "differ": differ}
