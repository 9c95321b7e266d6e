"""Farthest point sampling under cosine similarity (Algorithm 1).

Paper text, App. D.1 (Algorithm 1, FPS), with the summary's "前置知识 /
最远点采样" and the review's "작동 원리 ①" restating it:

* every query gets its average cosine similarity to the whole set (the sum
  runs over all N members, itself included);
* the seed is the query whose average is lowest;
* each unselected query keeps S_j, its largest cosine to any selected query;
* repeatedly the unselected query with the lowest S_j is added and S is
  raised to include the similarity to the new member, until m are chosen.

Readings where the pages are silent: ties go to the lower buffer slot, the
kept rows are returned in ascending original slot order (their temporal
order), and a zero norm is clamped to 1e-12 (it cannot occur for Gaussian
inputs).
"""

import numpy as np

NORM_FLOOR = 1e-12


def cosine_matrix(q):
    """C_ij = q_i . q_j / (|q_i| |q_j|) in float64."""
    q = np.asarray(q, dtype=np.float64)
    n = np.maximum(np.sqrt(np.sum(q * q, axis=1)), NORM_FLOOR)
    return (q @ q.T) / np.outer(n, n)


def fps(q, m):
    """Select m of the N rows of q.

    Returns (order, kept): ``order`` lists the picked row indices in the
    order they were picked (seed first); ``kept`` is the same set sorted
    ascending, which is the order the compressed buffer stores them in.
    With N <= m every row is kept.
    """
    q = np.asarray(q, dtype=np.float64)
    n_rows = q.shape[0]
    if n_rows <= m:
        idx = list(range(n_rows))
        return idx, idx
    c = cosine_matrix(q)
    avg = c.sum(axis=1) / n_rows
    seed = int(np.argmin(avg))  # first minimum: the lowest slot wins a tie
    order = [seed]
    chosen = np.zeros(n_rows, dtype=bool)
    chosen[seed] = True
    s = c[:, seed].copy()
    while len(order) < m:
        cand = np.where(chosen, np.inf, s)
        r = int(np.argmin(cand))
        order.append(r)
        chosen[r] = True
        s = np.maximum(s, c[:, r])
    return order, sorted(order)


def fps_margins(q, m):
    """For each step of the oracle's own run, the gap between the winning
    value and the runner-up (seed: average cosine; later picks: S_j).

    A GPU result may differ from the oracle only where such a gap is inside
    the acceptance tolerance; the parity tests use this to decide whether a
    set must match exactly.
    """
    q = np.asarray(q, dtype=np.float64)
    n_rows = q.shape[0]
    if n_rows <= m:
        return []
    c = cosine_matrix(q)
    avg = c.sum(axis=1) / n_rows
    srt = np.sort(avg)
    gaps = [float(srt[1] - srt[0])]
    seed = int(np.argmin(avg))
    chosen = np.zeros(n_rows, dtype=bool)
    chosen[seed] = True
    s = c[:, seed].copy()
    picks = 1
    while picks < m:
        cand = np.where(chosen, np.inf, s)
        srt = np.sort(cand)
        gaps.append(float(srt[1] - srt[0]) if np.isfinite(srt[1]) else np.inf)
        r = int(np.argmin(cand))
        chosen[r] = True
        s = np.maximum(s, c[:, r])
        picks += 1
    return gaps


def replay_check(q, order, tol):
    """Check a pick order produced elsewhere, step by step, in float64.

    The seed's average cosine must be within ``tol`` of the lowest average;
    each later pick's S (built from the earlier picks of ``order`` itself)
    must be within ``tol`` of the lowest S over rows not yet picked.
    Returns (ok, worst_excess).
    """
    q = np.asarray(q, dtype=np.float64)
    n_rows = q.shape[0]
    c = cosine_matrix(q)
    avg = c.sum(axis=1) / n_rows
    worst = avg[order[0]] - avg.min()
    chosen = np.zeros(n_rows, dtype=bool)
    chosen[order[0]] = True
    s = c[:, order[0]].copy()
    for r in order[1:]:
        if chosen[r]:
            return False, np.inf
        best = np.min(np.where(chosen, np.inf, s))
        worst = max(worst, s[r] - best)
        chosen[r] = True
        s = np.maximum(s, c[:, r])
    return bool(worst <= tol), float(worst)
