"""Pins of FPS (Algorithm 1): brute force, special cases, the pages' example."""
import inspect
import math
import os
import textwrap

import numpy as np
import pytest

from oracle.fps import cosine_matrix, fps, fps_margins, replay_check

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cos(a, b):
    num = math.fsum(float(x) * float(y) for x, y in zip(a, b))
    na = math.sqrt(math.fsum(float(x) ** 2 for x in a))
    nb = math.sqrt(math.fsum(float(y) ** 2 for y in b))
    return num / (max(na, 1e-12) * max(nb, 1e-12))


def _brute_fps(q, m):
    """Recompute every quantity from scratch at every step with plain loops."""
    n = len(q)
    avg = [math.fsum(_cos(q[i], q[j]) for j in range(n)) / n for i in range(n)]
    best = min(range(n), key=lambda i: (avg[i], i))
    order = [best]
    while len(order) < m:
        rest = [j for j in range(n) if j not in order]
        far = {j: max(_cos(q[j], q[k]) for k in order) for j in rest}
        order.append(min(rest, key=lambda j: (far[j], j)))
    return order


@pytest.mark.parametrize("seed", range(12))
def test_matches_brute_force_on_tiny_sets(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(3, 11))
    d = int(r.integers(2, 7))
    q = r.standard_normal((n, d))
    for m in range(1, n + 1):
        order, kept = fps(q, m)
        if m >= n:
            assert order == list(range(n))
            continue
        assert order == _brute_fps(q, m), (seed, m)
        assert kept == sorted(order)


def test_cosine_matrix_entries():
    r = np.random.default_rng(5)
    q = r.standard_normal((6, 5))
    c = cosine_matrix(q)
    for i in range(6):
        for j in range(6):
            assert abs(c[i, j] - _cos(q[i], q[j])) < 1e-14


def test_m_at_least_n_keeps_everything():
    q = np.random.default_rng(0).standard_normal((7, 4))
    assert fps(q, 7) == (list(range(7)), list(range(7)))
    assert fps(q, 9)[1] == list(range(7))


def test_m_one_is_lowest_average_similarity():
    q = np.random.default_rng(1).standard_normal((9, 3))
    avg = [np.mean([_cos(q[i], q[j]) for j in range(9)]) for i in range(9)]
    assert fps(q, 1)[0] == [int(np.argmin(avg))]


def test_orthonormal_ties_go_to_lowest_slots():
    q = np.eye(8)
    for m in range(1, 8):
        assert fps(q, m)[0] == list(range(m))


def test_antipode_is_second_pick():
    r = np.random.default_rng(2)
    base = r.standard_normal(6)
    others = base + 0.2 * r.standard_normal((5, 6))
    q = np.vstack([others, -base])  # -base: lowest average similarity
    order = fps(q, 2)[0]
    assert order[0] == 5
    # The seed's antipodal neighbours: the second pick is the most opposite one.
    s = [_cos(q[j], q[5]) for j in range(5)]
    assert order[1] == int(np.argmin(s))
    q2 = np.vstack([q, base])  # exact antipode of the seed
    assert fps(q2, 2)[0][1] == 6


def test_pages_worked_example_three_directions():
    rows, clusters = [], []
    m, expected = None, None
    with open(os.path.join(GOLDEN, "fps_three_directions.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "m":
                m = int(parts[1])
            elif parts[0] == "expected_clusters":
                expected = sorted(int(x) for x in parts[1:])
            else:
                a = math.radians(float(parts[0]))
                rows.append([math.cos(a), math.sin(a)])
                clusters.append(int(parts[1]))
    order, _ = fps(np.array(rows), m)
    assert sorted(clusters[i] for i in order) == expected
    assert clusters[order[0]] == 180  # the seed the page names


def test_replay_accepts_own_order_and_rejects_bad_pick():
    r = np.random.default_rng(9)
    q = r.standard_normal((32, 16))
    order, _ = fps(q, 16)
    ok, worst = replay_check(q, order, 2e-3)
    assert ok and worst == 0.0
    # Replace the last pick by the unpicked row with the largest S: must fail.
    c = cosine_matrix(q)
    s = c[:, order[:-1]].max(axis=1)
    s[order[:-1]] = -np.inf
    bad = order[:-1] + [int(np.argmax(s))]
    ok, worst = replay_check(q, bad, 2e-3)
    assert not ok and worst > 2e-3


# ---------------------------------------------------------------------------
# fps_margins and replay_check decide, in every GPU parity check of FPS,
# whether a picked set must equal the oracle's and whether a pick order is a
# valid FPS run.  Both are pinned against plain-loop recomputations and hand
# values; each pin is a function of the implementation so that the mutation
# tests below can show it rejects planted mistakes.

def _avg_brute(q):
    n = len(q)
    return [math.fsum(_cos(q[i], q[j]) for j in range(n)) / n for i in range(n)]


def _greedy_from(q, seed, m):
    """Algorithm 1's farthest-point loop from a given seed, plain loops."""
    n = len(q)
    order = [seed]
    while len(order) < m:
        rest = [j for j in range(n) if j not in order]
        far = {j: max(_cos(q[j], q[k]) for k in order) for j in rest}
        order.append(min(rest, key=lambda j: (far[j], j)))
    return order


def _brute_margins(q, m):
    """Runner-up gap of every step of the oracle's run, recomputed from scratch."""
    n = len(q)
    lo = sorted(_avg_brute(q))
    gaps = [lo[1] - lo[0]]
    order = _brute_fps(q, m)
    for step in range(1, m):
        picked = order[:step]
        far = sorted(max(_cos(q[j], q[k]) for k in picked) for j in range(n) if j not in picked)
        gaps.append(far[1] - far[0] if len(far) > 1 else math.inf)
    return gaps


def _brute_replay_excess(q, order):
    """Largest step excess of a pick order: the seed's average over the lowest
    average, then each pick's S over the lowest S of the rows not yet picked."""
    avg = _avg_brute(q)
    worst = avg[order[0]] - min(avg)
    for step in range(1, len(order)):
        picked = order[:step]
        s = {j: max(_cos(q[j], q[k]) for k in picked) for j in range(len(q)) if j not in picked}
        worst = max(worst, s[order[step]] - min(s.values()))
    return worst


def pin_margins(margins_fn):
    # Hand example: unit vectors at 0, 60 and 180 degrees.  Cosines 1/2, -1,
    # -1/2 give averages 1/6, 1/3, -1/6: the seed is the 180-degree row with
    # a gap of 1/3 to the runner-up; S = (-1, -1/2) then picks the 0-degree
    # row with a gap of 1/2.
    q = np.array([[1.0, 0.0], [0.5, math.sqrt(3) / 2], [-1.0, 0.0]])
    got = margins_fn(q, 2)
    assert len(got) == 2
    assert abs(got[0] - 1 / 3) < 1e-12 and abs(got[1] - 0.5) < 1e-12, got
    assert margins_fn(q, 3) == [] and margins_fn(q, 5) == []
    for seed in range(8):
        r = np.random.default_rng(100 + seed)
        n = int(r.integers(3, 11))
        q = r.standard_normal((n, int(r.integers(2, 7))))
        for m in range(1, n):
            got = margins_fn(q, m)
            want = _brute_margins(q, m)
            assert len(got) == m == len(want), (seed, m)
            for a, b in zip(got, want):
                assert abs(a - b) < 1e-12, (seed, m, got, want)


def pin_replay(replay_fn):
    r = np.random.default_rng(21)
    q = r.standard_normal((10, 5))
    own = _brute_fps(q, 6)
    ok, worst = replay_fn(q, own, 2e-3)
    assert ok and abs(worst) < 1e-12
    # A seed that is not the lowest-average row, followed by valid picks from
    # it: only the seed step is off, by its average's excess.
    avg = _avg_brute(q)
    wrong = int(np.argmax(avg))
    order = _greedy_from(q, wrong, 6)
    ok, worst = replay_fn(q, order, 2e-3)
    assert not ok and abs(worst - (avg[wrong] - min(avg))) < 1e-12, worst
    # A seed tied with the lowest average is accepted: with every row present
    # twice (the copy scaled, so its cosines are the same), the copy of the
    # lowest-average row ties with it.
    p = int(np.argmin(avg))
    q2 = np.vstack([q, 3.0 * q])
    order = _greedy_from(q2, len(q) + p, 6)
    ok, worst = replay_fn(q2, order, 2e-3)
    assert ok and worst < 1e-12, worst
    # Arbitrary orders: the reported excess equals the plain-loop recomputation.
    for k in range(6):
        perm = [int(x) for x in np.random.default_rng(40 + k).permutation(10)[:6]]
        ok, worst = replay_fn(q, perm, 2e-3)
        want = _brute_replay_excess(q, perm)
        assert abs(worst - want) < 1e-12 and ok == (want <= 2e-3), (perm, worst, want)
    # A row picked twice is never a valid run, even where every order ties:
    # rows all parallel have every cosine 1, so any order of distinct rows is
    # valid and only the repeat is not.
    par = np.outer([1.0, 2.0, 0.5, 3.0, 1.5], r.standard_normal(4))
    assert replay_fn(par, [3, 0, 4], 2e-3)[0]
    assert not replay_fn(par, [3, 0, 0], 2e-3)[0]
    assert not replay_fn(q, own[:5] + [own[2]], 2e-3)[0]


def test_margins_pinned():
    pin_margins(fps_margins)


def test_replay_pinned():
    pin_replay(replay_check)


def _mutant(fn, old, new):
    """fn with the first occurrence of `old` in its source replaced by `new`."""
    src = textwrap.dedent(inspect.getsource(fn))
    assert old in src, old
    ns = dict(vars(inspect.getmodule(fn)))
    exec(compile(src.replace(old, new, 1), f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]


MARGIN_MUTANTS = [
    ("gaps = [float(srt[1] - srt[0])]", "gaps = [0.0]"),                      # seed gap lost
    ("gaps.append(float(srt[1] - srt[0]) if np.isfinite(srt[1]) else np.inf)",
     "gaps.append(0.0)"),                                                     # pick gaps lost
    ("srt = np.sort(avg)", "srt = np.sort(avg)[::-1]"),                       # wrong end
    ("avg = c.sum(axis=1) / n_rows", "avg = c.max(axis=1)"),                  # not the mean
    ("s = np.maximum(s, c[:, r])", "s = np.minimum(s, c[:, r])"),             # wrong update
]
# Not listed: leaving the picked rows in the argmin or the sorted gap.  A
# picked row's S is its cosine with itself, 1, the largest value S takes, so
# with at least two rows unpicked (m < N) that mutant gives the same margins
# on every input: it is equivalent, not a mistake a pin could catch.

REPLAY_MUTANTS = [
    ("worst = avg[order[0]] - avg.min()", "worst = 0.0"),                     # seed ignored
    ("s = np.maximum(s, c[:, r])", "s = c[:, r]"),                            # no running max
    ("worst = max(worst, s[r] - best)", "worst = max(worst, best - s[r])"),   # sign
    ("if chosen[r]:", "if False:"),                                          # repeats accepted
]
# Not listed: leaving the picked rows in the minimum of S (equivalent, as for
# the margins: a picked row's S is 1, the largest S can be).


@pytest.mark.parametrize("old,new", MARGIN_MUTANTS)
def test_margin_pin_rejects_mutant(old, new):
    with pytest.raises(Exception):
        pin_margins(_mutant(fps_margins, old, new))


@pytest.mark.parametrize("old,new", REPLAY_MUTANTS)
def test_replay_pin_rejects_mutant(old, new):
    with pytest.raises(Exception):
        pin_replay(_mutant(replay_check, old, new))
