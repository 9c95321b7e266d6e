"""Pins of FPS (Algorithm 1): brute force, special cases, the pages' example."""
import math
import os

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
    gaps = fps_margins(q, 16)
    assert len(gaps) == 16 and min(gaps) >= 0
    # Replace the last pick by the unpicked row with the largest S: must fail.
    c = cosine_matrix(q)
    s = c[:, order[:-1]].max(axis=1)
    s[order[:-1]] = -np.inf
    bad = order[:-1] + [int(np.argmax(s))]
    ok, worst = replay_check(q, bad, 2e-3)
    assert not ok and worst > 2e-3
