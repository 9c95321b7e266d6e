"""Pins of selection and compaction against brute force and invariants."""
import numpy as np
import pytest

from oracle.compact import compact
from oracle.select import select


def _brute(score, L, b_kv, P, R):
    forced = set(range(P)) | set(range(L - R, L))
    middle = [j for j in range(P, L - R)]
    ranked = sorted(middle, key=lambda j: (-score[j], j))
    return sorted(forced | set(ranked[: b_kv - P - R]))


@pytest.mark.parametrize("seed", range(10))
def test_select_matches_brute_force_with_ties(seed):
    r = np.random.default_rng(seed)
    L = int(r.integers(40, 300))
    P = int(r.integers(0, 12))
    R = 16
    b = int(r.integers(P + R, L))
    score = r.choice([0.1, 0.2, 0.25, 0.5, 1e-30, 0.0], size=L)  # many ties
    kept = select(score, L, b, P, R)
    assert kept.tolist() == _brute(score, L, b, P, R)


def test_select_invariants():
    r = np.random.default_rng(1)
    L, P, R, b = 500, 8, 16, 300
    score = r.random(L)
    kept = select(score, L, b, P, R)
    assert len(kept) == b and np.all(np.diff(kept) > 0)
    assert set(range(P)) <= set(kept.tolist())
    assert set(range(L - R, L)) <= set(kept.tolist())
    mid = np.zeros(L, bool)
    mid[P:L - R] = True
    keep = np.zeros(L, bool)
    keep[kept] = True
    assert score[keep & mid].min() >= score[~keep & mid].max()


def test_select_rejects_bad_budgets():
    with pytest.raises(ValueError):
        select(np.ones(50), 50, 20, 8, 16)   # P + R > b
    with pytest.raises(ValueError):
        select(np.ones(50), 50, 50, 8, 16)   # b == L


def test_compact_matches_loop():
    r = np.random.default_rng(2)
    L, d = 64, 8
    k, v = r.standard_normal((L, d)), r.standard_normal((L, d))
    kpos = np.arange(L) * 3 + 5
    kept = np.sort(r.choice(L, 40, replace=False))
    k2, v2, p2 = compact(k, v, kpos, kept)
    for i, j in enumerate(kept):
        assert np.array_equal(k2[i], k[j]) and np.array_equal(v2[i], v[j])
        assert p2[i] == kpos[j]
    assert np.all(np.diff(p2) > 0)
