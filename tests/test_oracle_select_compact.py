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


def test_fill_holes_hand_example():
    # b_kv = 5 of L = 8 slots, kept = [0, 2, 3, 6, 7]: the holes below 5 are
    # slots 1 and 4, the kept slots at or past 5 are 6 and 7, so slot 1
    # takes token 6 and slot 4 takes token 7; slots 0, 2, 3 stay.
    from oracle.compact import fill_holes
    keys = np.arange(8.0)[:, None] * np.ones((1, 2))
    kpos = np.arange(100, 108)
    k, v, p, moves = fill_holes(keys, -keys, kpos, [0, 2, 3, 6, 7], 5)
    assert moves == [(1, 6), (4, 7)]
    assert k[:, 0].tolist() == [0, 6, 2, 3, 7]
    assert v[:, 0].tolist() == [0, -6, -2, -3, -7]
    assert p.tolist() == [100, 106, 102, 103, 107]


def test_fill_holes_is_a_permutation_of_the_sorted_compaction():
    # Same kept rows, any order: sorting the output by position gives the
    # position-ordered compaction; kept slots below b_kv never move; every
    # move goes from a slot >= b_kv to an evicted slot < b_kv.
    from oracle.compact import compact, fill_holes
    from oracle.select import select
    r = np.random.default_rng(11)
    for L, b in ((300, 200), (256, 128), (97, 96), (64, 16)):
        keys = r.standard_normal((L, 4))
        vals = r.standard_normal((L, 4))
        kpos = np.arange(L) * 3 + 5
        sc = r.random(L)
        kept = select(sc, L, b, 4, 8)
        k, v, p, moves = fill_holes(keys, vals, kpos, kept, b)
        ks, vs, ps = compact(keys, vals, kpos, kept)
        order = np.argsort(p)
        assert np.array_equal(p[order], ps) and np.array_equal(k[order], ks)
        assert np.array_equal(v[order], vs)
        stay = [j for j in kept if j < b]
        assert np.array_equal(k[stay], keys[stay])
        assert len(moves) == sum(1 for j in kept if j >= b)
        assert all(s >= b > h and h not in set(kept.tolist()) for h, s in moves)
