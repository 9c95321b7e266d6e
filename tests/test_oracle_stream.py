"""Pins of the Continual-FPS cadence and the cache-size closed form."""
import os
from collections import Counter

import numpy as np

from oracle.evict import evict_unit
from oracle.stream import UnitStream, kv_cache_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_cadence_per_eviction_interval():
    # Derived from the summary's steps (2), (3), (6): after an eviction the
    # buffer holds 16; 128 - 16 = 112 collected queries trigger 112 / 16 = 7
    # fill-and-compress events, the beacon fix then finds 16 rows (a no-op),
    # 16 recents are set aside, and the eviction's merge compresses 32 -> 16.
    g, d, b_kv, P = 1, 8, 64, 4
    st = UnitStream(g, d, b_max=b_kv + 128, b_kv=b_kv, prefix=P, theta=1e4)
    r = np.random.default_rng(0)
    st.prefill(r.standard_normal((P, d)), r.standard_normal((P, d)),
               r.standard_normal((g, P, d)))
    n_steps = 3 * 128 + 120
    for _ in range(n_steps):
        st.step(r.standard_normal(d), r.standard_normal(d), r.standard_normal((g, d)))
    ev = [e for e, _ in st.events]
    cuts = [i for i, e in enumerate(ev) if e == "evict"]
    assert len(cuts) == 3
    for a, b in zip(cuts[:-1], cuts[1:]):
        c = Counter(ev[a + 1:b + 1])
        assert c["collect_fps"] == 7
        assert c["beacon_fix_noop"] == 1 and c["beacon_fix_fps"] == 0
        assert c["merge_fps"] == 1 and c["evict"] == 1
    first = (b_kv + 128) - P  # steps until the first eviction
    assert st.keys.shape[0] == b_kv + (n_steps - first - 2 * 128)
    since = n_steps - first - 2 * 128  # collected since the last merge
    assert all(b.shape[0] == 16 + since % 16 for b in st.buf)


def test_kv_cache_size_claim():
    vals = {}
    with open(os.path.join(GOLDEN, "kv_cache_size.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    gb = kv_cache_bytes(int(vals["layers"]), int(vals["kv_heads"]), int(vals["d_head"]),
                        int(vals["seq"]), int(vals["batch"]), int(vals["bytes_per_elem"])) / 1e9
    assert gb > vals["claim_gb_more_than"]
    assert abs(gb - 77.3) < 0.05


def test_evict_unit_invariants_and_merge():
    r = np.random.default_rng(3)
    L, d, g, b, P = 160, 16, 2, 96, 8
    keys, vals = r.standard_normal((L, d)), r.standard_normal((L, d))
    out = evict_unit(keys, vals, np.arange(L), L, r.standard_normal((g, 16, d)),
                     r.standard_normal((g, 16, d)), L, b, P, 16, 1e4)
    kept = out["kept"]
    assert len(kept) == b and set(range(P)) <= set(kept) and set(range(L - 16, L)) <= set(kept)
    assert np.array_equal(out["keys"], keys[kept])
    assert out["buf"].shape == (g, 16, d)
    # Compaction in position order moves every kept slot above its rank and
    # no prefix slot.
    moved = sum(1 for k, slot in enumerate(kept) if slot != k)
    assert moved == sum(1 for k in range(P, b) if kept[k] > k) and moved <= b - P


def test_initial_recent_policy_keeps_the_first_generated_queries():
    # Initial+Recent (paper text §5.3, Table 3): the reference rows are the
    # first 16 queries generated after the prompt, unchanged by evictions;
    # the recents are the last 16 queries before each eviction, and the
    # eviction scores with exactly those two sets.
    g, d, b_kv, P = 2, 8, 64, 4
    st = UnitStream(g, d, b_max=b_kv + 128, b_kv=b_kv, prefix=P, theta=1e4, beacons="initial")
    r = np.random.default_rng(5)
    st.prefill(r.standard_normal((P, d)), r.standard_normal((P, d)),
               r.standard_normal((g, P, d)))
    qs = []
    first = (b_kv + 128) - P
    for _ in range(first + 128 + 5):
        k, v, q = r.standard_normal(d), r.standard_normal(d), r.standard_normal((g, d))
        qs.append(q)
        if len(qs) == first:  # about to evict: check what it will score with
            pre = (st.keys.copy(), st.values.copy(), st.kpos.copy(), st.t)
        st.step(k, v, q)
        if len(qs) == first:
            keys, vals, kpos, t = pre
            keys = np.vstack([keys, k[None]])
            vals = np.vstack([vals, v[None]])
            kpos = np.append(kpos, t)
            beacons = np.stack([np.stack([qs[i][h] for i in range(16)]) for h in range(g)])
            recents = np.stack([np.stack([qs[i][h] for i in range(first - 16, first)])
                                for h in range(g)])
            ref = evict_unit(keys, vals, kpos, b_kv + 128, beacons, recents, t + 1, b_kv, P,
                             16, 1e4, merge=False)
            assert np.array_equal(st.last_evict["kept"], ref["kept"])
            assert np.array_equal(st.last_evict["score"], ref["score"])
    want = np.stack([np.stack([qs[i][h] for i in range(16)]) for h in range(g)])
    assert np.array_equal(np.stack(st.buf), want)
    ev = [e for e, _ in st.events]
    assert ev.count("evict") == 2 and "merge_fps" not in ev and "collect_fps" not in ev
    assert ev[:2] == ["prefill", "initial_set"] and ev.count("recent_start") == 2
    try:
        UnitStream(g, d, 192, 64, P, 1e4, beacons="random")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown beacon policy must be rejected")


def test_unsorted_compaction_keeps_the_same_evictions():
    # Filling holes only permutes the kept tokens, and scoring, selection
    # (up to the slot order of ties) and the causal masks do not depend on
    # the order of the older tokens: over three eviction intervals the kept
    # positions, as sets, match the position-ordered run.
    g, d, b_kv, P = 1, 8, 64, 4
    runs = {}
    for unsorted in (False, True):
        st = UnitStream(g, d, b_max=b_kv + 128, b_kv=b_kv, prefix=P, theta=1e4, unsorted=unsorted)
        r = np.random.default_rng(21)
        st.prefill(r.standard_normal((P, d)), r.standard_normal((P, d)),
                   r.standard_normal((g, P, d)))
        kept_sets = []
        for _ in range((b_kv + 128 - P) + 2 * 128 + 3):
            n_ev = st.events.count(("evict", b_kv + 128))
            st.step(r.standard_normal(d), r.standard_normal(d), r.standard_normal((g, d)))
            if st.events.count(("evict", b_kv + 128)) > n_ev:
                kept_sets.append(sorted(st.kpos.tolist()))
        runs[unsorted] = (kept_sets, st)
    assert runs[False][0] == runs[True][0] and len(runs[True][0]) == 3
    # The unsorted cache is a permutation with the prefix in place.
    st = runs[True][1]
    assert st.kpos[:P].tolist() == list(range(P))
    assert sorted(st.kpos.tolist()) != st.kpos.tolist()
