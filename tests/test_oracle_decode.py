"""Pins of the decode-attention oracle and of scoring from known denominators."""
import numpy as np
import scipy.special

from oracle.bf16 import round_f64_to_bf16
from oracle.decode import (beacon_lse, decode_attention, logsumexp_rows, rotated_queries,
                           score_from_lse)
from oracle.score import logits, observation_set, score_unit


def _bf16(x):
    return round_f64_to_bf16(np.asarray(x, np.float64))


def test_decode_matches_library_softmax_and_logsumexp():
    r = np.random.default_rng(3)
    L, d, g = 77, 16, 3
    keys, values = _bf16(r.standard_normal((L, d))), _bf16(r.standard_normal((L, d)))
    q = r.standard_normal((g, d)).astype(np.float32)
    out, lse = decode_attention(keys, values, q, 41, 1e4)
    qhat = rotated_queries(q, 41, 1e4)
    s = qhat @ keys.T / np.sqrt(d)
    assert np.allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=1e-14, atol=1e-14)
    assert np.allclose(out, scipy.special.softmax(s, axis=-1) @ values, rtol=1e-12, atol=1e-14)


def test_decode_identical_keys_average_the_values():
    # Every logit equal: W = 1/L, out = mean of V, lse = s + log L.
    r = np.random.default_rng(4)
    L, d = 50, 8
    k = _bf16(r.standard_normal(d))
    keys = np.tile(k, (L, 1))
    values = r.standard_normal((L, d))
    q = r.standard_normal((2, d)).astype(np.float32)
    out, lse = decode_attention(keys, values, q, 9, 1e4)
    s = rotated_queries(q, 9, 1e4) @ k / np.sqrt(d)
    assert np.allclose(out, np.tile(values.mean(axis=0), (2, 1)), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, s + np.log(L), rtol=1e-14, atol=1e-14)


def test_decode_hand_values():
    # d = 4, position 0 (no rotation), q = e0 (bf16-exact): s = k[0] / 2.
    # Logits ln 3 and 0: weights 3/4 and 1/4, lse = ln 4.
    q = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    keys = np.array([[2 * np.log(3.0), 5.0, -1.0, 2.0], [0.0, 1.0, 1.0, 1.0]])
    values = np.array([[4.0, 0.0, 8.0, 1.0], [0.0, 4.0, 0.0, 1.0]])
    out, lse = decode_attention(keys, values, q, 0, 1e4)
    assert np.allclose(out[0], [3.0, 1.0, 6.0, 1.0], rtol=1e-14, atol=1e-14)
    assert np.isclose(lse[0], np.log(4.0), rtol=1e-15)
    # One slot: the output is that slot's value, lse its logit.
    out1, lse1 = decode_attention(keys[:1], values[:1], q, 0, 1e4)
    assert np.array_equal(out1[0], values[0]) and np.isclose(lse1[0], np.log(3.0))


def test_decode_query_is_rotated_to_its_position():
    # Relative-position property: rotating the query by t and the keys by
    # -t' is the same attention as rotating it by t - t' (up to the bf16
    # rounding, which is why the query is made bf16-exact after rotation by
    # checking against the explicit rotation).
    r = np.random.default_rng(5)
    d = 8
    q = r.standard_normal((1, d)).astype(np.float32)
    keys = _bf16(r.standard_normal((6, d)))
    _, lse_a = decode_attention(keys, keys, q, 0, 1e4)
    _, lse_b = decode_attention(keys, keys, q, 37, 1e4)
    assert not np.allclose(lse_a, lse_b)  # the position matters
    qh = rotated_queries(q, 37, 1e4)
    assert np.allclose(lse_b, scipy.special.logsumexp(qh @ keys.T / np.sqrt(d), axis=-1),
                       rtol=1e-14)


def test_beacon_lse_is_row_logsumexp_of_the_scoring_logits():
    r = np.random.default_rng(6)
    g, d, L = 2, 16, 40
    keys = _bf16(r.standard_normal((L, d)))
    beacons = r.standard_normal((g, 16, d)).astype(np.float32)
    got = beacon_lse(keys, beacons, 100, 1e4)
    qhat = observation_set(beacons, np.zeros((g, 0, d)), 100, np.zeros(0), 1e4)
    s = logits(qhat, keys, 1 / np.sqrt(d))
    assert np.allclose(got, scipy.special.logsumexp(s, axis=-1), rtol=1e-14, atol=1e-14)


def test_logsumexp_rows_survives_large_logits():
    s = np.array([[1000.0, 1000.0], [-1000.0, -1000.0 + np.log(3.0)]])
    assert np.allclose(logsumexp_rows(s), [1000 + np.log(2.0), -1000 + np.log(4.0)],
                       rtol=1e-15)


def _event(seed, g=2, L=150, d=16, theta=1e4):
    r = np.random.default_rng(seed)
    keys = _bf16(r.standard_normal((L, d)))
    beacons = r.standard_normal((g, 16, d)).astype(np.float32)
    recents = r.standard_normal((g, 16, d)).astype(np.float32)
    return keys, beacons, recents


def _fused_lse(keys, beacons, recents, t, lse_from, theta):
    """Denominators as the fused path gathers them: the beacons' over the
    slots present at lse_from, each recent query's from its own decode step
    (the cache then held slots 0 .. L-16+i)."""
    L = keys.shape[0]
    g = beacons.shape[0]
    lse = np.zeros((g, 32))
    lse[:, :16] = beacon_lse(keys[:lse_from], beacons, t, theta)
    for i in range(16):
        _, li = decode_attention(keys[:L - 16 + i + 1], keys[:L - 16 + i + 1],
                                 recents[:, i], L - 16 + i, theta)
        lse[:, 16 + i] = li
    return lse


def test_score_from_decode_denominators_equals_two_pass_score():
    # The eviction's scores from denominators gathered during decoding equal
    # the plain definition (score.score_unit, pinned on its own), for the
    # fused step at the beacon fix (L - 16), at a tile-unaligned point, at
    # the very start (all slots added at eviction) and at L (nothing added).
    keys, beacons, recents = _event(7)
    L = keys.shape[0]
    taus = np.arange(L - 16, L)
    for agg in ("max", "mean"):
        ref = score_unit(keys, beacons, recents, L, taus, 1e4, aggregate=agg)
        for lse_from in (L - 16, 101, 0, L):
            lse = _fused_lse(keys, beacons, recents, L, lse_from, 1e4)
            got = score_from_lse(keys, beacons, recents, L, taus, 1e4, lse, lse_from,
                                 aggregate=agg)
            assert np.allclose(got, ref, rtol=1e-12, atol=0), (agg, lse_from)


def test_score_from_lse_rejects_a_missing_tail():
    # Leaving out the slots appended after the fused pass (claiming the
    # beacons' denominator was complete) changes the scores: the tail merge
    # is not a no-op.
    keys, beacons, recents = _event(8)
    L = keys.shape[0]
    taus = np.arange(L - 16, L)
    ref = score_unit(keys, beacons, recents, L, taus, 1e4)
    lse = _fused_lse(keys, beacons, recents, L, L - 16, 1e4)
    wrong = score_from_lse(keys, beacons, recents, L, taus, 1e4, lse, L)
    assert not np.allclose(wrong, ref, rtol=1e-6, atol=0)
