"""Pins of the scoring definition: softmax, masking, pooling, hand values."""
import numpy as np
import scipy.special

from oracle.score import (attention_weights, logits, observation_set, pooled_score,
                          score_unit, visibility)


def _case(seed=0, g=2, L=96, d=16):
    r = np.random.default_rng(seed)
    keys = r.standard_normal((L, d))
    beacons = r.standard_normal((g, 16, d))
    recents = r.standard_normal((g, 16, d))
    taus = np.arange(L - 16, L)
    return keys, beacons, recents, taus


def test_rows_sum_to_one_and_match_library_softmax():
    keys, b, rc, taus = _case()
    L = keys.shape[0]
    sc, qhat, s, w = score_unit(keys, b, rc, L, taus, 1e4, return_all=True)
    assert np.allclose(w.sum(axis=-1), 1.0, atol=1e-12, rtol=0)
    # A beacon row has no mask: it is the plain softmax of its logits.
    assert np.allclose(w[1, 3], scipy.special.softmax(s[1, 3]), rtol=1e-13, atol=0)
    # A recent row: softmax of its visible prefix, zeros after.
    i = 5
    vis = L - 16 + i + 1
    assert np.allclose(w[0, 16 + i, :vis], scipy.special.softmax(s[0, 16 + i, :vis]),
                       rtol=1e-13, atol=0)
    assert np.all(w[0, 16 + i, vis:] == 0)


def test_score_is_brute_force_max_and_lse_form():
    keys, b, rc, taus = _case(1, g=3, L=64, d=8)
    L = keys.shape[0]
    sc, qhat, s, w = score_unit(keys, b, rc, L, taus, 1e4, return_all=True)
    vis = visibility(L, 16, 16)
    for j in range(L):
        best = 0.0
        for h in range(3):
            for r_ in range(32):
                if vis[r_, j]:
                    best = max(best, w[h, r_, j])
        assert sc[j] == best
    # Independent closed form: exp(max_r (s_rj - LSE_r)) over visible rows.
    sm = np.where(vis[None], s, -np.inf)
    lse = scipy.special.logsumexp(sm, axis=-1, keepdims=True)
    alt = np.exp((sm - lse).reshape(-1, L).max(axis=0))
    assert np.allclose(sc, alt, rtol=1e-12, atol=0)


def test_score_bounds():
    keys, b, rc, taus = _case(2, g=4, L=200, d=32)
    L = keys.shape[0]
    sc = score_unit(keys, b, rc, L, taus, 1e6)
    assert np.all(sc > 0) and np.all(sc <= 1)
    assert sc.sum() >= 1 - 1e-12
    assert sc.sum() <= 4 * 32 + 1e-9


def test_identical_keys_give_closed_form_mask_values():
    # Every logit of a row is equal, so each row is uniform over what it sees:
    # beacon rows 1/L, recent row i 1/(L-15+i).  The pooled score of a slot is
    # the largest weight among the rows that see it.
    L, d = 80, 16
    r = np.random.default_rng(3)
    k = r.standard_normal(d)
    keys = np.tile(k, (L, 1))
    b, rc = r.standard_normal((2, 16, d)), r.standard_normal((2, 16, d))
    sc = score_unit(keys, b, rc, L, np.arange(L - 16, L), 1e4)
    want = np.empty(L)
    want[: L - 15] = 1.0 / (L - 15)
    for i in range(1, 16):
        want[L - 16 + i] = 1.0 / (L - 15 + i)
    assert np.allclose(sc, want, rtol=1e-12, atol=0)


def test_logit_scale_hand_value():
    qhat = np.array([[[1.0, 2.0, 0.0, 0.0]]])
    keys = np.array([[3.0, 1.0, 5.0, 0.0]])
    assert np.allclose(logits(qhat, keys, 1 / 2.0), [[[2.5]]])


def test_observation_rows_at_position_zero_are_rounded_queries():
    r = np.random.default_rng(4)
    b, rc = r.standard_normal((1, 16, 8)), r.standard_normal((1, 16, 8))
    q = observation_set(b, rc, 0, np.zeros(16), 1e4)
    import torch
    want = torch.from_numpy(np.concatenate([b, rc], axis=1).astype(np.float32)).to(
        torch.bfloat16).double().numpy()
    assert np.array_equal(q, want)


def test_beacons_rotate_to_t_recents_to_their_positions():
    # For a key rotated to position p, the logit depends only on (query pos - p):
    # a beacon at t against a key stored at t equals the unrotated dot product.
    r = np.random.default_rng(6)
    d = 8
    b = np.zeros((1, 16, d))
    b[0, 0] = [1, 0, 0, 0, 0, 0, 0, 0]
    rc = np.zeros((1, 16, d))
    rc[0, 0] = [1, 0, 0, 0, 0, 0, 0, 0]
    q = observation_set(b, rc, 3, np.arange(16) + 10, 1e4)
    from oracle.bf16 import round_f64_to_bf16
    assert np.allclose(q[0, 0], round_f64_to_bf16(
        [np.cos(3.0), 0, 0, 0, np.sin(3.0), 0, 0, 0]))
    assert np.allclose(q[0, 16], round_f64_to_bf16(
        [np.cos(10.0), 0, 0, 0, np.sin(10.0), 0, 0, 0]))
    _ = r


def test_pooled_score_and_weights_shapes():
    s = np.zeros((2, 32, 40))
    w = attention_weights(s, visibility(40, 16, 16))
    assert pooled_score(w).shape == (40,)


def test_mean_pooling_sums_to_one_and_brute_force():
    # Every softmax row sums to 1, so the average of the rows sums to 1 over
    # the slots; and each slot's value is the plain average over all
    # g x 32 rows, hidden rows counting as 0.
    keys, b, rc, taus = _case(7, g=3, L=70, d=8)
    L = keys.shape[0]
    sc, _, _, w = score_unit(keys, b, rc, L, taus, 1e4, return_all=True, aggregate="mean")
    assert abs(sc.sum() - 1.0) < 1e-12
    vis = visibility(L, 16, 16)
    for j in (0, 17, L - 16, L - 9, L - 1):
        tot = 0.0
        for h in range(3):
            for r_ in range(32):
                tot += w[h, r_, j] if vis[r_, j] else 0.0
        assert abs(sc[j] - tot / 96) < 1e-15
    mx = score_unit(keys, b, rc, L, taus, 1e4)
    assert np.all(sc <= mx) and np.all(sc >= mx / 96 - 1e-18)


def test_mean_pooling_identical_keys_closed_form():
    # Uniform rows: beacon rows give 1/L to every slot, recent row i gives
    # 1/(L-15+i) to slots 0..L-16+i.  The mean over the 2 x 32 rows is
    # (16/L + sum over recent rows that see j of 1/(L-15+i)) / 32.
    L, d = 80, 16
    r = np.random.default_rng(8)
    keys = np.tile(r.standard_normal(d), (L, 1))
    b, rc = r.standard_normal((2, 16, d)), r.standard_normal((2, 16, d))
    sc = score_unit(keys, b, rc, L, np.arange(L - 16, L), 1e4, aggregate="mean")
    want = np.empty(L)
    for j in range(L):
        tot = 16.0 / L
        for i in range(16):
            if j <= L - 16 + i:
                tot += 1.0 / (L - 15 + i)
        want[j] = tot / 32
    assert np.allclose(sc, want, rtol=1e-12, atol=0)


def test_mean_equals_max_for_a_single_row():
    # One head, one recent row and no beacons: both poolings return that row.
    r = np.random.default_rng(9)
    L, d = 30, 8
    keys = r.standard_normal((L, d))
    b = np.zeros((1, 0, d))
    rc = r.standard_normal((1, 1, d))
    a = score_unit(keys, b, rc, L, [L - 1], 1e4, aggregate="mean")
    m = score_unit(keys, b, rc, L, [L - 1], 1e4)
    assert np.array_equal(a, m)
    try:
        pooled_score(np.zeros((1, 1, 3)), "median")
    except ValueError:
        pass
    else:
        raise AssertionError("unknown pooling must be rejected")
