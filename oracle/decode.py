"""Decode attention with the observation rows' softmax statistics.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages point at fusing the beacon scoring into the attention kernel as a
way to remove the eviction step's extra latency (summary, "未来方向": fold
beacon scoring into the attention kernel; the summary's "局限与改进" notes
that no kernel-level fusion is discussed).  The arithmetic that makes it
possible is plain softmax algebra:

* decode attention (paper text §2.1: softmax(q k^T / sqrt(d)) V under the
  causal mask) of the query generated at step tau attends to exactly the
  cache slots a recent observation row i sees at the next eviction (its own
  key and everything before it, paper text §4.3), so its log-sum-exp is that
  row's softmax denominator;
* the beacons are fixed once the cache reaches B_max - R (summary step (3))
  and are rotated to the eviction's step t (paper text §4.3), so their
  log-sum-exp over the slots present at that point can be accumulated while
  the attention pass reads the keys, and the slots appended afterwards are
  added with log(e^a + e^b).

With those denominators known, the eviction's scores need the logits once:
W[r, j] = exp(s[r, j] - LSE_r).

Everything is float64; the queries meet the keys after the same rounding
the scoring uses (rotate in float64, then float32, then bfloat16).
"""

import numpy as np

from .bf16 import round_f64_to_bf16
from .rope import rope
from .score import logits, observation_set, pooled_score, visibility


def _scale(d, scale):
    return 1.0 / np.sqrt(d) if scale is None else scale


def rotated_queries(q, pos, theta):
    """Pre-RoPE queries [n, d] rotated to pos (scalar or [n]), rounded to bf16."""
    q = np.asarray(q, dtype=np.float64)
    p = np.broadcast_to(np.asarray(pos, dtype=np.float64), q.shape[:-1])
    return round_f64_to_bf16(rope(q, p, theta))


def logsumexp_rows(s):
    """log sum_j exp(s[..., j]) with the row maximum taken out first; an
    empty row sums to 0, so its log is -inf."""
    s = np.asarray(s, dtype=np.float64)
    if s.shape[-1] == 0:
        return np.full(s.shape[:-1], -np.inf)
    mx = s.max(axis=-1, keepdims=True)
    return (mx + np.log(np.exp(s - mx).sum(axis=-1, keepdims=True)))[..., 0]


def decode_attention(keys, values, q, t_q, theta, scale=None):
    """Attention of one new query per head of a KV group over its cache.

    keys, values: [L, d] (bfloat16 values widened to float64), the new
    token's key already in slot L - 1, so every slot is visible.
    q: [g, d] pre-RoPE queries of the g heads, rotated to t_q.
    Returns (out [g, d] = softmax(s) V, lse [g] = log sum_j exp(s_j)) with
    s = qhat . k_j * scale.
    """
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    qhat = rotated_queries(q, t_q, theta)
    s = qhat @ keys.T * _scale(keys.shape[1], scale)
    lse = logsumexp_rows(s)
    w = np.exp(s - lse[:, None])
    return w @ values, lse


def beacon_lse(keys, beacons, t_obs, theta, scale=None):
    """log sum_j exp(s_bj) of each beacon row over the slots in `keys`.

    keys: [n, d]; beacons: [g, n_beacon, d] pre-RoPE, rotated to t_obs.
    Returns [g, n_beacon].
    """
    keys = np.asarray(keys, dtype=np.float64)
    b = np.asarray(beacons, dtype=np.float64)
    qhat = rotated_queries(b.reshape(-1, b.shape[-1]), t_obs, theta)
    s = qhat @ keys.T * _scale(keys.shape[1], scale)
    return logsumexp_rows(s).reshape(b.shape[:2])


def score_from_lse(keys, beacons, recents, t, taus, theta, lse_in, lse_from,
                   scale=None, aggregate="max"):
    """Pooled score of every slot from known softmax denominators.

    lse_in: [g, n_beacon + n_recent]: for beacon rows the log-sum-exp over
    slots [0, lse_from); for recent rows the complete log-sum-exp over the
    slots they see.  The beacon rows' slots [lse_from, L) are added here:
    LSE = log(exp(lse_in) + sum over those slots of exp(s)).
    Then W = exp(s - LSE) on visible slots (0 elsewhere) and the scores are
    pooled as in score.pooled_score.
    """
    keys = np.asarray(keys, dtype=np.float64)
    L, d = keys.shape
    nb = np.asarray(beacons).shape[1]
    nr = np.asarray(recents).shape[1]
    qhat = observation_set(beacons, recents, t, taus, theta)
    s = logits(qhat, keys, _scale(d, scale))
    lse = np.array(lse_in, dtype=np.float64, copy=True)
    if lse_from < L:
        tail = np.concatenate([lse[:, :nb, None], s[:, :nb, lse_from:]], axis=-1)
        lse[:, :nb] = logsumexp_rows(tail)
    vis = visibility(L, nb, nr)
    w = np.where(vis[None], np.exp(s - lse[:, :, None]), 0.0)
    return pooled_score(w, aggregate)
