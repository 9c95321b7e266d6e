"""Observation-set scoring: RoPE alignment, attention weights, max pooling.

(Mean pooling, the pages' ablation of the pooling step, is an option.)

Paper text, §4.3: when the cache is full at decoding step t, the observation
set combines the beacon queries, rotated to t, and the most recent queries,
kept at their own positions tau; its attention weights W over the current
cache (|Q_obs| x L) are max-pooled over all queries and all heads of the
GQA group.  Summary, "方法步骤详情" step (4) and the review's §4.3 give the
pooled score as Score[j] = max over heads h in the group and queries q of
W[h, q, j].  Paper text, §2.1-§2.2: W is scaled dot-product attention,
softmax(q k^T / sqrt(d)) under the causal mask.

Readings where the pages are silent (each listed with its reason in the
design notes):

* the softmax runs over all L live slots, prefix and recent slots included;
* a recent query at slot L - n_recent + i sees slots 0 .. L - n_recent + i
  (its own key included); beacon rows see every slot, since every cached
  position is before t;
* each query head contributes its own beacons and recents, so a KV group of
  g heads has g * (n_beacon + n_recent) observation rows;
* the rotated rows are rounded to bfloat16 (through float32) before the
  product, matching the bfloat16 cache; everything after is float64.
"""

import numpy as np

from .bf16 import round_f64_to_bf16
from .rope import rope


def observation_set(beacons, recents, t, taus, theta):
    """Rotated, bf16-rounded observation rows of one KV group.

    beacons: [g, n_beacon, d] pre-RoPE queries, rotated to position t.
    recents: [g, n_recent, d] pre-RoPE queries, row i rotated to taus[i].
    Returns [g, n_beacon + n_recent, d] float64 holding bfloat16 values.
    """
    beacons = np.asarray(beacons, dtype=np.float64)
    recents = np.asarray(recents, dtype=np.float64)
    qb = rope(beacons, np.full(beacons.shape[:-1], t, dtype=np.float64), theta)
    tau = np.broadcast_to(np.asarray(taus, dtype=np.float64), recents.shape[:-1])
    qr = rope(recents, tau, theta)
    return round_f64_to_bf16(np.concatenate([qb, qr], axis=1))


def visibility(L, n_beacon, n_recent):
    """Boolean [n_beacon + n_recent, L]: which slots each observation row sees."""
    vis = np.ones((n_beacon + n_recent, L), dtype=bool)
    slots = np.arange(L)
    for i in range(n_recent):
        vis[n_beacon + i] = slots <= L - n_recent + i
    return vis


def logits(qhat, keys, scale):
    """s[h, r, j] = qhat[h, r] . k_j * scale (scale = 1/sqrt(d))."""
    return np.einsum("hrd,jd->hrj", np.asarray(qhat, np.float64),
                     np.asarray(keys, np.float64)) * scale


def attention_weights(s, vis):
    """Row softmax of s over visible slots; hidden slots get weight 0."""
    s = np.where(vis[None], s, -np.inf)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    return e / e.sum(axis=-1, keepdims=True)


def pooled_score(w, aggregate="max"):
    """Pool W[h, r, j] over every head and observation row of the group.

    "max": Score[j] = max over (h, r) of W[h, r, j] (the method's pooling,
    paper text §4.3).  "mean": Score[j] = the average of W[h, r, j] over all
    N = heads x rows of the group, rows that cannot see slot j counting with
    weight 0 (the mean-aggregation ablation, paper text §5.3 / Table 2, and
    the average form of the importance score in §2.2; over a group the
    average runs over all queries and heads, as the max does).
    """
    flat = w.reshape(-1, w.shape[-1])
    if aggregate == "max":
        return flat.max(axis=0)
    if aggregate == "mean":
        return flat.sum(axis=0) / flat.shape[0]
    raise ValueError(f"aggregate must be 'max' or 'mean', not {aggregate!r}")


def score_unit(keys, beacons, recents, t, taus, theta, scale=None,
               return_all=False, aggregate="max"):
    """Score every slot of one KV group's cache.

    keys: [L, d] (bfloat16 values widened to float64).
    aggregate: "max" (the method) or "mean" (the ablation), see pooled_score.
    Returns score [L] (and, with return_all, qhat, logits and weights).
    """
    keys = np.asarray(keys, dtype=np.float64)
    L, d = keys.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    n_beacon = np.asarray(beacons).shape[1]
    n_recent = np.asarray(recents).shape[1]
    qhat = observation_set(beacons, recents, t, taus, theta)
    s = logits(qhat, keys, scale)
    w = attention_weights(s, visibility(L, n_beacon, n_recent))
    sc = pooled_score(w, aggregate)
    if return_all:
        return sc, qhat, s, w
    return sc
