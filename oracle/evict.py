"""One eviction event of one KV group, composed from the pinned parts.

Summary, "方法步骤详情" steps (4)-(6) and paper text, App. D.2: score the
cache with the observation set, keep prefix + recent + Top-K, compact the
cache in position order, then merge the beacon and recent queries and
compress them back to the minimum buffer size with FPS.

Parity unpinned as a whole: the pages print no worked eviction, so this
composite is trusted through its parts (rope, bf16, score, select, compact,
fps), each pinned separately.
"""

import numpy as np

from .compact import compact, fill_holes
from .fps import fps
from .score import score_unit
from .select import select


def evict_unit(keys, values, kpos, L, beacons, recents, t, b_kv, prefix,
               recent_tok, theta, n_min=16, scale=None, merge=True, aggregate="max",
               unsorted=False):
    """keys/values: [>=L, d]; kpos: [>=L]; beacons/recents: [g, 16, d].

    aggregate: the pooling of the scores, "max" (the method) or "mean".
    unsorted: compact by filling the evicted slots (compact.fill_holes)
    instead of in position order.

    Returns a dict with score [L], kept [b_kv], the compacted keys, values
    and positions, and (with merge) the merged buffer [g, n_min, d] plus the
    per-head FPS pick orders.
    """
    keys = np.asarray(keys, dtype=np.float64)[:L]
    values = np.asarray(values, dtype=np.float64)[:L]
    kpos = np.asarray(kpos, dtype=np.int64)[:L]
    n_recent = np.asarray(recents).shape[1]
    taus = kpos[L - n_recent:L]
    sc = score_unit(keys, beacons, recents, t, taus, theta, scale, aggregate=aggregate)
    kept = select(sc, L, b_kv, prefix, recent_tok)
    if unsorted:
        k2, v2, p2, _ = fill_holes(keys, values, kpos, kept, b_kv)
    else:
        k2, v2, p2 = compact(keys, values, kpos, kept)
    out = {"score": sc, "kept": kept, "keys": k2, "values": v2, "kpos": p2}
    if merge:
        bufs, orders = [], []
        for h in range(np.asarray(beacons).shape[0]):
            merged = np.concatenate([np.asarray(beacons[h], np.float64),
                                     np.asarray(recents[h], np.float64)])
            order, keep_rows = fps(merged, n_min)
            bufs.append(merged[keep_rows])
            orders.append(order)
        out["buf"] = np.stack(bufs)
        out["fps_order"] = orders
    return out

