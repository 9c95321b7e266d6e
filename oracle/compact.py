"""Compaction: index the cache along the sequence axis with the keep set.

Paper text, §2.2: the compressed cache is obtained by indexing the sequence
dimension with the retained index set; summary, "方法步骤详情" step (5):
written back in position order.  Reading: kept keys keep their original
absolute positions, so the position array is indexed the same way.

``fill_holes`` is the unsorted variant: the ThinKV pages note that attention
is invariant to the order of the cached tokens and reuse evicted slots in
place instead of gathering.  Here the kept tokens at slots >= B_KV move into
the evicted slots below B_KV and every other kept token stays where it is,
so slots [0, B_KV) hold the kept set, not in position order.
"""

import numpy as np


def compact(keys, values, kpos, kept):
    kept = np.asarray(kept, dtype=np.int64)
    return (np.take(keys, kept, axis=0), np.take(values, kept, axis=0),
            np.take(kpos, kept, axis=0))


def fill_holes(keys, values, kpos, kept, b_kv):
    """Kept tokens past b_kv fill the evicted slots below b_kv.

    kept: the ascending keep set (b_kv slots).  The i-th lowest evicted slot
    below b_kv (a "hole") receives the i-th lowest kept slot at or above
    b_kv.  Returns the first b_kv rows of keys, values and positions after
    the moves, and the (hole, source) pairs.
    """
    kept = np.asarray(kept, dtype=np.int64)
    low = kept[kept < b_kv]
    high = kept[kept >= b_kv]
    holes = np.setdiff1d(np.arange(b_kv), low)
    assert holes.size == high.size
    k = np.array(keys[:b_kv], copy=True)
    v = np.array(values[:b_kv], copy=True)
    p = np.array(kpos[:b_kv], copy=True)
    k[holes] = keys[high]
    v[holes] = values[high]
    p[holes] = kpos[high]
    return k, v, p, list(zip(holes.tolist(), high.tolist()))
