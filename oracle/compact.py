"""Compaction: index the cache along the sequence axis with the keep set.

Paper text, §2.2: the compressed cache is obtained by indexing the sequence
dimension with the retained index set; summary, "方法步骤详情" step (5):
written back in position order.  Reading: kept keys keep their original
absolute positions, so the position array is indexed the same way.
"""

import numpy as np


def compact(keys, values, kpos, kept):
    kept = np.asarray(kept, dtype=np.int64)
    return (np.take(keys, kept, axis=0), np.take(values, kept, axis=0),
            np.take(kpos, kept, axis=0))
