"""Keep-set construction (selection) for one KV group.

Summary, "方法步骤详情" step (5): the prefix tokens {1..n_prefix} and the
most recent tokens {L-n_recent+1..L} are always kept; the rest of the budget
is filled by Top-K on the score, and the kept entries are written back in
position order.  Paper text, §2.2 (top-B_KV retention) and App. D.2.

Readings: positions here are 0-based slots, so the forced set is
[0, P) U [L-R, L); the budget B_KV counts the forced slots (exactly B_KV
entries are kept); ties in score go to the lower slot.
"""

import numpy as np


def select(score, L, b_kv, prefix, recent_tok):
    """Return the kept slots of one unit, ascending, length b_kv."""
    score = np.asarray(score, dtype=np.float64)[:L]
    if not (prefix + recent_tok <= b_kv < L):
        raise ValueError("need prefix + recent_tok <= b_kv < L")
    forced = np.concatenate([np.arange(prefix), np.arange(L - recent_tok, L)])
    middle = np.arange(prefix, L - recent_tok)
    k = b_kv - prefix - recent_tok
    # np.lexsort orders by its last key first: score descending, then slot.
    order = np.lexsort((middle, -score[middle]))
    chosen = middle[order[:k]]
    return np.sort(np.concatenate([forced, chosen])).astype(np.int64)
