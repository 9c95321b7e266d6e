"""Continual-FPS state machine of one KV group during decoding.

Summary, "方法步骤详情" steps (1)-(6), and paper text, §4.2 and App. D.2:

1. prefill: the cache takes every prefill token; each query head compresses
   its prefill pre-RoPE queries with FPS to B_Q^min = 16 rows;
2. decoding: each new pre-RoPE query is appended to its head's buffer; when
   the buffer reaches B_Q^max = 32 it is compressed back to 16 with FPS
   ("fill and compress");
3. when the cache length reaches B_max - n_recent, the buffer is compressed
   (if it holds more than 16) and frozen as the beacon set; the following
   n_recent queries are kept aside as recent queries with their positions;
4.-5. when the cache reaches B_max the cache is scored and compacted
   (``evict.evict_unit``);
6. afterwards beacons and recents are merged and compressed back to 16, and
   collection resumes.

Readings: positions are 0-based and the next token's position is t; the
query of the token that brings the cache to B_max - n_recent still goes to
the buffer; the cache is trimmed to the workload's B_KV (the pages' 7/8
rule is one choice of B_KV).

``beacons="initial"`` is the Initial+Recent comparison of paper text §5.3
(Table 3): the historical reference set is the first n_beacon queries
generated after the prompt, kept as they are for the whole run (no FPS, no
merge); everything else -- recents, scoring with the references rotated to
t, selection, compaction -- is unchanged.
"""

import numpy as np

from .evict import evict_unit
from .fps import fps


class UnitStream:
    """Exact per-unit replay of the decode-time policy (slow; small units)."""

    def __init__(self, g, d, b_max, b_kv, prefix, theta, recent_tok=16,
                 n_recent_q=16, buf_min=16, buf_max=32, beacons="fps", unsorted=False):
        if beacons not in ("fps", "initial"):
            raise ValueError(f"beacons must be 'fps' or 'initial', not {beacons!r}")
        self.policy = beacons
        self.unsorted = unsorted  # compact by filling holes (cache not in position order)
        self.g, self.d = g, d
        self.b_max, self.b_kv, self.prefix = b_max, b_kv, prefix
        self.theta, self.recent_tok = theta, recent_tok
        self.n_recent_q, self.buf_min, self.buf_max = n_recent_q, buf_min, buf_max
        self.keys = np.zeros((0, d))
        self.values = np.zeros((0, d))
        self.kpos = np.zeros(0, dtype=np.int64)
        self.t = 0
        self.buf = [np.zeros((0, d)) for _ in range(g)]
        self.recents = [[] for _ in range(g)]
        self.phase = "collect"
        self.events = []  # (kind, cache length) log

    def prefill(self, keys, values, queries):
        """keys/values: [P, d]; queries: [g, P, d] pre-RoPE prefill queries."""
        p = keys.shape[0]
        self.keys = np.asarray(keys, np.float64).copy()
        self.values = np.asarray(values, np.float64).copy()
        self.kpos = np.arange(p, dtype=np.int64)
        self.t = p
        if self.policy == "initial":  # references come from the generation
            self.events.append(("prefill", p))
            return
        for h in range(self.g):
            _, keep = fps(queries[h], self.buf_min)
            self.buf[h] = np.asarray(queries[h], np.float64)[keep]
        self.events.append(("prefill_fps", p))

    def _compress(self, kind):
        for h in range(self.g):
            _, keep = fps(self.buf[h], self.buf_min)
            self.buf[h] = self.buf[h][keep]
        self.events.append((kind, self.keys.shape[0]))

    def step(self, k, v, q):
        """Decode one token: k, v: [d]; q: [g, d] pre-RoPE queries."""
        self.keys = np.vstack([self.keys, np.asarray(k, np.float64)[None]])
        self.values = np.vstack([self.values, np.asarray(v, np.float64)[None]])
        self.kpos = np.append(self.kpos, self.t)
        L = self.keys.shape[0]
        if self.policy == "initial":
            if self.phase == "collect":
                if self.buf[0].shape[0] < self.buf_min:
                    for h in range(self.g):
                        self.buf[h] = np.vstack([self.buf[h],
                                                 np.asarray(q[h], np.float64)[None]])
                    if self.buf[0].shape[0] == self.buf_min:
                        self.events.append(("initial_set", L))
                if L == self.b_max - self.n_recent_q:
                    self.events.append(("recent_start", L))
                    self.phase = "recent"
            else:
                for h in range(self.g):
                    self.recents[h].append(np.asarray(q[h], np.float64))
            self.t += 1
            if L == self.b_max:
                self._evict()
            return
        if self.phase == "collect":
            for h in range(self.g):
                self.buf[h] = np.vstack([self.buf[h], np.asarray(q[h], np.float64)[None]])
            if self.buf[0].shape[0] >= self.buf_max:
                self._compress("collect_fps")
            if L == self.b_max - self.n_recent_q:
                if self.buf[0].shape[0] > self.buf_min:
                    self._compress("beacon_fix_fps")
                else:
                    self.events.append(("beacon_fix_noop", L))
                self.phase = "recent"
        else:
            for h in range(self.g):
                self.recents[h].append(np.asarray(q[h], np.float64))
        self.t += 1
        if L == self.b_max:
            self._evict()

    def _evict(self):
        L = self.keys.shape[0]
        beacons = np.stack(self.buf)
        recents = np.stack([np.stack(r) for r in self.recents])
        initial = self.policy == "initial"
        out = evict_unit(self.keys, self.values, self.kpos, L, beacons, recents,
                         self.t, self.b_kv, self.prefix, self.recent_tok,
                         self.theta, n_min=self.buf_min, merge=not initial,
                         unsorted=self.unsorted)
        self.keys, self.values, self.kpos = out["keys"], out["values"], out["kpos"]
        if not initial:
            self.buf = [out["buf"][h] for h in range(self.g)]
        self.recents = [[] for _ in range(self.g)]
        self.phase = "collect"
        self.events.append(("evict", L))
        if not initial:
            self.events.append(("merge_fps", self.keys.shape[0]))
        self.last_evict = out
        return out


def kv_cache_bytes(layers, kv_heads, d_head, tokens, batch, bytes_per_elem=2):
    """Bytes of a KV cache holding ``tokens`` per sequence.

    Review page, "문제 1": two tensors (K and V) per layer and KV head, each
    d_head wide, for every token of every sequence.
    """
    return 2 * layers * kv_heads * d_head * tokens * batch * bytes_per_elem
