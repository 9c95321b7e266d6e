"""Decode-time driver of the eviction path: host control flow only.

Summary, "方法步骤详情" steps (1)-(6); paper text §4.2 and App. D.2.  Every
unit gains one token per decode step (all units in lockstep), so one library
call covers all units at each point of the policy:

1. prefill: the prompt's keys, values and positions go into the cache; each
   query head compresses its prompt queries with FPS to 16 rows;
2. collect: each step appends the head's new pre-RoPE query to its buffer,
   and a buffer reaching 32 rows is compressed back to 16 (bkv_fps_update);
3. when the cache length reaches B_max - 16, heads holding more than 16 rows
   are compressed (the beacon fix); the next 16 queries are collected as
   recent queries instead (bkv_fps_update in append-only mode);
4.-6. when the cache reaches B_max, bkv_evict scores, selects and compacts
   the cache to B_KV and merges beacons and recents back to 16 rows.

With beacon_policy="initial" (the Initial+Recent comparison, paper text
§5.3 and Table 3) the reference rows are instead the first 16 queries
generated after the prompt, appended and then left alone: no FPS at any
point and no merge after an eviction.  With unsorted=True the evictions
compact by filling the evicted slots (bkv_compact_unsorted): the cache is
then not in position order, which scoring and the slot-based masks do not
need (every slot below the recent window holds an older token).

Writing the new token's key, value and position into the cache is the
decoder's own work and is done here with plain tensor writes; every step of
the policy runs in the library.  An optional observer is called with
(event, stage, stream) before ("pre") and after ("post") every FPS and
eviction event, for verification.
"""
from dataclasses import replace

import torch

from . import bkv


class Stream:
    def __init__(self, n_units, group, d_head, b_max, b_kv, prefix, theta, recent_tok=16,
                 device="cuda", observer=None, beacon_policy="fps", unsorted=False):
        if b_max - b_kv < recent_tok or b_kv < prefix + recent_tok:
            raise ValueError("need prefix + recent_tok <= b_kv <= b_max - recent_tok")
        if beacon_policy not in ("fps", "initial"):
            raise ValueError(f"beacon_policy must be 'fps' or 'initial', not {beacon_policy!r}")
        self.policy = beacon_policy
        dev = torch.device(device)
        self.shape = bkv.Shape(n_units, group, d_head, b_max, prefix, theta,
                               recent_tok=recent_tok, unsorted=unsorted)
        self.rshape = replace(self.shape, buf_cap=self.shape.n_recent_q)
        U, nq = n_units, n_units * group
        self.b_max, self.b_kv, self.recent_tok = b_max, b_kv, recent_tok
        self.K = torch.zeros((U, b_max, d_head), dtype=torch.bfloat16, device=dev)
        self.V = torch.zeros_like(self.K)
        self.kpos = torch.zeros((U, b_max), dtype=torch.int32, device=dev)
        self.buf = torch.zeros((nq, self.shape.buf_cap, d_head), dtype=torch.float32, device=dev)
        self.count = torch.zeros((nq,), dtype=torch.int32, device=dev)
        self.recents = torch.zeros((nq, self.shape.n_recent_q, d_head), dtype=torch.float32,
                                   device=dev)
        self.rcount = torch.zeros((nq,), dtype=torch.int32, device=dev)
        self.score = torch.zeros((U, b_max), dtype=torch.float32, device=dev)
        self.kept = torch.zeros((U, b_kv), dtype=torch.int32, device=dev)
        self.sel = torch.zeros((nq, 16), dtype=torch.int32, device=dev)
        self.ws = bkv.alloc_workspace(self.shape, b_max, b_kv, dev)
        self.L = 0        # live slots (all units)
        self.t = 0        # position of the next token
        self.rows = 0     # rows in every head's buffer
        self.phase = "collect"
        self.events = []  # (kind, cache length)
        self.observer = observer
        self.n_evictions = 0

    def _note(self, kind, stage):
        if self.observer is not None:
            self.observer(kind, stage, self)

    def prefill(self, keys, values, queries):
        """keys, values: bf16 [U, P, d]; queries: fp32 [U*g, P, d] (P <= 8192)."""
        P = keys.shape[1]
        if P < 17 or P > 8192 or P >= self.b_max - self.recent_tok:
            raise ValueError(f"prompt length {P} not supported")
        self.K[:, :P] = keys
        self.V[:, :P] = values
        self.kpos[:, :P] = torch.arange(P, dtype=torch.int32, device=self.K.device)
        self.L = self.t = P
        if self.policy == "initial":  # the references come from the generation
            if self.b_max - self.recent_tok - P < 16:
                raise ValueError("prompt too long: 16 generated queries must precede the "
                                 "recent window")
            self.count.zero_()
            self.rows = 0
            self.events.append(("prefill", P))
            return
        pshape = replace(self.shape, buf_cap=P)
        qbuf = queries.contiguous().clone()
        pcount = torch.full_like(self.count, P)
        self.prompt_queries = qbuf
        self._note("prefill_fps", "pre")
        bkv.fps_update(pshape, qbuf, pcount, trigger=P, m=16, sel_order=self.sel)
        self.buf[:, :16] = qbuf[:, :16]
        self.count.fill_(16)
        self.rows = 16
        self.events.append(("prefill_fps", P))
        self._note("prefill_fps", "post")

    def step(self, k, v, q):
        """One decode step: k, v bf16 [U, d]; q fp32 [U*g, d]."""
        L = self.L
        self.last_q = q  # the step's queries, for observers
        self.K[:, L] = k
        self.V[:, L] = v
        self.kpos[:, L] = self.t
        self.L = L = L + 1
        if self.policy == "initial":
            self._step_initial(q, L)
        elif self.phase == "collect":
            compress = self.rows + 1 >= 32
            if compress:
                self._note("collect_fps", "pre")
            # Every head holds the same number of rows, so the host knows when the
            # buffer fills: other steps append only (trigger past the capacity).
            bkv.fps_update(self.shape, self.buf, self.count, q[:, None],
                           trigger=32 if compress else self.shape.buf_cap + 1, m=16,
                           sel_order=self.sel if compress else None)
            self.rows = 16 if compress else self.rows + 1
            if compress:
                self.events.append(("collect_fps", L))
                self._note("collect_fps", "post")
            if L == self.b_max - self.recent_tok:
                if self.rows > 16:
                    self._note("beacon_fix_fps", "pre")
                    bkv.fps_update(self.shape, self.buf, self.count, None, trigger=17, m=16,
                                   sel_order=self.sel)
                    self.rows = 16
                    self.events.append(("beacon_fix_fps", L))
                    self._note("beacon_fix_fps", "post")
                else:
                    self.events.append(("beacon_fix_noop", L))
                self.phase = "recent"
                self.rcount.zero_()
        else:
            # recent query: appended to the recents buffer, never compressed
            bkv.fps_update(self.rshape, self.recents, self.rcount, q[:, None],
                           trigger=self.rshape.buf_cap + 1, m=16)
        self.t += 1
        if L == self.b_max:
            self._evict()

    def _step_initial(self, q, L):
        if self.phase == "collect":
            if self.rows < 16:  # one of the first 16 generated queries: append only
                bkv.fps_update(self.shape, self.buf, self.count, q[:, None],
                               trigger=self.shape.buf_cap + 1, m=16)
                self.rows += 1
                if self.rows == 16:
                    self.events.append(("initial_set", L))
            if L == self.b_max - self.recent_tok:
                self.events.append(("recent_start", L))
                self.phase = "recent"
                self.rcount.zero_()
        else:
            bkv.fps_update(self.rshape, self.recents, self.rcount, q[:, None],
                           trigger=self.rshape.buf_cap + 1, m=16)

    def _evict(self):
        L = self.L
        initial = self.policy == "initial"
        self._note("evict", "pre")
        bkv.evict(self.shape, self.K, self.V, self.kpos, L, self.buf, self.recents, self.t,
                  self.b_kv, buf=None if initial else self.buf,
                  count=None if initial else self.count, score_out=self.score,
                  kept_out=self.kept, ws=self.ws)
        self.L = self.b_kv
        if not initial:
            self.rows = 16
        self.phase = "collect"
        self.n_evictions += 1
        self.events.append(("evict", L))
        if not initial:
            self.events.append(("merge_fps", self.b_kv))
        self._note("evict", "post")
