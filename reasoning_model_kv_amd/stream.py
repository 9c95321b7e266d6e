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

With fused_decode=True the steps' decode attention (bkv_decode_attend) also
gathers the scores' softmax denominators: at the beacon fix it adds the
beacon rows, rotated to the coming eviction's step, and at each recent step
the new query's own log-sum-exp is kept; the eviction then scores with
bkv_evict_lse (bkv_evict with the scores from those denominators: one read
of the keys).  The attention output of those steps is left in
`attn_out`; other steps' attention is the decoder's own business and is not
run here.

Writing the new token's key, value and position into the cache is the
decoder's own work and is done here with plain tensor writes; every step of
the policy runs in the library.  An optional observer is called with
(event, stage, stream) before ("pre") and after ("post") every FPS and
eviction event, for verification (or only the event kinds in `observe`).
"""
from dataclasses import replace

import torch

from . import bkv


class Stream:
    def __init__(self, n_units, group, d_head, b_max, b_kv, prefix, theta, recent_tok=16,
                 device="cuda", observer=None, beacon_policy="fps", unsorted=False,
                 fused_decode=False, observe=None):
        # The recent phase starts when the cache reaches b_max - n_recent_q, so
        # that n_recent_q queries are collected before the eviction at b_max;
        # after an eviction the cache holds b_kv slots and must lie below that
        # point again, or the next interval would never switch phase.
        n_recent_q = 16
        if not (b_kv < b_max - n_recent_q and prefix + recent_tok <= b_kv):
            raise ValueError(f"need prefix + recent_tok <= b_kv < b_max - n_recent_q "
                             f"({n_recent_q}); got prefix {prefix}, recent_tok {recent_tok}, "
                             f"b_kv {b_kv}, b_max {b_max}")
        if beacon_policy not in ("fps", "initial"):
            raise ValueError(f"beacon_policy must be 'fps' or 'initial', not {beacon_policy!r}")
        self.policy = beacon_policy
        if fused_decode and beacon_policy != "fps":
            raise ValueError("fused_decode needs the Continual-FPS beacons")
        self.fused = fused_decode
        dev = torch.device(device)
        self.shape = bkv.Shape(n_units, group, d_head, b_max, prefix, theta,
                               recent_tok=recent_tok, unsorted=unsorted)
        self.rshape = replace(self.shape, buf_cap=self.shape.n_recent_q)
        U, nq = n_units, n_units * group
        self.b_max, self.b_kv, self.recent_tok = b_max, b_kv, recent_tok
        self.n_recent_q = self.shape.n_recent_q
        assert self.n_recent_q == n_recent_q
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
        self._steps = torch.arange(b_max, dtype=torch.int32, device=dev)  # run(): position offsets
        self.ws = bkv.alloc_workspace(self.shape, b_max, b_kv, dev)
        self.L = 0        # live slots (all units)
        self.t = 0        # position of the next token
        self.rows = 0     # rows in every head's buffer
        self.phase = "collect"
        self.events = []  # (kind, cache length)
        self.observer = observer
        self.observe = None if observe is None else frozenset(observe)
        self.n_evictions = 0
        if fused_decode:
            self.attn_out = torch.zeros((nq, d_head), dtype=torch.float32, device=dev)
            self.lse_q = torch.zeros((nq,), dtype=torch.float32, device=dev)
            self.lse_obs = torch.zeros((nq, 16), dtype=torch.float32, device=dev)
            self.lse_in = torch.zeros((U, group, 32), dtype=torch.float32, device=dev)
            self.lse_from = 0
            self.t_obs = -1

    # Checkpoint and resume: every piece of the policy's state is either a
    # tensor the caller could save or one of these host fields.
    _TENSORS = ("K", "V", "kpos", "buf", "count", "recents", "rcount", "score", "kept", "sel")
    _FUSED_TENSORS = ("attn_out", "lse_q", "lse_obs", "lse_in")
    _HOST = ("L", "t", "rows", "phase", "events", "n_evictions")
    _FUSED_HOST = ("lse_from", "t_obs")

    def state_dict(self):
        """The whole state as a dict of tensors (copies on the host) and plain
        values, loadable with torch.load(weights_only=True)."""
        names_t = self._TENSORS + (self._FUSED_TENSORS if self.fused else ())
        names_h = self._HOST + (self._FUSED_HOST if self.fused else ())
        sd = {n: getattr(self, n).detach().cpu().clone() for n in names_t}
        sd.update({n: getattr(self, n) for n in names_h if n != "events"})
        sd["events"] = [list(e) for e in self.events]
        sd["prompt_queries"] = (self.prompt_queries.detach().cpu().clone()
                                if hasattr(self, "prompt_queries") else None)
        return sd

    def load_state_dict(self, sd):
        """Restore a state_dict() of a Stream built with the same arguments."""
        names_t = self._TENSORS + (self._FUSED_TENSORS if self.fused else ())
        names_h = self._HOST + (self._FUSED_HOST if self.fused else ())
        for n in names_t:
            dst = getattr(self, n)
            if tuple(sd[n].shape) != tuple(dst.shape) or sd[n].dtype != dst.dtype:
                raise ValueError(f"state {n}: {tuple(sd[n].shape)} {sd[n].dtype} does not match "
                                 f"{tuple(dst.shape)} {dst.dtype}")
            dst.copy_(sd[n])
        for n in names_h:
            if n != "events":
                setattr(self, n, sd[n])
        self.events = [tuple(e) for e in sd["events"]]
        if sd.get("prompt_queries") is not None:
            self.prompt_queries = sd["prompt_queries"].to(self.K.device)

    def _observed(self, kind):
        return self.observer is not None and (self.observe is None or kind in self.observe)

    def _note(self, kind, stage):
        if self._observed(kind):
            self.observer(kind, stage, self)

    def prefill(self, keys, values, queries):
        """keys, values: bf16 [U, P, d]; queries: fp32 [U*g, P, d] (P <= 8192)."""
        P = keys.shape[1]
        if P < 17 or P > 8192 or P >= self.b_max - self.n_recent_q:
            raise ValueError(f"prompt length {P} not supported")
        self.K[:, :P] = keys
        self.V[:, :P] = values
        self.kpos[:, :P] = torch.arange(P, dtype=torch.int32, device=self.K.device)
        self.L = self.t = P
        if self.policy == "initial":  # the references come from the generation
            if self.b_max - self.n_recent_q - P < 16:
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
            if L == self.b_max - self.n_recent_q:
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
                if self.fused:
                    # This step's attention, plus the fixed beacons rotated to
                    # the eviction's step (n_recent_q more tokens from here).
                    self.t_obs = self.t + 1 + self.n_recent_q
                    bkv.decode_attend(self.shape, self.K, self.V, L, q, self.t, self.attn_out,
                                      self.lse_q, self.buf, self.t_obs, self.lse_obs)
                    self.lse_in[:, :, :16] = self.lse_obs.view(-1, self.shape.group, 16)
                    self.lse_from = L
        else:
            # recent query: appended to the recents buffer, never compressed
            bkv.fps_update(self.rshape, self.recents, self.rcount, q[:, None],
                           trigger=self.rshape.buf_cap + 1, m=16)
            if self.fused:
                # The step's attention; its log-sum-exp is recent row i's
                # denominator (this cache is exactly what that row sees).
                i = L - 1 - (self.b_max - self.n_recent_q)
                bkv.decode_attend(self.shape, self.K, self.V, L, q, self.t, self.attn_out,
                                  self.lse_q)
                self.lse_in[:, :, 16 + i] = self.lse_q.view(-1, self.shape.group)
        self.t += 1
        if L == self.b_max:
            self._evict()

    def run(self, k, v, q):
        """n decode steps at once: k, v bf16 [n, U, d]; q fp32 [n, U*g, d].

        Leaves the same state at every policy event and at the end as n calls
        of step().  Between events nothing reads the cache, the positions or
        the query buffers (attention is the caller's), so a stretch of steps
        that only append is issued together: one bkv_fps_update appending its
        queries (the fill step with n_new rows, read in place from the
        step-major block through the strided entry point) and one write each
        of the K, V and position slots, instead of four launches per step.
        Steps that fix the beacons, switch phase or evict, and the recent
        phase's steps with fused decode (each attends), run through step().
        The step that completes the initial references ends its stretch, and
        so does a step that compresses unless that event is observed (the
        fill call appends, then compresses); an observed one runs alone, so
        the observer sees the states step() shows it."""
        n = k.shape[0]
        s = 0
        while s < n:
            m = min(self._append_run(), n - s)
            if m <= 1:
                self.step(k[s], v[s], q[s])
                s += 1
            else:
                self._append_steps(k[s:s + m], v[s:s + m], q[s:s + m])
                s += m

    def _append_run(self):
        """How many steps from here only append (and write the cache)."""
        L, lim = self.L, self.b_max - self.n_recent_q
        if self.phase == "recent":
            return 0 if self.fused else self.b_max - 1 - L   # the step reaching b_max evicts
        room = lim - 1 - L                                     # the step reaching lim switches phase
        if self.policy == "initial":  # completing the references notifies no observer
            return min(room, 16 - self.rows) if self.rows < 16 else room
        fold = not self._observed("collect_fps")
        return min(room, (32 if fold else 31) - self.rows)     # the step reaching 32 rows compresses

    def _append_steps(self, k, v, q):
        m, L, t = k.shape[0], self.L, self.t
        self.last_q = q[-1]
        self.K[:, L:L + m] = k.transpose(0, 1)
        self.V[:, L:L + m] = v.transpose(0, 1)
        torch.add(self._steps[:m].expand(self.kpos.shape[0], m), t, out=self.kpos[:, L:L + m])
        self.L, self.t = L + m, t + m
        if self.phase == "recent":
            bkv.fps_update(self.rshape, self.recents, self.rcount, q.transpose(0, 1),
                           trigger=self.rshape.buf_cap + 1, m=16)
        elif self.policy == "fps":
            compress = self.rows + m >= 32
            bkv.fps_update(self.shape, self.buf, self.count, q.transpose(0, 1),
                           trigger=32 if compress else self.shape.buf_cap + 1, m=16,
                           sel_order=self.sel if compress else None)
            self.rows = 16 if compress else self.rows + m
            if compress:
                self.events.append(("collect_fps", L + m))
        elif self.rows < 16:
            bkv.fps_update(self.shape, self.buf, self.count, q.transpose(0, 1),
                           trigger=self.shape.buf_cap + 1, m=16)
            self.rows += m
            if self.rows == 16:
                self.events.append(("initial_set", L + m))

    def _step_initial(self, q, L):
        if self.phase == "collect":
            if self.rows < 16:  # one of the first 16 generated queries: append only
                bkv.fps_update(self.shape, self.buf, self.count, q[:, None],
                               trigger=self.shape.buf_cap + 1, m=16)
                self.rows += 1
                if self.rows == 16:
                    self.events.append(("initial_set", L))
            if L == self.b_max - self.n_recent_q:
                self.events.append(("recent_start", L))
                self.phase = "recent"
                self.rcount.zero_()
        else:
            bkv.fps_update(self.rshape, self.recents, self.rcount, q[:, None],
                           trigger=self.rshape.buf_cap + 1, m=16)

    def _evict(self):
        L = self.L
        initial = self.policy == "initial"
        # The merge appends the recents to buffers that must hold exactly the
        # beacons (the library leaves a head whose rows would not fit
        # unchanged); every head holds self.rows rows.
        if not initial and self.rows != self.shape.n_beacon:
            raise RuntimeError(f"eviction with {self.rows} buffer rows per head; the merge "
                               f"needs exactly {self.shape.n_beacon}")
        self._note("evict", "pre")
        if self.fused:
            if self.t != self.t_obs:
                raise RuntimeError("eviction step differs from the beacons' rotation step")
            bkv.evict_lse(self.shape, self.K, self.V, self.kpos, L, self.buf, self.recents,
                          self.t, self.lse_in, self.lse_from, self.b_kv, buf=self.buf,
                          count=self.count, score_out=self.score, kept_out=self.kept,
                          ws=self.ws)
        else:
            bkv.evict(self.shape, self.K, self.V, self.kpos, L, self.buf, self.recents,
                      self.t, self.b_kv, buf=None if initial else self.buf,
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
