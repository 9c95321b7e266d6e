"""Host control flow of the decode-time driver, without a GPU.

The library calls of reasoning_model_kv_amd.stream are replaced by recorders,
so the driver runs on CPU tensors; what is checked is its cadence: when it
compresses, fixes the beacons, collects recent queries and evicts.  The
float64 oracle's UnitStream (summary, "方法步骤详情" steps (1)-(6)) logs the same
events for the same lengths, and the two logs must be equal.
"""
import numpy as np
import pytest
import torch

import oracle
from reasoning_model_kv_amd import stream as smod


class Recorder:
    def __init__(self):
        self.calls = []

    def fps_update(self, shape, buf, count, new_q=None, trigger=32, m=16, sel_order=None,
                   n_overflow=None, stream=None):
        self.calls.append(("fps", shape.buf_cap, trigger, 0 if new_q is None else new_q.shape[-2]))

    def evict(self, shape, K, V, kpos, L, beacons, recents, t, b_kv, **kw):
        self.calls.append(("evict", L, t, kw.get("buf") is not None))

    def evict_lse(self, shape, K, V, kpos, L, beacons, recents, t, lse_in, lse_from, b_kv, **kw):
        self.calls.append(("evict_lse", L, t, lse_from))

    def decode_attend(self, shape, K, V, L, q, t_q, out, lse_q, beacons=None, t_obs=0,
                      lse_obs=None, stream=None):
        self.calls.append(("decode", L, t_q, None if beacons is None else t_obs))


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    for name in ("fps_update", "evict", "evict_lse", "decode_attend"):
        monkeypatch.setattr(smod.bkv, name, getattr(r, name))
    return r


def test_guard_needs_room_for_the_recent_window():
    # After an eviction the cache holds b_kv slots; the recent phase starts at
    # b_max - 16, which must come after it.
    with pytest.raises(ValueError):
        smod.Stream(1, 1, 64, b_max=80, b_kv=64, prefix=4, theta=1e4, device="cpu")
    with pytest.raises(ValueError):
        smod.Stream(1, 1, 64, b_max=200, b_kv=32, prefix=20, theta=1e4, recent_tok=16,
                    device="cpu")
    smod.Stream(1, 1, 64, b_max=81, b_kv=64, prefix=4, theta=1e4, device="cpu")


def _run_both(b_max, b_kv, prefix, recent_tok, n_steps, policy="fps", rec=None):
    g, d = 1, 64
    st = smod.Stream(1, g, d, b_max=b_max, b_kv=b_kv, prefix=prefix, theta=1e4,
                     recent_tok=recent_tok, device="cpu", beacon_policy=policy)
    ora = oracle.stream.UnitStream(g, d, b_max=b_max, b_kv=b_kv, prefix=prefix, theta=1e4,
                                   recent_tok=recent_tok,
                                   beacons="fps" if policy == "fps" else "initial")
    r = np.random.default_rng(0)
    P = 20
    k, v, q = r.standard_normal((P, d)), r.standard_normal((P, d)), r.standard_normal((g, P, d))
    ora.prefill(k, v, q)
    st.prefill(torch.zeros(1, P, d, dtype=torch.bfloat16), torch.zeros(1, P, d, dtype=torch.bfloat16),
               torch.zeros(g, P, d))
    for _ in range(n_steps):
        ora.step(r.standard_normal(d), r.standard_normal(d), r.standard_normal((g, d)))
        st.step(torch.zeros(1, d, dtype=torch.bfloat16), torch.zeros(1, d, dtype=torch.bfloat16),
                torch.zeros(g, d))
    return st, ora


@pytest.mark.parametrize("b_max,b_kv,prefix,recent_tok", [
    (64 + 128, 64, 4, 16),     # the workloads' trigger at B_KV + 128
    (64 + 17, 64, 4, 16),      # the smallest gap the guard allows
    (64 + 40, 64, 4, 32),      # 32 kept recent tokens, 16 recent queries
])
def test_cadence_matches_the_oracle(rec, b_max, b_kv, prefix, recent_tok):
    n_steps = 3 * (b_max - b_kv) + (b_max - 20) + 5
    st, ora = _run_both(b_max, b_kv, prefix, recent_tok, n_steps, rec=rec)
    assert [tuple(e) for e in st.events] == [tuple(e) for e in ora.events]
    assert st.n_evictions == 4
    # Each eviction scores 16 recent queries gathered after the beacon fix.
    calls = rec.calls
    ev = [i for i, c in enumerate(calls) if c[0] == "evict"]
    assert len(ev) == 4
    for i in ev:
        assert calls[i][1] == b_max and calls[i][3]
        recent = 0
        j = i - 1
        while calls[j][0] == "fps" and calls[j][1] == 16:   # appends to the recents
            assert calls[j][2] == 17 and calls[j][3] == 1
            recent += 1
            j -= 1
        assert recent == 16
    assert st.L == ora.keys.shape[0] and st.t == ora.t


def test_initial_policy_cadence_matches_the_oracle(rec):
    st, ora = _run_both(64 + 128, 64, 4, 16, 2 * 128 + 180, policy="initial", rec=rec)
    assert [tuple(e) for e in st.events] == [tuple(e) for e in ora.events]
    assert all(not c[3] for c in rec.calls if c[0] == "evict")  # no merge


def test_eviction_refuses_a_buffer_that_is_not_the_beacons(rec):
    st, _ = _run_both(64 + 128, 64, 4, 16, 10, rec=rec)
    st.rows = 20
    with pytest.raises(RuntimeError):
        st._evict()


@pytest.mark.parametrize("policy", ["fps", "initial"])
def test_run_batches_appends_with_the_same_cadence(rec, policy):
    """Stream.run issues each stretch of append-only steps (with no observer,
    up to and including a compressing step) as one fill call of n_new rows
    and keeps every other call, and the event log, as step() makes them; the
    oracle's log is the same."""
    b_max, b_kv, prefix, n_steps = 200, 160, 8, 400
    g, d, P = 1, 64, 20

    def make():
        st = smod.Stream(1, g, d, b_max=b_max, b_kv=b_kv, prefix=prefix, theta=1e4,
                         device="cpu", beacon_policy=policy)
        st.prefill(torch.zeros(1, P, d, dtype=torch.bfloat16),
                   torch.zeros(1, P, d, dtype=torch.bfloat16), torch.zeros(g, P, d))
        return st

    a = make()
    for _ in range(n_steps):
        a.step(torch.zeros(1, d, dtype=torch.bfloat16), torch.zeros(1, d, dtype=torch.bfloat16),
               torch.zeros(g, d))
    calls_a = list(rec.calls)
    rec.calls.clear()
    b = make()
    done = 0
    for m in (7, 128, 1, 64, 200):
        b.run(torch.zeros(m, 1, d, dtype=torch.bfloat16), torch.zeros(m, 1, d, dtype=torch.bfloat16),
              torch.zeros(m, g, d))
        done += m
    assert done == n_steps
    calls_b = list(rec.calls)
    assert a.events == b.events and (a.L, a.t, a.rows, a.phase) == (b.L, b.t, b.rows, b.phase)
    assert a.n_evictions == b.n_evictions >= 2

    def split(calls):  # (rows appended per buffer, every other call in order)
        rows = {}
        other = []
        for c in calls:
            if c[0] == "fps":
                rows[c[1]] = rows.get(c[1], 0) + c[3]
                if c[2] != c[1] + 1:  # not append-only (trigger within the capacity): a
                    other.append(c[:3])  # compression, whatever rows it appended first
            else:
                other.append(c)
        return rows, other

    rows_a, other_a = split(calls_a)
    rows_b, other_b = split(calls_b)
    assert rows_a == rows_b and other_a == other_b
    assert len(calls_b) < len(calls_a) / 4
    ora = oracle.stream.UnitStream(g, d, b_max=b_max, b_kv=b_kv, prefix=prefix, theta=1e4,
                                   beacons=policy)
    r = np.random.default_rng(0)
    ora.prefill(r.standard_normal((P, d)), r.standard_normal((P, d)),
                r.standard_normal((g, P, d)))
    for _ in range(n_steps):
        ora.step(r.standard_normal(d), r.standard_normal(d), r.standard_normal((g, d)))
    assert b.events == ora.events
