"""Decode-time streaming run (Stream driver over the C ABI) against the oracle.

The policy's event cadence must equal the oracle state machine's
(oracle.stream.UnitStream, same prompt length, B_max, B_KV).  Every event is
checked on the GPU's own state just before it ("lockstep with resync"): each
FPS compression by replaying its pick order in float64; each eviction by the
oracle's scores and kept set on the pre-eviction cache, exact compaction
with the GPU's kept set, and the merged buffer.  Small run: every unit and
head, under the method's Continual FPS and under the Initial+Recent
comparison (the first 16 generated queries as fixed references).  Qwen3-14B shape (40 layers x batch 16 x 8 KV heads, group 5): the
first two eviction intervals on sampled units and heads, and the whole
32,768-step run with every 16th eviction checked.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check_fps, check_kept, check_scores, log
from reasoning_model_kv_amd import stream as bstream

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Checker:
    """Observer: snapshots sampled state before each event, checks after."""

    def __init__(self, w, units, policy="fps", unsorted=False, every_evict=1, every_fps=1):
        self.w, self.units, self.policy, self.unsorted = w, list(units), policy, unsorted
        self.heads = [u * w.group + h for u in self.units for h in range(w.group)]
        self.pre = None
        self.n = {"fps": 0, "evict": 0, "exact_fps": 0}
        self.worst = 0.0
        # Check every every_evict-th eviction and every every_fps-th FPS event
        # (counting from the first); the others run unobserved.
        self.every = {"evict": every_evict, "fps": every_fps}
        self.seen = {"evict": 0, "fps": 0}
        self.checking = True
        self.checked_evictions = []

    def __call__(self, kind, stage, st):
        cls = "evict" if kind == "evict" else "fps"
        if stage == "pre":
            self.checking = self.seen[cls] % self.every[cls] == 0
            self.seen[cls] += 1
        if not self.checking:
            return
        hi = torch.tensor(self.heads, device=st.buf.device)
        if stage == "pre":
            if kind == "prefill_fps":
                self.pre = {"rows": st.prompt_queries[hi].cpu().numpy()}
            elif kind in ("collect_fps", "beacon_fix_fps"):
                rows = st.buf[hi].cpu().numpy()
                n = st.rows
                if kind == "collect_fps":  # the step's query is appended first
                    rows[:, n] = st.last_q[hi].cpu().numpy()
                    n += 1
                self.pre = {"rows": rows[:, :n]}
            else:
                ui = torch.tensor(self.units, device=st.K.device)
                self.pre = {"K": st.K[ui].float().cpu().numpy(),
                            "V": st.V[ui].float().cpu().numpy(),
                            "P": st.kpos[ui].cpu().numpy(), "L": st.L, "t": st.t,
                            "beacons": st.buf[hi, :16].cpu().numpy(),
                            "recents": st.recents[hi].cpu().numpy()}
            return
        if kind != "evict":
            sel = st.sel[hi].cpu().numpy()
            out = st.buf[hi, :16].cpu().numpy()
            for i, q in enumerate(self.heads):
                rows = self.pre["rows"][i]
                self.n["exact_fps"] += check_fps(rows, sel[i], 16, f"{kind} head {q}")
                assert np.array_equal(out[i], rows[np.sort(sel[i])]), f"{kind} head {q} rows"
            self.n["fps"] += 1
            return
        w, pre, g = self.w, self.pre, self.w.group
        L, b = pre["L"], w.b_kv
        ui = torch.tensor(self.units, device=st.K.device)
        K1, V1, P1 = (st.K[ui].float().cpu().numpy(), st.V[ui].float().cpu().numpy(),
                      st.kpos[ui].cpu().numpy())
        sc, kept = st.score[ui].cpu().numpy(), st.kept[ui].cpu().numpy()
        merged_out = st.buf[hi, :16].cpu().numpy()
        for i, u in enumerate(self.units):
            hs = slice(i * g, (i + 1) * g)
            initial = self.policy == "initial"
            ref = oracle.evict.evict_unit(pre["K"][i], pre["V"][i], pre["P"][i], L,
                                          pre["beacons"][hs], pre["recents"][hs], pre["t"], b,
                                          w.prefix, w.recent_tok, w.theta, merge=not initial)
            where = f"evict at L={L} unit {u}"
            self.worst = max(self.worst, check_scores(sc[i, :L], ref["score"], where))
            check_kept(kept[i], ref["score"], L, b, w.prefix, w.recent_tok, where)
            if self.unsorted:
                ek, ev, ep, _ = oracle.compact.fill_holes(pre["K"][i], pre["V"][i], pre["P"][i],
                                                          kept[i], b)
            else:
                ek, ev, ep = oracle.compact.compact(pre["K"][i], pre["V"][i], pre["P"][i],
                                                    kept[i])
            assert np.array_equal(K1[i, :b], ek), where + " K"
            assert np.array_equal(V1[i, :b], ev), where + " V"
            assert np.array_equal(P1[i, :b], ep), where + " kpos"
            if initial:  # no merge: the reference rows stay as they were
                assert np.array_equal(merged_out[hs], pre["beacons"][hs]), where + " refs"
                continue
            for h in range(g):
                merged = np.concatenate([pre["beacons"][i * g + h], pre["recents"][i * g + h]])
                out = merged_out[i * g + h]
                idx = [int(np.nonzero((merged == row).all(axis=1))[0][0]) for row in out]
                assert idx == sorted(idx) and len(set(idx)) == 16, where + " merged rows"
                if min(oracle.fps.fps_margins(merged, 16)) > 2e-3:
                    order, _ = oracle.fps.fps(merged, 16)
                    assert sorted(order) == idx, where + " merged FPS set"
        self.n["evict"] += 1
        self.checked_evictions.append(self.seen["evict"] - 1)


def _oracle_events(w, n_steps, policy="fps"):
    """Event cadence of the oracle state machine (values do not affect it)."""
    st = oracle.stream.UnitStream(1, 4, w.L, w.b_kv, w.prefix, w.theta, beacons=policy)
    r = np.random.default_rng(0)
    st.prefill(r.standard_normal((w.prefix, 4)), r.standard_normal((w.prefix, 4)),
               r.standard_normal((1, w.prefix, 4)))
    for _ in range(n_steps):
        st.step(r.standard_normal(4), r.standard_normal(4), r.standard_normal((1, 4)))
    return st.events


def _run(w, n_steps, units, chunk=128, policy="fps", unsorted=False, fused=False,
         every_evict=1, every_fps=1, batched=False):
    chk = Checker(w, units, policy, unsorted, every_evict, every_fps)
    st = bstream.Stream(w.n_units, w.group, w.d_head, w.L, w.b_kv, w.prefix, w.theta,
                        device=DEV, observer=chk, beacon_policy=policy, unsorted=unsorted,
                        fused_decode=fused)
    gen = synth.StreamInputs(w, DEV)
    st.prefill(*gen.prompt())
    done = 0
    c = 0
    while done < n_steps:
        k, v, q = gen.chunk(c, chunk)
        c += 1
        m = min(chunk, n_steps - done)
        if batched:  # stretches of appends issued together (Stream.run)
            st.run(k[:m], v[:m], q[:m])
        else:
            for s in range(m):
                st.step(k[s], v[s], q[s])
        done += m
    torch.cuda.synchronize()
    return st, chk


def test_stream_small_all_units():
    w = synth.WORKLOADS["stream_small"]
    n = w.stream_steps
    log(f"stream {w.name}: U={w.n_units} g={w.group} B_max={w.L} B_KV={w.b_kv} steps={n}")
    st, chk = _run(w, n, range(w.n_units))
    assert st.events == _oracle_events(w, n)
    first = w.L - w.prefix
    assert st.n_evictions == 1 + (n - first) // 128
    assert chk.n["evict"] == st.n_evictions and chk.n["fps"] > 10
    log(f"  events {len(st.events)}, evictions {st.n_evictions}, FPS events {chk.n['fps']}, "
        f"exact FPS sets {chk.n['exact_fps']}, max score rel err {chk.worst:.3g}")


def test_stream_qwen3_14b_two_intervals_sampled():
    w = synth.WORKLOADS["qwen3_14b_stream"]
    n = (w.L - w.prefix) + 128 + 40  # two evictions, then into the third interval
    units = [0, 2047, w.n_units - 1]
    log(f"stream {w.name}: U={w.n_units} g={w.group} steps={n} sampled units {units}")
    st, chk = _run(w, n, units)
    assert st.events == _oracle_events(w, n)
    assert st.n_evictions == 2 and chk.n["evict"] == 2
    assert st.L == w.b_kv + 40
    assert torch.all(st.count == 16 + 40 % 16)
    log(f"  FPS events {chk.n['fps']}, exact FPS sets {chk.n['exact_fps']}, "
        f"max score rel err {chk.worst:.3g}")


def test_stream_qwen3_14b_full_run_sampled():
    """All 32,768 decode steps of the Qwen3-14B shape (5120 units, 226
    evictions per unit), driven as the streaming bench drives them (chunks of
    128 steps through Stream.run): the cadence equals the oracle's over the whole run,
    every 16th eviction and every 64th FPS event is checked in lockstep on
    three units spread over the cache, and at the end every unit's positions
    are strictly ascending and every head holds the rows the cadence says."""
    w = synth.WORKLOADS["qwen3_14b_stream"]
    n = w.stream_steps
    units = [0, 2047, w.n_units - 1]
    log(f"stream {w.name}: all {n} steps, units {units}, every 16th eviction checked")
    st, chk = _run(w, n, units, every_evict=16, every_fps=64, batched=True)
    assert st.events == _oracle_events(w, n)
    first = w.L - w.prefix
    assert st.n_evictions == 1 + (n - first) // 128 == 226
    assert chk.checked_evictions == list(range(0, st.n_evictions, 16))
    assert chk.checked_evictions[-1] >= 208  # checks reach the end of the run
    L = st.L
    assert torch.all(st.kpos[:, 1:L] > st.kpos[:, :L - 1])
    assert torch.all(st.kpos[:, L - 1] == st.t - 1)
    assert torch.all(st.count == st.rows)
    log(f"  evictions {st.n_evictions} ({len(chk.checked_evictions)} checked), FPS events "
        f"checked {chk.n['fps']}, exact FPS sets {chk.n['exact_fps']}, "
        f"max score rel err {chk.worst:.3g}")


def test_stream_small_initial_recent_all_units():
    """Initial+Recent: the first 16 generated queries are the references."""
    w = synth.WORKLOADS["stream_small"]
    n = w.stream_steps
    log(f"stream {w.name} (Initial+Recent): U={w.n_units} g={w.group} steps={n}")
    st, chk = _run(w, n, range(w.n_units), policy="initial")
    assert st.events == _oracle_events(w, n, "initial")
    assert chk.n["evict"] == st.n_evictions >= 2 and chk.n["fps"] == 0
    assert torch.all(st.count == 16)
    log(f"  evictions {st.n_evictions}, max score rel err {chk.worst:.3g}")


def test_stream_small_unsorted_compaction_all_units():
    """Evictions that fill holes: same cadence, exact hole filling at every
    eviction, and the cache stays a permutation with the prefix in place."""
    w = synth.WORKLOADS["stream_small"]
    n = w.stream_steps
    log(f"stream {w.name} (unsorted compaction): U={w.n_units} steps={n}")
    st, chk = _run(w, n, range(w.n_units), unsorted=True)
    assert st.events == _oracle_events(w, n)
    assert chk.n["evict"] == st.n_evictions >= 2
    P = w.prefix
    assert torch.equal(st.kpos[:, :P], torch.arange(P, dtype=torch.int32,
                                                    device=st.kpos.device).expand(w.n_units, -1))
    live = st.kpos[:, :st.L]
    assert torch.all(torch.sort(live, dim=1).values[:, 1:] > torch.sort(live, dim=1).values[:, :-1])
    log(f"  evictions {st.n_evictions}, max score rel err {chk.worst:.3g}")


def test_stream_long_prompt_prefill():
    """A 1000-token prompt: the prefill FPS runs on the long-buffer path."""
    w = synth.shrink(synth.WORKLOADS["stream_small"], prefix=1000, L=1280, b_kv=1152,
                     stream_steps=300)
    n = w.stream_steps
    log(f"stream long prompt: U={w.n_units} g={w.group} P={w.prefix} B_max={w.L} steps={n}")
    st, chk = _run(w, n, range(w.n_units))
    assert st.events == _oracle_events(w, n)
    assert st.n_evictions == 1 and chk.n["evict"] == 1 and chk.n["fps"] > 5
    log(f"  FPS events {chk.n['fps']}, exact FPS sets {chk.n['exact_fps']}, "
        f"max score rel err {chk.worst:.3g}")


@pytest.mark.parametrize("unsorted", [False, True])
def test_stream_small_fused_decode_all_units(unsorted):
    """Denominators gathered by decode attention (beacon rows at the beacon
    fix, each recent query's own step), one key read at each eviction: same
    cadence, and every eviction checked against the two-pass definition."""
    w = synth.WORKLOADS["stream_small"]
    n = w.stream_steps
    log(f"stream {w.name} (fused decode, unsorted={unsorted}): U={w.n_units} steps={n}")
    st, chk = _run(w, n, range(w.n_units), unsorted=unsorted, fused=True)
    assert st.events == _oracle_events(w, n)
    assert chk.n["evict"] == st.n_evictions >= 2 and chk.n["fps"] > 10
    log(f"  evictions {st.n_evictions}, max score rel err {chk.worst:.3g}")


def test_stream_qwen3_14b_fused_decode_sampled():
    w = synth.WORKLOADS["qwen3_14b_stream"]
    n = (w.L - w.prefix) + 128 + 40
    units = [0, 2047, w.n_units - 1]
    log(f"stream {w.name} (fused decode): steps={n} sampled units {units}")
    st, chk = _run(w, n, units, fused=True)
    assert st.events == _oracle_events(w, n)
    assert st.n_evictions == 2 and chk.n["evict"] == 2
    log(f"  max score rel err {chk.worst:.3g}")


@pytest.mark.parametrize("policy,unsorted,fused", [("fps", False, False), ("fps", True, False),
                                                   ("initial", False, False), ("fps", False, True)])
def test_stream_run_equals_step(policy, unsorted, fused):
    """Stream.run (stretches of appends issued together) leaves every tensor
    and host field bit for bit as step() does, over three evictions, with
    chunks that start and end inside stretches.  The one exception is the
    dead rows of the beacon buffers (at or past a head's count): a fill call
    that appends and compresses reads its new rows from its input without
    storing them, so after a stretch that ends in a compression those rows
    keep older queries; nothing reads them before they are appended over."""
    w = synth.WORKLOADS["stream_small"]
    n = 700
    log(f"stream run vs step ({policy}, unsorted={unsorted}, fused={fused}): {n} steps")
    gen = synth.StreamInputs(w, DEV)
    prompt = gen.prompt()
    chunks = [gen.chunk(c, 128) for c in range((n + 127) // 128)]
    k = torch.cat([c[0] for c in chunks])[:n]
    v = torch.cat([c[1] for c in chunks])[:n]
    q = torch.cat([c[2] for c in chunks])[:n]

    def make():
        st = bstream.Stream(w.n_units, w.group, w.d_head, w.L, w.b_kv, w.prefix, w.theta,
                            device=DEV, beacon_policy=policy, unsorted=unsorted,
                            fused_decode=fused)
        st.prefill(*prompt)
        return st

    a, b = make(), make()
    for i in range(n):
        a.step(k[i], v[i], q[i])
    s0 = 0
    for m in (37, 128, 1, 200, 99, 235):  # 700 steps in uneven chunks
        b.run(k[s0:s0 + m], v[s0:s0 + m], q[s0:s0 + m])
        s0 += m
    assert s0 == n
    torch.cuda.synchronize()
    assert a.n_evictions == b.n_evictions >= 3
    assert a.events == b.events and (a.L, a.t, a.rows, a.phase) == (b.L, b.t, b.rows, b.phase)
    for name in ("K", "V"):
        assert torch.equal(getattr(a, name).view(torch.int16), getattr(b, name).view(torch.int16)), name
    names = ["kpos", "count", "recents", "rcount", "kept", "score", "sel"]
    if fused:
        names += ["lse_in", "lse_obs"]
    for name in names:
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.all(a.count == a.rows)
    assert torch.equal(a.buf[:, :a.rows], b.buf[:, :a.rows]), "live beacon-buffer rows"
    log(f"  evictions {a.n_evictions}, events {len(a.events)}")


@pytest.mark.parametrize("fused", [False, True])
def test_stream_checkpoint_resume_bit_identical(fused):
    """A run snapshotted in its recent-query phase (state_dict through
    torch.save / torch.load(weights_only=True)) and resumed in a new driver
    continues bit for bit like the original, through two more evictions."""
    import io
    w = synth.WORKLOADS["stream_small"]
    n1, n2 = 340, 300
    log(f"stream checkpoint/resume (fused={fused}): {n1} steps, snapshot, {n2} more")
    gen = synth.StreamInputs(w, DEV)
    prompt = gen.prompt()
    chunks = [gen.chunk(c, 128) for c in range((n1 + n2 + 127) // 128)]

    def step(st, i):
        k, v, q = chunks[i // 128]
        st.step(k[i % 128], v[i % 128], q[i % 128])

    def make():
        return bstream.Stream(w.n_units, w.group, w.d_head, w.L, w.b_kv, w.prefix, w.theta,
                              device=DEV, fused_decode=fused)

    a = make()
    a.prefill(*prompt)
    for i in range(n1):
        step(a, i)
    assert a.phase == "recent"
    blob = io.BytesIO()
    torch.save(a.state_dict(), blob)
    for i in range(n1, n1 + n2):
        step(a, i)
    blob.seek(0)
    b = make()
    b.load_state_dict(torch.load(blob, weights_only=True))
    for i in range(n1, n1 + n2):
        step(b, i)
    torch.cuda.synchronize()
    assert a.n_evictions == b.n_evictions >= 3
    assert a.events == b.events and (a.L, a.t, a.rows, a.phase) == (b.L, b.t, b.rows, b.phase)
    for n in ("K", "V"):
        assert torch.equal(getattr(a, n).view(torch.int16), getattr(b, n).view(torch.int16)), n
    for n in ("kpos", "buf", "count", "recents", "rcount", "kept", "score"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    log(f"  evictions {a.n_evictions}, events {len(a.events)}")
