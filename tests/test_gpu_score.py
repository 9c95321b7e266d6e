"""Scoring kernel (bkv_score) against the float64 oracle on the GPU.

The kernel streams each unit's keys in tiles of 64 through a ring of three
LDS tiles (two passes); the cases cover a single tile, several tiles and
ring turns, a ragged last tile, a last tile that some recent rows cannot
see at all, recent positions that need the direct RoPE path (all or some of
the rows), and groups of
2, 4, 5 and 7 (which change the number of loader wavefronts).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check_scores, log
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(name):
    if name == "tiny_g7":
        return synth.shrink(synth.WORKLOADS["tiny"], group=7, d_head=128, theta=1e6)
    if name == "tiny_g5":
        return synth.shrink(synth.WORKLOADS["tiny"], group=5, d_head=128, theta=1e6,
                            h_kv=3)
    if name == "tiny_g8":
        return synth.shrink(synth.WORKLOADS["tiny"], group=8, d_head=128, theta=1e6)
    return synth.WORKLOADS[name]


def _run(w, L=None, l_cap=None, t=None, kpos_offset=0, shift_first_recents=0, aggregate="max"):
    L = L or w.L
    l_cap = l_cap or L
    w2 = synth.shrink(w, L=L)
    inp = synth.workload_inputs(w2)
    inp["kpos"] = inp["kpos"] + kpos_offset
    if shift_first_recents:  # recent rows 0..7 earlier, rows 8..15 at t-8..t-1
        inp["kpos"][:, L - 16:L - 8] -= shift_first_recents
    t = t if t is not None else L + kpos_offset
    dev = synth.to_device(inp, DEV, l_cap=l_cap)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, l_cap, w.prefix, w.theta,
                      recent_tok=w.recent_tok, n_beacon=w.n_beacon, n_recent_q=w.n_recent_q,
                      aggregate=aggregate)
    score = torch.full((w.n_units, l_cap), -1.0, device=DEV)
    qobs = torch.zeros((w.n_units, w.group * 32, w.d_head), dtype=torch.bfloat16, device=DEV)
    beacons = dev["buf"] if w.n_beacon else None
    bkv.score(shape, dev["keys"], dev["kpos"], L, beacons, dev["recents"], t, score, qobs)
    torch.cuda.synchronize()
    return inp, score.cpu().numpy(), qobs.cpu(), t


CASES = [
    ("tiny", None, None, 0),          # 256 slots: 4 tiles, one ring turn
    ("tiny", 203, 256, 0),            # ragged tail, l_cap > L
    ("tiny", 40, 64, 0),              # one tile; recent rows masked inside it
    ("tiny", 64, 64, 0),              # exactly one full tile
    ("tiny", 128, 128, 0),            # exactly two tiles
    ("tiny", 150, 150, 37),           # recent positions != t-16+i: direct RoPE path
    ("tiny", 517, 600, 0),            # 5-key last tile, invisible to recent rows 0..10
    ("tiny", 700, 700, 37),           # eleven tiles, direct RoPE path
    ("tiny", 300, 300, "partial"),    # recent rows 0..7 moved, 8..15 from the table
    ("tiny_g7", 300, 320, 0),         # group 7
    ("tiny_g7", 40, 64, 0),           # group 7, one tile
    ("tiny_g7", 100, 128, 0),         # group 7, two tiles
    ("tiny_g7", 150, 192, 37),        # group 7, three tiles, direct RoPE path
    ("tiny_g7", 250, 256, 0),         # group 7, four tiles
    ("tiny_g5", 1000, 1000, 0),       # group 5
    ("tiny_g5", 517, 600, 0),         # group 5, 5-key last tile
    ("tiny_g8", 300, 320, 0),         # group 8: eight wavefronts (512 threads)
    ("qwen3_4b_layer", None, None, 0),
]


@pytest.mark.parametrize("name,L,l_cap,t_shift", CASES)
def test_score_matches_oracle(name, L, l_cap, t_shift):
    w = _workload(name)
    log(f"score {name} L={L or w.L} l_cap={l_cap} t_shift={t_shift}")
    if t_shift == "partial":
        inp, sc, qobs, t = _run(w, L, l_cap, shift_first_recents=3)
    else:
        inp, sc, qobs, t = _run(w, L, l_cap, None if not t_shift else (L or w.L) + t_shift)
    L = L or w.L
    worst = 0.0
    flips = 0
    for u in range(w.n_units):
        beacons = inp["buf"][u][:, :16]
        taus = inp["kpos"][u][L - 16:L]
        ref, qhat, _, _ = oracle.score.score_unit(inp["keys"][u], beacons, inp["recents"][u],
                                                  t, taus, w.theta, return_all=True)
        worst = max(worst, check_scores(sc[u, :L], ref, f"{name} unit {u}"))
        if sc.shape[1] > L:
            assert np.all(sc[u, L:] == -1.0), "slots past L must be untouched"
        got_q = qobs[u].float().numpy().reshape(w.group, 32, w.d_head)
        neq = got_q != qhat
        flips += int(neq.sum())
        if neq.any():  # rounding-boundary flips only: one bf16 ulp
            ulp = np.abs(qhat[neq]) * 2.0 ** -7
            assert np.all(np.abs(got_q[neq] - qhat[neq]) <= ulp)
    assert flips <= 1e-4 * qobs.numel()
    log(f"  max rel err {worst:.3g}, bf16 rounding flips {flips}")


MEAN_CASES = [
    ("tiny", 203, 256),       # ragged tail, l_cap > L
    ("tiny", 40, 64),         # one tile, recent rows masked inside it
    ("tiny_g7", 300, 320),    # group 7: seven wavefronts, the 128-VGPR form
    ("tiny_g5", 1000, 1000),  # group 5
    ("tiny_g8", 203, 256),    # group 8
    ("qwen3_4b_layer", None, None),
]


@pytest.mark.parametrize("name,L,l_cap", MEAN_CASES)
def test_score_mean_pooling_matches_oracle(name, L, l_cap):
    w = _workload(name)
    log(f"score mean pooling {name} L={L or w.L} l_cap={l_cap}")
    inp, sc, _, t = _run(w, L, l_cap, aggregate="mean")
    L = L or w.L
    worst = 0.0
    for u in range(w.n_units):
        beacons = inp["buf"][u][:, :16]
        taus = inp["kpos"][u][L - 16:L]
        ref = oracle.score.score_unit(inp["keys"][u], beacons, inp["recents"][u], t, taus,
                                      w.theta, aggregate="mean")
        worst = max(worst, check_scores(sc[u, :L], ref, f"{name} mean unit {u}"))
        assert abs(sc[u, :L].astype(np.float64).sum() - 1.0) < 1e-4
        if sc.shape[1] > L:
            assert np.all(sc[u, L:] == -1.0), "slots past L must be untouched"
    log(f"  max rel err {worst:.3g}")


def _window(w):
    """The baselines' observation set: the 32 most recent queries, no beacons."""
    return synth.shrink(w, n_beacon=0, n_recent_q=32, recent_tok=32)


WINDOW_CASES = [
    ("tiny", None, None, 0),          # 4 tiles
    ("tiny", 203, 256, 0),            # ragged tail, l_cap > L
    ("tiny", 40, 64, 0),              # one tile: 32 recent rows masked inside it
    ("tiny", 517, 600, 0),            # 5-key last tile
    ("tiny", 300, 300, 37),           # positions != t-32+i: direct RoPE path, all rows
    ("tiny", 300, 300, "partial"),    # rows 0..7 moved
    ("tiny_g7", 300, 320, 0),         # group 7 (the 128-VGPR form)
    ("tiny_g7", 40, 64, 0),           # group 7, one tile
    ("tiny_g7", 150, 150, 0),         # group 7, three tiles
    ("tiny_g5", 1000, 1000, 0),       # group 5
    ("qwen3_4b_layer", None, None, 0),
]


@pytest.mark.parametrize("aggregate", ["max", "mean"])
@pytest.mark.parametrize("name,L,l_cap,t_shift", WINDOW_CASES)
def test_score_recent_window_matches_oracle(name, L, l_cap, t_shift, aggregate):
    w = _window(_workload(name))
    log(f"score 32-query window {name} L={L or w.L} l_cap={l_cap} t_shift={t_shift} "
        f"{aggregate}")
    if t_shift == "partial":
        inp, sc, qobs, t = _run(w, L, l_cap, shift_first_recents=3, aggregate=aggregate)
    else:
        inp, sc, qobs, t = _run(w, L, l_cap, None if not t_shift else (L or w.L) + t_shift,
                                aggregate=aggregate)
    L = L or w.L
    worst, flips = 0.0, 0
    for u in range(w.n_units):
        none = np.zeros((w.group, 0, w.d_head))
        taus = inp["kpos"][u][L - 32:L]
        ref, qhat, _, _ = oracle.score.score_unit(inp["keys"][u], none, inp["recents"][u], t,
                                                  taus, w.theta, return_all=True,
                                                  aggregate=aggregate)
        worst = max(worst, check_scores(sc[u, :L], ref, f"{name} unit {u}"))
        if sc.shape[1] > L:
            assert np.all(sc[u, L:] == -1.0), "slots past L must be untouched"
        got_q = qobs[u].float().numpy().reshape(w.group, 32, w.d_head)
        neq = got_q != qhat
        flips += int(neq.sum())
        if neq.any():
            ulp = np.abs(qhat[neq]) * 2.0 ** -7
            assert np.all(np.abs(got_q[neq] - qhat[neq]) <= ulp)
    assert flips <= 1e-4 * qobs.numel()
    log(f"  max rel err {worst:.3g}, bf16 rounding flips {flips}")


# Pass 1 sums exp2(logit * scale * log2 e) against a fixed reference; a
# workgroup with a row total outside [2^-60, 2^100] redoes pass 1 with a
# running maximum.  These cases put rows outside that range, so the scores
# come from the second path; they must still match the oracle.
RESCUE_SCALES = [
    (40.0, "logits up to several hundred: row totals overflow the fast range"),
    (6.0, "some rows above 2^100, most inside"),
]


@pytest.mark.parametrize("sm_scale,why", RESCUE_SCALES)
def test_score_large_logits_take_the_running_max_path(sm_scale, why):
    w = synth.WORKLOADS["tiny"]
    L = 300
    w2 = synth.shrink(w, L=L)
    inp = synth.workload_inputs(w2)
    dev = synth.to_device(inp, DEV)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, L, w.prefix, w.theta,
                      recent_tok=w.recent_tok, sm_scale=sm_scale)
    log(f"score with sm_scale {sm_scale}: {why}")
    score = torch.full((w.n_units, L), -1.0, device=DEV)
    bkv.score(shape, dev["keys"], dev["kpos"], L, dev["buf"], dev["recents"], L, score)
    torch.cuda.synchronize()
    sc = score.cpu().numpy()
    top = 0.0
    for u in range(w.n_units):
        taus = inp["kpos"][u][L - 16:L]
        ref, _, logits, _ = oracle.score.score_unit(inp["keys"][u], inp["buf"][u][:, :16],
                                                    inp["recents"][u], L, taus, w.theta,
                                                    scale=sm_scale, return_all=True)
        top = max(top, float(np.max(logits[:, :16])))  # beacon rows see every slot
        check_scores(sc[u], ref, f"sm_scale {sm_scale} unit {u}")
    # The case really leaves the fast range: some beacon row's log-sum-exp (at
    # least its largest logit) exceeds 100 log2 units.
    assert top * 1.4426950408889634 > 100, top
