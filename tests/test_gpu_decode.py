"""Decode attention with beacon denominators (bkv_decode_attend) and scoring
from known denominators (bkv_score_lse) against the float64 oracle.

The decode kernel streams keys and values in tiles of 32 through rings of
three LDS tiles; the cases cover one slot, a single partial tile, ragged
tails with l_cap > L, several ring turns, groups of 1, 2, 3, 4, 5, 7 and 8
and both head sizes, a long cache, and the 128-register form that groups
larger than four use.  The scoring cases place lse_from so that the tail pass covers one
tile (the prologue then loads the first tile the backward walk needs beyond
it, and the walk visits the buffers in the reflected order), two tiles,
every tile (lse_from = 0) and no slot at all (lse_from = L); the 32-query
window and the full-size path are covered too.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import TOL, check_kept, check_scores, log
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workload(name):
    if name == "tiny_g7":
        return synth.shrink(synth.WORKLOADS["tiny"], group=7, d_head=128, theta=1e6)
    if name == "tiny_g5":
        return synth.shrink(synth.WORKLOADS["tiny"], group=5, d_head=128, theta=1e6, h_kv=3)
    if name == "tiny_g1":
        return synth.shrink(synth.WORKLOADS["tiny"], group=1)
    if name == "tiny_g3":
        return synth.shrink(synth.WORKLOADS["tiny"], group=3, d_head=128, theta=1e6)
    if name == "tiny_g8":
        return synth.shrink(synth.WORKLOADS["tiny"], group=8, d_head=64)
    if name == "tiny_g8_128":
        return synth.shrink(synth.WORKLOADS["tiny"], group=8, d_head=128, theta=1e6)
    if name == "long_g4":
        return synth.shrink(synth.WORKLOADS["tiny"], group=4, d_head=128, theta=1e6, h_kv=1)
    return synth.WORKLOADS[name]


def _setup(w, L, l_cap):
    w2 = synth.shrink(w, L=L)
    inp = synth.workload_inputs(w2)
    dev = synth.to_device(inp, DEV, l_cap=l_cap)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, l_cap, w.prefix, w.theta,
                      recent_tok=w.recent_tok)
    return inp, dev, shape


def _decode(shape, dev, L, q, t_q, beacons=None, t_obs=0):
    nq, d = shape.n_units * shape.group, shape.d_head
    out = torch.full((nq, d), float("nan"), device=DEV)
    lse_q = torch.full((nq,), float("nan"), device=DEV)
    lse_obs = torch.full((nq, 16), float("nan"), device=DEV) if beacons is not None else None
    bkv.decode_attend(shape, dev["keys"], dev["values"], L, q, t_q, out, lse_q, beacons, t_obs,
                      lse_obs)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse_q.cpu().numpy(), (None if lse_obs is None else
                                                     lse_obs.cpu().numpy())


DECODE_CASES = [
    ("tiny", 256, 256),           # d 64, g 2: 8 tiles of 32, ring turns
    ("tiny", 1, 64),              # one slot
    ("tiny", 20, 64),             # one partial tile
    ("tiny", 33, 64),             # one key in the second tile
    ("tiny", 203, 256),           # ragged tail, l_cap > L
    ("tiny_g1", 150, 160),        # one head per group (one loader wavefront)
    ("tiny_g3", 97, 128),         # three wavefronts, two of them loaders
    ("tiny_g8", 129, 160),        # eight wavefronts (512 threads), d 64
    ("tiny_g8_128", 257, 288),    # eight wavefronts, d 128: the 128-VGPR form
    ("tiny_g7", 300, 320),        # group 7, d 128
    ("tiny_g5", 1000, 1000),      # group 5
    ("qwen3_4b_layer", 2176, 2176),
    ("long_g4", 9000, 9001),      # a long cache: 282 tiles of 32 keys
]


@pytest.mark.parametrize("with_beacons", [True, False])
@pytest.mark.parametrize("name,L,l_cap", DECODE_CASES)
def test_decode_attend_matches_oracle(name, L, l_cap, with_beacons):
    w = _workload(name)
    log(f"decode {name} L={L} l_cap={l_cap} beacons={with_beacons}")
    inp, dev, shape = _setup(w, max(L, 16), l_cap)
    _check_decode(w, inp, dev, shape, L, with_beacons)


@pytest.mark.parametrize("name,L", [("tiny_g7", 300), ("tiny", 203), ("qwen3_4b_layer", 700)])
def test_decode_late_logit_jump(name, L):
    """Key j and its negation, both scaled by 64 (exact in bf16), in a late
    tile: for most rows one of them has a logit far above all earlier ones
    (measured in float64 on these inputs: the new query's jumps past its lazy
    threshold of 8 log2 units for 86-100% of the heads, the beacon rows' past
    64 for 46-82% of the rows), so after many tiles both rescale paths run;
    the output and every log-sum-exp still match the oracle."""
    w = _workload(name)
    log(f"decode late jump {name} L={L}")
    inp, dev, shape = _setup(w, L, L)
    j = L - 40
    inp["keys"][:, j] *= 64.0
    inp["keys"][:, j + 1] = -inp["keys"][:, j]
    dev["keys"][:, j] *= 64.0
    dev["keys"][:, j + 1] = -dev["keys"][:, j]
    _check_decode(w, inp, dev, shape, L, True)


def _check_decode(w, inp, dev, shape, L, with_beacons):
    g, d = w.group, w.d_head
    # The step's query: buffer row 20 of each head, at the newest slot's position.
    q_host = inp["buf"][:, :, 20]                           # [U, g, d]
    q = torch.from_numpy(np.ascontiguousarray(q_host.reshape(-1, d))).to(DEV)
    t_q = int(inp["kpos"][0, L - 1])
    t_obs = L + 16
    beacons = dev["buf"] if with_beacons else None
    out, lse_q, lse_obs = _decode(shape, dev, L, q, t_q, beacons, t_obs)
    worst_o, worst_l = 0.0, 0.0
    for u in range(w.n_units):
        keys, vals = inp["keys"][u][:L], inp["values"][u][:L]
        ref_o, ref_l = oracle.decode.decode_attention(keys, vals, q_host[u], t_q, w.theta)
        # |out error| <= TOL * sum_j W_j |V_j|: the bound a relative error TOL
        # in every softmax weight gives.
        qhat = oracle.decode.rotated_queries(q_host[u], t_q, w.theta)
        s = qhat @ np.asarray(keys, np.float64).T / np.sqrt(d)
        wts = np.exp(s - ref_l[:, None])
        bound = TOL * (wts @ np.abs(np.asarray(vals, np.float64))) + 1e-6
        err = np.abs(out[u * g:(u + 1) * g] - ref_o)
        assert np.all(err <= bound), f"unit {u}: output error {err.max():.3g}"
        worst_o = max(worst_o, float((err / bound).max()))
        dl = np.abs(lse_q[u * g:(u + 1) * g] - ref_l)
        assert np.all(dl <= TOL), f"unit {u}: lse_q error {dl.max():.3g}"
        worst_l = max(worst_l, float(dl.max()))
        if with_beacons:
            ref_b = oracle.decode.beacon_lse(keys, inp["buf"][u][:, :16], t_obs, w.theta)
            db = np.abs(lse_obs[u * g:(u + 1) * g] - ref_b)
            assert np.all(db <= TOL), f"unit {u}: lse_obs error {db.max():.3g}"
            worst_l = max(worst_l, float(db.max()))
    log(f"  output err / bound {worst_o:.3g}, max lse abs err {worst_l:.3g}")


def _lse_from_decode(shape, dev, inp, L, lse_from, t):
    """The denominators as decoding gathers them, all on the GPU: the beacons'
    from the step whose cache held lse_from slots, recent query i's from its
    own step (cache of L - 16 + i + 1 slots)."""
    U, g, d = shape.n_units, shape.group, shape.d_head
    lse = torch.empty((U, g, 32), device=DEV)
    if lse_from > 0:
        q = dev["recents"][:, 0].contiguous()
        _, _, lo = _decode(shape, dev, lse_from, q, int(inp["kpos"][0, lse_from - 1]),
                           dev["buf"], t)
        lse[:, :, :16] = torch.from_numpy(lo.reshape(U, g, 16)).to(DEV)
    else:
        lse[:, :, :16] = -float("inf")
    for i in range(16):
        q = dev["recents"][:, i].contiguous()
        _, lq, _ = _decode(shape, dev, L - 16 + i + 1, q, int(inp["kpos"][0, L - 16 + i]))
        lse[:, :, 16 + i] = torch.from_numpy(lq.reshape(U, g)).to(DEV)
    return lse.contiguous()


SCORE_CASES = [
    ("tiny", 256, 256, 240, "max"),        # tail pass: last tile only
    ("tiny", 203, 256, 187, "max"),        # tail pass: last two tiles
    ("tiny", 256, 256, 0, "max"),          # every tile (nothing known for the beacons)
    ("tiny", 256, 256, 256, "max"),        # no slot added
    ("tiny", 40, 64, 24, "max"),           # one tile in all
    ("tiny", 100, 128, 84, "max"),         # two tiles: pass 1 on one, the other from the prologue
    ("tiny", 150, 192, 100, "max"),        # three tiles, pass 1 on two: the third at pass 2's start
    ("tiny", 517, 600, 501, "max"),        # 5-key last tile
    ("tiny", 256, 256, 240, "mean"),
    ("tiny_g7", 300, 320, 284, "max"),     # group 7 (the 128-VGPR form)
    ("tiny_g5", 1000, 1000, 984, "max"),
    ("tiny_g7", 256, 256, 0, "max"),       # group 7: every tile in the tail pass
    ("tiny_g7", 256, 256, 256, "max"),     # group 7: no slot added
    ("tiny_g7", 150, 192, 100, "max"),     # group 7: three tiles, pass 1 on two
    ("tiny_g7", 40, 64, 24, "max"),        # group 7: one tile in all
    ("tiny_g5", 517, 600, 501, "mean"),    # group 5: 5-key last tile, mean pooling
    ("tiny_g8", 300, 300, 284, "mean"),    # group of eight (d 64), mean pooling
    ("tiny_g8_128", 300, 320, 284, "max"), # group of eight, d 128
    ("tiny_g3", 129, 160, 113, "max"),     # three heads, a 1-key last tile
    ("qwen3_4b_layer", 2176, 2176, 2160, "max"),
]


@pytest.mark.parametrize("name,L,l_cap,lse_from,aggregate", SCORE_CASES)
def test_score_lse_matches_oracle(name, L, l_cap, lse_from, aggregate):
    w = _workload(name)
    log(f"score_lse {name} L={L} l_cap={l_cap} lse_from={lse_from} {aggregate}")
    inp, dev, shape = _setup(w, L, l_cap)
    shape.aggregate = aggregate
    t = L
    lse = _lse_from_decode(shape, dev, inp, L, lse_from, t)
    score = torch.full((w.n_units, l_cap), -1.0, device=DEV)
    bkv.score_lse(shape, dev["keys"], dev["kpos"], L, dev["buf"], dev["recents"], t, lse,
                  lse_from, score)
    torch.cuda.synchronize()
    sc = score.cpu().numpy()
    worst, n_diff = 0.0, 0
    B = min(w.b_kv, L - 1)
    for u in range(w.n_units):
        beacons = inp["buf"][u][:, :16]
        taus = inp["kpos"][u][L - 16:L]
        ref = oracle.score.score_unit(inp["keys"][u], beacons, inp["recents"][u], t, taus,
                                      w.theta, aggregate=aggregate)
        worst = max(worst, check_scores(sc[u, :L], ref, f"{name} unit {u}"))
        if l_cap > L:
            assert np.all(sc[u, L:] == -1.0), "slots past L must be untouched"
        if aggregate == "max" and B > w.prefix + w.recent_tok:
            kept = oracle.select.select(sc[u, :L].astype(np.float64), L, B, w.prefix,
                                        w.recent_tok)
            n_diff += check_kept(kept, ref, L, B, w.prefix, w.recent_tok, f"unit {u}")
    log(f"  max rel err {worst:.3g}, kept-set differences in the tie band {n_diff}")


def test_score_lse_agrees_with_two_pass_kernel():
    # Same unit, same kernel family: one read with known denominators vs the
    # two-pass call; both within the tolerance of each other.
    w = synth.WORKLOADS["qwen3_4b_layer"]
    inp, dev, shape = _setup(w, w.L, w.L)
    lse = _lse_from_decode(shape, dev, inp, w.L, w.L - 16, w.L)
    s1 = torch.empty((w.n_units, w.L), device=DEV)
    s2 = torch.empty((w.n_units, w.L), device=DEV)
    bkv.score(shape, dev["keys"], dev["kpos"], w.L, dev["buf"], dev["recents"], w.L, s1)
    bkv.score_lse(shape, dev["keys"], dev["kpos"], w.L, dev["buf"], dev["recents"], w.L, lse,
                  w.L - 16, s2)
    torch.cuda.synchronize()
    a, b = s1.cpu().numpy().astype(np.float64), s2.cpu().numpy().astype(np.float64)
    rel = np.abs(a - b) / b
    log(f"score_lse vs score: max rel diff {rel.max():.3g}")
    assert rel.max() <= 2 * TOL


def test_fused_path_full_size_sampled():
    """Qwen3-4B shape, all 4608 units, in the launch configuration the bench
    times: beacon denominators from decode attention at L - 16, the recent
    rows' from their own steps, then bkv_score_lse.  Sampled units against the
    oracle; every unit against the two-pass kernel within twice the tolerance."""
    w = synth.WORKLOADS["qwen3_4b_full_b2048"]
    U, g, d, L = w.n_units, w.group, w.d_head, w.L
    log(f"fused path full size: U={U} g={g} L={L}")
    dev = synth.device_inputs(w, DEV)
    shape = bkv.Shape(U, g, d, L, w.prefix, w.theta, recent_tok=w.recent_tok)
    K, V, P = dev["keys"], dev["values"], dev["kpos"]
    lse = torch.empty((U, g, 32), device=DEV)
    out = torch.empty((U * g, d), device=DEV)
    lq = torch.empty((U * g,), device=DEV)
    lo = torch.empty((U * g, 16), device=DEV)
    bkv.decode_attend(shape, K, V, L - 16, dev["buf"][:, 30].contiguous(), int(P[0, L - 17]),
                      out, lq, dev["buf"], L, lo)
    lse[:, :, :16] = lo.view(U, g, 16)
    for i in range(16):
        bkv.decode_attend(shape, K, V, L - 16 + i + 1, dev["recents"][:, i].contiguous(),
                          int(P[0, L - 16 + i]), out, lq)
        lse[:, :, 16 + i] = lq.view(U, g)
    s1 = torch.empty((U, L), device=DEV)
    s2 = torch.empty((U, L), device=DEV)
    bkv.score_lse(shape, K, P, L, dev["buf"], dev["recents"], L, lse, L - 16, s1)
    bkv.score(shape, K, P, L, dev["buf"], dev["recents"], L, s2)
    torch.cuda.synchronize()
    rel = ((s1 - s2).abs() / s2).max().item()
    assert rel <= 2 * TOL, rel
    worst = 0.0
    for u in (0, 1777, U - 1):
        ref = oracle.score.score_unit(K[u].float().cpu().numpy(),
                                      dev["buf"][u * g:(u + 1) * g, :16].cpu().numpy(),
                                      dev["recents"][u * g:(u + 1) * g].cpu().numpy(), L,
                                      P[u, L - 16:L].cpu().numpy(), w.theta)
        worst = max(worst, check_scores(s1[u].cpu().numpy(), ref, f"unit {u}"))
    log(f"  one-read vs two-pass max rel diff {rel:.3g}; sampled max rel err {worst:.3g}")


@pytest.mark.parametrize("name", ["r1_qwen_7b", "qwen3_4b_full_b2048"])
def test_decode_full_size_sampled(name):
    """Decode attention with the beacon rows at the beacon fix (L - 16
    slots) over every unit of the full workload, in the launch configuration
    the bench times (R1-Distill-Qwen-7B: groups of seven, the 128-VGPR form);
    sampled units against the oracle."""
    w = synth.WORKLOADS[name]
    U, g, d, L = w.n_units, w.group, w.d_head, w.L
    Lf = L - 16
    log(f"decode full size {name}: U={U} g={g} L={Lf}")
    dev = synth.device_inputs(w, DEV)
    shape = bkv.Shape(U, g, d, L, w.prefix, w.theta, recent_tok=w.recent_tok)
    K, V, P = dev["keys"], dev["values"], dev["kpos"]
    q = dev["buf"][:, 30].contiguous()
    t_q = int(P[0, Lf - 1])
    out = torch.empty((U * g, d), device=DEV)
    lq = torch.empty((U * g,), device=DEV)
    lo = torch.empty((U * g, 16), device=DEV)
    bkv.decode_attend(shape, K, V, Lf, q, t_q, out, lq, dev["buf"], L, lo)
    torch.cuda.synchronize()
    worst_o, worst_l = 0.0, 0.0
    for u in (0, U // 2 + 7, U - 1):
        keys = K[u, :Lf].float().cpu().numpy()
        vals = V[u, :Lf].float().cpu().numpy()
        qu = q[u * g:(u + 1) * g].cpu().numpy()
        ref_o, ref_l = oracle.decode.decode_attention(keys, vals, qu, t_q, w.theta)
        qhat = oracle.decode.rotated_queries(qu, t_q, w.theta)
        s = qhat @ np.asarray(keys, np.float64).T / np.sqrt(d)
        bound = TOL * (np.exp(s - ref_l[:, None]) @ np.abs(np.asarray(vals, np.float64))) + 1e-6
        err = np.abs(out[u * g:(u + 1) * g].cpu().numpy() - ref_o)
        assert np.all(err <= bound), f"unit {u}: output error {err.max():.3g}"
        worst_o = max(worst_o, float((err / bound).max()))
        dl = np.abs(lq[u * g:(u + 1) * g].cpu().numpy() - ref_l)
        ref_b = oracle.decode.beacon_lse(keys, dev["buf"][u * g:(u + 1) * g, :16].cpu().numpy(),
                                         L, w.theta)
        db = np.abs(lo[u * g:(u + 1) * g].cpu().numpy() - ref_b)
        assert dl.max() <= TOL and db.max() <= TOL, f"unit {u}: lse errors {dl.max():.3g} {db.max():.3g}"
        worst_l = max(worst_l, float(dl.max()), float(db.max()))
    log(f"  output err / bound {worst_o:.3g}, max lse abs err {worst_l:.3g}")


@pytest.mark.parametrize("L,l_cap", [(256, 256), (203, 256)])
def test_score_lse_recent_window(L, l_cap):
    """The baselines' window of 32 recent queries (no beacons): every row's
    denominator comes from that query's own decode step, and the one-read
    scores equal the oracle's two-pass definition."""
    w = synth.shrink(synth.WORKLOADS["tiny"], n_beacon=0, n_recent_q=32, recent_tok=32)
    log(f"score_lse 32-query window L={L} l_cap={l_cap}")
    inp, dev, _ = _setup(w, L, l_cap)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, l_cap, w.prefix, w.theta, recent_tok=32,
                      n_beacon=0, n_recent_q=32)
    U, g = w.n_units, w.group
    lse = torch.empty((U, g, 32), device=DEV)
    for i in range(32):
        q = dev["recents"][:, i].contiguous()
        _, lq, _ = _decode(shape, dev, L - 32 + i + 1, q, int(inp["kpos"][0, L - 32 + i]))
        lse[:, :, i] = torch.from_numpy(lq.reshape(U, g)).to(DEV)
    score = torch.full((U, l_cap), -1.0, device=DEV)
    bkv.score_lse(shape, dev["keys"], dev["kpos"], L, None, dev["recents"], L, lse, L, score)
    torch.cuda.synchronize()
    sc = score.cpu().numpy()
    worst = 0.0
    for u in range(U):
        none = np.zeros((g, 0, w.d_head))
        ref = oracle.score.score_unit(inp["keys"][u], none, inp["recents"][u], L,
                                      inp["kpos"][u][L - 32:L], w.theta)
        worst = max(worst, check_scores(sc[u, :L], ref, f"unit {u}"))
        if l_cap > L:
            assert np.all(sc[u, L:] == -1.0)
    log(f"  max rel err {worst:.3g}")


# Known denominators outside the fast pass-1 range: a beacon row starting at
# 150 (its total overflows 2^100) or, with no slot added, at -50 (its total
# falls below 2^-60).  The workgroup then redoes pass 1 with a running
# maximum; the scores must still follow the given denominators.
@pytest.mark.parametrize("lse_from,special", [(240, 150.0), (256, -50.0)])
def test_score_lse_out_of_range_denominators(lse_from, special):
    w = _workload("tiny")
    L = 256
    log(f"score_lse with a beacon denominator of {special}, lse_from={lse_from}")
    inp, dev, shape = _setup(w, L, L)
    r = np.random.default_rng(5)
    lse_np = r.uniform(-5.0, 5.0, size=(w.n_units, w.group, 32)).astype(np.float32)
    lse_np[0, 0, 3] = special
    lse = torch.from_numpy(lse_np).to(DEV)
    score = torch.full((w.n_units, L), -1.0, device=DEV)
    bkv.score_lse(shape, dev["keys"], dev["kpos"], L, dev["buf"], dev["recents"], L, lse,
                  lse_from, score)
    torch.cuda.synchronize()
    sc = score.cpu().numpy()
    for u in range(w.n_units):
        taus = inp["kpos"][u][L - 16:L]
        ref = oracle.decode.score_from_lse(inp["keys"][u], inp["buf"][u][:, :16],
                                           inp["recents"][u], L, taus, w.theta,
                                           lse_np[u].astype(np.float64), lse_from)
        check_scores(sc[u], ref, f"unit {u}")
