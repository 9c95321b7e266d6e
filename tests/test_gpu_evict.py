"""Whole eviction step (bkv_fps_update + bkv_evict) against the oracle.

Small workloads are checked on every unit; the full-size Qwen3-4B step
(36 layers x batch 16 x 8 KV heads, the benchmark's launch configuration)
and the R1-Distill-Qwen-7B shape (group of 7) are checked on sampled units
plus properties that hold for every unit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check_fps, check_kept, check_scores, log
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(w, l_cap, aggregate="max"):
    return bkv.Shape(w.n_units, w.group, w.d_head, l_cap, w.prefix, w.theta,
                     recent_tok=w.recent_tok, aggregate=aggregate)


def _step(w, dev, l_cap, aggregate="max"):
    """The benchmark's step: Continual-FPS compress, then evict with merge."""
    shape = _shape(w, l_cap, aggregate)
    nq = w.n_qheads
    count = torch.full((nq,), 31, dtype=torch.int32, device=DEV)
    newq = dev["buf"][:, 31:32].contiguous()
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    buf0 = dev["buf"].clone()
    bkv.fps_update(shape, dev["buf"], count, newq, trigger=32, m=16, sel_order=sel)
    beacons_after_fps = dev["buf"][:, :16].clone()
    score = torch.zeros((w.n_units, l_cap), device=DEV)
    kept = torch.zeros((w.n_units, w.b_kv), dtype=torch.int32, device=DEV)
    K0, V0, P0 = dev["keys"].clone(), dev["values"].clone(), dev["kpos"].clone()
    bkv.evict(shape, dev["keys"], dev["values"], dev["kpos"], w.L, dev["buf"], dev["recents"],
              dev["t"], w.b_kv, buf=dev["buf"], count=count, score_out=score, kept_out=kept)
    torch.cuda.synchronize()
    return dict(buf0=buf0, sel=sel, beacons=beacons_after_fps, score=score, kept=kept,
                K0=K0, V0=V0, P0=P0, count=count)


def _check_unit(w, u, inp_u, res, where, aggregate="max"):
    L = w.L
    g = w.group
    qh = slice(u * g, (u + 1) * g)
    buf0 = res["buf0"][qh].cpu().numpy()
    sel = res["sel"][qh].cpu().numpy()
    for h in range(g):
        check_fps(buf0[h, :32], sel[h], 16, f"{where} fps head {h}")
    beacons = res["beacons"][qh].cpu().numpy()
    ref = oracle.evict.evict_unit(inp_u["keys"], inp_u["values"], inp_u["kpos"], L, beacons,
                                  inp_u["recents"], L, w.b_kv, w.prefix, w.recent_tok, w.theta,
                                  aggregate=aggregate)
    rel = check_scores(res["score"][u, :L].cpu().numpy(), ref["score"], where)
    kept = res["kept"][u].cpu().numpy()
    nd = check_kept(kept, ref["score"], L, w.b_kv, w.prefix, w.recent_tok, where)
    # Compaction is exact given the GPU's own kept set.
    K0 = res["K0"][u].view(torch.int16).cpu().numpy()
    got = res["K1"][u, :w.b_kv].view(torch.int16).cpu().numpy()
    assert np.array_equal(got, K0[kept]), f"{where}: K compaction"
    V0 = res["V0"][u].view(torch.int16).cpu().numpy()
    assert np.array_equal(res["V1"][u, :w.b_kv].view(torch.int16).cpu().numpy(), V0[kept])
    assert np.array_equal(res["P1"][u, :w.b_kv].cpu().numpy(), res["P0"][u].cpu().numpy()[kept])
    # Rolling update: merged buffer is a valid FPS pick of beacons + recents.
    merged = np.concatenate([beacons, inp_u["recents"]], axis=1)
    out = res["buf1"][qh, :16].cpu().numpy()
    for h in range(g):
        idx = [int(np.nonzero((merged[h] == row).all(axis=1))[0][0]) for row in out[h]]
        assert idx == sorted(idx) and len(set(idx)) == 16, f"{where}: merged rows"
        ref_order, _ = oracle.fps.fps(merged[h], 16)
        if min(oracle.fps.fps_margins(merged[h], 16)) > 2e-3:
            assert sorted(ref_order) == idx, f"{where}: merged FPS set"
    return rel, nd


@pytest.mark.parametrize("name", ["tiny", "qwen3_4b_layer"])
def test_evict_small_all_units(name):
    w = synth.WORKLOADS[name]
    log(f"evict {name}: U={w.n_units} L={w.L} B={w.b_kv}")
    inp = synth.workload_inputs(w)
    dev = synth.to_device(inp, DEV)
    res = _step(w, dev, w.L)
    res.update(K1=dev["keys"], V1=dev["values"], P1=dev["kpos"], buf1=dev["buf"])
    assert torch.all(res["count"] == 16)
    worst, ndiff = 0.0, 0
    for u in range(w.n_units):
        unit = {k: inp[k][u] for k in ("keys", "values", "kpos", "recents")}
        rel, nd = _check_unit(w, u, unit, res, f"{name} unit {u}")
        worst, ndiff = max(worst, rel), ndiff + nd
    log(f"  max score rel err {worst:.3g}; kept-set tie-band differences {ndiff}")


@pytest.mark.parametrize("name,samples", [
    ("tiny", None),
    ("qwen3_4b_layer", None),
    ("r1_qwen_7b", [0, 1791, 3583]),   # group 7: the score kernel's 128-VGPR form
])
def test_evict_mean_pooling(name, samples):
    """The mean-aggregation ablation through the whole step."""
    w = synth.WORKLOADS[name]
    log(f"evict mean pooling {name}: U={w.n_units} g={w.group} L={w.L} B={w.b_kv}")
    if samples is None:
        inp = synth.workload_inputs(w)
        dev = synth.to_device(inp, DEV)
        samples = list(range(w.n_units))
        host = {u: {k: inp[k][u] for k in ("keys", "values", "kpos", "recents")}
                for u in samples}
    else:
        dev = synth.device_inputs(w, DEV)
        host = {u: {"keys": dev["keys"][u].float().cpu().numpy(),
                    "values": dev["values"][u].float().cpu().numpy(),
                    "kpos": dev["kpos"][u].cpu().numpy(),
                    "recents": dev["recents"][u * w.group:(u + 1) * w.group].cpu().numpy()}
                for u in samples}
    res = _step(w, dev, w.L, aggregate="mean")
    res.update(K1=dev["keys"], V1=dev["values"], P1=dev["kpos"], buf1=dev["buf"])
    # Every unit: the average of softmax rows sums to 1 over the slots.
    tot = res["score"][:, :w.L].double().sum(dim=1)
    assert torch.all((tot - 1).abs() < 1e-3), float((tot - 1).abs().max())
    worst, ndiff = 0.0, 0
    for u in samples:
        rel, nd = _check_unit(w, u, host[u], res, f"{name} mean unit {u}", aggregate="mean")
        worst, ndiff = max(worst, rel), ndiff + nd
    log(f"  max score rel err {worst:.3g}; kept-set tie-band differences {ndiff}")


@pytest.mark.parametrize("name,samples", [
    ("tiny", None),
    ("qwen3_4b_layer", None),
    ("r1_qwen_7b", [0, 1791, 3583]),
])
def test_evict_recent_window(name, samples):
    """The baselines' observation set (32 most recent queries, no beacons, the
    last 32 tokens kept): score, select and compact, no rolling update."""
    w = synth.shrink(synth.WORKLOADS[name], n_beacon=0, n_recent_q=32, recent_tok=32)
    log(f"evict 32-query window {name}: U={w.n_units} g={w.group} L={w.L} B={w.b_kv}")
    if samples is None:
        inp = synth.workload_inputs(w)
        dev = synth.to_device(inp, DEV)
        samples = list(range(w.n_units))
        host = {u: {k: inp[k][u] for k in ("keys", "values", "kpos", "recents")}
                for u in samples}
    else:
        dev = synth.device_inputs(w, DEV)
        host = {u: {"keys": dev["keys"][u].float().cpu().numpy(),
                    "values": dev["values"][u].float().cpu().numpy(),
                    "kpos": dev["kpos"][u].cpu().numpy(),
                    "recents": dev["recents"][u * w.group:(u + 1) * w.group].cpu().numpy()}
                for u in samples}
    shape = bkv.Shape(w.n_units, w.group, w.d_head, w.L, w.prefix, w.theta, recent_tok=32,
                      n_beacon=0, n_recent_q=32)
    score = torch.zeros((w.n_units, w.L), device=DEV)
    kept = torch.zeros((w.n_units, w.b_kv), dtype=torch.int32, device=DEV)
    K0, V0, P0 = dev["keys"].clone(), dev["values"].clone(), dev["kpos"].clone()
    bkv.evict(shape, dev["keys"], dev["values"], dev["kpos"], w.L, None, dev["recents"],
              dev["t"], w.b_kv, score_out=score, kept_out=kept)
    torch.cuda.synchronize()
    _all_unit_properties(w, kept)
    worst, ndiff = 0.0, 0
    for u in samples:
        hu = host[u]
        ref = oracle.evict.evict_unit(hu["keys"], hu["values"], hu["kpos"], w.L,
                                      np.zeros((w.group, 0, w.d_head)), hu["recents"], w.L,
                                      w.b_kv, w.prefix, 32, w.theta, merge=False)
        worst = max(worst, check_scores(score[u].cpu().numpy(), ref["score"], f"{name} {u}"))
        ku = kept[u].cpu().numpy()
        ndiff += check_kept(ku, ref["score"], w.L, w.b_kv, w.prefix, 32, f"{name} {u}")
        k16 = K0[u].view(torch.int16).cpu().numpy()
        assert np.array_equal(dev["keys"][u, :w.b_kv].view(torch.int16).cpu().numpy(), k16[ku])
        v16 = V0[u].view(torch.int16).cpu().numpy()
        assert np.array_equal(dev["values"][u, :w.b_kv].view(torch.int16).cpu().numpy(), v16[ku])
        assert np.array_equal(dev["kpos"][u, :w.b_kv].cpu().numpy(), P0[u].cpu().numpy()[ku])
    log(f"  max score rel err {worst:.3g}; kept-set tie-band differences {ndiff}")


@pytest.mark.parametrize("name,samples", [
    ("tiny", None),
    ("qwen3_4b_layer", None),
    ("qwen3_4b_full_b2048", [0, 2303, 4607]),
])
def test_evict_unsorted_compaction(name, samples):
    """bkv_evict with BKV_FLAG_UNSORTED: scores, kept set and merge as usual;
    the cache holds the kept tokens with the tail ones in the evicted slots."""
    w = synth.WORKLOADS[name]
    log(f"evict unsorted {name}: U={w.n_units} g={w.group} L={w.L} B={w.b_kv}")
    if samples is None:
        inp = synth.workload_inputs(w)
        dev = synth.to_device(inp, DEV)
        samples = list(range(w.n_units))
        host = {u: {k: inp[k][u] for k in ("keys", "values", "kpos", "recents")}
                for u in samples}
    else:
        dev = synth.device_inputs(w, DEV)
        host = {u: {"keys": dev["keys"][u].float().cpu().numpy(),
                    "values": dev["values"][u].float().cpu().numpy(),
                    "kpos": dev["kpos"][u].cpu().numpy(),
                    "recents": dev["recents"][u * w.group:(u + 1) * w.group].cpu().numpy()}
                for u in samples}
    shape = bkv.Shape(w.n_units, w.group, w.d_head, w.L, w.prefix, w.theta,
                      recent_tok=w.recent_tok, unsorted=True)
    nq = w.n_qheads
    count = torch.full((nq,), 31, dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, dev["buf"], count, dev["buf"][:, 31:32].contiguous(), trigger=32, m=16)
    beacons = dev["buf"][:, :16].clone()
    score = torch.zeros((w.n_units, w.L), device=DEV)
    kept = torch.zeros((w.n_units, w.b_kv), dtype=torch.int32, device=DEV)
    K0, V0, P0 = dev["keys"].clone(), dev["values"].clone(), dev["kpos"].clone()
    bkv.evict(shape, dev["keys"], dev["values"], dev["kpos"], w.L, dev["buf"], dev["recents"],
              dev["t"], w.b_kv, buf=dev["buf"], count=count, score_out=score, kept_out=kept)
    torch.cuda.synchronize()
    _all_unit_properties(w, kept)
    # Every unit: the positions in [0, b_kv) are exactly the kept tokens' positions.
    got_pos = torch.sort(dev["kpos"][:, :w.b_kv], dim=1).values
    want_pos = torch.gather(P0, 1, kept.long())
    assert torch.equal(got_pos, want_pos)
    worst = 0.0
    for u in samples:
        hu = host[u]
        g = w.group
        ref = oracle.evict.evict_unit(hu["keys"], hu["values"], hu["kpos"], w.L,
                                      beacons[u * g:(u + 1) * g].cpu().numpy(), hu["recents"],
                                      w.L, w.b_kv, w.prefix, w.recent_tok, w.theta, merge=False)
        worst = max(worst, check_scores(score[u].cpu().numpy(), ref["score"], f"{name} {u}"))
        ku = kept[u].cpu().numpy()
        check_kept(ku, ref["score"], w.L, w.b_kv, w.prefix, w.recent_tok, f"{name} {u}")
        ek, ev, ep, _ = oracle.compact.fill_holes(K0[u].view(torch.int16).cpu().numpy(),
                                                  V0[u].view(torch.int16).cpu().numpy(),
                                                  P0[u].cpu().numpy(), ku, w.b_kv)
        assert np.array_equal(dev["keys"][u, :w.b_kv].view(torch.int16).cpu().numpy(), ek)
        assert np.array_equal(dev["values"][u, :w.b_kv].view(torch.int16).cpu().numpy(), ev)
        assert np.array_equal(dev["kpos"][u, :w.b_kv].cpu().numpy(), ep)
    assert torch.all(count == 16)
    log(f"  max score rel err {worst:.3g}")


def _all_unit_properties(w, kept):
    P, R, L = w.prefix, w.recent_tok, w.L
    assert torch.all(kept[:, 1:] > kept[:, :-1])
    if P:
        assert torch.equal(kept[:, :P], torch.arange(P, device=DEV, dtype=torch.int32).expand(
            w.n_units, -1))
    assert torch.equal(kept[:, -R:], torch.arange(L - R, L, device=DEV,
                                                  dtype=torch.int32).expand(w.n_units, -1))


@pytest.mark.parametrize("name,samples", [
    ("qwen3_4b_full_b2048", [0, 1, 777, 2303, 4095, 4607]),
    ("qwen3_4b_full_b128", [0, 2304, 4607]),    # L = 256: a unit of four key tiles
    ("qwen3_4b_full_b512", [0, 1500, 4607]),    # L = 640: the 16-register select
    ("qwen3_4b_full_b1024", [0, 3100, 4607]),   # L = 1152: the 36-register select
    ("qwen3_4b_full_b4096", [0, 3001, 4607]),   # L = 4224
    ("r1_qwen_7b", [0, 1791, 3583]),
])
def test_evict_full_size_sampled(name, samples):
    w = synth.WORKLOADS[name]
    log(f"evict full size {name}: U={w.n_units} g={w.group} L={w.L} B={w.b_kv}")
    dev = synth.device_inputs(w, DEV)
    host = {u: {"keys": dev["keys"][u].float().cpu().numpy(),
                "values": dev["values"][u].float().cpu().numpy(),
                "kpos": dev["kpos"][u].cpu().numpy(),
                "recents": dev["recents"][u * w.group:(u + 1) * w.group].cpu().numpy()}
            for u in samples}
    res = _step(w, dev, w.L)
    res.update(K1=dev["keys"], V1=dev["values"], P1=dev["kpos"], buf1=dev["buf"])
    assert torch.all(res["count"] == 16)
    _all_unit_properties(w, res["kept"])
    sc = res["score"][:, :w.L]
    assert torch.all(sc > 0) and torch.all(sc <= 1)
    assert torch.all(sc.sum(dim=1) >= 1 - 1e-3)
    worst = 0.0
    for u in samples:
        rel, _ = _check_unit(w, u, host[u], res, f"{name} unit {u}")
        worst = max(worst, rel)
    log(f"  sampled max score rel err {worst:.3g}")


def test_in_place_equals_out_of_place_full_size():
    w = synth.WORKLOADS["qwen3_4b_full_b2048"]
    log("compact race check: in place vs out of place, full size")
    dev = synth.device_inputs(w, DEV)
    shape = _shape(w, w.L)
    score = torch.zeros((w.n_units, w.L), device=DEV)
    kept = torch.zeros((w.n_units, w.b_kv), dtype=torch.int32, device=DEV)
    bkv.score(shape, dev["keys"], dev["kpos"], w.L, dev["buf"], dev["recents"], w.L, score)
    bkv.select(shape, score, w.L, w.b_kv, kept)
    Ko = torch.empty((w.n_units, w.b_kv, w.d_head), dtype=torch.bfloat16, device=DEV)
    Vo, Po = torch.empty_like(Ko), torch.empty((w.n_units, w.b_kv), dtype=torch.int32,
                                                device=DEV)
    bkv.compact(shape, dev["keys"], dev["values"], dev["kpos"], w.L, kept, w.b_kv, Ko, Vo, Po,
                out_cap=w.b_kv)
    bkv.compact(shape, dev["keys"], dev["values"], dev["kpos"], w.L, kept, w.b_kv)
    torch.cuda.synchronize()
    assert torch.equal(dev["keys"][:, :w.b_kv].view(torch.int16), Ko.view(torch.int16))
    assert torch.equal(dev["values"][:, :w.b_kv].view(torch.int16), Vo.view(torch.int16))
    assert torch.equal(dev["kpos"][:, :w.b_kv], Po)
