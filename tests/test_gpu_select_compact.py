"""Selection and compaction kernels against the oracle (bit-exact).

Selection runs on one wavefront per unit up to L = 8192 and on a workgroup
per unit beyond; both are covered.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import log
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("L,b_kv,P,R,kind", [
    (256, 128, 8, 16, "cont"),
    (2176, 2048, 256, 16, "cont"),
    (1000, 24, 8, 16, "cont"),      # nothing chosen: only forced slots
    (1000, 999, 0, 16, "ties"),     # evict exactly one
    (777, 300, 33, 16, "ties"),     # many equal scores around the cut
    (4224, 4096, 512, 16, "ties"),
    (300, 150, 0, 0, "zeros"),      # all-equal scores, no forced slots
    (8192, 8000, 8, 16, "cont"),    # largest unit of the one-wavefront kernel
    (8193, 7000, 8, 16, "ties"),    # beyond it: the workgroup kernel
    (9001, 5000, 8, 16, "cont"),
])
def test_select_bit_exact(L, b_kv, P, R, kind):
    U = 37
    log(f"select L={L} b_kv={b_kv} P={P} R={R} {kind}")
    r = np.random.default_rng(L + b_kv)
    if kind == "cont":
        s = r.random((U, L)).astype(np.float32) * 1e-3
    elif kind == "ties":
        s = r.choice(np.array([1e-6, 2e-6, 2e-6, 5e-4, 0.25, 0.0], np.float32), size=(U, L))
    else:
        s = np.zeros((U, L), np.float32)
    l_cap = L + 5
    sc = torch.zeros((U, l_cap), dtype=torch.float32, device=DEV)
    sc[:, :L] = torch.from_numpy(s).to(DEV)
    kept = torch.full((U, b_kv), -1, dtype=torch.int32, device=DEV)
    shape = bkv.Shape(U, 1, 64, l_cap, P, 1e4, recent_tok=R)
    bkv.select(shape, sc, L, b_kv, kept)
    torch.cuda.synchronize()
    k = kept.cpu().numpy()
    for u in range(U):
        ref = oracle.select.select(s[u].astype(np.float64), L, b_kv, P, R)
        assert np.array_equal(k[u], ref), f"unit {u}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,b_kv", [
    (256, 128), (519, 301),             # four wavefronts per part
    (700, 600), (1100, 1023),           # eight
    (2176, 2048), (4224, 4096),         # sixteen, one to eight rounds of 512 tokens
    (1000, 999),                        # one eviction
])
def test_compact_in_place_and_out_of_place(d, L, b_kv):
    """Unit 0: nothing moves; unit 1: only the last entry moves; unit 2:
    every kept slot but the first comes from the tail (each token moves by
    L - b_kv, further than a round when L - b_kv > 512)."""
    U = 13
    log(f"compact d={d} L={L} b_kv={b_kv}")
    r = np.random.default_rng(d + L)
    l_cap = L + 3
    K = r.standard_normal((U, l_cap, d)).astype(np.float32)
    V = r.standard_normal((U, l_cap, d)).astype(np.float32)
    kpos = (np.arange(l_cap)[None].repeat(U, 0) * 2 + 11).astype(np.int32)
    kept = np.stack([np.sort(r.choice(L, b_kv, replace=False)) for _ in range(U)]).astype(np.int32)
    kept[0] = np.arange(b_kv)           # nothing moves
    kept[1, : b_kv - 1] = np.arange(b_kv - 1)
    kept[1, -1] = L - 1                  # only the last entry moves
    kept[2, 0] = 0
    kept[2, 1:] = np.arange(L - b_kv + 1, L)
    Kt = torch.from_numpy(K).to(torch.bfloat16).to(DEV)
    Vt = torch.from_numpy(V).to(torch.bfloat16).to(DEV)
    Pt = torch.from_numpy(kpos).to(DEV)
    kt = torch.from_numpy(kept).to(DEV)
    shape = bkv.Shape(U, 1, d, l_cap, 0, 1e4)
    Ko = torch.zeros((U, b_kv, d), dtype=torch.bfloat16, device=DEV)
    Vo = torch.zeros_like(Ko)
    Po = torch.zeros((U, b_kv), dtype=torch.int32, device=DEV)
    Kh, Vh = Kt.cpu(), Vt.cpu()
    bkv.compact(shape, Kt, Vt, Pt, L, kt, b_kv, Ko, Vo, Po, out_cap=b_kv)
    K2, V2, P2 = Kt.clone(), Vt.clone(), Pt.clone()
    bkv.compact(shape, K2, V2, P2, L, kt, b_kv)
    torch.cuda.synchronize()
    for u in range(U):
        ek, ev, ep = oracle.compact.compact(Kh[u].view(torch.int16).numpy(),
                                            Vh[u].view(torch.int16).numpy(), kpos[u], kept[u])
        assert np.array_equal(Ko[u].cpu().view(torch.int16).numpy(), ek)
        assert np.array_equal(Vo[u].cpu().view(torch.int16).numpy(), ev)
        assert np.array_equal(Po[u].cpu().numpy(), ep)
    # In place equals out of place, and the tail past b_kv is untouched.
    assert torch.equal(K2[:, :b_kv].view(torch.int16), Ko.view(torch.int16))
    assert torch.equal(V2[:, :b_kv].view(torch.int16), Vo.view(torch.int16))
    assert torch.equal(P2[:, :b_kv], Po)
    assert torch.equal(K2[:, b_kv:].view(torch.int16), Kt[:, b_kv:].view(torch.int16))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,b_kv", [(256, 128), (2176, 2048), (519, 301), (5000, 1000),
                                    (70, 65)])
def test_compact_unsorted_bit_exact(d, L, b_kv):
    """Hole filling against the oracle's fill_holes, every unit, bit for bit.

    (5000, 1000): 3,800+ holes per unit, more than one pass of the kernel's
    1024-hole window; units 0-2: nothing moves, one move, every kept slot at
    or past b_kv but the first."""
    U = 13
    log(f"compact unsorted d={d} L={L} b_kv={b_kv}")
    r = np.random.default_rng(3 * d + L)
    l_cap = L + 3
    K = r.standard_normal((U, l_cap, d)).astype(np.float32)
    V = r.standard_normal((U, l_cap, d)).astype(np.float32)
    kpos = (np.arange(l_cap)[None].repeat(U, 0) * 2 + 11).astype(np.int32)
    kept = np.stack([np.sort(r.choice(L, b_kv, replace=False)) for _ in range(U)]).astype(np.int32)
    kept[0] = np.arange(b_kv)                       # nothing moves
    kept[1, : b_kv - 1] = np.arange(b_kv - 1)
    kept[1, -1] = L - 1                             # one move
    kept[2, 0] = 0
    kept[2, 1:] = np.arange(L - b_kv + 1, L)        # all but slot 0 come from the tail
    Kt = torch.from_numpy(K).to(torch.bfloat16).to(DEV)
    Vt = torch.from_numpy(V).to(torch.bfloat16).to(DEV)
    Pt = torch.from_numpy(kpos).to(DEV)
    kt = torch.from_numpy(kept).to(DEV)
    Kh, Vh = Kt.cpu().view(torch.int16).numpy(), Vt.cpu().view(torch.int16).numpy()
    shape = bkv.Shape(U, 1, d, l_cap, 0, 1e4)
    bkv.compact_unsorted(shape, Kt, Vt, Pt, L, kt, b_kv)
    torch.cuda.synchronize()
    Kg, Vg, Pg = Kt.cpu().view(torch.int16).numpy(), Vt.cpu().view(torch.int16).numpy(), Pt.cpu()
    for u in range(U):
        ek, ev, ep, moves = oracle.compact.fill_holes(Kh[u], Vh[u], kpos[u], kept[u], b_kv)
        assert np.array_equal(Kg[u, :b_kv], ek), f"unit {u} K"
        assert np.array_equal(Vg[u, :b_kv], ev), f"unit {u} V"
        assert np.array_equal(Pg[u, :b_kv].numpy(), ep), f"unit {u} kpos"
        # slots at and past b_kv are read, never written
        assert np.array_equal(Kg[u, b_kv:], Kh[u, b_kv:]), f"unit {u} tail"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L,b_kv,P,kind", [
    (256, 128, 8, "cont"),      # 4 score registers per lane
    (1000, 24, 8, "cont"),      # only the forced slots kept
    (777, 300, 33, "ties"),     # many equal scores around the cut
    (2176, 2048, 8, "cont"),    # the Qwen3-4B step's shape
    (4224, 4096, 512, "ties"),  # the wide kernel (72 score registers per lane)
    (5000, 1000, 8, "cont"),    # the LDS-staged selection
])
def test_select_compact_matches_the_two_calls(d, L, b_kv, P, kind):
    """Selection and compaction in one call: the oracle's kept set exactly,
    and K, V, positions equal to the oracle's compaction of the inputs."""
    U, R = 21, 16
    log(f"select_compact d={d} L={L} b_kv={b_kv} P={P} {kind}")
    r = np.random.default_rng(L + d)
    if kind == "cont":
        s = r.random((U, L)).astype(np.float32) * 1e-3
    else:
        s = r.choice(np.array([1e-6, 2e-6, 2e-6, 5e-4, 0.25, 0.0], np.float32), size=(U, L))
    l_cap = L + 7
    sc = torch.zeros((U, l_cap), dtype=torch.float32, device=DEV)
    sc[:, :L] = torch.from_numpy(s).to(DEV)
    K = torch.from_numpy(r.standard_normal((U, l_cap, d)).astype(np.float32)).to(
        torch.bfloat16).to(DEV)
    V = torch.from_numpy(r.standard_normal((U, l_cap, d)).astype(np.float32)).to(
        torch.bfloat16).to(DEV)
    kpos = torch.from_numpy((np.arange(l_cap)[None].repeat(U, 0) * 3 + 5).astype(np.int32)).to(DEV)
    Kh, Vh, Ph = K.cpu(), V.cpu(), kpos.cpu().numpy()
    kept = torch.full((U, b_kv), -1, dtype=torch.int32, device=DEV)
    shape = bkv.Shape(U, 1, d, l_cap, P, 1e4, recent_tok=R)
    bkv.select_compact(shape, sc, L, b_kv, K, V, kpos, kept)
    torch.cuda.synchronize()
    k = kept.cpu().numpy()
    for u in range(U):
        ref = oracle.select.select(s[u].astype(np.float64), L, b_kv, P, R)
        assert np.array_equal(k[u], ref), f"unit {u} kept"
        ek, ev, ep = oracle.compact.compact(Kh[u].view(torch.int16).numpy(),
                                            Vh[u].view(torch.int16).numpy(), Ph[u], ref)
        assert np.array_equal(K[u, :b_kv].cpu().view(torch.int16).numpy(), ek), f"unit {u} K"
        assert np.array_equal(V[u, :b_kv].cpu().view(torch.int16).numpy(), ev), f"unit {u} V"
        assert np.array_equal(kpos[u, :b_kv].cpu().numpy(), ep), f"unit {u} kpos"
    # Slots past b_kv are left as they were.
    assert torch.equal(K[:, b_kv:].cpu().view(torch.int16), Kh[:, b_kv:].view(torch.int16))


def test_select_compact_full_size_equals_two_calls():
    """Qwen3-4B shape, all 4608 units: the in-place call against select
    followed by an out-of-place compaction, bit for bit."""
    import synth
    w = synth.WORKLOADS["qwen3_4b_full_b2048"]
    log(f"select_compact full size: U={w.n_units} L={w.L} B={w.b_kv}")
    dev = synth.device_inputs(w, DEV)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, w.L, w.prefix, w.theta,
                      recent_tok=w.recent_tok)
    score = torch.zeros((w.n_units, w.L), device=DEV)
    bkv.score(shape, dev["keys"], dev["kpos"], w.L, dev["buf"], dev["recents"], w.L, score)
    kept_a = torch.zeros((w.n_units, w.b_kv), dtype=torch.int32, device=DEV)
    kept_b = torch.zeros_like(kept_a)
    bkv.select(shape, score, w.L, w.b_kv, kept_a)
    Ko = torch.empty((w.n_units, w.b_kv, w.d_head), dtype=torch.bfloat16, device=DEV)
    Vo, Po = torch.empty_like(Ko), torch.empty((w.n_units, w.b_kv), dtype=torch.int32,
                                                device=DEV)
    bkv.compact(shape, dev["keys"], dev["values"], dev["kpos"], w.L, kept_a, w.b_kv, Ko, Vo, Po,
                out_cap=w.b_kv)
    bkv.select_compact(shape, score, w.L, w.b_kv, dev["keys"], dev["values"], dev["kpos"],
                       kept_b)
    torch.cuda.synchronize()
    assert torch.equal(kept_a, kept_b)
    assert torch.equal(dev["keys"][:, :w.b_kv].view(torch.int16), Ko.view(torch.int16))
    assert torch.equal(dev["values"][:, :w.b_kv].view(torch.int16), Vo.view(torch.int16))
    assert torch.equal(dev["kpos"][:, :w.b_kv], Po)
