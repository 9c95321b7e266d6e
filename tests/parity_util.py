"""Acceptance rules shared by the GPU parity tests (compare HIP vs oracle).

* scores: |s_gpu - s_ora| <= 2e-3 * s_ora + 1e-30 element-wise;
* kept sets: exactly b_kv entries, forced slots present, ascending; every
  slot in the symmetric difference with the oracle's set has an oracle score
  within 2e-3 (relative) of the oracle's K'-th largest middle score s*;
* FPS: the GPU's pick order replayed in float64 is a valid FPS run within
  2e-3 at every step, and the picked set equals the oracle's whenever every
  oracle step wins by more than 2e-3.
"""
import sys

import numpy as np

import oracle

TOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_scores(got, want, where=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bound = TOL * want + 1e-30
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{where}: {bad.size} scores out of tolerance, first slot {bad[0]}: "
                           f"gpu {got[bad[0]]:.9g} oracle {want[bad[0]]:.9g}")
    return float(np.max(err / (want + 1e-30)))


def check_kept(kept_gpu, score_ora, L, b_kv, prefix, recent_tok, where=""):
    kept_gpu = np.asarray(kept_gpu, np.int64)
    assert kept_gpu.shape == (b_kv,), where
    assert np.all(np.diff(kept_gpu) > 0), f"{where}: kept not strictly ascending"
    assert kept_gpu[0] >= 0 and kept_gpu[-1] < L, where
    s = set(kept_gpu.tolist())
    assert set(range(prefix)) <= s, f"{where}: prefix slot missing"
    assert set(range(L - recent_tok, L)) <= s, f"{where}: recent slot missing"
    ref = oracle.select.select(score_ora, L, b_kv, prefix, recent_tok)
    diff = s ^ set(ref.tolist())
    if diff:
        mid = np.sort(np.asarray(score_ora, np.float64)[prefix:L - recent_tok])[::-1]
        s_star = mid[b_kv - prefix - recent_tok - 1]
        for j in diff:
            assert abs(score_ora[j] - s_star) <= TOL * s_star, (
                f"{where}: slot {j} (score {score_ora[j]:.6g}) differs outside the tie band "
                f"around {s_star:.6g}")
    return len(diff)


def check_fps(rows, order, m, where=""):
    """rows: [N, d] buffer before compression; order: GPU pick order."""
    order = [int(x) for x in order]
    assert len(order) == m and len(set(order)) == m, f"{where}: bad pick list {order}"
    assert all(0 <= r < rows.shape[0] for r in order), where
    ok, worst = oracle.fps.replay_check(rows, order, TOL)
    assert ok, f"{where}: FPS replay off by {worst:.3g}"
    ref_order, _ = oracle.fps.fps(rows, m)
    margins = oracle.fps.fps_margins(rows, m)
    if min(margins) > TOL:
        assert sorted(order) == sorted(ref_order), f"{where}: FPS set differs"
        return True
    return False
