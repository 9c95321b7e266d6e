"""Host-side pieces of bench.py: the algorithmic-byte model and the guards."""
import subprocess
import sys

import numpy as np

import bench
import synth


def test_stage_bytes_model():
    w = synth.WORKLOADS["qwen3_4b_full_b2048"]
    U, g, d, L, B, P, R = w.n_units, w.group, w.d_head, w.L, w.b_kv, w.prefix, w.recent_tok
    n_mv = 12345
    sb = bench.stage_bytes(w, n_mv)
    # The one-launch selection and compaction moves what the two stages move.
    assert sb["select_compact"] == sb["select"] + sb["compact"]
    # Keys read once, fp32 observation rows, recent positions, fp32 scores out.
    assert sb["score"] == U * (L * d * 2 + g * 32 * d * 4 + 16 * 4 + L * 4)
    # A moved token: K and V rows read and written (bf16) plus its position.
    assert sb["compact"] - U * B * 4 == n_mv * (4 * d * 2 + 8)
    assert sb["select"] == U * ((L - P - R) * 4 + B * 4)
    # FPS: 48 rows of d fp32 per head (31 + 1 in, 16 out; or 16 + 16 in, 16 out) + the count.
    assert sb["fps_compress"] == sb["fps_merge"] == U * g * (48 * d * 4 + 8)


def test_source_digest_of_several_files_differs_from_one():
    assert bench.source_digest("compact.hip") != bench.source_digest(("compact.hip",
                                                                      "select_wave.h"))
    assert bench.source_digest(["compact.hip"]) == bench.source_digest("compact.hip")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--workload", "nope"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "unknown workload" in r.stderr


def test_moved_token_count():
    # Hand cases: nothing evicted below the last kept slot moves nothing; a
    # gap at slot 2 moves every later kept slot; unsorted moves only the
    # kept slots at or past b_kv.
    assert bench.moved_token_count([[0, 1, 2, 3]], 4, False) == 0
    assert bench.moved_token_count([[0, 1, 3, 4]], 4, False) == 2
    assert bench.moved_token_count([[1, 2, 3, 4]], 4, False) == 4
    assert bench.moved_token_count([[0, 1, 3, 4]], 4, True) == 1
    assert bench.moved_token_count([[0, 5, 6, 7]], 4, True) == 3
    # Random keep sets against an explicit loop.
    r = np.random.default_rng(0)
    for _ in range(20):
        L, b = int(r.integers(10, 60)), int(r.integers(2, 9))
        kept = np.array([np.sort(r.choice(L, size=b, replace=False)) for _ in range(3)])
        want_sorted = sum(1 for row in kept for k, slot in enumerate(row) if slot != k)
        want_fill = sum(1 for row in kept for slot in row if slot >= b)
        assert bench.moved_token_count(kept, b, False) == want_sorted
        assert bench.moved_token_count(kept, b, True) == want_fill


def test_parity_sample_accepts_the_oracle_and_rejects_mistakes():
    """The bench's parity leg, fed outputs built by the oracle itself (CPU
    tensors), passes; a wrong keep set or a wrong compacted row fails it."""
    import torch

    import oracle
    w = synth.WORKLOADS["tiny"]
    inp = synth.workload_inputs(w)
    U, g, d, L, B = w.n_units, w.group, w.d_head, w.L, w.b_kv
    K0 = torch.from_numpy(inp["keys"]).to(torch.bfloat16)
    V0 = torch.from_numpy(inp["values"]).to(torch.bfloat16)
    P0 = torch.from_numpy(inp["kpos"])
    buf0 = torch.from_numpy(inp["buf"].reshape(U * g, 32, d))
    rec = torch.from_numpy(inp["recents"].reshape(U * g, 16, d))
    newq = buf0[:, 31:32].clone()
    beacons = np.stack([buf0[q].numpy()[oracle.fps.fps(buf0[q].numpy(), 16)[1]]
                        for q in range(U * g)])
    K, V, kpos = K0.clone(), V0.clone(), P0.clone()
    buf, score = buf0.clone(), torch.zeros(U, L)
    kept = torch.zeros(U, B, dtype=torch.int64)
    for u in range(U):
        ref = oracle.evict.evict_unit(K0[u].float().numpy(), V0[u].float().numpy(), P0[u].numpy(),
                                      L, beacons[u * g:(u + 1) * g], rec[u * g:(u + 1) * g].numpy(),
                                      L, B, w.prefix, w.recent_tok, w.theta)
        score[u] = torch.from_numpy(ref["score"].astype(np.float32))
        kept[u] = torch.from_numpy(ref["kept"])
        K[u, :B], V[u, :B], kpos[u, :B] = K0[u, kept[u]], V0[u, kept[u]], P0[u, kept[u]]
        for h in range(g):
            buf[u * g + h, :16] = torch.from_numpy(ref["buf"][h])
    args = (w, [0, U - 1], K0, V0, P0, buf0, newq, rec, beacons)
    good = bench.parity_sample(*args, K, V, kpos, buf, score, kept, False, "max", False)
    assert good["ok"] and good["kept_diff_outside_tie_band"] == 0 and good["compaction_exact"]
    assert good["fps_rows_are_distinct_inputs"] and good["max_score_rel_err"] < 1e-6
    # Swap the best kept middle slot for the worst evicted one.
    s = score[0].numpy()
    k0 = set(kept[0].tolist())
    mid = [j for j in range(w.prefix, L - w.recent_tok)]
    best = max((j for j in mid if j in k0), key=lambda j: s[j])
    worst = min((j for j in mid if j not in k0), key=lambda j: s[j])
    bad = kept.clone()
    bad[0] = torch.tensor(sorted((k0 - {best}) | {worst}))
    r = bench.parity_sample(*args, K, V, kpos, buf, score, bad, False, "max", False)
    assert not r["ok"] and r["kept_diff_outside_tie_band"] == 2
    K2 = K.clone()
    K2[U - 1, 5] = K2[U - 1, 5] + 1
    r = bench.parity_sample(*args, K2, V, kpos, buf, score, kept, False, "max", False)
    assert not r["ok"] and not r["compaction_exact"]
    buf2 = buf.clone()
    buf2[1, 3] = buf2[1, 3] * 1.5    # a merged row that is no input row
    r = bench.parity_sample(*args, K, V, kpos, buf2, score, kept, False, "max", False)
    assert not r["ok"] and not r["fps_rows_are_distinct_inputs"]
