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
