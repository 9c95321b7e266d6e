"""The seeded generators: determinism, shapes, storage types."""
import numpy as np

import synth


def test_unit_inputs_deterministic_and_bf16_valued():
    w = synth.WORKLOADS["tiny"]
    a = synth.unit_inputs(w, 1)
    b = synth.unit_inputs(w, 1)
    for k in ("keys", "values", "buf", "recents", "kpos"):
        assert np.array_equal(a[k], b[k])
    assert a["keys"].shape == (w.L, w.d_head)
    assert a["buf"].shape == (w.group, 32, w.d_head)
    assert a["recents"].shape == (w.group, 16, w.d_head)
    assert np.array_equal(synth.to_bf16_values(a["keys"]), a["keys"])
    c = synth.unit_inputs(w, 0)
    assert not np.array_equal(a["keys"], c["keys"])


def test_outlier_channels_are_per_layer():
    w = synth.WORKLOADS["qwen3_4b_layer"]
    ch = synth.outlier_channels(w, 0)
    assert len(ch) == 4
    k, _ = synth.unit_keys_values(synth.shrink(w, L=300), 0)
    assert np.std(k[:, ch]) > 4 * np.std(np.delete(k, ch, axis=1))
