"""bkv_evict_noalloc (scratch in the library's fixed array) against bkv_evict
(scratch in a caller's workspace): the same kernels, so every output must be
bit-identical.  Two calls in a row on one device, the second smaller than the
first, so the second runs on a scratch still holding the first call's data."""
import sys

import pytest
import torch

import synth
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(w):
    if w.n_units > 64:
        return synth.device_inputs(w, DEV)
    return synth.to_device(synth.workload_inputs(w), DEV)


def _run(w, noalloc, outputs):
    """One compress + eviction on fresh inputs; returns every output."""
    d = _inputs(w)
    shape = bkv.Shape(w.n_units, w.group, w.d_head, w.L, w.prefix, w.theta,
                      recent_tok=w.recent_tok)
    nq = w.n_units * w.group
    count = torch.full((nq,), 31, dtype=torch.int32, device=DEV)
    newq = d["buf"][:, 31:32].contiguous()
    bkv.fps_update(shape, d["buf"], count, newq, trigger=32, m=16)
    score = torch.full((w.n_units, w.L), -1.0, device=DEV) if outputs else None
    kept = torch.full((w.n_units, w.b_kv), -1, dtype=torch.int32, device=DEV) if outputs else None
    args = (shape, d["keys"], d["values"], d["kpos"], w.L, d["buf"], d["recents"], d["t"], w.b_kv)
    if noalloc:
        bkv.evict_noalloc(*args, buf=d["buf"], count=count, score_out=score, kept_out=kept)
    else:
        bkv.evict(*args, buf=d["buf"], count=count, score_out=score, kept_out=kept)
    torch.cuda.synchronize()
    out = {"K": d["keys"], "V": d["values"], "kpos": d["kpos"], "buf": d["buf"], "count": count}
    if outputs:
        out.update(score=score, kept=kept)
    return out


def _same(a, b, where):
    for k in a:
        assert a[k].shape == b[k].shape, (where, k)
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k]), \
            f"{where}: {k} differs"


@pytest.mark.parametrize("outputs", [False, True])
def test_noalloc_equals_evict_twice_second_smaller(outputs):
    # 4608 units at L = 256 (score and kept in the scratch: 7 MB), then the
    # two-unit tiny case.
    for name in ("qwen3_4b_full_b128", "tiny"):
        w = synth.WORKLOADS[name]
        _log(f"noalloc vs evict: {name} U={w.n_units} L={w.L} B={w.b_kv} outputs={outputs}")
        ref = _run(w, noalloc=False, outputs=outputs)
        got = _run(w, noalloc=True, outputs=outputs)
        _same(ref, got, name)
