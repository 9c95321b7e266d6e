"""FPS kernel (bkv_fps_update) against the float64 oracle on the GPU."""
import numpy as np
import pytest
import torch

import synth
from parity_util import check_fps, log
from reasoning_model_kv_amd import bkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(w, **kw):
    base = dict(n_units=w.n_units, group=w.group, d_head=w.d_head, l_cap=w.L,
                prefix=w.prefix, rope_theta=w.theta)
    base.update(kw)
    return bkv.Shape(**base)


@pytest.mark.parametrize("name", ["tiny", "qwen3_4b_layer"])
def test_compress_32_to_16(name):
    w = synth.WORKLOADS[name]
    log(f"fps compress {name}: Uq={w.n_qheads} d={w.d_head}")
    inp = synth.workload_inputs(w)
    host = inp["buf"].reshape(w.n_qheads, 32, w.d_head)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((w.n_qheads,), 32, dtype=torch.int32, device=DEV)
    sel = torch.full((w.n_qheads, 16), -7, dtype=torch.int32, device=DEV)
    bkv.fps_update(_shape(w), buf, count, trigger=32, m=16, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == 16)
    sel, out = sel.cpu().numpy(), buf.cpu().numpy()
    exact = 0
    for q in range(w.n_qheads):
        exact += check_fps(host[q], sel[q], 16, f"{name} head {q}")
        assert np.array_equal(out[q, :16], host[q][np.sort(sel[q])]), f"head {q} rows"
    log(f"  {exact}/{w.n_qheads} heads outside near-ties matched exactly")


def test_append_only_and_triggers():
    w = synth.WORKLOADS["tiny"]
    nq, d = w.n_qheads, w.d_head
    r = np.random.default_rng(5)
    host = r.standard_normal((nq, 32, d)).astype(np.float32)
    shape = _shape(w)
    # count 10 + 1 new row, trigger 32: append only.
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), 10, dtype=torch.int32, device=DEV)
    newq = torch.from_numpy(r.standard_normal((nq, 1, d)).astype(np.float32)).to(DEV)
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, newq, trigger=32, m=16, sel_order=sel)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert torch.all(count == 11) and torch.all(sel == -1)
    assert np.array_equal(out[:, 10], newq.cpu().numpy()[:, 0])
    assert np.array_equal(np.delete(out, 10, axis=1), np.delete(host, 10, axis=1))
    # Beacon fix on heads holding exactly 16: nothing changes.
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), 16, dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, trigger=17, m=16)
    torch.cuda.synchronize()
    assert torch.all(count == 16) and np.array_equal(buf.cpu().numpy(), host)
    # Mixed counts: 20 -> compress, 16 -> unchanged.
    buf = torch.from_numpy(host.copy()).to(DEV)
    cnt = np.array([20, 16, 20, 16][:nq], dtype=np.int32)
    count = torch.from_numpy(cnt).to(DEV)
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, trigger=17, m=16, sel_order=sel)
    torch.cuda.synchronize()
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    for q in range(nq):
        if cnt[q] == 20:
            check_fps(host[q, :20], sel[q], 16, f"beacon fix head {q}")
            assert np.array_equal(out[q, :16], host[q, :20][np.sort(sel[q])])
        else:
            assert np.all(sel[q] == -1) and np.array_equal(out[q], host[q])
    # Merge: 16 beacons + 16 appended recents, trigger 32.
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), 16, dtype=torch.int32, device=DEV)
    rec = r.standard_normal((nq, 16, d)).astype(np.float32)
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, torch.from_numpy(rec).to(DEV), trigger=32, m=16,
                   sel_order=sel)
    torch.cuda.synchronize()
    merged = np.concatenate([host[:, :16], rec], axis=1)
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    for q in range(nq):
        check_fps(merged[q], sel[q], 16, f"merge head {q}")
        assert np.array_equal(out[q, :16], merged[q][np.sort(sel[q])])


@pytest.mark.parametrize("name,n_new", [("tiny", 1), ("tiny", 3), ("qwen3_4b_layer", 1),
                                         ("qwen3_4b_layer", 2), ("qwen3_4b_layer", 3)])
def test_append_only_many_heads_per_workgroup(name, n_new):
    """trigger = buf_cap + 1 (append only): rows land at each head's count,
    counts advance, heads without room are left unchanged and counted as
    overflow, sel_order reads -1.  New rows of up to 64 16-byte chunks per
    head take the batched append kernel (tiny: 1 and 3 rows; d = 128: 1 and 2
    rows); 3 rows at d = 128 take the per-head kernel."""
    w = synth.WORKLOADS[name]
    nq, d = w.n_qheads, w.d_head
    r = np.random.default_rng(11 + n_new)
    host = r.standard_normal((nq, 32, d)).astype(np.float32)
    shape = _shape(w)
    cnt = np.array([(7 * q) % 33 for q in range(nq)], dtype=np.int32)  # some heads are full
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.from_numpy(cnt.copy()).to(DEV)
    newq = r.standard_normal((nq, n_new, d)).astype(np.float32)
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    ovf = torch.zeros((1,), dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, torch.from_numpy(newq).to(DEV), trigger=33, m=16,
                   sel_order=sel, n_overflow=ovf)
    torch.cuda.synchronize()
    out, cnt2 = buf.cpu().numpy(), count.cpu().numpy()
    fits = cnt + n_new <= 32
    assert int(ovf.item()) == int((~fits).sum())
    assert torch.all(sel == -1)
    for q in range(nq):
        if fits[q]:
            assert cnt2[q] == cnt[q] + n_new
            assert np.array_equal(out[q, cnt[q]:cnt[q] + n_new], newq[q])
            rest = np.delete(out[q], np.arange(cnt[q], cnt[q] + n_new), axis=0)
            assert np.array_equal(rest, np.delete(host[q], np.arange(cnt[q], cnt[q] + n_new),
                                                  axis=0))
        else:
            assert cnt2[q] == cnt[q] and np.array_equal(out[q], host[q])


def test_overflow_leaves_heads_unchanged():
    w = synth.WORKLOADS["tiny"]
    nq, d = w.n_qheads, w.d_head
    host = np.random.default_rng(6).standard_normal((nq, 32, d)).astype(np.float32)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), 31, dtype=torch.int32, device=DEV)
    newq = torch.ones((nq, 2, d), dtype=torch.float32, device=DEV)
    ovf = torch.zeros(1, dtype=torch.int32, device=DEV)
    bkv.fps_update(_shape(w), buf, count, newq, trigger=32, m=16, n_overflow=ovf)
    torch.cuda.synchronize()
    assert int(ovf.item()) == nq
    assert torch.all(count == 31) and np.array_equal(buf.cpu().numpy(), host)


@pytest.mark.parametrize("d,n", [(128, 256), (64, 200), (128, 33)])
def test_prefill_block_path(d, n):
    """Buffers above 32 rows (prefill FPS over up to 256 queries)."""
    nq, cap = 6, 256
    log(f"fps prefill block path d={d} N={n}")
    r = np.random.default_rng(n + d)
    host = r.standard_normal((nq, cap, d)).astype(np.float32)
    host[:, : n // 3] += 3.0 * r.standard_normal((nq, 1, d)).astype(np.float32)
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=cap)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), n, dtype=torch.int32, device=DEV)
    sel = torch.zeros((nq, 16), dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, trigger=17, m=16, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == 16)
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    for q in range(nq):
        check_fps(host[q, :n], sel[q], 16, f"prefill head {q}")
        assert np.array_equal(out[q, :16], host[q, :n][np.sort(sel[q])])


@pytest.mark.parametrize("d,n,cap,nq,m,n_new", [
    (128, 257, 300, 8, 16, 0),     # just past the workgroup-per-row path
    (64, 100, 300, 3, 16, 2),      # every unpicked row fits the shortlist from the start
    (128, 150, 300, 2, 64, 0),     # the unpicked rows come to fit the shortlist midway
    (64, 1000, 1000, 6, 16, 1),    # the last row arrives as a new query
    (128, 2000, 2048, 4, 64, 0),   # the largest kept set of the long path
    (128, 4096, 4096, 3, 16, 5),
    (64, 8192, 8192, 1, 16, 0),    # the largest buffer
    (128, 8192, 8192, 1, 64, 0),   # the largest buffer and kept set: 72 KB of LDS
])
def test_long_buffer_fps(d, n, cap, nq, m, n_new):
    """Buffers of more than 256 rows (prefill FPS over a long prompt): rows
    streamed from memory on every pass."""
    log(f"fps long buffer d={d} N={n} cap={cap} heads={nq} m={m} n_new={n_new}")
    r = np.random.default_rng(n + d + m)
    host = r.standard_normal((nq, cap, d)).astype(np.float32)
    host[:, : n // 4] += 3.0 * r.standard_normal((nq, 1, d)).astype(np.float32)
    host[:, n // 2: n // 2 + 50] += 5.0 * r.standard_normal((nq, 1, d)).astype(np.float32)
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=cap)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), n - n_new, dtype=torch.int32, device=DEV)
    newq = (torch.from_numpy(host[:, n - n_new:n].copy()).to(DEV) if n_new else None)
    sel = torch.full((nq, m), -7, dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, newq, trigger=n, m=m, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == m)
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    exact = 0
    for q in range(nq):
        exact += check_fps(host[q, :n], sel[q], m, f"long head {q}")
        assert np.array_equal(out[q, :m], host[q, :n][np.sort(sel[q])]), f"head {q} rows"
    log(f"  {exact}/{nq} heads outside near-ties matched exactly")


@pytest.mark.parametrize("d,n,m", [(128, 1500, 32), (64, 700, 16)])
def test_long_buffer_fps_duplicate_rows(d, n, m):
    """Rows drawn from 40 distinct vectors: equal cosines everywhere, so the
    slot breaks every tie, inside the shortlist and at its bound."""
    nq = 2
    log(f"fps long buffer, duplicated rows d={d} N={n} m={m}")
    r = np.random.default_rng(d + n)
    base = r.standard_normal((nq, 40, d)).astype(np.float32)
    host = np.ascontiguousarray(base[:, r.integers(0, 40, n)])
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=n)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), n, dtype=torch.int32, device=DEV)
    sel = torch.full((nq, m), -7, dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, trigger=n, m=m, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == m)
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    for q in range(nq):
        check_fps(host[q], sel[q], m, f"duplicated head {q}")
        assert np.array_equal(out[q, :m], host[q][np.sort(sel[q])]), f"head {q} rows"


def test_long_buffer_fps_degenerate_rows():
    """Zero rows, rows with a NaN or an infinity among ordinary ones: no
    parity is defined for such rows, but the call finishes and keeps m
    distinct rows of the buffer."""
    d, n, nq, m = 128, 900, 3, 16
    r = np.random.default_rng(21)
    host = r.standard_normal((nq, n, d)).astype(np.float32)
    host[0, 100:140] = 0.0
    host[1, 5, 7] = np.nan
    host[1, 300:310, 0] = np.inf
    host[2, :] = host[2, :1]          # every row the same
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=n)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), n, dtype=torch.int32, device=DEV)
    sel = torch.full((nq, m), -7, dtype=torch.int32, device=DEV)
    bkv.fps_update(shape, buf, count, trigger=n, m=m, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == m)
    out, sel = buf.cpu().numpy(), sel.cpu().numpy()
    for q in range(nq):
        assert len(set(sel[q].tolist())) == m and sel[q].min() >= 0 and sel[q].max() < n
        assert np.array_equal(out[q, :m], host[q][np.sort(sel[q])], equal_nan=True)
    # Identical rows tie everywhere: the lowest slots win, seed first.
    assert sel[2].tolist() == list(range(m))


@pytest.mark.parametrize("name,n", [("qwen3_4b_full_b2048", 2048), ("qwen3_4b_layer", 8192)])
def test_long_buffer_fps_full_size_sampled(name, n):
    """The prefill FPS at the benchmark's sizes (every query head of the
    Qwen3-4B step with its 2048-row prompt: 18,432 heads; one layer with
    8192-row prompts), in the launch bench.py --prefill-fps times; sampled
    heads against the oracle."""
    w = synth.shrink(synth.WORKLOADS[name], prefix=n)
    log(f"fps long buffer full size {w.name}: {w.n_qheads} heads x {n} rows")
    _, _, q = synth.StreamInputs(w, DEV).prompt()
    q0 = q.contiguous()
    del q
    nq, d, m = w.n_qheads, w.d_head, 16
    buf = q0.clone()
    count = torch.full((nq,), n, dtype=torch.int32, device=DEV)
    sel = torch.full((nq, m), -7, dtype=torch.int32, device=DEV)
    shape = bkv.Shape(w.n_units, w.group, d, 64, 0, w.theta, buf_cap=n)
    bkv.fps_update(shape, buf, count, trigger=n, m=m, sel_order=sel)
    torch.cuda.synchronize()
    assert torch.all(count == m)
    sel = sel.cpu().numpy()
    assert np.all((sel >= 0) & (sel < n))
    exact = 0
    heads = sorted({0, 1, nq // 3, nq // 2, nq - 1})
    for h in heads:
        rows = q0[h].cpu().numpy()
        exact += check_fps(rows, sel[h], m, f"{w.name} head {h}")
        assert np.array_equal(buf[h, :m].cpu().numpy(), rows[np.sort(sel[h])]), f"head {h} rows"
    log(f"  {exact}/{len(heads)} sampled heads outside near-ties matched exactly")


def test_long_buffer_append_only():
    d, cap, nq = 128, 600, 5
    r = np.random.default_rng(3)
    host = r.standard_normal((nq, cap, d)).astype(np.float32)
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=cap)
    buf = torch.from_numpy(host.copy()).to(DEV)
    count = torch.full((nq,), 500, dtype=torch.int32, device=DEV)
    newq = torch.from_numpy(r.standard_normal((nq, 40, d)).astype(np.float32)).to(DEV)
    bkv.fps_update(shape, buf, count, newq, trigger=cap + 1, m=16)
    torch.cuda.synchronize()
    assert torch.all(count == 540)
    got = buf.cpu().numpy()
    assert np.array_equal(got[:, 500:540], newq.cpu().numpy())
    assert np.array_equal(got[:, :500], host[:, :500])
    assert np.array_equal(got[:, 540:], host[:, 540:])


@pytest.mark.parametrize("d,cap,cnt,n_new,trigger,m", [
    (128, 32, 16, 16, 32, 16),     # fill and compress with 16 new rows (one wavefront per head)
    (128, 32, 10, 7, 33, 16),      # append only, many heads per workgroup
    (64, 16, 3, 9, 17, 16),        # append only into a recents-sized buffer
    (128, 64, 40, 24, 64, 16),     # one workgroup per head (buffers of up to 256 rows)
])
def test_strided_new_rows(d, cap, cnt, n_new, trigger, m):
    """bkv_fps_update_strided reading a step-major block of new rows
    ([n_new, heads, d], transposed as a view) leaves the buffers, counts and
    pick orders bit for bit as bkv_fps_update does with the same rows copied
    head-major; appended rows equal the inputs.  (Buffers of more than 256
    rows take head-major rows only; test_abi checks the refusal.)"""
    nq = 6
    log(f"strided new rows d={d} cap={cap} count={cnt} n_new={n_new} trigger={trigger}")
    r = np.random.default_rng(cap + n_new)
    host = r.standard_normal((nq, cap, d)).astype(np.float32)
    block = torch.from_numpy(r.standard_normal((n_new, nq, d)).astype(np.float32)).to(DEV)
    shape = bkv.Shape(n_units=nq, group=1, d_head=d, l_cap=64, prefix=0, rope_theta=1e6,
                      buf_cap=cap)
    out = []
    for view in (block.transpose(0, 1).contiguous(), block.transpose(0, 1)):
        buf = torch.from_numpy(host.copy()).to(DEV)
        count = torch.full((nq,), cnt, dtype=torch.int32, device=DEV)
        sel = torch.full((nq, m), -7, dtype=torch.int32, device=DEV)
        bkv.fps_update(shape, buf, count, view, trigger=trigger, m=m, sel_order=sel)
        torch.cuda.synchronize()
        out.append((buf.cpu().numpy(), count.cpu().numpy(), sel.cpu().numpy()))
    (b0, c0, s0), (b1, c1, s1) = out
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    live = int(c0[0])
    assert np.all(c0 == live)
    assert np.array_equal(b0[:, :live], b1[:, :live])
    if trigger > cap:  # append only: the rows land after the old ones, unchanged
        assert live == cnt + n_new
        assert np.array_equal(b1[:, cnt:live], block.transpose(0, 1).cpu().numpy())
        assert np.array_equal(b1[:, :cnt], host[:, :cnt])
    else:
        assert live == m and np.all(s1 >= 0)
