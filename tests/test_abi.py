"""Host-only checks of the C ABI: exports, validation, error codes.

No call here reaches a kernel launch: every call either fails validation,
has n_units == 0, or is stopped by the fault-injection hook, all of which
return before the library touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

from reasoning_model_kv_amd import bkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    return bkv.load_library()


def _shape(**kw):
    base = dict(n_units=4, group=4, d_head=128, l_cap=512, prefix=8, rope_theta=1e6)
    base.update(kw)
    return bkv.Shape(**base)


def test_exports_every_declared_symbol(lib):
    with open(os.path.join(ROOT, "include", "bkv.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(bkv_\w+)\(", header, re.M))
    assert declared == set(bkv.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.bkv_abi_version() == bkv.ABI_VERSION


def _call_score(lib, shape, L=300, t=300, ws_bytes=1 << 20, K=FAKE, score=FAKE, ws=FAKE):
    return lib.bkv_score(ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), K, FAKE, L,
                         FAKE, FAKE, t, score, None, ws, ws_bytes, None)


def test_score_validation(lib):
    s = _shape()
    assert _call_score(lib, s, K=None) == bkv.BKV_EINVAL
    assert _call_score(lib, s, L=600) == bkv.BKV_EINVAL          # L > l_cap
    assert _call_score(lib, s, L=8) == bkv.BKV_EINVAL            # L < n_recent_q
    assert _call_score(lib, s, t=-1) == bkv.BKV_EINVAL
    assert _call_score(lib, s, ws_bytes=16) == bkv.BKV_ENOSPC
    assert "workspace" in bkv.last_error()
    assert _call_score(lib, _shape(d_head=96)) == bkv.BKV_ENOTSUP
    assert _call_score(lib, _shape(group=9)) == bkv.BKV_ENOTSUP
    assert _call_score(lib, _shape(group=0)) == bkv.BKV_EINVAL
    assert _call_score(lib, _shape(n_beacon=8)) == bkv.BKV_ENOTSUP
    assert _call_score(lib, _shape(n_beacon=0)) == bkv.BKV_ENOTSUP    # 0 beacons needs 32 recents
    assert _call_score(lib, _shape(n_units=0, n_beacon=0, n_recent_q=32)) == bkv.BKV_OK
    assert _call_score(lib, _shape(rope_theta=0.0)) == bkv.BKV_EINVAL
    bad_flags = _shape()
    pol = bad_flags.policy()
    pol.flags = 4                                                 # unknown flag bit
    assert lib.bkv_score(ctypes.byref(bad_flags.dims()), ctypes.byref(pol), FAKE, FAKE, 300,
                         FAKE, FAKE, 300, FAKE, None, FAKE, 1 << 20, None) == bkv.BKV_EINVAL
    assert "flags" in bkv.last_error()
    assert _call_score(lib, _shape(n_units=0, aggregate="mean")) == bkv.BKV_OK
    with pytest.raises(ValueError):
        _shape(aggregate="median").policy()
    assert _call_score(lib, _shape(buf_cap=9000)) == bkv.BKV_ENOTSUP
    big = _shape(n_units=1, l_cap=1 << 23)                        # 2^31 key bytes per unit
    assert _call_score(lib, big, L=1 << 23, t=1 << 23) == bkv.BKV_ENOTSUP
    assert "2^31" in bkv.last_error()
    assert _call_score(lib, _shape(n_units=0)) == bkv.BKV_OK     # no-op, no launch
    assert bkv.last_error() == ""


def test_select_validation(lib):
    s = _shape(prefix=8)
    call = lambda L, b: lib.bkv_select(ctypes.byref(s.dims()), ctypes.byref(s.policy()),
                                        FAKE, L, b, FAKE, None)
    assert call(300, 20) == bkv.BKV_EINVAL    # b_kv < P + R
    assert call(300, 300) == bkv.BKV_EINVAL   # b_kv == L
    assert call(600, 100) == bkv.BKV_EINVAL   # L > l_cap
    s0 = _shape(n_units=0)
    assert lib.bkv_select(ctypes.byref(s0.dims()), ctypes.byref(s0.policy()), FAKE, 300, 100,
                          FAKE, None) == bkv.BKV_OK


def test_compact_validation(lib):
    s = _shape()
    d = ctypes.byref(s.dims())
    assert lib.bkv_compact(d, FAKE, FAKE, FAKE, 300, FAKE, 0, None, None, None, 0,
                           None) == bkv.BKV_EINVAL
    assert lib.bkv_compact(d, FAKE, FAKE, FAKE, 300, FAKE, 301, None, None, None, 0,
                           None) == bkv.BKV_EINVAL
    # partially given outputs
    assert lib.bkv_compact(d, FAKE, FAKE, FAKE, 300, FAKE, 200, FAKE, None, None, 200,
                           None) == bkv.BKV_EINVAL
    # out_cap too small
    o = ctypes.c_void_p(0x20000)
    assert lib.bkv_compact(d, FAKE, FAKE, FAKE, 300, FAKE, 200, o, o, o, 100,
                           None) == bkv.BKV_EINVAL
    # aliasing outputs
    assert lib.bkv_compact(d, FAKE, FAKE, FAKE, 300, FAKE, 200, FAKE, o, o, 200,
                           None) == bkv.BKV_EINVAL


def test_compact_unsorted_validation(lib):
    s = _shape()
    d = ctypes.byref(s.dims())
    call = lambda K, L, b: lib.bkv_compact_unsorted(d, K, FAKE, FAKE, L, FAKE, b, None)
    assert call(None, 300, 200) == bkv.BKV_EINVAL    # NULL K
    assert call(FAKE, 300, 0) == bkv.BKV_EINVAL      # b_kv = 0
    assert call(FAKE, 300, 301) == bkv.BKV_EINVAL    # b_kv > L
    assert call(FAKE, 600, 200) == bkv.BKV_EINVAL    # L > l_cap
    s0 = _shape(n_units=0)
    assert lib.bkv_compact_unsorted(ctypes.byref(s0.dims()), FAKE, FAKE, FAKE, 300, FAKE, 200,
                                    None) == bkv.BKV_OK


def test_fps_validation(lib):
    s = _shape()
    call = lambda nq, n_new, trig, m: lib.bkv_fps_update(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, FAKE, nq, n_new, trig, m, None,
        None, None)
    assert call(None, 0, 32, 32) == bkv.BKV_EINVAL     # m == trigger
    assert call(None, 0, 34, 16) == bkv.BKV_EINVAL     # trigger > buf_cap + 1
    assert call(None, 0, 32, 0) == bkv.BKV_EINVAL      # m < 1
    assert call(FAKE, 0, 32, 16) == bkv.BKV_EINVAL     # new_q without rows
    assert call(None, 1, 32, 16) == bkv.BKV_EINVAL     # rows without new_q
    assert call(FAKE, 33, 32, 16) == bkv.BKV_EINVAL    # n_new > buf_cap
    # (n_units = 0: validation only, nothing is launched)
    long = _shape(buf_cap=1000, n_units=0)
    lcall = lambda trig, m: lib.bkv_fps_update(
        ctypes.byref(long.dims()), ctypes.byref(long.policy()), FAKE, FAKE, None, 0, trig, m,
        None, None, None)
    assert lcall(1000, 65) == bkv.BKV_ENOTSUP          # long buffers keep at most 64
    assert lcall(1001, 65) == bkv.BKV_OK               # append only: no limit on m
    # new_q not 16-byte aligned (no units: the checks run before the early
    # return, and nothing could be launched if they did not)
    z = _shape(n_units=0)
    assert lib.bkv_fps_update(ctypes.byref(z.dims()), ctypes.byref(z.policy()), FAKE, FAKE,
                              ctypes.c_void_p(0x10004), 1, 32, 16, None, None,
                              None) == bkv.BKV_EINVAL


def test_fps_strided_validation(lib):
    # No units: every check runs before the library's early return, so a
    # check that failed to refuse would still launch nothing.
    s = _shape(n_units=0)
    scall = lambda nq, n_new, hs, rs: lib.bkv_fps_update_strided(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, FAKE, nq, n_new, hs, rs, 32, 16,
        None, None, None)
    d = s.d_head
    assert scall(FAKE, 2, d, d - 4) == bkv.BKV_EINVAL             # row stride below d_head
    assert scall(FAKE, 2, d + 2, 2 * d) == bkv.BKV_EINVAL         # head stride not a multiple of 4
    assert scall(FAKE, 2, -4, d) == bkv.BKV_EINVAL                # negative head stride
    assert scall(ctypes.c_void_p(0x10008), 2, d, 2 * d) == bkv.BKV_EINVAL  # misaligned new_q
    assert scall(FAKE, 0, d, d) == bkv.BKV_EINVAL                 # new_q without rows
    assert scall(FAKE, 33, d, d) == bkv.BKV_EINVAL                # n_new > buf_cap
    assert scall(FAKE, 2, 4 * d, d) == bkv.BKV_OK                 # valid: accepted, no launch
    big = _shape(n_units=0, buf_cap=1000)
    bcall = lambda n_new, hs, rs, trig: lib.bkv_fps_update_strided(
        ctypes.byref(big.dims()), ctypes.byref(big.policy()), FAKE, FAKE, FAKE, n_new, hs, rs,
        trig, 16, None, None, None)
    assert bcall(100, d, 6 * d, 1000) == bkv.BKV_ENOTSUP          # long buffers: head-major only
    assert bcall(100, 100 * d, d, 1000) == bkv.BKV_OK             # ... which they take
    assert bcall(2, d, 6 * d, 1001) == bkv.BKV_OK                 # small appends: any strides


def test_evict_validation_and_workspace(lib):
    s = _shape(l_cap=2176)
    need = bkv.workspace_bytes(s, 2176, 2048)
    table = bkv.workspace_bytes(s, 2176, 0)
    assert table >= 17 * 64 * 16
    assert need >= table + 4 * 2176 * 4 + 4 * 2048 * 4
    call = lambda ws_bytes, buf=None, count=None: lib.bkv_evict(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, FAKE, FAKE, 2176, FAKE, FAKE,
        2176, 2048, buf, count, None, None, FAKE, ws_bytes, None)
    assert call(need - 1) == bkv.BKV_ENOSPC
    assert call(need, buf=FAKE) == bkv.BKV_EINVAL      # buf without count
    w32 = _shape(l_cap=2176, n_beacon=0, n_recent_q=32, recent_tok=32)
    need32 = bkv.workspace_bytes(w32, 2176, 2048)
    assert lib.bkv_evict(ctypes.byref(w32.dims()), ctypes.byref(w32.policy()), FAKE, FAKE, FAKE,
                         2176, None, FAKE, 2176, 2048, FAKE, FAKE, None, None, FAKE, need32,
                         None) == bkv.BKV_EINVAL            # no beacons: no rolling update
    assert "buf" in bkv.last_error()
    with pytest.raises(bkv.BkvError):
        bkv.workspace_bytes(s, 2176, 2176)


def test_fault_injection_reports_hip_error(lib, monkeypatch):
    s = _shape()
    monkeypatch.setenv("BKV_FAULT_INJECT", "bkv_score")
    assert _call_score(lib, s) == bkv.BKV_EHIP
    assert "injected" in bkv.last_error()
    monkeypatch.setenv("BKV_FAULT_INJECT", "all")
    assert lib.bkv_select(ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, 300, 100,
                          FAKE, None) == bkv.BKV_EHIP


def test_missing_library_fails_loudly(tmp_path):
    import importlib
    mod = importlib.import_module("reasoning_model_kv_amd.bkv")
    with pytest.raises(ImportError):
        mod.load_library.__wrapped__(str(tmp_path / "nope.so")) if hasattr(
            mod.load_library, "__wrapped__") else _load_missing(mod, tmp_path)


def _load_missing(mod, tmp_path):
    saved = mod._lib
    mod._lib = None
    try:
        mod.load_library(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def _call_score_lse(lib, shape, L=300, lse_from=284, lse=FAKE):
    return lib.bkv_score_lse(ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), FAKE,
                             FAKE, L, FAKE, FAKE, L, lse, lse_from, FAKE, FAKE, 1 << 20, None)


def test_score_lse_validation(lib):
    s = _shape()
    assert _call_score_lse(lib, s, lse=None) == bkv.BKV_EINVAL
    assert "lse_in" in bkv.last_error()
    assert _call_score_lse(lib, s, lse_from=-1) == bkv.BKV_EINVAL
    assert _call_score_lse(lib, s, lse_from=301) == bkv.BKV_EINVAL   # beyond L
    assert _call_score_lse(lib, s, L=600) == bkv.BKV_EINVAL          # L > l_cap
    assert _call_score_lse(lib, _shape(d_head=96)) == bkv.BKV_ENOTSUP
    assert _call_score_lse(lib, _shape(n_units=0)) == bkv.BKV_OK
    assert _call_score_lse(lib, _shape(n_units=0), lse_from=300) == bkv.BKV_OK


def _call_decode(lib, shape, L=300, t_q=299, beacons=FAKE, t_obs=316, lse_obs=FAKE, out=FAKE,
                 q=FAKE):
    return lib.bkv_decode_attend(ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), FAKE,
                                 FAKE, L, q, t_q, beacons, t_obs, out, FAKE, lse_obs, None)


def test_decode_attend_validation(lib, monkeypatch):
    s = _shape()
    assert _call_decode(lib, s, q=None) == bkv.BKV_EINVAL
    assert _call_decode(lib, s, out=None) == bkv.BKV_EINVAL
    assert _call_decode(lib, s, lse_obs=None) == bkv.BKV_EINVAL      # beacons need lse_obs
    assert _call_decode(lib, s, L=0) == bkv.BKV_EINVAL
    assert _call_decode(lib, s, L=513) == bkv.BKV_EINVAL             # L > l_cap
    assert _call_decode(lib, s, t_q=-1) == bkv.BKV_EINVAL
    assert _call_decode(lib, s, t_obs=-1) == bkv.BKV_EINVAL
    assert _call_decode(lib, _shape(n_beacon=0, n_recent_q=32)) == bkv.BKV_EINVAL
    assert _call_decode(lib, _shape(d_head=32)) == bkv.BKV_ENOTSUP
    assert _call_decode(lib, _shape(group=9)) == bkv.BKV_ENOTSUP
    big = _shape(n_units=1, l_cap=1 << 23)
    assert _call_decode(lib, big, L=1 << 23) == bkv.BKV_ENOTSUP
    assert _call_decode(lib, _shape(n_units=0), beacons=None, lse_obs=None) == bkv.BKV_OK
    monkeypatch.setenv("BKV_FAULT_INJECT", "bkv_decode_attend")
    assert _call_decode(lib, s) == bkv.BKV_EHIP


def test_select_compact_validation(lib, monkeypatch):
    s = _shape(prefix=8)
    call = lambda L, b, K=FAKE: lib.bkv_select_compact(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, L, b, K, FAKE, FAKE, FAKE, None)
    assert call(300, 100, K=None) == bkv.BKV_EINVAL
    assert call(300, 300) == bkv.BKV_EINVAL        # b_kv must be < L
    assert call(300, 20) == bkv.BKV_EINVAL         # below prefix + recent
    assert call(600, 100) == bkv.BKV_EINVAL        # L > l_cap
    s0 = _shape(n_units=0, prefix=8)
    assert lib.bkv_select_compact(ctypes.byref(s0.dims()), ctypes.byref(s0.policy()), FAKE, 300,
                                  100, FAKE, FAKE, FAKE, FAKE, None) == bkv.BKV_OK
    monkeypatch.setenv("BKV_FAULT_INJECT", "bkv_select_compact")
    assert call(300, 100) == bkv.BKV_EHIP


def test_evict_lse_validation(lib):
    s = _shape(prefix=8)
    need = bkv.workspace_bytes(s, 300, 200)
    call = lambda lse=FAKE, lse_from=284, L=300: lib.bkv_evict_lse(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, FAKE, FAKE, L, FAKE, FAKE, L,
        lse, lse_from, 200, None, None, None, None, FAKE, need, None)
    assert call(lse=None) == bkv.BKV_EINVAL
    assert call(lse_from=-1) == bkv.BKV_EINVAL
    assert call(lse_from=301) == bkv.BKV_EINVAL
    s0 = _shape(n_units=0, prefix=8)
    assert lib.bkv_evict_lse(ctypes.byref(s0.dims()), ctypes.byref(s0.policy()), FAKE, FAKE, FAKE,
                             300, FAKE, FAKE, 300, FAKE, 284, 200, None, None, None, None, FAKE,
                             need, None) == bkv.BKV_OK


def test_evict_noalloc_scratch_limit(lib, monkeypatch):
    """The fixed scratch (16 MiB) must hold the RoPE table plus the score and
    kept arrays the caller does not pass; beyond it the call is refused before
    anything reaches the HIP runtime."""
    big = _shape(n_units=4608, l_cap=2176)
    call = lambda s, score=None, kept=None, L=2176, b=2048: lib.bkv_evict_noalloc(
        ctypes.byref(s.dims()), ctypes.byref(s.policy()), FAKE, FAKE, FAKE, L, FAKE, FAKE, L, b,
        FAKE, FAKE, score, kept, None)
    assert call(big) == bkv.BKV_ENOSPC
    assert "16777216" in bkv.last_error() and "score_out" in bkv.last_error()
    assert call(big, score=FAKE) == bkv.BKV_ENOSPC        # kept alone: 37.7 MB
    monkeypatch.setenv("BKV_FAULT_INJECT", "bkv_evict_noalloc")
    assert call(big, score=FAKE, kept=FAKE) == bkv.BKV_EHIP   # table only: fits
    small = _shape(n_units=8, l_cap=2176)
    assert call(small) == bkv.BKV_EHIP                      # 8 units: 135 KB fits
    assert "injected" in bkv.last_error()
    assert call(_shape(n_units=0, l_cap=2176)) == bkv.BKV_OK
    assert call(small, b=2176) == bkv.BKV_EINVAL            # b_kv must be < L
