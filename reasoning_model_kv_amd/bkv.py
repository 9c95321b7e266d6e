"""Thin ctypes binding of libbkv.so: argument marshalling only.

Every function takes torch tensors, checks dtype / device / contiguity,
passes raw device pointers and the current HIP stream to the C entry point
of the same name, and raises ``BkvError`` on a non-zero return code.  All
computation happens in the library's kernels; nothing here falls back to
another implementation.
"""

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbkv.so")

BKV_OK, BKV_EINVAL, BKV_ENOTSUP, BKV_ENOSPC, BKV_EHIP = 0, -1, -2, -3, -4
ABI_VERSION = 1
BKV_FLAG_MEAN = 1      # policy flag: mean pooling (include/bkv.h)
BKV_FLAG_UNSORTED = 2  # policy flag: bkv_evict fills holes instead of shifting

EXPORTS = ("bkv_abi_version", "bkv_last_error", "bkv_workspace_bytes", "bkv_fps_update",
           "bkv_score", "bkv_select", "bkv_compact", "bkv_compact_unsorted", "bkv_evict",
           "bkv_score_lse", "bkv_decode_attend", "bkv_select_compact", "bkv_evict_lse",
           "bkv_evict_noalloc", "bkv_fps_update_strided")


class BkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("n_units", ctypes.c_int64), ("group", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("l_cap", ctypes.c_int64)]


class Policy(ctypes.Structure):
    _fields_ = [("n_beacon", ctypes.c_int32), ("n_recent_q", ctypes.c_int32),
                ("buf_cap", ctypes.c_int32), ("prefix", ctypes.c_int32),
                ("recent_tok", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("sm_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


@dataclass
class Shape:
    """Python mirror of bkv_dims + bkv_policy."""
    n_units: int
    group: int
    d_head: int
    l_cap: int
    prefix: int
    rope_theta: float
    recent_tok: int = 16
    buf_cap: int = 32
    n_beacon: int = 16
    n_recent_q: int = 16
    sm_scale: float = 0.0
    aggregate: str = "max"  # pooling of the attention weights: "max" or "mean"
    unsorted: bool = False  # bkv_evict compacts by filling holes (not in position order)

    def dims(self):
        return Dims(self.n_units, self.group, self.d_head, self.l_cap)

    def policy(self):
        if self.aggregate not in ("max", "mean"):
            raise ValueError(f"aggregate must be 'max' or 'mean', not {self.aggregate!r}")
        flags = (BKV_FLAG_MEAN if self.aggregate == "mean" else 0) | (
            BKV_FLAG_UNSORTED if self.unsorted else 0)
        return Policy(self.n_beacon, self.n_recent_q, self.buf_cap, self.prefix,
                      self.recent_tok, flags, float(self.rope_theta), float(self.sm_scale), 0)

    @property
    def scale(self):
        return self.sm_scale if self.sm_scale > 0 else 1.0 / math.sqrt(self.d_head)


_lib = None

_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_PD = ctypes.POINTER(Dims)
_PP = ctypes.POINTER(Policy)


def load_library(path=LIB_PATH):
    """Load libbkv.so and declare its signatures; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950) before using the library")
    lib = ctypes.CDLL(path)
    lib.bkv_abi_version.restype = ctypes.c_int
    lib.bkv_abi_version.argtypes = []
    lib.bkv_last_error.restype = ctypes.c_char_p
    lib.bkv_last_error.argtypes = []
    lib.bkv_workspace_bytes.restype = ctypes.c_size_t
    lib.bkv_workspace_bytes.argtypes = [_PD, _PP, _I64, _I64]
    lib.bkv_fps_update.restype = ctypes.c_int
    lib.bkv_fps_update.argtypes = [_PD, _PP, _VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP]
    lib.bkv_fps_update_strided.restype = ctypes.c_int
    lib.bkv_fps_update_strided.argtypes = [_PD, _PP, _VP, _VP, _VP, _I32, _I64, _I64, _I32, _I32,
                                           _VP, _VP, _VP]
    lib.bkv_score.restype = ctypes.c_int
    lib.bkv_score.argtypes = [_PD, _PP, _VP, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP,
                              ctypes.c_size_t, _VP]
    lib.bkv_select.restype = ctypes.c_int
    lib.bkv_select.argtypes = [_PD, _PP, _VP, _I64, _I64, _VP, _VP]
    lib.bkv_compact.restype = ctypes.c_int
    lib.bkv_compact.argtypes = [_PD, _VP, _VP, _VP, _I64, _VP, _I64, _VP, _VP, _VP, _I64, _VP]
    lib.bkv_compact_unsorted.restype = ctypes.c_int
    lib.bkv_compact_unsorted.argtypes = [_PD, _VP, _VP, _VP, _I64, _VP, _I64, _VP]
    lib.bkv_evict.restype = ctypes.c_int
    lib.bkv_evict.argtypes = [_PD, _PP, _VP, _VP, _VP, _I64, _VP, _VP, _I64, _I64, _VP, _VP,
                              _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.bkv_evict_noalloc.restype = ctypes.c_int
    lib.bkv_evict_noalloc.argtypes = [_PD, _PP, _VP, _VP, _VP, _I64, _VP, _VP, _I64, _I64, _VP,
                                      _VP, _VP, _VP, _VP]
    lib.bkv_score_lse.restype = ctypes.c_int
    lib.bkv_score_lse.argtypes = [_PD, _PP, _VP, _VP, _I64, _VP, _VP, _I64, _VP, _I64, _VP,
                                  _VP, ctypes.c_size_t, _VP]
    lib.bkv_evict_lse.restype = ctypes.c_int
    lib.bkv_evict_lse.argtypes = [_PD, _PP, _VP, _VP, _VP, _I64, _VP, _VP, _I64, _VP, _I64, _I64,
                                  _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.bkv_select_compact.restype = ctypes.c_int
    lib.bkv_select_compact.argtypes = [_PD, _PP, _VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP]
    lib.bkv_decode_attend.restype = ctypes.c_int
    lib.bkv_decode_attend.argtypes = [_PD, _PP, _VP, _VP, _I64, _VP, _I64, _VP, _I64, _VP,
                                      _VP, _VP, _VP]
    if lib.bkv_abi_version() != ABI_VERSION:
        raise ImportError(f"libbkv ABI {lib.bkv_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def last_error():
    return load_library().bkv_last_error().decode()


def _check(rc):
    if rc != BKV_OK:
        raise BkvError(rc, last_error())


def _ptr(t, dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, n, name):
    """Refuse a tensor smaller than the layout the call implies."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name}: {t.numel()} elements < {n} required by the shape")


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bits(t, name, allow_none=False):
    """bf16 tensors travel as their 16-bit patterns."""
    return _ptr(t, torch.bfloat16, name, allow_none)


def workspace_bytes(shape, L, b_kv=0):
    lib = load_library()
    n = lib.bkv_workspace_bytes(ctypes.byref(shape.dims()), ctypes.byref(shape.policy()),
                                int(L), int(b_kv))
    if n == 0:
        raise BkvError(BKV_EINVAL, last_error())
    return n


def alloc_workspace(shape, L, b_kv=0, device="cuda"):
    return torch.empty(workspace_bytes(shape, L, b_kv), dtype=torch.uint8, device=device)


def fps_update(shape, buf, count, new_q=None, trigger=32, m=16, sel_order=None,
               n_overflow=None, stream=None):
    lib = load_library()
    n_new = 0 if new_q is None else int(new_q.shape[-2])
    nq, d, cap = shape.n_units * shape.group, shape.d_head, shape.buf_cap
    _need(buf, nq * cap * d, "buf")
    _need(count, nq, "count")
    _need(new_q, nq * n_new * d, "new_q")
    _need(sel_order, nq * m, "sel_order")
    _need(n_overflow, 1, "n_overflow")
    if new_q is not None and not new_q.is_contiguous():
        # A strided view [U*g, n_new, d] (unit stride along d), e.g. a block of
        # steps' queries [n_new, U*g, d] transposed: bkv_fps_update_strided.
        if tuple(new_q.shape) != (nq, n_new, d) or new_q.stride(2) != 1:
            raise ValueError(f"new_q: a strided view must be [{nq}, n_new, {d}] with unit "
                             f"stride along d, got {tuple(new_q.shape)} strides {new_q.stride()}")
        if new_q.dtype != torch.float32 or not new_q.is_cuda:
            raise TypeError("new_q: expected a float32 device tensor")
        _check(lib.bkv_fps_update_strided(
            ctypes.byref(shape.dims()), ctypes.byref(shape.policy()),
            _ptr(buf, torch.float32, "buf"), _ptr(count, torch.int32, "count"),
            ctypes.c_void_p(new_q.data_ptr()), n_new, new_q.stride(0), new_q.stride(1),
            int(trigger), int(m), _ptr(sel_order, torch.int32, "sel_order", True),
            _ptr(n_overflow, torch.int32, "n_overflow", True), _stream(stream)))
        return
    _check(lib.bkv_fps_update(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()),
        _ptr(buf, torch.float32, "buf"), _ptr(count, torch.int32, "count"),
        _ptr(new_q, torch.float32, "new_q", True), n_new, int(trigger), int(m),
        _ptr(sel_order, torch.int32, "sel_order", True),
        _ptr(n_overflow, torch.int32, "n_overflow", True), _stream(stream)))


def _need_score_inputs(shape, K, kpos, beacons, recents):
    U, d, cap, nq = shape.n_units, shape.d_head, shape.l_cap, shape.n_units * shape.group
    _need(K, U * cap * d, "K")
    _need(kpos, U * cap, "kpos")
    _need(beacons, nq * shape.buf_cap * d, "beacons")
    _need(recents, nq * shape.n_recent_q * d, "recents")


def score(shape, K, kpos, L, beacons, recents, t, score_out, qobs_out=None, ws=None,
          stream=None):
    lib = load_library()
    _need_score_inputs(shape, K, kpos, beacons, recents)
    _need(score_out, shape.n_units * shape.l_cap, "score")
    _need(qobs_out, shape.n_units * shape.group * 32 * shape.d_head, "qobs_out")
    if ws is None:
        ws = alloc_workspace(shape, L, 0, K.device)
    _check(lib.bkv_score(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"),
        _ptr(kpos, torch.int32, "kpos"), int(L), _ptr(beacons, torch.float32, "beacons", shape.n_beacon == 0),
        _ptr(recents, torch.float32, "recents"), int(t), _ptr(score_out, torch.float32, "score"),
        _bits(qobs_out, "qobs_out", True), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)))


def score_lse(shape, K, kpos, L, beacons, recents, t, lse_in, lse_from, score_out, ws=None,
              stream=None):
    lib = load_library()
    _need_score_inputs(shape, K, kpos, beacons, recents)
    _need(score_out, shape.n_units * shape.l_cap, "score")
    _need(lse_in, shape.n_units * shape.group * 32, "lse_in")
    if ws is None:
        ws = alloc_workspace(shape, L, 0, K.device)
    _check(lib.bkv_score_lse(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"),
        _ptr(kpos, torch.int32, "kpos"), int(L), _ptr(beacons, torch.float32, "beacons", shape.n_beacon == 0),
        _ptr(recents, torch.float32, "recents"), int(t), _ptr(lse_in, torch.float32, "lse_in"),
        int(lse_from), _ptr(score_out, torch.float32, "score"), _ptr(ws, torch.uint8, "ws"),
        ws.numel(), _stream(stream)))


def decode_attend(shape, K, V, L, q, t_q, out, lse_q, beacons=None, t_obs=0, lse_obs=None,
                  stream=None):
    lib = load_library()
    U, d, cap, nq = shape.n_units, shape.d_head, shape.l_cap, shape.n_units * shape.group
    _need(K, U * cap * d, "K")
    _need(V, U * cap * d, "V")
    _need(q, nq * d, "q")
    _need(out, nq * d, "out")
    _need(lse_q, nq, "lse_q")
    _need(beacons, nq * shape.buf_cap * d, "beacons")
    _need(lse_obs, nq * 16, "lse_obs")
    _check(lib.bkv_decode_attend(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"), _bits(V, "V"),
        int(L), _ptr(q, torch.float32, "q"), int(t_q),
        _ptr(beacons, torch.float32, "beacons", True), int(t_obs),
        _ptr(out, torch.float32, "out"), _ptr(lse_q, torch.float32, "lse_q"),
        _ptr(lse_obs, torch.float32, "lse_obs", True), _stream(stream)))


def select(shape, score_t, L, b_kv, kept, stream=None):
    lib = load_library()
    _need(score_t, shape.n_units * shape.l_cap, "score")
    _need(kept, shape.n_units * int(b_kv), "kept")
    _check(lib.bkv_select(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()),
        _ptr(score_t, torch.float32, "score"), int(L), int(b_kv),
        _ptr(kept, torch.int32, "kept"), _stream(stream)))


def select_compact(shape, score_t, L, b_kv, K, V, kpos, kept, stream=None):
    lib = load_library()
    U, d, cap = shape.n_units, shape.d_head, shape.l_cap
    _need(score_t, U * cap, "score")
    _need(kept, U * int(b_kv), "kept")
    _need(K, U * cap * d, "K")
    _need(V, U * cap * d, "V")
    _need(kpos, U * cap, "kpos")
    _check(lib.bkv_select_compact(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()),
        _ptr(score_t, torch.float32, "score"), int(L), int(b_kv), _bits(K, "K"), _bits(V, "V"),
        _ptr(kpos, torch.int32, "kpos"), _ptr(kept, torch.int32, "kept"), _stream(stream)))


def compact(shape, K, V, kpos, L, kept, b_kv, K_out=None, V_out=None, kpos_out=None,
            out_cap=0, stream=None):
    lib = load_library()
    U, d, cap = shape.n_units, shape.d_head, shape.l_cap
    _need(K, U * cap * d, "K")
    _need(V, U * cap * d, "V")
    _need(kpos, U * cap, "kpos")
    _need(kept, U * int(b_kv), "kept")
    _need(K_out, U * int(out_cap) * d, "K_out")
    _need(V_out, U * int(out_cap) * d, "V_out")
    _need(kpos_out, U * int(out_cap), "kpos_out")
    _check(lib.bkv_compact(
        ctypes.byref(shape.dims()), _bits(K, "K"), _bits(V, "V"), _ptr(kpos, torch.int32, "kpos"),
        int(L), _ptr(kept, torch.int32, "kept"), int(b_kv), _bits(K_out, "K_out", True),
        _bits(V_out, "V_out", True), _ptr(kpos_out, torch.int32, "kpos_out", True),
        int(out_cap), _stream(stream)))


def compact_unsorted(shape, K, V, kpos, L, kept, b_kv, stream=None):
    """In place: kept tokens past b_kv fill the evicted slots below it."""
    lib = load_library()
    U, d, cap = shape.n_units, shape.d_head, shape.l_cap
    _need(K, U * cap * d, "K")
    _need(V, U * cap * d, "V")
    _need(kpos, U * cap, "kpos")
    _need(kept, U * int(b_kv), "kept")
    _check(lib.bkv_compact_unsorted(
        ctypes.byref(shape.dims()), _bits(K, "K"), _bits(V, "V"), _ptr(kpos, torch.int32, "kpos"),
        int(L), _ptr(kept, torch.int32, "kept"), int(b_kv), _stream(stream)))


def evict(shape, K, V, kpos, L, beacons, recents, t, b_kv, buf=None, count=None,
          score_out=None, kept_out=None, ws=None, stream=None):
    lib = load_library()
    _need_score_inputs(shape, K, kpos, beacons, recents)
    _need(V, shape.n_units * shape.l_cap * shape.d_head, "V")
    _need(buf, shape.n_units * shape.group * shape.buf_cap * shape.d_head, "buf")
    _need(count, shape.n_units * shape.group, "count")
    _need(score_out, shape.n_units * shape.l_cap, "score_out")
    _need(kept_out, shape.n_units * int(b_kv), "kept_out")
    if ws is None:
        ws = alloc_workspace(shape, L, b_kv, K.device)
    _check(lib.bkv_evict(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"), _bits(V, "V"),
        _ptr(kpos, torch.int32, "kpos"), int(L), _ptr(beacons, torch.float32, "beacons", shape.n_beacon == 0),
        _ptr(recents, torch.float32, "recents"), int(t), int(b_kv),
        _ptr(buf, torch.float32, "buf", True), _ptr(count, torch.int32, "count", True),
        _ptr(score_out, torch.float32, "score_out", True),
        _ptr(kept_out, torch.int32, "kept_out", True), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)))


def evict_noalloc(shape, K, V, kpos, L, beacons, recents, t, b_kv, buf=None, count=None,
                  score_out=None, kept_out=None, stream=None):
    lib = load_library()
    _need_score_inputs(shape, K, kpos, beacons, recents)
    _need(V, shape.n_units * shape.l_cap * shape.d_head, "V")
    _need(buf, shape.n_units * shape.group * shape.buf_cap * shape.d_head, "buf")
    _need(count, shape.n_units * shape.group, "count")
    _need(score_out, shape.n_units * shape.l_cap, "score_out")
    _need(kept_out, shape.n_units * int(b_kv), "kept_out")
    _check(lib.bkv_evict_noalloc(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"), _bits(V, "V"),
        _ptr(kpos, torch.int32, "kpos"), int(L), _ptr(beacons, torch.float32, "beacons", shape.n_beacon == 0),
        _ptr(recents, torch.float32, "recents"), int(t), int(b_kv),
        _ptr(buf, torch.float32, "buf", True), _ptr(count, torch.int32, "count", True),
        _ptr(score_out, torch.float32, "score_out", True),
        _ptr(kept_out, torch.int32, "kept_out", True), _stream(stream)))


def evict_lse(shape, K, V, kpos, L, beacons, recents, t, lse_in, lse_from, b_kv, buf=None,
              count=None, score_out=None, kept_out=None, ws=None, stream=None):
    lib = load_library()
    _need_score_inputs(shape, K, kpos, beacons, recents)
    _need(V, shape.n_units * shape.l_cap * shape.d_head, "V")
    _need(lse_in, shape.n_units * shape.group * 32, "lse_in")
    _need(buf, shape.n_units * shape.group * shape.buf_cap * shape.d_head, "buf")
    _need(count, shape.n_units * shape.group, "count")
    _need(score_out, shape.n_units * shape.l_cap, "score_out")
    _need(kept_out, shape.n_units * int(b_kv), "kept_out")
    if ws is None:
        ws = alloc_workspace(shape, L, b_kv, K.device)
    _check(lib.bkv_evict_lse(
        ctypes.byref(shape.dims()), ctypes.byref(shape.policy()), _bits(K, "K"), _bits(V, "V"),
        _ptr(kpos, torch.int32, "kpos"), int(L), _ptr(beacons, torch.float32, "beacons", shape.n_beacon == 0),
        _ptr(recents, torch.float32, "recents"), int(t), _ptr(lse_in, torch.float32, "lse_in"),
        int(lse_from), int(b_kv), _ptr(buf, torch.float32, "buf", True),
        _ptr(count, torch.int32, "count", True), _ptr(score_out, torch.float32, "score_out", True),
        _ptr(kept_out, torch.int32, "kept_out", True), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)))
