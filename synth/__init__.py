"""Seeded synthetic inputs shared by the oracle checks, the tests and the bench.

This package holds no arithmetic of the eviction method: it only draws
random numbers and converts them to the storage types (bfloat16 keys and
values via torch's round-to-nearest-even cast, float32 queries).  Both the
float64 oracle and the HIP library consume what it returns.

Two generators share one recipe.  ``unit_inputs`` gives every tensor of
every unit its own numpy stream,
``default_rng(SeedSequence([seed, workload_id, kind, index]))``, so small
cases are reproducible on any host.  ``device_inputs`` draws whole
full-size workloads on the device with torch's seeded generator (thousands
of units in well under a second); sampled units of such a workload are
copied to the host for the oracle.

Value structure (a stand-in for the reasoning traces the pages measure on;
see the design notes for the recipe and its reasons):

* keys, values ~ N(0, 1), optionally with a few outlier channels scaled up;
* a pre-RoPE query at nominal position p is *local* with probability
  1 - pi_g -- a copy of a key near p plus N(0, 0.3^2) noise -- or *global*
  with probability pi_g -- 8 times one of the head's cluster centres (unit
  vectors) plus the same noise;
* buffer queries take p uniform over [P, L - 16); recent query i takes
  p = its own position.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch

KIND_K, KIND_V, KIND_CENTRES, KIND_BUF, KIND_RECENT, KIND_OUTLIER, KIND_NEWQ = range(1, 8)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id, part of every seed
    layers: int
    batch: int
    h_kv: int
    group: int          # query heads per KV head
    d_head: int
    L: int              # live slots when eviction fires
    b_kv: int           # slots kept
    prefix: int
    theta: float
    recent_tok: int = 16
    n_beacon: int = 16
    n_recent_q: int = 16
    buf_cap: int = 32
    pi_global: float = 0.25
    n_centres: int = 3
    outlier_channels: int = 0
    outlier_scale: float = 6.0
    seed: int = 0
    l_cap: int = 0      # slot stride; 0 means L
    stream_steps: int = 0  # decode steps of a streaming run (L is then B_max)

    @property
    def n_units(self):
        return self.layers * self.batch * self.h_kv

    @property
    def n_qheads(self):
        return self.n_units * self.group

    @property
    def cap(self):
        return self.l_cap or self.L

    def layer_of(self, u):
        return u // (self.batch * self.h_kv)


def _tiny():
    return Workload("tiny", 1, layers=1, batch=1, h_kv=2, group=2, d_head=64,
                    L=256, b_kv=128, prefix=8, theta=1e4)


def _qwen3_4b_layer():
    return Workload("qwen3-4b-1layer-b1", 2, layers=1, batch=1, h_kv=8, group=4,
                    d_head=128, L=2176, b_kv=2048, prefix=256, theta=1e6,
                    pi_global=0.10, n_centres=6, outlier_channels=4)


def _qwen3_4b_full(b_kv):
    return Workload(f"qwen3-4b-36L-b16-B{b_kv}", 3, layers=36, batch=16, h_kv=8,
                    group=4, d_head=128, L=b_kv + 128, b_kv=b_kv, prefix=8,
                    theta=1e6)


def _r1_qwen_7b():
    return Workload("r1-distill-qwen-7b-28L-b32-B4096", 4, layers=28, batch=32,
                    h_kv=4, group=7, d_head=128, L=4224, b_kv=4096, prefix=512,
                    theta=1e6)


def _qwen3_14b_stream():
    # Streaming run: prompt of `prefix` tokens, then decode steps; eviction
    # fires when the cache reaches L = B_max = b_kv + 128.
    return Workload("qwen3-14b-40L-b16-stream", 5, layers=40, batch=16, h_kv=8, group=5,
                    d_head=128, L=4224, b_kv=4096, prefix=256, theta=1e6,
                    stream_steps=32768)


def _stream_small():
    return Workload("stream-small", 6, layers=1, batch=2, h_kv=2, group=5, d_head=128,
                    L=384, b_kv=256, prefix=32, theta=1e6, stream_steps=640)


WORKLOADS = {
    "tiny": _tiny(),
    "qwen3_4b_layer": _qwen3_4b_layer(),
    "qwen3_4b_full_b128": _qwen3_4b_full(128),
    "qwen3_4b_full_b512": _qwen3_4b_full(512),
    "qwen3_4b_full_b1024": _qwen3_4b_full(1024),
    "qwen3_4b_full_b2048": _qwen3_4b_full(2048),
    "qwen3_4b_full_b4096": _qwen3_4b_full(4096),
    "r1_qwen_7b": _r1_qwen_7b(),
    "qwen3_14b_stream": _qwen3_14b_stream(),
    "stream_small": _stream_small(),
}


def shrink(w, **kw):
    """A copy of a workload with some fields replaced (smaller test cases)."""
    return replace(w, **kw)


def _rng(w, kind, index):
    return np.random.default_rng(np.random.SeedSequence([w.seed, w.wid, kind, index]))


def to_bf16_values(x):
    """float32 -> bfloat16 (torch's RNE cast) -> float32 holding the bf16 values."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def outlier_channels(w, layer):
    if w.outlier_channels == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(w, KIND_OUTLIER, layer)
    return np.sort(r.choice(w.d_head, size=w.outlier_channels, replace=False))


def unit_keys_values(w, u):
    """Keys and values of unit u, [L, d] float32 holding bfloat16 values."""
    k = _rng(w, KIND_K, u).standard_normal((w.L, w.d_head), dtype=np.float32)
    ch = outlier_channels(w, w.layer_of(u))
    if ch.size:
        k[:, ch] *= np.float32(w.outlier_scale)
    v = _rng(w, KIND_V, u).standard_normal((w.L, w.d_head), dtype=np.float32)
    return to_bf16_values(k), to_bf16_values(v)


def _mixture(w, r, keys, centres, positions):
    """Pre-RoPE queries at the given nominal positions (float32)."""
    n = len(positions)
    q = np.empty((n, w.d_head), dtype=np.float32)
    is_global = r.random(n) < w.pi_global
    which = r.integers(0, w.n_centres, size=n)
    noise = r.standard_normal((n, w.d_head), dtype=np.float32) * np.float32(0.3)
    for i, p in enumerate(positions):
        if is_global[i]:
            q[i] = 8.0 * centres[which[i]]
        else:
            lo = max(0, int(p) - 31)
            j = int(r.integers(lo, int(p) + 1))
            q[i] = keys[min(j, keys.shape[0] - 1)]
    return q + noise


def head_centres(w, qh):
    c = _rng(w, KIND_CENTRES, qh).standard_normal((w.n_centres, w.d_head))
    return (c / np.linalg.norm(c, axis=1, keepdims=True)).astype(np.float32)


def unit_queries(w, u, keys):
    """Buffer rows [g, buf_cap, d] and recent queries [g, n_recent_q, d].

    The buffer is full (buf_cap rows); the last n_recent_q slots hold the
    most recent tokens, whose positions are their slots.
    """
    g, d = w.group, w.d_head
    buf = np.empty((g, w.buf_cap, d), dtype=np.float32)
    rec = np.empty((g, w.n_recent_q, d), dtype=np.float32)
    hi = max(w.prefix + 1, w.L - 16)
    for h in range(g):
        qh = u * g + h
        cen = head_centres(w, qh)
        rb = _rng(w, KIND_BUF, qh)
        pos = rb.integers(w.prefix, hi, size=w.buf_cap)
        buf[h] = _mixture(w, rb, keys, cen, pos)
        rr = _rng(w, KIND_RECENT, qh)
        rpos = np.arange(w.L - w.n_recent_q, w.L)
        rec[h] = _mixture(w, rr, keys, cen, rpos)
    return buf, rec


def new_queries(w, u, keys, n_new=1, step=0):
    """n_new further pre-RoPE queries per head of unit u, [g, n_new, d]."""
    g = w.group
    out = np.empty((g, n_new, w.d_head), dtype=np.float32)
    for h in range(g):
        qh = u * g + h
        r = np.random.default_rng(np.random.SeedSequence(
            [w.seed, w.wid, KIND_NEWQ, qh, step]))
        pos = np.full(n_new, w.L - 1)
        out[h] = _mixture(w, r, keys, head_centres(w, qh), pos)
    return out


def unit_inputs(w, u):
    """Everything one unit needs for a single eviction event at t = L.

    Returns dict(keys, values [L, d] float32 (bf16 values), kpos [L] int32,
    buf [g, buf_cap, d] float32, recents [g, n_recent_q, d] float32, t).
    The beacons are rows 0..n_beacon-1 of ``buf`` after it is compressed.
    """
    k, v = unit_keys_values(w, u)
    buf, rec = unit_queries(w, u, k)
    return {"keys": k, "values": v, "kpos": np.arange(w.L, dtype=np.int32),
            "buf": buf, "recents": rec, "t": w.L}


def workload_inputs(w, units=None):
    """Stack unit_inputs over ``units`` (default: all), host arrays."""
    units = range(w.n_units) if units is None else units
    parts = [unit_inputs(w, u) for u in units]
    out = {key: np.stack([p[key] for p in parts]) for key in
           ("keys", "values", "kpos", "buf", "recents")}
    out["t"] = w.L
    return out


# ---------------------------------------------------------------------------
# Bulk generation on the device (full-size workloads).
#
# Same recipe as above, drawn with torch's seeded device generator in chunks
# of units so that a 4608-unit cache is generated in well under a second.
# The numpy per-unit streams and this generator produce different numbers;
# each test or bench run uses one of them for both sides.  Sampled units of
# a device-generated workload are copied to the host for the oracle.


def _dev_gen(w, kind, chunk, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([w.seed, w.wid, kind, chunk]).generate_state(1)[0]))
    return g


def device_inputs(w, device="cuda", chunk_units=256, l_cap=None):
    """Whole-workload inputs as device tensors.

    Returns dict(keys, values: bf16 [U, l_cap, d]; kpos: int32 [U, l_cap];
    buf: fp32 [U*g, buf_cap, d]; recents: fp32 [U*g, n_recent_q, d]; t).
    Slots at and beyond L (when l_cap > L) hold zeros.
    """
    U, g, d, L = w.n_units, w.group, w.d_head, w.L
    cap = l_cap or w.cap
    dev = torch.device(device)
    keys = torch.zeros((U, cap, d), dtype=torch.bfloat16, device=dev)
    vals = torch.zeros((U, cap, d), dtype=torch.bfloat16, device=dev)
    kpos = torch.zeros((U, cap), dtype=torch.int32, device=dev)
    kpos[:, :L] = torch.arange(L, dtype=torch.int32, device=dev)
    buf = torch.empty((U * g, w.buf_cap, d), dtype=torch.float32, device=dev)
    rec = torch.empty((U * g, w.n_recent_q, d), dtype=torch.float32, device=dev)
    hi = max(w.prefix + 1, L - 16)
    for c0 in range(0, U, chunk_units):
        c1 = min(U, c0 + chunk_units)
        n = c1 - c0
        ci = c0 // chunk_units
        gk = _dev_gen(w, KIND_K, ci, dev)
        k = torch.randn((n, L, d), generator=gk, device=dev, dtype=torch.float32)
        if w.outlier_channels:
            layers = torch.tensor([w.layer_of(u) for u in range(c0, c1)])
            for layer in torch.unique(layers).tolist():
                rows = (layers == layer).nonzero().flatten().to(dev)
                ch = torch.from_numpy(outlier_channels(w, layer)).to(dev)
                sub = k[rows]
                sub[:, :, ch] *= w.outlier_scale
                k[rows] = sub
        kb = k.to(torch.bfloat16)
        keys[c0:c1, :L] = kb
        gv = _dev_gen(w, KIND_V, ci, dev)
        vals[c0:c1, :L] = torch.randn((n, L, d), generator=gv, device=dev,
                                      dtype=torch.float32).to(torch.bfloat16)
        kf = kb.to(torch.float32)  # local queries copy the stored (bf16) keys
        gq = _dev_gen(w, KIND_BUF, ci, dev)
        nq = n * g
        cen = torch.randn((nq, w.n_centres, d), generator=gq, device=dev)
        cen = cen / cen.norm(dim=-1, keepdim=True)
        unit_of = torch.arange(nq, device=dev) // g

        def mixture(pos):
            m = pos.shape[1]
            is_g = torch.rand((nq, m), generator=gq, device=dev) < w.pi_global
            which = torch.randint(0, w.n_centres, (nq, m), generator=gq, device=dev)
            lo = torch.clamp(pos - 31, min=0)
            j = lo + (torch.rand((nq, m), generator=gq, device=dev) *
                      (pos - lo + 1).to(torch.float32)).to(torch.int64)
            j = torch.minimum(j, pos)
            local = kf[unit_of[:, None], j]
            glob = 8.0 * torch.gather(cen, 1, which[..., None].expand(-1, -1, d))
            q = torch.where(is_g[..., None], glob, local)
            return q + 0.3 * torch.randn((nq, m, d), generator=gq, device=dev)

        pos_b = torch.randint(w.prefix, hi, (nq, w.buf_cap), generator=gq, device=dev)
        buf[c0 * g:c1 * g] = mixture(pos_b)
        pos_r = torch.arange(L - w.n_recent_q, L, device=dev).expand(nq, -1)
        rec[c0 * g:c1 * g] = mixture(pos_r)
    return {"keys": keys, "values": vals, "kpos": kpos, "buf": buf, "recents": rec, "t": L}


def to_device(inp, device="cuda", l_cap=None):
    """Move host unit inputs (workload_inputs) to device tensors in library layout."""
    dev = torch.device(device)
    k = inp["keys"]
    U, L, d = k.shape
    cap = l_cap or L
    keys = torch.zeros((U, cap, d), dtype=torch.bfloat16, device=dev)
    vals = torch.zeros((U, cap, d), dtype=torch.bfloat16, device=dev)
    kpos = torch.zeros((U, cap), dtype=torch.int32, device=dev)
    keys[:, :L] = torch.from_numpy(k).to(dev).to(torch.bfloat16)
    vals[:, :L] = torch.from_numpy(inp["values"]).to(dev).to(torch.bfloat16)
    kpos[:, :L] = torch.from_numpy(inp["kpos"]).to(dev)
    g = inp["buf"].shape[1]
    buf = torch.from_numpy(inp["buf"].reshape(U * g, *inp["buf"].shape[2:])).to(dev)
    rec = torch.from_numpy(inp["recents"].reshape(U * g, *inp["recents"].shape[2:])).to(dev)
    return {"keys": keys, "values": vals, "kpos": kpos, "buf": buf.contiguous(),
            "recents": rec.contiguous(), "t": inp["t"]}


# ---------------------------------------------------------------------------
# Streaming inputs (decode-time runs), generated on the device in chunks of
# steps.  A prompt of `prefix` tokens, then one key, value (bf16) and
# pre-RoPE query per query head (fp32) per unit and step.  Queries follow the
# same mixture: local queries copy one of the 32 most recently generated keys
# of their unit (+ noise), global ones a cluster centre of their head.

KIND_SPRE, KIND_SSTEP = 8, 9


class StreamInputs:
    """Seeded per-step inputs of a streaming workload on ``device``.

    prompt() -> keys, values [U, P, d] bf16; queries [U*g, P, d] fp32.
    chunk(c, n) -> keys, values [n, U, d] bf16; queries [n, U*g, d] fp32 for
    decode steps c*n .. c*n + n - 1 (chunks must be requested in order).
    """

    def __init__(self, w, device="cuda"):
        self.w = w
        self.dev = torch.device(device)
        U, g, d = w.n_units, w.group, w.d_head
        gc = _dev_gen(w, KIND_CENTRES, 0, self.dev)
        cen = torch.randn((U * g, w.n_centres, d), generator=gc, device=self.dev)
        self.centres = cen / cen.norm(dim=-1, keepdim=True)
        self.window = None  # [U, 32, d] fp32: the 32 most recent keys of each unit
        self.next_chunk = 0

    def _queries(self, gen, n_steps, keys_at):
        """keys_at(j): [n_steps, U*g, d] fp32, the key j (0..31) steps back from
        each step's own token for each query head's unit."""
        w = self.w
        U, g, d = w.n_units, w.group, w.d_head
        nq = U * g
        is_g = torch.rand((n_steps, nq), generator=gen, device=self.dev) < w.pi_global
        which = torch.randint(0, w.n_centres, (n_steps, nq), generator=gen, device=self.dev)
        j = torch.randint(0, 32, (n_steps, nq), generator=gen, device=self.dev)
        local = keys_at(j)
        glob = 8.0 * self.centres[torch.arange(nq, device=self.dev)[None, :], which]
        q = torch.where(is_g[..., None], glob, local)
        return q + 0.3 * torch.randn((n_steps, nq, d), generator=gen, device=self.dev)

    def _unit_of(self):
        return torch.arange(self.w.n_units * self.w.group, device=self.dev) // self.w.group

    def prompt(self):
        w = self.w
        U, g, d, P = w.n_units, w.group, w.d_head, w.prefix
        gen = _dev_gen(w, KIND_SPRE, 0, self.dev)
        k = torch.randn((U, P, d), generator=gen, device=self.dev).to(torch.bfloat16)
        v = torch.randn((U, P, d), generator=gen, device=self.dev).to(torch.bfloat16)
        kf = k.to(torch.float32)
        unit_of = self._unit_of()
        steps = torch.arange(P, device=self.dev)[:, None]

        def keys_at(j):  # prompt query i sees keys max(0, i - 31) .. i
            return kf[unit_of[None, :], torch.clamp(steps - j, min=0)]

        q = self._queries(gen, P, keys_at).permute(1, 0, 2).contiguous()  # [U*g, P, d]
        last = torch.clamp(torch.arange(P - 32, P, device=self.dev), min=0)
        self.window = kf[:, last].contiguous()                            # last 32 keys
        return k, v, q

    def chunk(self, c, n):
        if c != self.next_chunk:
            raise ValueError("stream chunks must be generated in order")
        self.next_chunk += 1
        w = self.w
        U, d = w.n_units, w.d_head
        gen = _dev_gen(w, KIND_SSTEP, c, self.dev)
        k = torch.randn((n, U, d), generator=gen, device=self.dev).to(torch.bfloat16)
        v = torch.randn((n, U, d), generator=gen, device=self.dev).to(torch.bfloat16)
        # keys of step s: allk[32 + s] is its own, allk[32 + s - j] is j steps back
        allk = torch.cat([self.window.permute(1, 0, 2), k.to(torch.float32)], dim=0)  # [32+n, U, d]
        unit_of = self._unit_of()
        steps = torch.arange(n, device=self.dev)[:, None]

        def keys_at(j):
            return allk[32 + steps - j, unit_of[None, :]]

        q = self._queries(gen, n, keys_at)
        self.window = allk[-32:].permute(1, 0, 2).contiguous()
        return k, v, q
