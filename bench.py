#!/usr/bin/env python3
"""Benchmark of the BeaconKV eviction step on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input, every stage through the C ABI on one stream:

  1. bkv_fps_update      append this step's pre-RoPE query and Continual-FPS
                         compress every head's buffer 32 -> 16     (a1, a2)
  2. bkv_score           RoPE-align beacons/recents, Q_obs . K^T on bf16
                         MFMA, row softmax, max over the GQA group (a4-a7)
  3. bkv_select          forced prefix/recent slots + Top-K      (a8)
  4. bkv_compact         in-place gather of K, V, positions      (a9)
  5. bkv_fps_update      merge the recent queries and compress 32 -> 16 (a10)

The timed step is stage 1 plus one bkv_evict (stages 2-5); a second loop
runs the stages as separate calls with HIP events between them on the
launch stream, for the per-stage breakdown and the roofline of the dominant
kernel.  Before each step the cache, positions and buffers are restored from
pristine copies and a 512 MB buffer is read to leave the caches cold and
clean; both happen outside the timed step.  Each timed step is bracketed by
torch.cuda.synchronize() on both sides.  The default line also carries, under
"variants", the same step with its softmax denominators taken from decode
attention (--fused-decode alone prints that line); --workload
qwen3_14b_stream runs the decode-time streaming policy and --prefill-fps N
the prefill FPS over N-row prompts.

Prints ONE JSON line (stdout).  Diagnostics go to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
# Worker processes of the CPU oracle baseline: the measurement host gives one
# GPU a share of 16 CPU cores, whatever the affinity mask shows.
CPU_WORKER_CAP = 16
TOL = 2e-3                      # acceptance tolerance (scores, tie bands, FPS margins)
METRIC = "KV-head·key-tokens scored/s + evictions/s at Qwen3-4B shape; % of HBM peak"
DEFAULT_WORKLOAD = "qwen3_4b_full_b2048"
KERNEL_SOURCES = {
    "fps_compress": "fps.hip", "score": "score.hip", "select": "select.hip",
    "compact": "compact.hip", "fps_merge": "fps.hip", "score_lse": "score.hip",
    "select_compact": ("select.hip", "select_wave.h", "compact.hip"),
    "fps_long_prefill": "fps.hip",
}


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--bkv", type=int, choices=(128, 512, 1024, 2048, 4096), default=0,
                   help="the Qwen3-4B 36-layer x batch-16 step at this B_KV (sets --workload)")
    p.add_argument("--seed", type=int, default=0,
                   help="master seed of the synthetic inputs (0: the workloads' own)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample (0 disables)")
    p.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    p.add_argument("--aggregate", choices=("max", "mean"), default="max",
                   help="pooling of the attention weights: the method's max, or the mean of "
                        "the aggregation ablation")
    p.add_argument("--observe", choices=("beacons", "recent32"), default="beacons",
                   help="observation set: the method's 16 beacons + 16 recent queries, or the "
                        "baselines' 32 most recent queries (no beacons, no FPS, 32 recent "
                        "tokens kept)")
    p.add_argument("--compaction", choices=("sorted", "unsorted"), default="sorted",
                   help="position-ordered compaction (the method), or the unsorted variant "
                        "that fills the evicted slots with the kept tokens past B_KV")
    p.add_argument("--beacon-policy", choices=("fps", "initial"), default="fps",
                   help="streaming workloads: the method's Continual FPS, or the Initial+Recent "
                        "comparison (the first 16 generated queries as fixed references)")
    p.add_argument("--prefill-fps", type=int, default=0, metavar="N",
                   help="time the prefill FPS instead: every query head of the workload "
                        "compresses an N-row prompt buffer to 16 (N up to 8192)")
    p.add_argument("--fused-decode", action="store_true",
                   help="the eviction with the softmax denominators gathered by decode "
                        "attention (bkv_decode_attend at the beacon fix and at each recent "
                        "query's step, then bkv_score_lse: one key read); the extra cost of the "
                        "beacon rows in decode attention is timed and charged to the step")
    p.add_argument("--no-variants", dest="variants", action="store_false",
                   help="skip the fused-decode variant that the default run appends to its line")
    p.add_argument("--stream-steps", type=int, default=0,
                   help="decode steps of a streaming workload (0: the workload's own)")
    return p.parse_args()


def moved_token_count(kept, b_kv, unsorted):
    """Tokens a compaction moves, from the ascending keep sets [U, b_kv].

    In position order the k-th kept slot moves unless it already is slot k;
    filling the holes instead moves only the kept slots at or past b_kv.
    """
    import numpy as np

    kept = np.asarray(kept).reshape(-1, b_kv)
    if unsorted:
        return int(np.count_nonzero(kept >= b_kv))
    return int(np.count_nonzero(kept != np.arange(b_kv)[None, :]))


def stage_bytes(w, n_mv_total):
    """Algorithmic HBM bytes per launch of each stage (what the method must move)."""
    U, g, d, L, B = w.n_units, w.group, w.d_head, w.L, w.b_kv
    nq = U * g
    P, R = w.prefix, w.recent_tok
    return {
        # read 31 buffer rows + the new query, write 16 rows and the count
        "fps_compress": nq * ((31 + 1 + 16) * d * 4 + 8),
        # K rows, 32 observation rows per head, the recent positions, score out
        "score": U * (L * d * 2 + g * 32 * d * 4 + w.n_recent_q * 4 + L * 4),
        # middle scores in, kept list out
        "select": U * ((L - P - R) * 4 + B * 4),
        # moved tokens: K and V row read + write, position read + write; kept in
        "compact": n_mv_total * (4 * d * 2 + 8) + U * B * 4,
        # 16 beacons + 16 recents in, 16 rows out, count
        "fps_merge": nq * ((16 + 16 + 16) * d * 4 + 8),
        # the two in one launch
        "select_compact": (U * ((L - P - R) * 4 + B * 4) +
                           n_mv_total * (4 * d * 2 + 8) + U * B * 4),
    }


def source_digest(names):
    """First 16 hex digits of the SHA-256 of the named source(s), concatenated."""
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        with open(os.path.join(ROOT, "reasoning_model_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from a committed counter summary, if it still
    matches the kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seconds):
    """The float64 oracle on a bounded sample of units, over the host cores.

    Runs before the GPU is touched (the workers are forked from this
    process).  Each worker generates a few units with the per-unit numpy
    generator (same recipe and shapes as the GPU run), waits at a barrier,
    then runs the oracle's full step over its share of the sample, cycling
    through its units.  Throughput = sampled units x L over the wall time
    from the barrier to the last worker's finish.
    """
    if seconds <= 0:
        return None
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, CPU_WORKER_CAP)
    unit0 = _host_unit(w, 0)
    _oracle_step(w, unit0)  # warm imports and caches
    reps = []
    for _ in range(3):
        t0 = time.perf_counter()
        _oracle_step(w, unit0)
        reps.append(time.perf_counter() - t0)
    one = min(reps)
    per_worker = max(1, int(seconds / max(one, 1e-3)))
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(cores + 1)
    q = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(w, i, per_worker, barrier, q))
             for i in range(cores)]
    for p in procs:
        p.start()
    barrier.wait()
    t0 = time.perf_counter()
    ends = [q.get() for _ in procs]
    dt = max(ends) - t0
    for p in procs:
        p.join()
    n = per_worker * cores
    return {"value": round(n * w.L / dt, 1), "unit": "KV-head·key-tokens/s", "cores": cores,
            "kind": "oracle",
            "value_1core": round(w.L / one, 1),
            "affinity_cores": affinity,
            "cores_cap": (f"{CPU_WORKER_CAP} worker processes at most: the CPU share of one GPU "
                          f"on the measurement host" if affinity > CPU_WORKER_CAP else None),
            "cpu_model": cpu_model(),
            "sample": (f"{n} unit-steps of {w.name} ({cores} workers x {per_worker}, each "
                       f"cycling over up to 8 host-generated units of the same recipe); full "
                       f"step per unit: FPS compress of {w.group} heads, score, select, compact, "
                       f"merge FPS; float64 numpy, one BLAS thread per worker, {dt:.1f} s wall")}


def parity_sample(w, units, K0, V0, P0, buf0, newq, rec, beacons, K, V, kpos, buf, score, kept,
                  window, aggregate, unsorted):
    """Compare sampled units of one eviction step with the oracle (see main)."""
    import numpy as np
    import torch

    import oracle
    g, d, L, B = w.group, w.d_head, w.L, w.b_kv
    worst, n_band, n_out, cmp_ok, fps_checked, fps_ok = 0.0, 0, 0, True, 0, True
    rows_ok = True
    for u in units:
        rows = rec[u * g:(u + 1) * g].cpu().numpy()
        ref = oracle.evict.evict_unit(
            K0[u].float().cpu().numpy(), V0[u].float().cpu().numpy(), P0[u].cpu().numpy(), L,
            beacons[u * g:(u + 1) * g], rows, L, B, w.prefix, w.recent_tok, w.theta,
            merge=not window, aggregate=aggregate, unsorted=unsorted)
        s_gpu, s_ref = score[u].cpu().numpy().astype(np.float64), ref["score"]
        worst = max(worst, float(np.max(np.abs(s_gpu - s_ref) / (s_ref + 1e-30))))
        kg = kept[u].cpu().numpy()
        diff = set(kg.tolist()) ^ set(ref["kept"].tolist())
        mid = np.sort(s_ref[w.prefix:L - w.recent_tok])[::-1]
        s_star = mid[B - w.prefix - w.recent_tok - 1]
        for j in diff:
            if abs(s_ref[j] - s_star) <= TOL * s_star:
                n_band += 1
            else:
                n_out += 1
        # The compacted cache holds the inputs at the GPU's kept slots.
        if unsorted:
            src = oracle.compact.fill_holes(np.arange(L), np.arange(L), np.arange(L), kg, B)[0]
        else:
            src = kg
        src = torch.as_tensor(np.asarray(src, np.int64), device=K0.device)
        cmp_ok &= bool(torch.equal(K[u, :B].cpu(), K0[u, src].cpu()) and
                       torch.equal(V[u, :B].cpu(), V0[u, src].cpu()) and
                       torch.equal(kpos[u, :B].cpu(), P0[u, src].cpu()))
        if window:
            continue
        for h in range(g):
            qh = u * g + h
            # FPS compress of the 31 buffered rows plus this step's query, then
            # the merge of the beacons the GPU scored with and the recents.
            full = np.concatenate([buf0[qh, :31].cpu().numpy(), newq[qh].cpu().numpy()])
            merged = np.concatenate([beacons[qh], rows[h]])
            for cand, got in ((full, beacons[qh]), (merged, buf[qh, :16].cpu().numpy())):
                # Every kept row is a distinct candidate row, in slot order.
                idx = [int(np.nonzero((cand == r).all(axis=1))[0][0])
                       if (cand == r).all(axis=1).any() else -1 for r in got]
                rows_ok &= min(idx) >= 0 and all(a < b for a, b in zip(idx, idx[1:]))
                if min(oracle.fps.fps_margins(cand, 16)) > TOL:
                    fps_checked += 1
                    fps_ok &= bool(np.array_equal(got, cand[oracle.fps.fps(cand, 16)[1]]))
    ok = worst <= TOL and n_out == 0 and cmp_ok and fps_ok and rows_ok
    return {"path": "the timed calls (fps_update, then bkv_evict)", "units": units,
            "max_score_rel_err": worst, "kept_diff_in_tie_band": n_band,
            "kept_diff_outside_tie_band": n_out, "compaction_exact": cmp_ok,
            "fps_rows_are_distinct_inputs": bool(rows_ok), "fps_sets_checked": fps_checked,
            "fps_sets_equal": fps_ok, "ok": bool(ok)}


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_worker(w, i, n_steps, barrier, q):
    _one_blas_thread()
    units = [_host_unit(w, (i * 8 + k) % w.n_units) for k in range(min(8, n_steps))]
    barrier.wait()
    for k in range(n_steps):
        _oracle_step(w, units[k % len(units)])
    q.put(time.perf_counter())


def _host_unit(w, u):
    import synth
    x = synth.unit_inputs(w, u)
    return {k: x[k] for k in ("keys", "values", "kpos", "buf", "recents")}


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_step(w, unit):
    import numpy as np

    import oracle
    if w.n_beacon == 0:  # the 32-query window: no FPS, no merge
        oracle.evict.evict_unit(unit["keys"], unit["values"], unit["kpos"], w.L,
                                np.zeros((w.group, 0, w.d_head)), unit["recents"], w.L, w.b_kv,
                                w.prefix, w.recent_tok, w.theta, merge=False)
        return True
    heads = []
    for h in range(w.group):
        _, keep = oracle.fps.fps(unit["buf"][h], 16)
        heads.append(unit["buf"][h][keep])
    beacons = np.stack(heads)
    oracle.evict.evict_unit(unit["keys"], unit["values"], unit["kpos"], w.L, beacons,
                            unit["recents"], w.L, w.b_kv, w.prefix, w.recent_tok, w.theta)
    return True


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        eprint("bench.py measures one GPU only: this eviction-step library runs on a single "
               "MI355X and has no multi-GPU path (every unit is independent; see the design "
               "notes for how it would shard). Run with --gpus 1.")
        sys.exit(2)

    import numpy as np

    import synth

    if args.bkv:
        args.workload = f"qwen3_4b_full_b{args.bkv}"
    if args.workload not in synth.WORKLOADS:
        eprint(f"unknown workload {args.workload!r}; known: {', '.join(synth.WORKLOADS)}")
        sys.exit(2)
    w = synth.WORKLOADS[args.workload]
    if args.seed:
        w = synth.shrink(w, seed=args.seed)
    if args.prefill_fps:
        prefill_fps_main(args, w)
        return
    if w.stream_steps:
        if args.fused_decode:
            eprint("--fused-decode times single eviction events; the streaming run's decode-time "
                   "denominators are exercised by the tests (Stream(fused_decode=True))")
            sys.exit(2)
        stream_main(args, w)
        return
    window = args.observe == "recent32"
    if args.fused_decode:
        print(json.dumps(fused_main(args, w)), flush=True)
        return
    if window:
        w = synth.shrink(w, n_beacon=0, n_recent_q=32, recent_tok=32)
    cpu = None
    if args.cpu_seconds > 0:
        eprint(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s of CPU work per core)")
        cpu = cpu_baseline(w, args.cpu_seconds)
        eprint(f"[bench] cpu baseline: {cpu}")

    import torch

    from reasoning_model_kv_amd import bkv

    bkv.load_library()
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    U, g, d, L, B = w.n_units, w.group, w.d_head, w.L, w.b_kv
    nq = U * g
    eprint(f"[bench] workload {w.name}: U={U} g={g} d={d} L={L} B_KV={B} P={w.prefix}")

    t0 = time.perf_counter()
    inp = synth.device_inputs(w, dev)
    torch.cuda.synchronize()
    eprint(f"[bench] inputs generated in {time.perf_counter() - t0:.2f} s")
    K0, V0, P0 = inp["keys"], inp["values"], inp["kpos"]
    buf0, rec = inp["buf"], inp["recents"]
    newq = buf0[:, 31:32].clone()          # this step's query (appended at count 31)
    K, V, kpos = torch.empty_like(K0), torch.empty_like(V0), torch.empty_like(P0)
    buf = torch.empty_like(buf0)
    count = torch.empty((nq,), dtype=torch.int32, device=dev)
    score = torch.empty((U, L), dtype=torch.float32, device=dev)
    kept = torch.empty((U, B), dtype=torch.int32, device=dev)
    # Cache flush before each timed step: a read-only pass over 512 MB (twice
    # the 256 MB last-level cache), so that the step starts with cold caches
    # holding no dirty lines of the untimed state restore (their write-back
    # would otherwise land in the first timed kernel).
    scrub = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    shape = bkv.Shape(U, g, d, L, w.prefix, w.theta, recent_tok=w.recent_tok,
                      n_beacon=w.n_beacon, n_recent_q=w.n_recent_q, aggregate=args.aggregate,
                      unsorted=args.compaction == "unsorted")
    ws = bkv.alloc_workspace(shape, L, 0, dev)
    stream = torch.cuda.current_stream()

    def restore():
        K.copy_(K0)
        V.copy_(V0)
        kpos.copy_(P0)
        buf.copy_(buf0)
        count.fill_(31)
        scrub.sum()

    # The step as a caller runs it: the decode-time FPS compress, then one
    # bkv_evict (score, select, compact and the buffer merge).
    ws_e = bkv.alloc_workspace(shape, L, B, dev)
    eva = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def step_evict():
        eva[0].record(stream)
        if not window:
            bkv.fps_update(shape, buf, count, newq, trigger=32, m=16)
        eva[1].record(stream)
        if window:
            bkv.evict(shape, K, V, kpos, L, None, rec, L, B, score_out=score, kept_out=kept,
                      ws=ws_e)
        else:
            bkv.evict(shape, K, V, kpos, L, buf, rec, L, B, buf=buf, count=count,
                      score_out=score, kept_out=kept, ws=ws_e)
        eva[2].record(stream)

    # The same work as separate calls, with events between them, for the
    # per-stage breakdown and the roofline of the dominant kernel: the
    # kernels bkv_evict runs, one call each.
    sel = ["select", "compact"]
    names = (["score"] + sel if window else ["fps_compress", "score"] + sel + ["fps_merge"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]

    def step():
        calls = {
            "fps_compress": lambda: bkv.fps_update(shape, buf, count, newq, trigger=32, m=16),
            "score": lambda: bkv.score(shape, K, kpos, L, None if window else buf, rec, L,
                                       score, ws=ws),
            "select": lambda: bkv.select(shape, score, L, B, kept),
            "compact": lambda: (bkv.compact_unsorted(shape, K, V, kpos, L, kept, B)
                                if shape.unsorted else bkv.compact(shape, K, V, kpos, L, kept, B)),
            "fps_merge": lambda: bkv.fps_update(shape, buf, count, rec, trigger=32, m=16),
        }
        ev[0].record(stream)
        for j, n in enumerate(names):
            calls[n]()
            ev[j + 1].record(stream)

    for i in range(args.warmup):
        for fn in (step_evict, step):
            restore()
            torch.cuda.synchronize()
            fn()
            torch.cuda.synchronize()
    eprint(f"[bench] {args.warmup} warmup steps done")

    # Moved tokens of this (deterministic) eviction, for the compaction bytes.
    n_mv = moved_token_count(kept.cpu().numpy(), B, shape.unsorted)

    wall, gpu_evict, gpu_fps_c = [], [], []
    for i in range(args.steps):
        restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step_evict()
        torch.cuda.synchronize()
        wall.append(time.perf_counter() - t0)
        gpu_fps_c.append(eva[0].elapsed_time(eva[1]))
        gpu_evict.append(eva[1].elapsed_time(eva[2]))
    eprint(f"[bench] {args.steps} timed steps done (fps compress + bkv_evict)")
    stage_ms = {n: [] for n in names}
    for i in range(args.steps):
        restore()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            stage_ms[n].append(ev[j].elapsed_time(ev[j + 1]))
    eprint(f"[bench] {args.steps} timed steps done (separate calls, for the breakdown)")

    ms_step = 1e3 * float(np.mean(wall))
    gpu_ms = {n: float(np.mean(v)) for n, v in stage_ms.items()}
    gpu_step_ms = float(np.mean(gpu_fps_c)) + float(np.mean(gpu_evict))
    sbytes = {n: b for n, b in stage_bytes(w, n_mv).items() if n in names}
    total_bytes = sum(sbytes.values())
    flops = 2.0 * U * g * 32 * d * L  # one pass of Q_obs . K^T per unit

    stages = {}
    for n in names:
        t = gpu_ms[n] * 1e-3
        gbs = sbytes[n] / t / 1e9
        stages[n] = {"us": round(gpu_ms[n] * 1e3, 2), "alg_bytes": sbytes[n],
                     "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    stages["score"]["TFLOPs"] = round(flops / (gpu_ms["score"] * 1e-3) / 1e12, 2)
    stages["score"]["mfma_frac"] = round(stages["score"]["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4)

    dom = max(names, key=lambda n: gpu_ms[n])
    achieved = sbytes[dom] / (gpu_ms[dom] * 1e-3) / 1e9
    traffic = traffic_from_profile(dom, w.name)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic}

    # Sampled parity check of one more step, run as the timed step runs it
    # (the FPS compress, then bkv_evict with the same arguments), against the
    # oracle on a few units: scores within the tolerance, kept sets equal
    # outside the tie band, the compacted cache equal to the inputs at the
    # GPU's kept slots, and the two FPS results equal to the oracle's sets
    # where every pick wins by more than the tolerance.
    check = None
    if not args.no_check:
        import oracle
        sample_units = [0, U // 3, U - 1]
        restore()
        torch.cuda.synchronize()
        if not window:
            bkv.fps_update(shape, buf, count, newq, trigger=32, m=16)
            beacons = buf[:, :16].cpu().numpy()
            bkv.evict(shape, K, V, kpos, L, buf, rec, L, B, buf=buf, count=count,
                      score_out=score, kept_out=kept, ws=ws_e)
        else:
            beacons = np.zeros((U * g, 0, d))
            bkv.evict(shape, K, V, kpos, L, None, rec, L, B, score_out=score, kept_out=kept,
                      ws=ws_e)
        torch.cuda.synchronize()
        check = parity_sample(w, sample_units, K0, V0, P0, buf0, newq, rec, beacons, K, V, kpos,
                              buf, score, kept, window, args.aggregate, shape.unsorted)
        eprint(f"[bench] parity of the timed path on units {sample_units}: {check}")

    t_step = gpu_step_ms * 1e-3
    out = {
        "metric": METRIC,
        "value": round(U * L / (ms_step * 1e-3), 1),
        "unit": "KV-head·key-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [round(1e3 * float(np.percentile(wall, q)), 4)
                                    for q in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "units": U, "layers": w.layers, "batch": w.batch,
                   "kv_heads": w.h_kv, "group": g, "d_head": d, "L": L, "b_kv": B,
                   "prefix": w.prefix, "recent": w.recent_tok, "rope_theta": w.theta,
                   "pooling": args.aggregate, "compaction": args.compaction,
                   "observation": "recent32" if window else "beacons16+recent16"},
        "unit_evictions_per_s": round(U / (ms_step * 1e-3), 1),
        "steps_per_s": round(1e3 / ms_step, 2),
        "step": ("bkv_evict (32-query window, no FPS)" if window else
                 "bkv_fps_update (compress) + bkv_evict"),
        "gpu_ms_per_step": round(gpu_step_ms, 4),
        "gpu_ms_evict": round(float(np.mean(gpu_evict)), 4),
        "gpu_ms_separate_calls": round(sum(gpu_ms.values()), 4),
        "alg_bytes_per_step": total_bytes,
        "hbm_frac_step": round(total_bytes / t_step / 1e9 / HBM_PEAK_GBS, 4),
        "moved_tokens": n_mv,
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": check,
    }
    if (args.variants and not window and args.aggregate == "max"
            and args.compaction == "sorted"):
        # The same step with its denominators from decode attention, in the
        # same run (the standalone measurement's buffers released first).
        del K, V, kpos, K0, V0, P0, buf, buf0, rec, scrub, inp
        torch.cuda.empty_cache()
        f = fused_main(args, w)
        fv = {k: f[k] for k in ("value", "ms_per_step", "gpu_ms_per_step",
                                "gpu_ms_beacon_rows_in_decode", "hbm_frac_step", "step")}
        fv["score_us"] = f["stages"]["score"]["us"]
        fv["parity"] = f["parity"]
        out["variants"] = {"fused_decode": fv}
    print(json.dumps(out), flush=True)



def fused_main(args, w):
    """The eviction step with its softmax denominators taken from decode
    attention.  Untimed set-up (work decoding does anyway): bkv_decode_attend
    over each recent query's own cache gives the recent rows' denominators.
    Timed: the decode attention of the step at the beacon fix (cache of L-16
    slots) with and without the beacon rows (the difference is charged to the
    eviction step), and the step itself: FPS compress, bkv_score_lse (one key
    read), select, compact, merge FPS."""
    import numpy as np
    import torch

    import synth
    from reasoning_model_kv_amd import bkv

    bkv.load_library()
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    U, g, d, L, B = w.n_units, w.group, w.d_head, w.L, w.b_kv
    nq = U * g
    L_fix = L - w.recent_tok
    eprint(f"[bench] fused decode: workload {w.name}: U={U} g={g} d={d} L={L} B_KV={B}")
    inp = synth.device_inputs(w, dev)
    torch.cuda.synchronize()
    K0, V0, P0 = inp["keys"], inp["values"], inp["kpos"]
    buf0, rec = inp["buf"], inp["recents"]
    newq = buf0[:, 31:32].clone()
    K, V, kpos = torch.empty_like(K0), torch.empty_like(V0), torch.empty_like(P0)
    buf = torch.empty_like(buf0)
    count = torch.empty((nq,), dtype=torch.int32, device=dev)
    score = torch.empty((U, L), dtype=torch.float32, device=dev)
    kept = torch.empty((U, B), dtype=torch.int32, device=dev)
    # Cache flush before each timed step: a read-only pass over 512 MB (twice
    # the 256 MB last-level cache), so that the step starts with cold caches
    # holding no dirty lines of the untimed state restore (their write-back
    # would otherwise land in the first timed kernel).
    scrub = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    shape = bkv.Shape(U, g, d, L, w.prefix, w.theta, recent_tok=w.recent_tok)
    ws = bkv.alloc_workspace(shape, L, 0, dev)
    stream = torch.cuda.current_stream()
    out = torch.empty((nq, d), dtype=torch.float32, device=dev)
    lse_q = torch.empty((nq,), dtype=torch.float32, device=dev)
    lse_obs = torch.empty((nq, 16), dtype=torch.float32, device=dev)
    lse_in = torch.empty((U, g, 32), dtype=torch.float32, device=dev)
    q_fix = buf0[:, 30].contiguous()     # the query of the step at the beacon fix

    def restore():
        K.copy_(K0)
        V.copy_(V0)
        kpos.copy_(P0)
        buf.copy_(buf0)
        count.fill_(31)
        scrub.sum()

    # Denominators of the recent rows: each recent query's decode step.
    K.copy_(K0)
    V.copy_(V0)
    for i in range(16):
        qi = rec[:, i].contiguous()
        bkv.decode_attend(shape, K, V, L - 16 + i + 1, qi, int(P0[0, L - 16 + i]), out, lse_q)
        lse_in[:, :, 16 + i] = lse_q.view(U, g)

    def decode_fix(with_beacons):
        # The beacons are the compressed buffer's rows 0..15 (the state
        # before this step's compress is the same up to the appended row).
        if with_beacons:
            bkv.decode_attend(shape, K, V, L_fix, q_fix, int(P0[0, L_fix - 1]), out, lse_q,
                              buf, L, lse_obs)
        else:
            bkv.decode_attend(shape, K, V, L_fix, q_fix, int(P0[0, L_fix - 1]), out, lse_q)

    names = ["fps_compress", "score", "select", "compact", "fps_merge"]
    calls = {
        "fps_compress": lambda: bkv.fps_update(shape, buf, count, newq, trigger=32, m=16),
        "score": lambda: bkv.score_lse(shape, K, kpos, L, buf, rec, L, lse_in, L_fix, score,
                                       ws=ws),
        "select": lambda: bkv.select(shape, score, L, B, kept),
        "compact": lambda: bkv.compact(shape, K, V, kpos, L, kept, B),
        "fps_merge": lambda: bkv.fps_update(shape, buf, count, rec, trigger=32, m=16),
    }
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    evd = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def prepare():
        # State before the step, plus the beacons' denominators as the fused
        # decode step leaves them (from the compressed buffer of this state).
        restore()
        bkv.fps_update(shape, buf, count, newq, trigger=32, m=16)
        decode_fix(True)
        lse_in[:, :, :16] = lse_obs.view(U, g, 16)
        buf.copy_(buf0)
        count.fill_(31)
        scrub.sum()

    def step():
        ev[0].record(stream)
        for j, n in enumerate(names):
            calls[n]()
            ev[j + 1].record(stream)

    def decodes():
        scrub.sum()
        evd[0].record(stream)
        decode_fix(False)
        evd[1].record(stream)
        scrub.sum()
        torch.cuda.synchronize()
        evd[2].record(stream)
        decode_fix(True)
        ev_end = torch.cuda.Event(enable_timing=True)
        ev_end.record(stream)
        torch.cuda.synchronize()
        return evd[0].elapsed_time(evd[1]), evd[2].elapsed_time(ev_end)

    for _ in range(args.warmup):
        prepare()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        decodes()
    stage_ms = {n: [] for n in names}
    wall = []
    dec_plain, dec_fused = [], []
    for _ in range(args.steps):
        prepare()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        wall.append(time.perf_counter() - t0)
        for j, n in enumerate(names):
            stage_ms[n].append(ev[j].elapsed_time(ev[j + 1]))
        a, b = decodes()
        dec_plain.append(a)
        dec_fused.append(b)
    eprint(f"[bench] {args.steps} timed steps done (fused-decode eviction)")

    n_mv = moved_token_count(kept.cpu().numpy(), B, False)
    gpu_ms = {n: float(np.mean(v)) for n, v in stage_ms.items()}
    sbytes = {n: b for n, b in stage_bytes(w, n_mv).items() if n in names}
    sbytes["score"] += U * g * 32 * 4          # the known denominators read
    extra_ms = max(0.0, float(np.mean(dec_fused)) - float(np.mean(dec_plain)))
    step_ms = sum(gpu_ms.values()) + extra_ms
    total_bytes = sum(sbytes.values())
    stages = {}
    for n in names:
        gbs = sbytes[n] / (gpu_ms[n] * 1e-3) / 1e9
        stages[n] = {"us": round(gpu_ms[n] * 1e3, 2), "alg_bytes": sbytes[n],
                     "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    flops = 2.0 * U * g * 32 * d * L
    stages["score"]["TFLOPs"] = round(flops / (gpu_ms["score"] * 1e-3) / 1e12, 2)
    dec_bytes = U * (2 * L_fix * d * 2) + nq * d * 4 * 2
    dec = {"L": L_fix, "us_plain": round(float(np.mean(dec_plain)) * 1e3, 2),
           "us_with_beacon_rows": round(float(np.mean(dec_fused)) * 1e3, 2),
           "alg_bytes": dec_bytes,
           "hbm_frac_plain": round(dec_bytes / (np.mean(dec_plain) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                   4)}
    dom = max(names, key=lambda n: gpu_ms[n])
    achieved = sbytes[dom] / (gpu_ms[dom] * 1e-3) / 1e9

    check = None
    if not args.no_check:
        import oracle
        sample = [0, U // 3, U - 1]
        prepare()
        bkv.fps_update(shape, buf, count, newq, trigger=32, m=16)
        beacons = buf[:, :16].cpu().numpy()
        bkv.score_lse(shape, K, kpos, L, buf, rec, L, lse_in, L_fix, score, ws=ws)
        torch.cuda.synchronize()
        worst = 0.0
        for u in sample:
            taus = P0[u, L - 16:L].cpu().numpy()
            ref = oracle.score.score_unit(K0[u, :L].float().cpu().numpy(),
                                          beacons[u * g:(u + 1) * g],
                                          rec[u * g:(u + 1) * g].cpu().numpy(), L, taus, w.theta)
            s_gpu = score[u].cpu().numpy()
            worst = max(worst, float(np.max(np.abs(s_gpu - ref) / (ref + 1e-30))))
        check = {"units": sample, "max_score_rel_err": worst}
        eprint(f"[bench] parity on units {sample}: {check}")

    ms_wall = 1e3 * float(np.mean(wall)) + extra_ms
    out_line = {
        "metric": METRIC,
        "value": round(U * L / (ms_wall * 1e-3), 1),
        "unit": "KV-head·key-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "units": U, "layers": w.layers, "batch": w.batch,
                   "kv_heads": w.h_kv, "group": g, "d_head": d, "L": L, "b_kv": B,
                   "prefix": w.prefix, "recent": w.recent_tok, "rope_theta": w.theta,
                   "pooling": "max", "compaction": "sorted",
                   "observation": "beacons16+recent16",
                   "denominators": "from decode attention (beacons at L-16, recents at their steps)"},
        "unit_evictions_per_s": round(U / (ms_wall * 1e-3), 1),
        "step": ("bkv_fps_update (compress) + bkv_score_lse + bkv_select + bkv_compact + "
                 "bkv_fps_update (merge), plus the beacon rows' extra time in decode attention"),
        "gpu_ms_per_step": round(step_ms, 4),
        "gpu_ms_beacon_rows_in_decode": round(extra_ms, 4),
        "alg_bytes_per_step": total_bytes,
        "hbm_frac_step": round(total_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "moved_tokens": n_mv,
        "stages": stages,
        "decode_attention": dec,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("score_lse" if dom == "score" else dom,
                                                     w.name)},
        "cpu_baseline": None,
        "parity": check,
    }
    return out_line

def stream_main(args, w):
    """Streaming decode run (the Qwen3-14B-shaped workload): the whole policy
    over `stream_steps` decode steps of all units in lockstep.  Each chunk of
    128 steps is generated on the device before its steps are timed; HIP
    events on the launch stream time the chunks (decode-step upkeep:
    writing each token's K/V, append / fill-and-compress, beacon fix, recent
    capture, evictions) and, inside them, every eviction event."""
    import numpy as np
    import torch

    import synth
    from reasoning_model_kv_amd import bkv
    from reasoning_model_kv_amd import stream as bstream

    cpu = None
    if args.cpu_seconds > 0:
        # The oracle's eviction event per unit (the GPU is not touched yet).
        eprint(f"[bench] oracle CPU baseline (~{args.cpu_seconds:.0f} s of CPU work per core)")
        c = cpu_baseline(w, args.cpu_seconds)
        cpu = dict(c, value=round(c["value"] / w.L, 2), unit="unit-evictions/s")
        eprint(f"[bench] cpu baseline: {cpu}")
    bkv.load_library()
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    n_steps = args.stream_steps or w.stream_steps
    U, g, d = w.n_units, w.group, w.d_head
    cs = torch.cuda.current_stream()
    ev_marks = []

    def observer(kind, stage, st):
        if kind == "evict":
            e = torch.cuda.Event(enable_timing=True)
            e.record(cs)
            ev_marks.append(e)

    st = bstream.Stream(U, g, d, w.L, w.b_kv, w.prefix, w.theta, device=dev, observer=observer,
                        beacon_policy=args.beacon_policy,
                        unsorted=args.compaction == "unsorted", observe={"evict"})
    gen = synth.StreamInputs(w, dev)
    st.prefill(*gen.prompt())
    torch.cuda.synchronize()
    eprint(f"[bench] stream {w.name}: U={U} g={g} B_max={w.L} B_KV={w.b_kv} P={w.prefix} "
           f"steps={n_steps}")
    chunk_ms, done, c, moved = [], 0, 0, []
    t_wall = time.perf_counter()
    while done < n_steps:
        n = min(128, n_steps - done)
        k, v, q = gen.chunk(c, 128)
        c += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(cs)
        before = st.n_evictions
        st.run(k[:n], v[:n], q[:n])
        e1.record(cs)
        torch.cuda.synchronize()
        chunk_ms.append(e0.elapsed_time(e1))
        if st.n_evictions > before and len(moved) < 4:
            kept = st.kept.cpu().numpy()
            moved.append(int(np.count_nonzero(kept >= w.b_kv)) if st.shape.unsorted else
                         int(np.count_nonzero(kept != np.arange(w.b_kv)[None, :])))
        done += n
        if c % 32 == 0:
            eprint(f"[bench] {done} steps, {st.n_evictions} evictions")
    wall = time.perf_counter() - t_wall
    evict_ms = [ev_marks[i].elapsed_time(ev_marks[i + 1]) for i in range(0, len(ev_marks), 2)]
    gpu_ms = float(np.sum(chunk_ms))
    n_ev = st.n_evictions
    unit_ev = n_ev * U
    mean_ev = float(np.mean(evict_ms)) if evict_ms else float("nan")
    L = w.L
    n_mv = float(np.mean(moved)) if moved else 0.0
    ev_bytes = (U * (L * d * 2 + g * 32 * d * 4 + 16 * 4 + L * 4)       # score
                + U * ((L - w.prefix - w.recent_tok) * 4 + w.b_kv * 4)  # select
                + n_mv * (4 * d * 2 + 8) + U * w.b_kv * 4               # compaction
                + U * g * ((16 + 16 + 16) * d * 4 + 8))                 # merge FPS
    cache_bytes = 2 * U * L * d * 2
    out = {
        "metric": "unit-evictions/s sustained over a streaming decode run (Qwen3-14B shape)",
        "value": round(unit_ev / (gpu_ms * 1e-3), 1),
        "unit": "unit-evictions/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": 0,
        "ms_per_step": round(gpu_ms / n_steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "units": U, "layers": w.layers, "batch": w.batch,
                   "kv_heads": w.h_kv, "group": g, "d_head": d, "B_max": L, "b_kv": w.b_kv,
                   "prefix": w.prefix, "recent": w.recent_tok, "rope_theta": w.theta,
                   "beacons": "continual FPS" if args.beacon_policy == "fps" else
                              "first 16 generated queries (Initial+Recent)",
                   "compaction": args.compaction},
        "evictions": n_ev,
        "evict_ms_mean": round(mean_ev, 4),
        "evict_hbm_frac": round(ev_bytes / (mean_ev * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_upkeep_ms_per_step": round((gpu_ms - float(np.sum(evict_ms))) / n_steps, 5),
        "gpu_s_total": round(gpu_ms * 1e-3, 3),
        "wall_s_total": round(wall, 3),
        "peak_cache_bytes": cache_bytes,
        "full_cache_bytes_at_end": 2 * U * (w.prefix + n_steps) * d * 2,
        "torch_max_memory_allocated": torch.cuda.max_memory_allocated(),
        "moved_tokens_per_eviction": n_mv,
        # The eviction events dominate the bytes; their algorithmic bytes over
        # their event-timed duration.
        "roofline": {"kernel": "eviction event (bkv_evict)", "bound": "hbm",
                     "achieved": round(ev_bytes / (mean_ev * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ev_bytes / (mean_ev * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def prefill_fps_main(args, w):
    """Prefill FPS over long prompts: each query head's N prompt queries
    (the streaming recipe's prompt, synth.StreamInputs) are compressed to 16
    beacons by one bkv_fps_update on an N-row buffer."""
    import numpy as np
    import torch

    import oracle
    import synth
    from reasoning_model_kv_amd import bkv

    N = args.prefill_fps
    if not 17 <= N <= 8192:
        eprint("--prefill-fps takes 17 <= N <= 8192")
        sys.exit(2)
    bkv.load_library()
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    w2 = synth.shrink(w, prefix=N)
    nq, d, m = w2.n_qheads, w2.d_head, 16
    t0 = time.perf_counter()
    _, _, q = synth.StreamInputs(w2, dev).prompt()
    q0 = q.contiguous()
    del q
    torch.cuda.synchronize()
    eprint(f"[bench] prefill FPS: {nq} heads x {N} rows x d={d}; inputs in "
           f"{time.perf_counter() - t0:.2f} s")
    buf = torch.empty_like(q0)
    count = torch.empty((nq,), dtype=torch.int32, device=dev)
    sel = torch.empty((nq, m), dtype=torch.int32, device=dev)
    shape = bkv.Shape(w2.n_units, w2.group, d, 64, 0, w2.theta, buf_cap=N)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for i in range(args.warmup + args.steps):
        buf.copy_(q0)
        count.fill_(N)
        torch.cuda.synchronize()
        ev[0].record(stream)
        bkv.fps_update(shape, buf, count, trigger=N, m=m, sel_order=sel)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(ev[0].elapsed_time(ev[1]))
    ms = float(np.mean(times))
    alg = nq * (N * d * 4 + m * d * 4 + 8)        # rows in, kept rows out, count
    # The long-buffer kernel reads every row in three full passes, then
    # gathers the shortlist rows (about one more pass on this recipe).
    full_passes = 3 if N > 256 else 1
    streamed = nq * N * d * 4 * full_passes
    check = None
    if not args.no_check:
        heads = [0, nq // 2, nq - 1]
        picks = sel.cpu().numpy()
        worst = 0.0
        ok = True
        for h in heads:
            rows = q0[h].double().cpu().numpy()
            good, off = oracle.fps.replay_check(rows, [int(x) for x in picks[h]], 2e-3)
            ok, worst = ok and good, max(worst, off)
            kept = buf[h, :m].cpu().numpy()
            ok = ok and np.array_equal(kept, q0[h].cpu().numpy()[np.sort(picks[h])])
        check = {"heads": heads, "valid_fps_runs": bool(ok), "worst_replay_gap": worst}
        eprint(f"[bench] parity on heads {heads}: {check}")
    cpu = None
    if args.cpu_seconds > 0:
        rows = q0[0].double().cpu().numpy()
        t1 = time.perf_counter()
        oracle.fps.fps(rows, m)
        dt = time.perf_counter() - t1
        cpu = {"value": round(N / dt, 1), "unit": "query rows compressed/s", "cores": 1,
               "kind": "oracle", "sample": f"one head's {N}-row prompt buffer, float64 numpy, "
                                           f"{dt:.2f} s"}
    out = {
        "metric": "prefill FPS: prompt query rows compressed to 16 beacons per second",
        "value": round(nq * N / (ms * 1e-3), 1),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "query_heads": nq, "prompt_rows": N, "d_head": d,
                   "kept": m},
        "alg_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
        "full_passes": full_passes,
        "full_pass_GBps": round(streamed / (ms * 1e-3) / 1e9, 1),
        # achieved: algorithmic bytes (the rows read once); the kernel itself
        # reads them in full_passes passes plus the shortlist gathers
        "roofline": {"kernel": "fps_long_kernel" if N > 256 else "fps_block_kernel",
                     "bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": (traffic_from_profile("fps_long_prefill", f"{w2.name}-N{N}")
                                 if N > 256 else None)},
        "cpu_baseline": cpu,
        "parity": check,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
