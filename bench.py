#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

Default workload: B=256 sequences, K=7 draft tokens, V=128256, bf16 logits, temperature 0.7,
top-k 50 on both distributions (Zipf-shaped synthetic logits, see workloads/synthetic.py).
A step is one spec_verify call over the whole batch: every target row (B*(K+1)) and draft row
(B*K) is read, distributions formed, drafts accepted or rejected, and the final token drawn.
Inputs are resident in HBM before the timed region; draft tokens are drawn on the GPU from the
draft rows (spec_sample) beforehand.  A workload whose inputs would fit twice in the 256 MB
last-level cache is timed over as many independently generated input sets as it takes to pass
that (at least 8), taken in turn.

Prints one JSON line (the last line of stdout).  value = logit elements per second over the
timed steps, which carry no instrumentation.  "roofline" covers the dominant kernel (the
row-streaming kernel), timed with HIP events recorded on the library's stream around that
kernel in a second pass of max(steps, 200) steps; that pass also gives the per-step median,
10th and 90th percentiles ("step_us").  "copy" is a 512 MiB device copy timed the same way, the
measured on-box bandwidth the step is also compared with.  "cpu_baseline" times the CPU oracle
(numpy, float64) on the host cores: the batch split by sequence over one process per core, each
repeating its share for a time budget; the oracle's results on the same inputs (its own draft
tokens and uniforms) are then checked against the GPU's, decision by decision, and the boundary
flips counted ("flips").
--workload tree_B32_N64_V32000_bf16 times greedy token-tree verification instead, and
--workload rest_B32_M64_L8_N64 the REST draft-tree construction.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify throughput: logit elems/s + % HBM peak, B=256 K=7 V=128256 bf16"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
KERNEL_SOURCE = os.path.join(ROOT, "speculative_sampling_verification_amd", "csrc",
                             "sv_kernels.hip")


def _hip_runtime():
    """The HIP runtime torch already loaded (the library binds to the same one)."""
    paths = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
    hip = ctypes.CDLL(paths[0])
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return hip


# Events only time the work (they are read after a full synchronisation), so they skip the
# system-scope fence of a recorded event: with it, each record writes back and invalidates the
# caches and leaves the GPU idle for several microseconds between kernels.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _new_event(hip, fence=False):
    e = ctypes.c_void_p()
    flags = 0 if fence else HIP_EVENT_DISABLE_SYSTEM_FENCE
    assert hip.hipEventCreateWithFlags(ctypes.byref(e), flags) == 0
    return e.value


def _elapsed(hip, a, b):
    f = ctypes.c_float()
    hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
    return f.value


def _destroy(hip, evs):
    for row in evs:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))


def _source_tag():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:12]


def _traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    tag = re.search(r"source_sha256_12:\s*([0-9a-f]+)", text)
    fetch = re.search(r"fetch_bytes_per_launch:\s*([0-9.e+]+)", text)
    write = re.search(r"write_bytes_per_launch:\s*([0-9.e+]+)", text)
    if not (tag and fetch and write) or tag.group(1) != _source_tag():
        return None
    return float(fetch.group(1)) + float(write.group(1))


def _pct(xs_ms):
    """median / p10 / p90 of per-step durations, in microseconds."""
    import numpy as np
    a = np.asarray(xs_ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()),
            "iterations": int(a.size)}


def _small_path(K, V, cfg):
    """Whether the library takes its single-launch path for small problems: dense rows (T > 0,
    nothing truncated) and all 2K+1 rows of a sequence in one workgroup's registers (V <= 256 L
    and 2K+1 <= 64 / L for L = 4, 8 or 16)."""
    dense = cfg["temperature"] > 0 and not (0 < cfg["top_k"] < V) and cfg["top_p"] >= 1.0
    return dense and any(V <= 256 * L and 2 * K + 1 <= 64 // L for L in (4, 8, 16))


def _n_sets(set_bytes):
    """Input sets to rotate: one if a set is larger than twice the last-level cache, else
    enough sets (at least 8, at most 64) to pass that."""
    if set_bytes > 2 * MALL_BYTES:
        return 1
    return int(min(64, max(8, math.ceil(2 * MALL_BYTES / max(1, set_bytes)) + 1)))


# ----------------------------------------------------------------------------- CPU baseline
# The oracle on the host cores: one process per core (at most 16, the machine's CPU share per GPU),
# each given a contiguous share of the batch.  Workers are started with the "spawn" method (a
# fresh interpreter that never touched the GPU) before their shares are sent; they do their
# untimed set-up (decoding, the oracle's own draft draws), wait for "go", run their share
# repeatedly until the time budget is spent, report, and then check the GPU's results for their
# share against the oracle (tests/parity.py) when the parent sends them.

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _decode(raw, dtype):
    """float32 logits from host bytes: fp32 as is, bf16 (raw 16-bit patterns) widened."""
    import numpy as np
    if dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32)
    return raw


def _oracle_worker(conn, root):
    sys.stdout = sys.stderr  # the benchmark's stdout carries only its JSON line
    sys.path[:0] = [root, os.path.join(root, "tests")]
    import numpy as np
    import oracle.spec_verify_oracle as O
    import parity
    job = conn.recv()
    kind, budget = job["kind"], job["budget"]
    if kind in ("verify", "mentored"):
        tf = _decode(job["target"], job["dtype"])
        df = _decode(job["draft"], job["dtype"])
        p = job["params"]
        T, k, P = np.float32(p["temperature"]), p["top_k"], np.float32(p["top_p"])
        K = tf.shape[1] - 1
        u_draw, u = job["u_draw"], job["u"]
        drafts = np.stack([O.sample_rows(df[:, j], u_draw[:, j], T, k, P) for j in range(K)],
                          axis=1).astype(np.int32) if K else np.zeros((tf.shape[0], 0), np.int32)
        conn.send(drafts)
        conn.recv()  # go
        reps, seqs = 0, 0
        t0 = time.perf_counter()
        while True:
            if kind == "verify":
                o = O.spec_verify(tf, df, drafts, u, T, k, P, np.float32(p["lenience"]))
                seqs += tf.shape[0]
            else:  # mentored: one sequence per call, the share cycled until the budget is spent
                b = reps % tf.shape[0]
                O.mentored_spec_verify(tf[b:b + 1], df[b:b + 1], drafts[b:b + 1], u[b:b + 1], T,
                                       k, P, np.float32(p["mentor_kl"]))
                seqs += 1
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                break
        conn.send({"seconds": dt, "sequences": seqs})
        g = conn.recv()
        res = {"checked": 0, "flips": {"accept": 0, "draw": 0, "topp": 0}, "mismatch": None}
        if g is not None:
            sel = slice(0, min(tf.shape[0], job["check_seqs"]))
            gs = {key: v[sel] for key, v in g.items()}
            try:
                flips, _ = parity.check(gs, tf[sel], df[sel], drafts[sel], u[sel], p,
                                        max_flips=1 << 30, label=job["label"])
                res["flips"] = flips
            except AssertionError as e:
                res["mismatch"] = str(e)[:400]
            res["checked"] = int(gs["tokens"].shape[0])
        conn.send(res)
    elif kind == "tree":
        x = _decode(job["logits"], job["dtype"])
        parent, tokens, D = job["parent"], job["tokens"], job["max_depth"]
        conn.send(None)
        conn.recv()
        reps = 0
        t0 = time.perf_counter()
        while True:
            o = O.tree_verify(x, parent, tokens, D)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                break
        conn.send({"seconds": dt, "sequences": reps * x.shape[0]})
        g = conn.recv()
        bad = (g["tokens"] != o["tokens"]).any(axis=1) | (g["n"] != o["n"])
        conn.send({"checked": int(x.shape[0]), "mismatch_sequences": int(bad.sum())})
    elif kind == "rest":
        c = job["candidates"]
        conn.send(None)
        conn.recv()
        done = 0
        t0 = time.perf_counter()
        while True:
            O.rest_build_tree(c[done % c.shape[0]], job["N"])
            done += 1
            dt = time.perf_counter() - t0
            if dt >= budget:
                break
        conn.send({"seconds": dt, "sequences": done})
        conn.recv()
        conn.send({})
    conn.close()


class OraclePool:
    """Worker processes for the oracle leg, one share of the batch each.  They are started
    before the benchmark touches the GPU and get their jobs later (submit)."""

    def __init__(self, n):
        import multiprocessing as mp
        ctx = mp.get_context("spawn")
        self.conns, self.procs = [], []
        old = os.environ.get("OMP_NUM_THREADS")
        os.environ["OMP_NUM_THREADS"] = "1"  # one core per worker
        try:
            for _ in range(n):
                a, b = ctx.Pipe()
                pr = ctx.Process(target=_oracle_worker, args=(b, ROOT), daemon=True)
                pr.start()
                self.conns.append(a)
                self.procs.append(pr)
        finally:
            if old is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = old

    def submit(self, jobs):
        """Send each worker its job; returns what each reports after its untimed set-up."""
        assert len(jobs) == len(self.conns)
        for c, job in zip(self.conns, jobs):
            c.send(job)
        return [c.recv() for c in self.conns]

    def timed(self):
        """Start every worker at once; wall seconds until the last one reports."""
        t0 = time.perf_counter()
        for c in self.conns:
            c.send("go")
        rep = [c.recv() for c in self.conns]
        return time.perf_counter() - t0, rep

    def finish(self, payloads):
        for c, p in zip(self.conns, payloads):
            c.send(p)
        out = [c.recv() for c in self.conns]
        for pr in self.procs:
            pr.join(timeout=60)
        return out


def _shares(B, n):
    n = max(1, min(n, B))
    edges = [round(i * B / n) for i in range(n + 1)]
    return [(edges[i], edges[i + 1]) for i in range(n)]


def _host_raw(t):
    """Host bytes of a logit tensor for the workers: fp32 as is, bf16 as raw 16-bit patterns."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view("uint16")
    return t.cpu().numpy()


def cpu_baseline_verify(svm, pool, name, cfg, target, draft, seconds, mentor_kl, kw):
    """The oracle on the host cores over the whole batch (each worker its share, repeated for
    the time budget), then the GPU on the same inputs (the oracle's draft draws, Philox
    uniforms) outside any timed region, checked against the oracle decision by decision."""
    import numpy as np
    import torch
    from workloads import synthetic as S
    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    shares = _shares(B, len(pool.conns))
    u_draw = S.philox_uniforms(101, (B, K))
    u = S.philox_uniforms(102, (B, K + 1))
    params = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"],
                  lenience=cfg["lenience"], mentor_kl=mentor_kl)
    traw, draw_ = _host_raw(target), _host_raw(draft)
    mentored = mentor_kl > 0
    jobs = [{"kind": "mentored" if mentored else "verify", "budget": seconds / len(shares),
             "target": traw[a:b], "draft": draw_[a:b], "dtype": cfg["dtype"], "params": params,
             "u_draw": u_draw[a:b], "u": u[a:b], "check_seqs": 1 if mentored else b - a,
             "label": f"bench {name} sequences {a}..{b - 1}"} for a, b in shares]
    drafts = np.concatenate(pool.submit(jobs), axis=0)
    wall, rep = pool.timed()
    seqs = sum(r["sequences"] for r in rep)
    # the GPU on the oracle's inputs, outside the timed regions
    dev = target.device
    g = svm.spec_verify(target, draft, torch.from_numpy(drafts).to(dev),
                        torch.from_numpy(u).to(dev), **kw)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items() if k != "rate"}
    res = pool.finish([{k: v[a:b] for k, v in g.items()} for a, b in shares])
    flips = {"accept": 0, "draw": 0, "topp": 0}
    for r in res:
        for k in flips:
            flips[k] += r["flips"][k]
    mism = [r["mismatch"] for r in res if r["mismatch"]]
    flips.update(sequences_checked=sum(r["checked"] for r in res), mismatches=len(mism))
    if mism:
        flips["first_mismatch"] = mism[0]
    cpu = {"value": seqs * (2 * K + 1) * V / wall, "unit": "logit elems/s", "cores": len(shares),
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": (f"{'mentored decoding, ' if mentored else ''}{seqs} sequences of the batch "
                      f"({(2 * K + 1) * V} logits each; each of {len(shares)} processes repeats "
                      f"its share of the {B} sequences for {seconds / len(shares):.2f} s), "
                      f"{wall:.2f} s wall, numpy float64"),
           "seconds": wall}
    return cpu, flips


# ----------------------------------------------------------------------------- timing
def _copy_reference(args, dev, hip):
    """A plain device copy of known size, timed with events: the measured on-box bandwidth
    (read + write bytes / time) and the reference kernel for calibrating rocprofv3 byte
    counters.  Returns GB/s or None."""
    import torch
    if args.copy_reference_mib <= 0:
        return None
    src = torch.empty(args.copy_reference_mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    evs = [[_new_event(hip) for _ in range(2)] for _ in range(5)]
    dst.copy_(src)
    for e in evs:
        hip.hipEventRecord(ctypes.c_void_p(e[0]), stream)
        dst.copy_(src)
        hip.hipEventRecord(ctypes.c_void_p(e[1]), stream)
    torch.cuda.synchronize()
    ms = sorted(_elapsed(hip, e[0], e[1]) for e in evs)[len(evs) // 2]
    _destroy(hip, evs)
    nbytes = 2 * src.numel()
    del src, dst
    return nbytes / (ms * 1e-3) / 1e9


def bench_tree(args, name, cfg):
    """Greedy token-tree verification: a step is one spec_verify_tree call over the batch.  The
    logits (131 MB per set) would fit the 256 MB last-level cache, so the timed steps rotate
    through independently generated input sets."""
    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, N, V, D = cfg["B"], cfg["N"], cfg["V"], cfg["max_depth"]
    pool = None if args.no_cpu_baseline else OraclePool(len(_shares(B, _cpu_workers())))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsets = _n_sets(B * N * V * S.elem_bytes(name))
    sets = []
    for seed in range(1, nsets + 1):
        logits, parent, tokens = S.workload_inputs(name, device=dev, seed=seed)
        sets.append((logits, torch.from_numpy(np.asarray(parent, np.int32)).to(dev),
                     torch.from_numpy(np.asarray(tokens, np.int32)).to(dev), parent, tokens))
    out = svm.spec_verify_tree(sets[0][0], sets[0][1], sets[0][2], D)
    torch.cuda.synchronize()
    hip = _hip_runtime()
    n_ev = max(args.steps, 200)
    evs = [[_new_event(hip, args.fenced_events) for _ in range(3)] for _ in range(n_ev)]
    for i in range(args.warmup):
        s = sets[i % len(sets)]
        svm.spec_verify_tree(s[0], s[1], s[2], D, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        svm.spec_verify_tree(s[0], s[1], s[2], D, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-step events in a second pass, for the kernel durations and the percentiles
    t0 = time.perf_counter()
    for i in range(n_ev):
        s = sets[i % len(sets)]
        svm.spec_verify_tree(s[0], s[1], s[2], D, out=out, events=evs[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    copy_gbs = _copy_reference(args, dev, hip)
    kern_ms = [_elapsed(hip, e[0], e[1]) for e in evs]
    step_ms = [_elapsed(hip, e[0], e[2]) for e in evs]
    _destroy(hip, evs)
    elems = B * N * V
    logit_bytes = elems * sets[0][0].element_size()
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    achieved = logit_bytes / (kern_avg * 1e-3) / 1e9
    step_gbs = logit_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": f"tree verify throughput: logit elems/s, greedy token tree B={B} N={N} V={V} "
                  f"{cfg['dtype']}",
        "value": elems / (ms_per_step * 1e-3),
        "unit": "logit elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": name, "B": B, "N": N, "V": V, "max_depth": D,
                   "planted": cfg["planted"], "input_sets": len(sets)},
        "roofline": {"bound": "hbm", "kernel": "k_chunk_argmax", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": _traffic_from_profiles("k_chunk_argmax", name),
                     "kernel_ms": kern_avg, "algorithmic_bytes_per_launch": logit_bytes,
                     "frac_of_copy": achieved / copy_gbs if copy_gbs else None},
        "rows_per_s": B * N / (ms_per_step * 1e-3),
        "step_gbs": step_gbs,
        "step_frac_hbm_peak": step_gbs / HBM_PEAK_GBS,
        "step_us": _pct(step_ms),
        "kernel_us": _pct(kern_ms),
        "copy_gbs": copy_gbs,
        "step_frac_of_copy": step_gbs / copy_gbs if copy_gbs else None,
        "ms_per_step_with_phase_events": wall_ev * 1e3 / n_ev,
        "mean_accepted_depth": float(out["num_accepted"].float().mean().item()),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if not args.no_cpu_baseline:
        s = sets[0]
        shares = _shares(B, len(pool.conns))
        raw = _host_raw(s[0])
        pool.submit([{"kind": "tree", "budget": args.cpu_seconds / len(shares),
                      "logits": raw[a:b], "dtype": cfg["dtype"], "parent": s[3][a:b],
                      "tokens": s[4][a:b], "max_depth": D} for a, b in shares])
        wall_c, rep = pool.timed()
        g = svm.spec_verify_tree(s[0], s[1], s[2], D)
        torch.cuda.synchronize()
        gn = {"tokens": g["tokens"].cpu().numpy(), "n": g["num_accepted"].cpu().numpy()}
        chk = pool.finish([{k: v[a:b] for k, v in gn.items()} for a, b in shares])
        trees = sum(r["sequences"] for r in rep)
        res["cpu_baseline"] = {
            "value": trees * N * V / wall_c, "unit": "logit elems/s", "cores": len(shares),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": f"{trees} trees of {N} nodes ({N * V} logits each; each of {len(shares)} "
                      f"processes repeats its share of the {B} trees), {wall_c:.2f} s wall, "
                      "numpy float64", "seconds": wall_c}
        res["mismatches_vs_oracle"] = {"sequences_checked": sum(r["checked"] for r in chk),
                                       "sequences_differing": sum(r["mismatch_sequences"]
                                                                  for r in chk)}
    print(json.dumps(res), flush=True)


def bench_rest(args, name, cfg):
    """REST draft-tree construction: a step is one spec_build_tree call over the batch (one
    workgroup per sequence; latency-bound: the data are a few hundred KB)."""
    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, M, L, N = cfg["B"], cfg["M"], cfg["L"], cfg["N"]
    pool = None if args.no_cpu_baseline else OraclePool(len(_shares(B, _cpu_workers())))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cands = S.workload_inputs(name, device=dev, seed=1)
    out = svm.spec_build_tree(cands, N)
    torch.cuda.synchronize()
    hip = _hip_runtime()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    n_ev = max(args.steps, 200)
    evs = [[_new_event(hip, args.fenced_events) for _ in range(2)] for _ in range(n_ev)]
    for _ in range(args.warmup):
        svm.spec_build_tree(cands, N, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        svm.spec_build_tree(cands, N, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(n_ev):
        hip.hipEventRecord(ctypes.c_void_p(evs[i][0]), stream)
        svm.spec_build_tree(cands, N, out=out)
        hip.hipEventRecord(ctypes.c_void_p(evs[i][1]), stream)
    torch.cuda.synchronize()
    kern_ms = [_elapsed(hip, e[0], e[1]) for e in evs]
    _destroy(hip, evs)
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    nbytes = B * M * L * 4 + B * N * 4 * 4 + B * 4 + B * N * N
    achieved = nbytes / (kern_avg * 1e-3) / 1e9
    res = {
        "metric": f"REST draft-tree build: trees/s, B={B} candidates M={M} of L={L} tokens, "
                  f"N={N} nodes",
        "value": B / (ms_per_step * 1e-3),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "M": M, "L": L, "N": N},
        "roofline": {"bound": "hbm", "kernel": "k_rest_tree", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "kernel_ms": kern_avg,
                     "algorithmic_bytes_per_launch": nbytes,
                     "note": "latency-bound: one workgroup per sequence, B workgroups"},
        "step_us": _pct(kern_ms),
        "mean_nodes": float(out["num_nodes"].float().mean().item()),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if not args.no_cpu_baseline:
        c = cands.cpu().numpy()
        shares = _shares(B, len(pool.conns))
        pool.submit([{"kind": "rest", "budget": args.cpu_seconds / len(shares),
                      "candidates": c[a:b], "N": N} for a, b in shares])
        wall_c, rep = pool.timed()
        pool.finish([None] * len(shares))
        done = sum(r["sequences"] for r in rep)
        res["cpu_baseline"] = {"value": done / wall_c, "unit": "trees/s", "cores": len(shares),
                               "kind": "oracle", "cpu_model": _cpu_model(),
                               "sample": f"{done} trees of the batch ({len(shares)} processes "
                                         f"each cycling its share), {wall_c:.2f} s wall",
                               "seconds": wall_c}
    print(json.dumps(res), flush=True)


def _analytics(svm, target, draft, kw, K, measured_tokens, step_inputs):
    """Acceptance rates of the batch on the GPU (beta = sum min(p, q/l) per position, alpha =
    their mean) and the blog's analytics for this K: expected tokens per call (compare with the
    measured mean, which assumes i.i.d. positions), wall-clock factor and optimal gamma for a
    draft costing c = 5% of the target.  Also the time of a verify step that returns the rates
    too (spec_verify_rates), against the separate acceptance-rate call."""
    import torch
    args = dict(temperature=kw["temperature"], top_k=kw["top_k"], top_p=kw["top_p"],
                lenience=kw["lenience"])
    beta = svm.spec_acceptance_rate(target, draft, **args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        svm.spec_acceptance_rate(target, draft, out=beta, **args)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / 10
    drafts, u = step_inputs
    out = svm.spec_verify(target, draft, drafts, u, want_rates=True, **args)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        svm.spec_verify(target, draft, drafts, u, want_rates=True, out=out, **args)
    torch.cuda.synchronize()
    ms_both = (time.perf_counter() - t0) * 1e3 / 20
    assert torch.equal(out["rate"], beta), "rates of spec_verify_rates differ"
    alpha = float(beta.double().mean().item())
    return {"alpha_mean_beta": alpha,
            "expected_tokens_per_call": svm.expected_tokens(alpha, K),
            "measured_tokens_per_call": measured_tokens,
            "walltime_speedup_c0.05": svm.walltime_speedup(alpha, K, 0.05),
            "optimal_gamma_c0.05": svm.optimal_gamma(alpha, 0.05, 64),
            "acceptance_rate_ms_per_call": ms,
            "verify_with_rates_ms_per_step": ms_both}


def bench_pipeline(args, name, cfg):
    """The draft -> verify hand-off with every uniform made on the GPU: a step draws the
    draft tokens from the draft rows (Philox uniforms, spec_sample) and verifies them (Philox
    uniforms, spec_verify); each step takes fresh counters.  By default the verify step takes
    the draft rows' summaries from the sampling call (spec_verify_presampled), so every logit
    is streamed once; --no-presampled streams the draft rows again in spec_verify."""
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    target, draft = S.workload_inputs(name, device=dev, seed=1)
    kw = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"])
    key = (0x5EED, 0xC0FFEE)
    nb_d, nb_v = (B * K + 3) // 4, (B * (K + 1) + 3) // 4
    u_d = torch.empty(B * K, dtype=torch.float32, device=dev)
    u_v = torch.empty((B, K + 1), dtype=torch.float32, device=dev)
    drafts = torch.empty((B, K), dtype=torch.int32, device=dev)
    out = None
    presampled = not args.no_presampled
    summary = svm.sample_summary(B * K, V, draft.dtype, device=dev, **kw) if presampled else None

    def step(i):
        nonlocal out
        c = i * (nb_d + nb_v)
        svm.spec_philox_uniform(key, c, B * K, out=u_d)
        svm.spec_sample(draft.view(B * K, V), u_d, out=drafts.view(B * K), summary=summary, **kw)
        svm.spec_philox_uniform(key, c + nb_d, B * (K + 1), out=u_v.view(-1))
        out = svm.spec_verify(target, draft, drafts, u_v, out=out, lenience=cfg["lenience"],
                              presampled=summary, **kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    elems = B * (2 * K + 1) * V + (0 if presampled else B * K * V)
    n = out["num_accepted"].cpu().numpy()
    res = {
        "metric": f"draft sampling + verify with device uniforms: logit elems/s, B={B} K={K} "
                  f"V={V} {cfg['dtype']}",
        "value": elems / (ms_per_step * 1e-3),
        "unit": "logit elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": name, "B": B, "K": K, "V": V, "temperature": cfg["temperature"],
                   "top_k": cfg["top_k"], "top_p": cfg["top_p"], "lenience": cfg["lenience"],
                   "pipeline": "philox -> spec_sample(draft rows) -> philox -> " +
                               ("spec_verify_presampled" if presampled else "spec_verify")},
        "roofline": None,
        "logits_read_per_step": elems,
        "mean_tokens_per_call": float(n.mean() + 1.0),
        "source_sha256_12": _source_tag(),
    }
    print(json.dumps(res), flush=True)


def bench_verify(args, name, cfg):
    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    pool = None if args.no_cpu_baseline else OraclePool(len(_shares(B, _cpu_workers())))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kw = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"],
              lenience=cfg["lenience"], mentor_kl=args.mentor_kl, want_probs=not args.no_probs)
    nsets = _n_sets(B * (2 * K + 1) * V * S.elem_bytes(name))
    sets = []
    for seed in range(1, nsets + 1):
        target, draft = S.workload_inputs(name, device=dev, seed=seed)
        u_draw = torch.from_numpy(S.philox_uniforms(2 + 10 * seed, (B * K,))).to(dev)
        drafts = svm.spec_sample(draft.view(B * K, V), u_draw, temperature=cfg["temperature"],
                                 top_k=cfg["top_k"], top_p=cfg["top_p"]).view(B, K)
        sets.append((target, draft, drafts))
    u = torch.from_numpy(S.philox_uniforms(3, (B, K + 1))).to(dev)
    target, draft, drafts = sets[0]
    out = svm.spec_verify(target, draft, drafts, u, **kw)
    torch.cuda.synchronize()

    hip = _hip_runtime()
    n_ev = max(args.steps, 200)
    evs = [[_new_event(hip, args.fenced_events) for _ in range(3)] for _ in range(n_ev)]
    for i in range(args.warmup):
        s = sets[i % nsets]
        svm.spec_verify(s[0], s[1], s[2], u, out=out, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = sets[i % nsets]
        svm.spec_verify(s[0], s[1], s[2], u, out=out, **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_last = out["num_accepted"].cpu().numpy()
    a_last = out["accept_prob"].cpu().numpy() if "accept_prob" in out else None
    # the same steps again with per-phase events (each record idles the GPU for a few
    # microseconds, so they stay out of the throughput loop), for the kernel durations and the
    # per-step percentiles
    t0 = time.perf_counter()
    for i in range(n_ev):
        s = sets[i % nsets]
        svm.spec_verify(s[0], s[1], s[2], u, out=out, events=evs[i], **kw)
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    # the step captured in a HIP graph per input set and replayed: the launch path of a serving
    # loop that replays its verify step (reported beside `value`, which is eager)
    graph_ms = None
    if not args.no_graph:
        graphs = []
        for s in sets:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                svm.spec_verify(s[0], s[1], s[2], u, out=out, **kw)
            graphs.append(gr)
        for i in range(args.warmup):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % nsets].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graphs

    copy_gbs = _copy_reference(args, dev, hip)
    kern_ms = [_elapsed(hip, e[0], e[1]) for e in evs]
    step_ms = [_elapsed(hip, e[0], e[2]) for e in evs]
    gpu_region_ms = _elapsed(hip, evs[0][0], evs[-1][2])
    _destroy(hip, evs)

    esz = target.element_size()
    elems = B * (2 * K + 1) * V
    logit_bytes = elems * esz
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    achieved = logit_bytes / (kern_avg * 1e-3) / 1e9
    if cfg["temperature"] == 0:
        dominant = "k_chunk_argmax"
    elif 0 < cfg["top_k"] <= 256:
        dominant = "k_topk_row"
    elif _small_path(K, V, cfg):
        dominant = "k_small"
    else:
        dominant = "k_chunk"
    traffic = _traffic_from_profiles(dominant, name)
    mentored = args.mentor_kl > 0
    step_gbs = logit_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC if (name == S.METRIC_WORKLOAD and not mentored and
                             cfg["lenience"] == 1.0) else
                  f"verify throughput: logit elems/s + % HBM peak, B={B} K={K} V={V} "
                  f"{cfg['dtype']}" + (f", mentored decoding D={args.mentor_kl}"
                                       if mentored else "") +
                  (f", lenience {cfg['lenience']}" if cfg["lenience"] != 1.0 else ""),
        "value": elems / (ms_per_step * 1e-3),
        "unit": "logit elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {2: "bf16", 4: "f32"}[esz],
        "data": "synthetic",
        "config": {"workload": name, "B": B, "K": K, "V": V, "temperature": cfg["temperature"],
                   "top_k": cfg["top_k"], "top_p": cfg["top_p"], "lenience": cfg["lenience"],
                   "mentor_kl": args.mentor_kl, "accept_probs_requested": not args.no_probs,
                   "input_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms": kern_avg,
                     "algorithmic_bytes_per_launch": logit_bytes,
                     "frac_of_copy": achieved / copy_gbs if copy_gbs else None},
        "rows_per_s": B * (2 * K + 1) / (ms_per_step * 1e-3),
        "step_gbs": step_gbs,
        "step_frac_hbm_peak": step_gbs / HBM_PEAK_GBS,
        "step_us": _pct(step_ms),
        "kernel_us": _pct(kern_ms),
        "copy_gbs": copy_gbs,
        "step_frac_of_copy": step_gbs / copy_gbs if copy_gbs else None,
        "gpu_event_ms_per_step": float(np.median(step_ms)),
        "gpu_region_ms_per_step": gpu_region_ms / n_ev,
        "ms_per_step_with_phase_events": wall_ev * 1e3 / n_ev,
        "graph_ms_per_step": graph_ms,
        "mean_accept_prob": float(a_last.mean()) if a_last is not None and a_last.size else None,
        "mean_tokens_per_call": float(n_last.mean() + 1.0),
        "accepted_hist": np.bincount(n_last, minlength=K + 1).tolist(),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if not mentored and K > 0:
        res["analytics"] = _analytics(svm, target, draft, kw, K, float(n_last.mean() + 1.0),
                                      (drafts, u))
    if not args.no_cpu_baseline:
        res["cpu_baseline"], res["flips"] = cpu_baseline_verify(
            svm, pool, name, cfg, target, draft, args.cpu_seconds, args.mentor_kl, kw)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the metric one)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU oracle budget in core-seconds, split over the worker processes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fenced-events", action="store_true",
                    help="record the per-step timing events with the default system-scope "
                         "fence (costs idle time between kernels)")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the draft -> verify hand-off with device uniforms instead: "
                         "Philox, draft sampling, Philox, verify")
    ap.add_argument("--lenience", type=float, default=None,
                    help="override the workload's lenience l (accept iff u < min(1, q/(l p)))")
    ap.add_argument("--no-presampled", action="store_true",
                    help="with --pipeline: stream the draft rows again in spec_verify instead of "
                         "taking their summaries from the sampling call")
    ap.add_argument("--mentor-kl", type=float, default=0.0,
                    help="KL bound D > 0: mentored decoding (top-k workloads)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay timing (graph_ms_per_step)")
    ap.add_argument("--no-probs", action="store_true",
                    help="do not request per-position accept probabilities (mentored decoding "
                         "then solves only the positions its shortcut cannot accept)")
    ap.add_argument("--copy-reference-mib", type=int, default=512,
                    help="after the timed steps, copy a tensor of this size (timed: the on-box "
                         "copy bandwidth; also the reference kernel of known size for "
                         "calibrating rocprofv3 byte counters); 0 disables")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark measures one GPU; --gpus {args.gpus} is not supported "
              "(the verify step is data-parallel over sequences and needs no exchange, so "
              "N GPUs would each run this benchmark on their own share)", file=sys.stderr)
        sys.exit(2)

    from workloads import synthetic as S
    name = args.workload or S.METRIC_WORKLOAD
    cfg = dict(S.WORKLOADS[name])
    if args.lenience is not None:
        cfg["lenience"] = args.lenience
    if cfg["gen"] == "tree":
        bench_tree(args, name, cfg)
    elif cfg["gen"] == "rest":
        bench_rest(args, name, cfg)
    elif args.pipeline:
        bench_pipeline(args, name, cfg)
    else:
        bench_verify(args, name, cfg)


if __name__ == "__main__":
    main()
