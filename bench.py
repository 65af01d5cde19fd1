#!/usr/bin/env python3
"""Verify-step throughput on one MI355X.

Default workload: B=256 sequences, K=7 draft tokens, V=128256, bf16 logits, temperature 0.7,
top-k 50 on both distributions (Zipf-shaped synthetic logits, see workloads/synthetic.py).
A step is one spec_verify call over the whole batch: every target row (B*(K+1)) and draft row
(B*K) is read, distributions formed, drafts accepted or rejected, and the final token drawn.
Inputs are resident in HBM before the timed region; draft tokens are drawn on the GPU from the
draft rows (spec_sample) beforehand.

Prints one JSON line.  value = logit elements per second over the timed steps, which carry no
instrumentation.  "roofline" covers the dominant kernel (the row-streaming kernel), timed with
HIP events recorded on the library's stream around that kernel in a second pass of as many
steps (ms_per_step_with_phase_events is that pass's rate: each event record leaves the GPU
idle for a few microseconds).  "cpu_baseline" times the CPU oracle (numpy, float64, single
process) on the same inputs: whole steps repeated for about 10 s.
--workload tree_B32_N64_V32000_bf16 times greedy token-tree verification instead, and
--workload rest_B32_M64_L8_N64 the REST draft-tree construction.
"""

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verify throughput: logit elems/s + % HBM peak, B=256 K=7 V=128256 bf16"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
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


def cpu_baseline(name, target, draft, seconds, mentor_kl=0.0, lenience=None):
    """Time the CPU oracle on the same inputs: whole steps (every sequence) repeated until
    `seconds` have passed (at least one step).  Mentored decoding, whose oracle solves every
    position over the full vocabulary, is timed on groups of 4 sequences instead, until the
    budget is spent."""
    import numpy as np
    import oracle.spec_verify_oracle as O
    from workloads import synthetic as S
    cfg = dict(S.WORKLOADS[name])
    if lenience is not None:
        cfg["lenience"] = lenience
    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    tf = target.float().cpu().numpy()
    df = draft.float().cpu().numpy()
    T, k, P = np.float32(cfg["temperature"]), cfg["top_k"], np.float32(cfg["top_p"])
    u_draw = S.philox_uniforms(101, (B, K))
    drafts = np.stack([O.sample_rows(df[:, j], u_draw[:, j], T, k, P) for j in range(K)], axis=1)
    u = S.philox_uniforms(102, (B, K + 1))
    if mentor_kl > 0:
        seqs = 0
        t0 = time.perf_counter()
        while True:
            sl = slice(seqs % B, seqs % B + 4)
            O.mentored_spec_verify(tf[sl], df[sl], drafts[sl], u[sl], T, k, P,
                                   np.float32(mentor_kl))
            seqs += tf[sl].shape[0]
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
        return {"value": seqs * (2 * K + 1) * V / dt, "unit": "logit elems/s", "cores": 1,
                "kind": "oracle",
                "sample": f"{seqs} sequences in groups of 4 ({(2 * K + 1) * V} logits each), "
                          f"{dt:.1f} s, numpy float64, one process"}
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.spec_verify(tf, df, drafts, u, T, k, P, np.float32(cfg["lenience"]))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    elems = reps * B * (2 * K + 1) * V
    return {"value": elems / dt, "unit": "logit elems/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole steps ({B} sequences, {B * (2 * K + 1) * V} logits each), "
                      f"{dt:.1f} s, numpy float64, one process"}


def cpu_baseline_tree(logits, parent, tokens, max_depth, seconds):
    """Time the CPU oracle's tree walk on the same inputs, whole steps repeated."""
    import oracle.spec_verify_oracle as O
    x = logits.float().cpu().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.tree_verify(x, parent, tokens, max_depth)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    B, N, V = x.shape
    return {"value": reps * B * N * V / dt, "unit": "logit elems/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} whole steps ({B} trees of {N} nodes, {B * N * V} logits each), "
                      f"{dt:.1f} s, numpy float64, one process"}


def _elapsed(hip, a, b):
    f = ctypes.c_float()
    hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
    return f.value


def bench_tree(args, name, cfg):
    """Greedy token-tree verification: a step is one spec_verify_tree call over the batch.  The
    logits (131 MB per set) would fit the 256 MB last-level cache, so the timed steps rotate
    through 8 independently generated input sets."""
    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, N, V, D = cfg["B"], cfg["N"], cfg["V"], cfg["max_depth"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = []
    for seed in range(1, 9):
        logits, parent, tokens = S.workload_inputs(name, device=dev, seed=seed)
        sets.append((logits, torch.from_numpy(np.asarray(parent, np.int32)).to(dev),
                     torch.from_numpy(np.asarray(tokens, np.int32)).to(dev), parent, tokens))
    out = svm.spec_verify_tree(sets[0][0], sets[0][1], sets[0][2], D)
    torch.cuda.synchronize()
    hip = _hip_runtime()

    def new_event():
        return _new_event(hip, args.fenced_events)

    evs = [[new_event() for _ in range(3)] for _ in range(args.steps)]
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
    # the same steps again with per-phase events, for the kernel durations
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        svm.spec_verify_tree(s[0], s[1], s[2], D, out=out, events=evs[i])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    _copy_reference(args, dev)
    kern_ms = [_elapsed(hip, e[0], e[1]) for e in evs]
    step_ms = [_elapsed(hip, e[0], e[2]) for e in evs]
    for row in evs:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    elems = B * N * V
    logit_bytes = elems * sets[0][0].element_size()
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = float(np.mean(kern_ms))
    achieved = logit_bytes / (kern_avg * 1e-3) / 1e9
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
                     "traffic": _traffic_from_profiles("k_chunk_argmax", name), "kernel_ms": kern_avg,
                     "algorithmic_bytes_per_launch": logit_bytes},
        "gpu_event_ms_per_step": float(np.median(step_ms)),
        "ms_per_step_with_phase_events": wall_ev * 1e3 / args.steps,
        "mean_accepted_depth": float(out["num_accepted"].float().mean().item()),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if not args.no_cpu_baseline:
        s = sets[0]
        res["cpu_baseline"] = cpu_baseline_tree(s[0], s[3], s[4], D, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def bench_rest(args, name, cfg):
    """REST draft-tree construction: a step is one spec_build_tree call over the batch (one
    workgroup per sequence; latency-bound: the data are a few hundred KB)."""
    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    B, M, L, N = cfg["B"], cfg["M"], cfg["L"], cfg["N"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cands = S.workload_inputs(name, device=dev, seed=1)
    out = svm.spec_build_tree(cands, N)
    torch.cuda.synchronize()
    hip = _hip_runtime()
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    evs = [[_new_event(hip, args.fenced_events) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        svm.spec_build_tree(cands, N, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        svm.spec_build_tree(cands, N, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(args.steps):
        hip.hipEventRecord(ctypes.c_void_p(evs[i][0]), stream)
        svm.spec_build_tree(cands, N, out=out)
        hip.hipEventRecord(ctypes.c_void_p(evs[i][1]), stream)
    torch.cuda.synchronize()
    kern_ms = [_elapsed(hip, e[0], e[1]) for e in evs]
    for row in evs:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))
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
        "mean_nodes": float(out["num_nodes"].float().mean().item()),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if not args.no_cpu_baseline:
        import oracle.spec_verify_oracle as O
        c = cands.cpu().numpy()
        done = 0
        t0 = time.perf_counter()
        while True:
            O.rest_build_tree(c[done % B], N)
            done += 1
            dt = time.perf_counter() - t0
            if dt >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": done / dt, "unit": "trees/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{done} trees of the same batch, {dt:.1f} s, one "
                                         "process"}
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
    import numpy as np
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


def _copy_reference(args, dev):
    """A plain copy kernel of known size, for calibrating rocprofv3 byte counters."""
    import torch
    if args.copy_reference_mib > 0:
        src = torch.empty(args.copy_reference_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="workload name (default: the metric one)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle timing budget: whole steps are repeated until it is spent")
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
                    help="after the timed steps, copy a tensor of this size 3 times (a plain "
                         "copy kernel of known size for calibrating rocprofv3 byte counters); "
                         "0 disables")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the verify step is data-parallel over sequences and needs no exchange, so "
              "N GPUs would each run this benchmark on their own share)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_sampling_verification_amd as svm
    from workloads import synthetic as S

    name = args.workload or S.METRIC_WORKLOAD
    cfg = dict(S.WORKLOADS[name])
    if args.lenience is not None:
        cfg["lenience"] = args.lenience
    if cfg["gen"] == "tree":
        bench_tree(args, name, cfg)
        return
    if cfg["gen"] == "rest":
        bench_rest(args, name, cfg)
        return
    if args.pipeline:
        bench_pipeline(args, name, cfg)
        return
    B, K, V = cfg["B"], cfg["K"], cfg["V"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    target, draft = S.workload_inputs(name, device=dev, seed=1)
    kw = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"],
              lenience=cfg["lenience"], mentor_kl=args.mentor_kl, want_probs=not args.no_probs)
    u_draw = torch.from_numpy(S.philox_uniforms(2, (B * K,))).to(dev)
    drafts = svm.spec_sample(draft.view(B * K, V), u_draw, temperature=cfg["temperature"],
                             top_k=cfg["top_k"], top_p=cfg["top_p"]).view(B, K)
    u = torch.from_numpy(S.philox_uniforms(3, (B, K + 1))).to(dev)
    out = svm.spec_verify(target, draft, drafts, u, **kw)
    torch.cuda.synchronize()

    hip = _hip_runtime()

    def new_event():
        return _new_event(hip, args.fenced_events)

    evs = [[new_event() for _ in range(3)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        svm.spec_verify(target, draft, drafts, u, out=out, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        svm.spec_verify(target, draft, drafts, u, out=out, **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same steps again with per-phase events (each record idles the GPU for a few
    # microseconds, so they stay out of the throughput loop), for the kernel durations
    t0 = time.perf_counter()
    for i in range(args.steps):
        svm.spec_verify(target, draft, drafts, u, out=out, events=evs[i], **kw)
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    # the same step captured once in a HIP graph and replayed K times: the launch path of a
    # serving loop that replays its verify step (reported beside `value`, which is eager)
    graph_ms = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            svm.spec_verify(target, draft, drafts, u, out=out, **kw)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    def elapsed(a, b):
        return _elapsed(hip, a, b)

    _copy_reference(args, dev)

    kern_ms = [elapsed(e[0], e[1]) for e in evs]
    step_ms = [elapsed(e[0], e[2]) for e in evs]
    gpu_region_ms = elapsed(evs[0][0], evs[-1][2])
    for row in evs:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))

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
    else:
        dominant = "k_chunk"
    traffic = _traffic_from_profiles(dominant, name)
    n = out["num_accepted"].cpu().numpy()
    a = out["accept_prob"].cpu().numpy() if "accept_prob" in out else None
    mentored = args.mentor_kl > 0
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
                   "mentor_kl": args.mentor_kl, "accept_probs_requested": not args.no_probs},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel_ms": kern_avg,
                     "algorithmic_bytes_per_launch": logit_bytes},
        "rows_per_s": B * (2 * K + 1) / (ms_per_step * 1e-3),
        "step_gbs": logit_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_hbm_peak": logit_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "gpu_event_ms_per_step": float(np.median(step_ms)),
        "gpu_region_ms_per_step": gpu_region_ms / args.steps,
        "ms_per_step_with_phase_events": wall_ev * 1e3 / args.steps,
        "graph_ms_per_step": graph_ms,
        "mean_accept_prob": float(a.mean()) if a is not None and a.size else None,
        "mean_tokens_per_call": float(n.mean() + 1.0),
        "accepted_hist": np.bincount(n, minlength=K + 1).tolist(),
        "timing_events": "system fence" if args.fenced_events else "no system fence",
        "source_sha256_12": _source_tag(),
    }
    if args.mentor_kl == 0.0:
        res["analytics"] = _analytics(svm, target, draft, kw, K, float(n.mean() + 1.0),
                                      (drafts, u))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(name, target, draft, args.cpu_seconds,
                                           args.mentor_kl, cfg["lenience"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
