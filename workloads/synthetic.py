"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only makes inputs: logits with the value distributions of the five verify
workloads, draft-token trees, and uniforms.  It holds none of the verification arithmetic
(no temperature, truncation, softmax, acceptance or resampling), so both the CPU oracle and
the HIP path can consume what it produces without sharing any of the method's code.

Recipes (all noise is i.i.d. per element and fresh for every row):

* ``normal``  (small fp32 case and the B=64 bf16 case): draft d ~ N(0, sd^2),
  target t = scale * d + N(0, noise^2).  Target row K has a fresh, unstored draft row behind it.
* ``zipf``    (B=256 K=7 V=128256 bf16 top-k case, the same shape with top-k 256 + top-p 0.9, and
  B=128 K=3 V=256000 fp32 top-p case):
  per (sequence, position) a random permutation gives each token a rank r in 1..V;
  base = -s*ln(r) + sigma*N(0,1); target = base + sigma*N(0,1) and draft = base + sigma*N(0,1),
  the target and draft rows of one position sharing ``base``.
* ``tree``    (REST-style greedy tree, B=32 N=64 V=32000 bf16): BFS expansion from node 0,
  each expanded node of depth < max_depth gets U{1..4} children until N nodes exist; node
  tokens are uniform over the vocabulary; logits N(0,1).  ``planted`` raises, for each
  internal node with probability 0.8, the logit of one random child's token to the row
  maximum + 1, so that accepted paths are non-trivial.
* ``rest``    (REST draft-tree construction, B=32 sequences x M=64 retrieved candidates of up
  to L=8 tokens, trees of N=64 nodes, token ids < 32000): per sequence, candidates are walks of
  a random order-1 chain from one start token; each token's successors are ``branch`` random
  token ids with probabilities proportional to 1/rank^s, drawn once per token, so that
  candidates share prefixes as retrieved continuations do; lengths are uniform in
  [L/2, L] (-1 after the end).
* uniforms: numpy Philox(seed) raw 64-bit words w -> float32((w >> 40) * 2^-24), which lies
  in [0, 1 - 2^-24] and converts exactly.

Large tensors are generated with torch on the requested device (seeded torch.Generator), small
integer structures and uniforms with numpy Philox on the host.
"""

from __future__ import annotations

import numpy as np
import torch

# Workload table: name -> parameters (shapes, dtype, generator, sampling parameters).
WORKLOADS = {
    "normal_B1_K4_V1000_f32": dict(
        B=1, K=4, V=1000, dtype="f32", gen="normal", draft_sd=2.0, scale=1.0, noise=0.5,
        temperature=1.0, top_k=0, top_p=1.0, lenience=1.0, steps=1000),
    "normal_B64_K4_V32000_bf16": dict(
        B=64, K=4, V=32000, dtype="bf16", gen="normal", draft_sd=3.0, scale=0.8, noise=1.5,
        temperature=1.0, top_k=0, top_p=1.0, lenience=1.0),
    "zipf_B256_K7_V128256_bf16_topk50": dict(
        B=256, K=7, V=128256, dtype="bf16", gen="zipf", s=1.1, sigma=1.0,
        temperature=0.7, top_k=50, top_p=1.0, lenience=1.0),
    "zipf_B256_K7_V128256_bf16_topk256_topp90": dict(
        B=256, K=7, V=128256, dtype="bf16", gen="zipf", s=1.1, sigma=1.0,
        temperature=0.7, top_k=256, top_p=0.9, lenience=1.0),
    "zipf_B128_K3_V256000_f32_topp95": dict(
        B=128, K=3, V=256000, dtype="f32", gen="zipf", s=1.1, sigma=2.0,
        temperature=1.0, top_k=0, top_p=0.95, lenience=1.0),
    "tree_B32_N64_V32000_bf16": dict(
        B=32, N=64, V=32000, dtype="bf16", gen="tree", max_depth=6, branch_max=4,
        planted=True),
    "rest_B32_M64_L8_N64": dict(
        B=32, M=64, L=8, N=64, V=32000, gen="rest", branch=4, s=1.2),
}

METRIC_WORKLOAD = "zipf_B256_K7_V128256_bf16_topk50"


def torch_dtype(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def philox_uniforms(seed, shape):
    """float32 uniforms in [0, 1 - 2^-24] from numpy's Philox bit generator."""
    bg = np.random.Philox(int(seed))
    n = int(np.prod(shape))
    raw = bg.random_raw(n).astype(np.uint64)
    u = (raw >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)
    return u.astype(np.float32).reshape(shape)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_logits(B, K, V, draft_sd, scale, noise, dtype="f32", device="cpu", seed=0):
    """(target [B, K+1, V], draft [B, K, V]) with draft ~ N(0, sd^2), target = scale*d + N(0, noise^2)."""
    g = _gen(device, seed)
    d = torch.randn((B, K + 1, V), generator=g, device=device, dtype=torch.float32) * draft_sd
    t = scale * d + noise * torch.randn((B, K + 1, V), generator=g, device=device,
                                        dtype=torch.float32)
    dt = torch_dtype(dtype)
    return t.to(dt).contiguous(), d[:, :K].to(dt).contiguous()


def zipf_logits(B, K, V, s=1.1, sigma=1.0, dtype="bf16", device="cpu", seed=0, chunk_rows=256):
    """(target [B, K+1, V], draft [B, K, V]) from the log-rank (Zipf) recipe described above."""
    g = _gen(device, seed)
    dt = torch_dtype(dtype)
    target = torch.empty((B, K + 1, V), dtype=dt, device=device)
    draft = torch.empty((B, K, V), dtype=dt, device=device)
    tflat = target.view(B * (K + 1), V)
    rows = B * (K + 1)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        n = r1 - r0
        rank = torch.argsort(torch.rand((n, V), generator=g, device=device), dim=1) + 1
        base = -s * torch.log(rank.to(torch.float32))
        del rank
        base += sigma * torch.randn((n, V), generator=g, device=device)
        t = base + sigma * torch.randn((n, V), generator=g, device=device)
        d = base + sigma * torch.randn((n, V), generator=g, device=device)
        tflat[r0:r1] = t.to(dt)
        rows_here = torch.arange(r0, r1, device=device)
        b_idx, k_idx = rows_here // (K + 1), rows_here % (K + 1)
        has_draft = k_idx < K
        if bool(has_draft.any()):
            dflat = draft.view(B * K, V)
            dflat[(b_idx * K + k_idx)[has_draft]] = d[has_draft].to(dt)
    return target, draft


def tree_structure(B, N, max_depth=6, branch_max=4, seed=0):
    """parent [B, N] int32 (parent[:,0] = -1, BFS order) and depth [B, N] int32."""
    rng = np.random.Generator(np.random.Philox(int(seed)))
    parent = np.full((B, N), -1, dtype=np.int32)
    depth = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        while True:
            par = [-1]
            dep = [0]
            frontier = 0
            while len(par) < N and frontier < len(par):
                if dep[frontier] < max_depth:
                    nchild = int(rng.integers(1, branch_max + 1))
                    for _ in range(nchild):
                        if len(par) == N:
                            break
                        par.append(frontier)
                        dep.append(dep[frontier] + 1)
                frontier += 1
            if len(par) == N:
                break  # otherwise the tree ran out of expandable nodes: draw again
        parent[b] = par
        depth[b] = dep
    return parent, depth


def tree_inputs(B, N, V, max_depth=6, branch_max=4, planted=True, dtype="bf16", device="cpu",
                seed=0):
    """(logits [B, N, V], parent [B, N] int32, node_tokens [B, N] int32) for the tree workload."""
    parent, _ = tree_structure(B, N, max_depth, branch_max, seed)
    rng = np.random.Generator(np.random.Philox(int(seed) + 7))
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    g = _gen(device, seed)
    logits = torch.randn((B, N, V), generator=g, device=device, dtype=torch.float32)
    if planted:
        for b in range(B):
            children = {}
            for i in range(1, N):
                children.setdefault(int(parent[b, i]), []).append(i)
            for node, kids in children.items():
                if rng.random() < 0.8:
                    child = kids[int(rng.integers(0, len(kids)))]
                    row = logits[b, node]
                    row[int(tokens[b, child])] = row.max() + 1.0
    return logits.to(torch_dtype(dtype)).contiguous(), parent, tokens


def rest_candidates(B, M, L, V, branch=4, s=1.2, seed=0):
    """candidates [B, M, L] int32 for the REST tree builder (recipe in the module header)."""
    rng = np.random.Generator(np.random.Philox(int(seed) + 11))
    probs = 1.0 / np.arange(1, branch + 1, dtype=np.float64) ** s
    probs /= probs.sum()
    out = np.full((B, M, L), -1, dtype=np.int32)
    for b in range(B):
        succ = {}
        start = int(rng.integers(0, V))
        for m in range(M):
            n = int(rng.integers((L + 1) // 2, L + 1))
            cur = start
            for t in range(n):
                if cur not in succ:
                    succ[cur] = rng.integers(0, V, size=branch)
                cur = int(succ[cur][int(rng.choice(branch, p=probs))])
                out[b, m, t] = cur
    return out


def workload_inputs(name, device="cpu", seed=0, **override):
    """Logits (+ tree structure) for a named workload; sizes may be overridden for tests."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    if cfg["gen"] == "normal":
        return normal_logits(cfg["B"], cfg["K"], cfg["V"], cfg["draft_sd"], cfg["scale"],
                             cfg["noise"], cfg["dtype"], device, seed)
    if cfg["gen"] == "zipf":
        return zipf_logits(cfg["B"], cfg["K"], cfg["V"], cfg["s"], cfg["sigma"], cfg["dtype"],
                           device, seed)
    if cfg["gen"] == "tree":
        return tree_inputs(cfg["B"], cfg["N"], cfg["V"], cfg["max_depth"], cfg["branch_max"],
                           cfg["planted"], cfg["dtype"], device, seed)
    if cfg["gen"] == "rest":
        c = rest_candidates(cfg["B"], cfg["M"], cfg["L"], cfg["V"], cfg["branch"], cfg["s"], seed)
        return torch.from_numpy(c).to(device)
    raise KeyError(name)


def logit_elements(name):
    """Logit elements one verify step reads: B*(2K+1)*V (tree: B*N*V)."""
    cfg = WORKLOADS[name]
    if cfg["gen"] == "tree":
        return cfg["B"] * cfg["N"] * cfg["V"]
    return cfg["B"] * (2 * cfg["K"] + 1) * cfg["V"]


def elem_bytes(name):
    return 2 if WORKLOADS[name]["dtype"] == "bf16" else 4

