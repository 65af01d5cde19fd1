"""GPU-vs-oracle parity checks (used by the GPU tests, smoke() and the benchmark's sampled
oracle check).

Inputs come from ``workloads.synthetic`` (seeded), draft tokens from the oracle's own draft
sampler, uniforms from numpy Philox; the same arrays go to the HIP library and to the oracle.

The bar (fixed for this method): accepted counts and tokens bit-exact, probabilities (a_k,
q_k(x~), p_k(x~)) within 1e-5 absolute + 1e-4 relative, except boundary flips, where a
floating-point decision sits within 1e-6 of its threshold.  Three kinds are admitted, each
counted:

  accept  an accept test decided the other way with |u_k - a_k| < 1e-6;
  draw    a final token whose CDF interval [C_{i-1}, C_i) lies within 1e-6 W of u W;
  topp    a row whose top-p running sum passes P within 1e-6 of it, read with a neighbouring
          cut: the GPU kept the oracle's set cut at another position j whose running sum c_j
          lies within 1e-6 of P (the oracle's distribution at nucleus P' = c_j, |P' - P| < 1e-6).

Every decision is checked against the oracle on exactly the rows it reads.  Accept test k reads
target row k and draft row k, and so does the final draw when the sequence stops at k; the bonus
draw reads target row K.  For each position the checker looks for one reading of that position's
two rows (the oracle's own first; the top-p alternatives only for rows inside the band) under
which every GPU output of the position equals the oracle's: the probabilities within tolerance,
the accept decision and the drawn token, up to accept and draw flips.  A reading of a row is
never used for a decision that does not read that row, and one reading must explain all the
outputs that read it.  Among the explanations, the one with the fewest flips is counted.
"""

import os
from collections import Counter

import numpy as np

import oracle.spec_verify_oracle as O

FLIP_BAND = 1e-6
ATOL, RTOL = 1e-5, 1e-4
FLIP_KINDS = ("accept", "draw", "topp")

# (case label, flip counts, sequences checked) of every check in this process; the test
# session prints them (tests/conftest.py) and the benchmark puts its own into its JSON line.
FLIP_LOG = []


# ---------------------------------------------------------------------------------- inputs
def make_inputs(target, draft, params, seed):
    """Draft tokens (oracle sampler on the draft rows) and uniforms for given logits."""
    from workloads import synthetic as S
    B, K1, V = target.shape
    K = K1 - 1
    df = draft.float().cpu().numpy() if K > 0 else None
    if K > 0:
        u_draw = S.philox_uniforms(seed + 1, (B, K))
        drafts = np.stack([O.sample_rows(df[:, k], u_draw[:, k], params["temperature"],
                                         params.get("top_k", 0), params.get("top_p", 1.0))
                           for k in range(K)], axis=1).astype(np.int32)
    else:
        drafts = np.zeros((B, 0), dtype=np.int32)
    u = S.philox_uniforms(seed + 2, (B, K + 1))
    return drafts, u


def run_gpu(target, draft, drafts, u, params, device="cuda"):
    import torch
    import speculative_sampling_verification_amd as svm
    t = target.to(device)
    d = draft.to(device) if draft is not None else None
    x = torch.from_numpy(np.ascontiguousarray(drafts)).to(device)
    uu = torch.from_numpy(np.ascontiguousarray(u)).to(device)
    out = svm.spec_verify(t, d, x, uu, temperature=params["temperature"],
                          top_k=params.get("top_k", 0), top_p=params.get("top_p", 1.0),
                          lenience=params.get("lenience", 1.0),
                          mentor_kl=params.get("mentor_kl", 0.0),
                          want_probs=params.get("want_probs", True))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _np(x):
    """Host float32 array of a torch tensor (on any device) or an array."""
    if x is None:
        return None
    if hasattr(x, "cpu") and hasattr(x, "float"):
        return x.float().cpu().numpy()
    return np.asarray(x, dtype=np.float32)


def _samp(params):
    return (np.float32(params["temperature"]), int(params.get("top_k", 0)),
            np.float32(params.get("top_p", 1.0)))


def run_oracle(target, draft, drafts, u, params):
    """The lossless oracle on the whole batch (its own reading of every row)."""
    tf = _np(target)
    df = _np(draft) if draft is not None else np.zeros((tf.shape[0], 0, tf.shape[2]))
    T, k, P = _samp(params)
    return O.spec_verify(tf, df, drafts, u, T, k, P, np.float32(params.get("lenience", 1.0)))


def run_oracle_mentored(target, draft, drafts, u, params):
    T, k, P = _samp(params)
    return O.mentored_spec_verify(_np(target), _np(draft), drafts, u, T, k, P,
                                  np.float32(params["mentor_kl"]))


# ---------------------------------------------------------------------------------- rules
class Lossless:
    """Accept test and final weights of the lossless rule with lenience l (the oracle's steps:
    accept_probability, then residual_weights, i.e. (q - p)_+ or q when that has no mass)."""

    def __init__(self, lenience=1.0):
        self.lenience = np.float32(lenience)

    def position(self, q, p, x):
        V = q.size
        inside = 0 <= x < V
        q_x = float(q[x]) if inside else 0.0
        p_x = float(p[x]) if inside else 0.0
        return {"a": float(O.accept_probability(q_x, p_x, self.lenience)), "q_x": q_x,
                "p_x": p_x, "weights": lambda: O.residual_weights(q, p)[0]}


class Mentored:
    """Mentored decoding with KL bound D: a = r at the draft token, replacement weights w (q
    when w has no mass), as the oracle's mentored_verify_sequence takes them."""

    def __init__(self, D):
        self.D = np.float32(D)

    def position(self, q, p, x):
        V = q.size
        sol = O.mentored_solve(q, p, self.D)
        inside = 0 <= x < V
        q_x = float(q[x]) if inside else 0.0
        p_x = float(p[x]) if inside else 0.0
        a = float(sol["r"][x]) if inside and (q_x > 0 or p_x > 0) else 0.0

        def weights():
            w = sol["w"]
            return w if np.sum(w) > 0 else q
        return {"a": a, "q_x": q_x, "p_x": p_x, "weights": weights}


def rule_for(params):
    if params.get("mentor_kl", 0.0) > 0 and params["temperature"] > 0:
        return Mentored(params["mentor_kl"])
    return Lossless(params.get("lenience", 1.0))


# ---------------------------------------------------------------------------------- readings
def row_readings(z, temperature, top_k, top_p):
    """The admissible distributions of one row: the oracle's own first, then (only when its
    top-p running sum passes P within FLIP_BAND) the distributions cut at each other position j
    whose running sum lies within FLIP_BAND of P -- the oracle at nucleus P' = c_j.  A GPU whose
    running sums are off by less than the band can only cut at one of these."""
    d = {}
    base = O.row_distribution(z, temperature, top_k, top_p, d)
    out = [base]
    if d.get("topp_margin", np.inf) < FLIP_BAND:
        c, js = d["topp_cumsum"], d["topp_cut"]
        P = float(top_p)
        lo = int(np.searchsorted(c, P - FLIP_BAND, side="right"))  # first c_j > P - band
        hi = min(int(np.searchsorted(c, P + FLIP_BAND, side="left")), c.size - 1)
        seen = {np.packbits(base > 0).tobytes()}
        for j in range(lo, hi + 1):
            if j == js:
                continue
            alt = O.row_distribution(z, temperature, top_k, float(c[j]))
            sig = np.packbits(alt > 0).tobytes()
            if sig not in seen:
                seen.add(sig)
                out.append(alt)
    return out


# ---------------------------------------------------------------------------------- checks
def _close(g, o):
    return abs(float(g) - float(o)) <= ATOL + RTOL * abs(float(o))


def check_sequence(gb, rows_t, rows_d, drafts_b, u_b, rule, label=""):
    """Check one sequence's GPU outputs gb = {n, tokens[K+1], and optionally a, q, p [K]}
    against the oracle.  rows_t[k] / rows_d[k] are the admissible readings of target / draft row
    k (the oracle's own first).  Returns (flips Counter, oracle n, oracle tokens) where the
    oracle's values are those of its own readings."""
    K = len(drafts_b)
    ng = int(gb["n"])
    tok = np.asarray(gb["tokens"]).astype(np.int64)
    uK = float(u_b[K])
    if not 0 <= ng <= K:
        raise AssertionError(f"{label}: accepted count {ng} outside [0, {K}]")
    np.testing.assert_array_equal(tok[:ng], np.asarray(drafts_b[:ng], dtype=np.int64),
                                  err_msg=f"{label}: accepted drafts")
    assert (tok[ng + 1:] == -1).all(), f"{label}: padding after position {ng}: {tok}"
    flips = Counter()
    cache = {}

    def position(k, i, j):  # the rule at position k under readings i (target) and j (draft)
        if (k, i, j) not in cache:
            cache[(k, i, j)] = rule.position(rows_t[k][i], rows_d[k][j], int(drafts_b[k]))
        return cache[(k, i, j)]

    # the oracle's own outcome (readings 0): its n and tokens
    n_o, tok_o = K, None
    for k in range(K + 1):
        if k < K:
            pos = position(k, 0, 0)
            if float(u_b[k]) < pos["a"]:
                continue
            n_o = k
            tok_o = O.inverse_cdf(pos["weights"](), uK)
        else:
            tok_o = O.inverse_cdf(rows_t[K][0], uK)
        break
    oracle_tokens = np.full(K + 1, -1, dtype=np.int64)
    oracle_tokens[:n_o] = np.asarray(drafts_b[:n_o], dtype=np.int64)
    oracle_tokens[n_o] = tok_o

    for k in range(K):
        best, failures = None, []
        for i in range(len(rows_t[k])):
            for j in range(len(rows_d[k])):
                pos = position(k, i, j)
                f = Counter(topp=int(i > 0) + int(j > 0))
                why = None
                if "a" in gb:
                    for key, ov in (("a", pos["a"]), ("q", pos["q_x"]), ("p", pos["p_x"])):
                        if why is None and not _close(gb[key][k], ov):
                            why = f"{key}={float(gb[key][k])!r} vs oracle {ov!r}"
                if why is None and k <= ng:
                    acc_o = float(u_b[k]) < pos["a"]
                    if acc_o != (k < ng):
                        if abs(float(u_b[k]) - pos["a"]) < FLIP_BAND:
                            f["accept"] += 1
                        else:
                            why = (f"GPU {'accepted' if k < ng else 'rejected'} with "
                                   f"u={float(u_b[k])!r}, oracle a={pos['a']!r}")
                if why is None and k == ng:
                    w = pos["weights"]()
                    t_o = O.inverse_cdf(w, uK)
                    if t_o != tok[ng]:
                        if O.inverse_cdf_margin(w, uK, int(tok[ng])) < FLIP_BAND:
                            f["draw"] += 1
                        else:
                            why = f"final token {tok[ng]} vs oracle {t_o}"
                if why is None:
                    cost = sum(f.values())
                    if best is None or cost < best[0]:
                        best = (cost, f)
                else:
                    failures.append(f"reading ({i},{j}): {why}")
                if best is not None and best[0] == 0:
                    break
            if best is not None and best[0] == 0:
                break
        if best is None:
            raise AssertionError(f"{label} position {k} (GPU n={ng}, oracle n={n_o}): no "
                                 f"admissible reading explains the GPU: {failures[:4]}")
        flips.update(best[1])
    if ng == K:
        best, failures = None, []
        for i, qt in enumerate(rows_t[K]):
            f = Counter(topp=int(i > 0))
            t_o = O.inverse_cdf(qt, uK)
            if t_o != tok[K]:
                if O.inverse_cdf_margin(qt, uK, int(tok[K])) < FLIP_BAND:
                    f["draw"] += 1
                else:
                    failures.append(f"reading {i}: bonus token {tok[K]} vs oracle {t_o}")
                    continue
            if best is None or sum(f.values()) < best[0]:
                best = (sum(f.values()), f)
            if best[0] == 0:
                break
        if best is None:
            raise AssertionError(f"{label} bonus draw: {failures[:4]}")
        flips.update(best[1])
    return flips, n_o, oracle_tokens


def check(g, target, draft, drafts, u, params, max_flip_frac=0.02, rule=None, label=None,
          max_flips=None):
    """Check GPU results g (spec_verify's dict, numpy) for every sequence of target [B, K+1, V]
    / draft [B, >=K, V] (torch or numpy, on the host) with drafts [B, K] and u [B, K+1].

    Returns (flips, oracle) with flips = {accept, draw, topp} counts and oracle = {n, tokens}
    from the oracle's own readings.  Raises AssertionError on any difference that is not a
    counted boundary flip, or when the flips exceed max_flips (default: max(1, max_flip_frac *
    B), or 0 when max_flip_frac is 0)."""
    tf = _np(target)
    df = _np(draft)
    B, K1, V = tf.shape
    K = K1 - 1
    T, k_, P = _samp(params)
    rule = rule or rule_for(params)
    label = label or os.environ.get("PYTEST_CURRENT_TEST", "check").split(" ")[0]
    flips = Counter({kind: 0 for kind in FLIP_KINDS})
    o_n = np.zeros(B, dtype=np.int64)
    o_tok = np.full((B, K + 1), -1, dtype=np.int64)
    for b in range(B):
        rows_t = [row_readings(tf[b, i], T, k_, P) for i in range(K + 1)]
        rows_d = [row_readings(df[b, i], T, k_, P) for i in range(K)]
        gb = {"n": g["num_accepted"][b], "tokens": g["tokens"][b]}
        if "accept_prob" in g and K > 0:
            gb.update(a=g["accept_prob"][b], q=g["q_draft"][b], p=g["p_draft"][b])
        f, o_n[b], o_tok[b] = check_sequence(gb, rows_t, rows_d, drafts[b], u[b], rule,
                                             f"{label} seq {b}")
        flips.update(f)
    flips = {kind: int(flips[kind]) for kind in FLIP_KINDS}
    FLIP_LOG.append((label, flips, B))
    print(f"[flips] {label}: {flips} over {B} sequences", flush=True)
    if max_flips is None:
        max_flips = 0 if max_flip_frac == 0 else max(1, int(max_flip_frac * B))
    assert sum(flips.values()) <= max_flips, (flips, max_flips)
    return flips, {"n": o_n, "tokens": o_tok}


def verify_case(target, draft, params, seed=0, max_flip_frac=0.02, rule=None, drafts=None,
                u=None):
    """Full parity check of spec_verify on given logits (mentored decoding when
    params["mentor_kl"] > 0, unless ``rule`` says otherwise); returns (flips, gpu, oracle)."""
    d0, u0 = make_inputs(target, draft, params, seed)
    drafts = d0 if drafts is None else drafts
    u = u0 if u is None else u
    g = run_gpu(target, draft, drafts, u, params)
    flips, o = check(g, target, draft, drafts, u, params, max_flip_frac, rule)
    return flips, g, o


verify_mentored_case = verify_case
