"""Plain CPU oracle for speculative-sampling verification (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import this
module.  The product path (the HIP library and its Python binding) never calls it and shares
no code with it.

Everything is computed in float64 with numpy, one row / one sequence at a time, in vocabulary
index order, so that each step can be checked against the pages by eye.  Notation follows the
page "Accelerating Large Language Model Decoding with Speculative Sampling" (Chen et al.
notes): q is the TARGET model's distribution, p the DRAFT model's, x~ a draft token, K the
number of draft tokens per call.  The page on "Fast Inference from Transformers via
Speculative Decoding" (Leviathan et al. blog) uses the opposite letters; its formulas are
restated here in the q=target / p=draft convention.

Where the pages leave a step open, the reading used is stated next to the step.

Pinning status: every public function here is pinned by tests under ``tests/`` that compare it
with closed forms, brute force, library routines or values printed on the pages (the REST tree
builder against a worked example built from the prefixes the REST article names, and brute
force over random candidate sets).
``expected_tokens_per_call`` and ``walltime_speedup`` / ``ops_factor`` are pinned to the values
printed on the Leviathan page (App. E figures); no function is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "row_distribution",
    "accept_probability",
    "residual_weights",
    "inverse_cdf",
    "inverse_cdf_margin",
    "verify_sequence",
    "verify_sequence_trials",
    "spec_verify",
    "sample_rows",
    "tree_verify",
    "rest_trie",
    "rest_build_tree",
    "philox4x64",
    "philox_uniforms",
    "kl_divergence",
    "mentored_solve",
    "mentored_verify_sequence",
    "mentored_spec_verify",
    "expected_tokens_per_call",
    "walltime_speedup",
    "ops_factor",
    "acceptance_rate",
    "optimal_gamma",
]


# ---------------------------------------------------------------------------------------------
# Per-row distribution: temperature, then top-k, then top-p.
#
# Page "Accelerating Large Language Model Decoding with Speculative Sampling", section A2
# (方法细节), paragraph on compatibility with standard sampling methods: nucleus, top-k and
# temperature are applied to the probabilities before the rejection scheme.  The Leviathan blog,
# section 方法细节 ("标准化采样框架"), says the same: argmax, top-k, nucleus and temperature are
# all a standard draw from an adjusted distribution.
#
# Readings (the pages are silent on these details):
#   * order: temperature -> top-k -> top-p, the same parameters for q and p;
#   * temperature 0 means argmax (one-hot, lowest index wins ties);
#   * top-k keeps every logit >= the k-th largest logit (ties at the boundary all kept);
#   * top-p keeps the smallest prefix of the probabilities sorted in decreasing order whose
#     running sum reaches P, plus every token tied with the last one taken, and renormalises;
#     when top-k is also on, top-p acts on the renormalised top-k distribution.
# ---------------------------------------------------------------------------------------------
def row_distribution(z, temperature, top_k=0, top_p=1.0, diagnostics=None):
    """Return the float64 probability vector of one row of logits ``z``.

    ``temperature``, ``top_p`` are used as float64 values of whatever the caller passes (the
    tests pass float32 values, the same numbers the GPU library receives).  ``diagnostics``,
    if a dict, receives ``topp_margin``: the distance of the running sum from P at the top-p
    boundary (min over the last excluded and the first included prefix), which says how close
    a floating-point decision was; when top-p is applied also ``topp_cumsum`` (the running sums
    in the order used, probability descending, index ascending) and ``topp_cut`` (the position
    j* in that order of the last token taken before ties are added).
    """
    z = np.asarray(z, dtype=np.float64).ravel()
    V = z.size
    T = float(temperature)
    if diagnostics is not None:
        diagnostics["topp_margin"] = np.inf

    if T == 0.0:
        prob = np.zeros(V)
        prob[int(np.argmax(z))] = 1.0  # np.argmax returns the first occurrence of the maximum
        return prob

    keep = np.ones(V, dtype=bool)
    k = int(top_k)
    if 0 < k < V:
        t_k = np.partition(z, V - k)[V - k]  # k-th largest logit, counted with multiplicity
        keep = z >= t_k

    y = np.full(V, -np.inf)
    y[keep] = z[keep] / T
    m = y[keep].max()
    e = np.zeros(V)
    e[keep] = np.exp(y[keep] - m)
    prob = e / e.sum()

    P = float(top_p)
    if P < 1.0:
        idx = np.arange(V)
        order = np.lexsort((idx, -prob))  # probability descending, index ascending on ties
        c = np.cumsum(prob[order])
        reached = np.nonzero(c >= P)[0]
        if reached.size:
            j_star = int(reached[0])
        else:  # rounding left the total just below P: take every kept token
            j_star = int(np.count_nonzero(prob > 0)) - 1
        t_p = prob[order[j_star]]
        if diagnostics is not None:
            before = c[j_star - 1] if j_star > 0 else 0.0
            diagnostics["topp_margin"] = float(min(abs(before - P), abs(c[j_star] - P)))
            diagnostics["topp_cumsum"] = c
            diagnostics["topp_cut"] = j_star
        keep_p = (prob >= t_p) & (prob > 0)
        prob = np.where(keep_p, prob, 0.0)
        prob = prob / prob.sum()
    return prob


# ---------------------------------------------------------------------------------------------
# Accept test.  Chen et al. notes, A2 "改进的拒绝采样": a draft token x~ drawn from p is kept
# with probability min(1, q(x~)/p(x~)).  Leviathan blog, 扩展方向 / App. F (lenience): the
# comparison is made after scaling, i.e. keep with probability min(1, q/(l p)), 0 < l <= 1.
# Edge cases (reading): p(x~)=0<q(x~) -> 1; p(x~)=q(x~)=0 -> 0 (an impossible token is rejected).
# ---------------------------------------------------------------------------------------------
def accept_probability(q_x, p_x, lenience=1.0):
    """min(1, q/(l*p)) with the edge cases above; works on scalars or arrays."""
    q_x = np.asarray(q_x, dtype=np.float64)
    p_x = np.asarray(p_x, dtype=np.float64)
    l = float(lenience)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(p_x > 0, q_x / (l * np.where(p_x > 0, p_x, 1.0)), 0.0)
    a = np.where(p_x > 0, np.minimum(1.0, ratio), np.where(q_x > 0, 1.0, 0.0))
    return a if a.ndim else float(a)


# ---------------------------------------------------------------------------------------------
# Residual distribution.  Chen et al. notes, A2 and Theorem 1: after a rejection the token is
# redrawn from (q - p)_+ where (f)_+ = max(0, f) / sum_x max(0, f).
# Reading: if the sum is 0 (q == p up to rounding, so a rejection had probability 0 in exact
# arithmetic) the draw falls back to q itself; the fallback is reported.
# With lenience the residual is left unchanged (App. F only changes the comparison).
# ---------------------------------------------------------------------------------------------
def residual_weights(q, p):
    """Return (w, fell_back): unnormalised weights max(0, q - p), or q if they sum to 0."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    w = np.maximum(0.0, q - p)
    if not w.sum() > 0.0:
        return q.copy(), True
    return w, False


# ---------------------------------------------------------------------------------------------
# Inverse-CDF draw of one index from unnormalised weights w with a uniform u in [0, 1).
# Reading (the pages only say "sample from"): cumulative sums C_i in vocabulary index order,
# W = C_{V-1}; the token is the smallest i with C_i > u*W; if rounding runs past the end, the
# last index with positive weight.
# ---------------------------------------------------------------------------------------------
def inverse_cdf(w, u):
    """Draw index/indices from weights ``w`` (1-D) using uniform(s) ``u`` (scalar or array).

    Because C is non-decreasing, the smallest i with C_i > u*W equals the number of i with
    C_i <= u*W; that count is what is computed here.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    W = C[-1]
    u_arr = np.atleast_1d(np.asarray(u, dtype=np.float64)).ravel()
    target = u_arr * W
    out = np.empty(u_arr.size, dtype=np.int64)
    block = max(1, 4_000_000 // max(1, w.size))
    for s0 in range(0, u_arr.size, block):
        s1 = min(u_arr.size, s0 + block)
        out[s0:s1] = np.count_nonzero(C[None, :] <= target[s0:s1, None], axis=1)
    positive = np.nonzero(w > 0)[0]
    last_positive = int(positive[-1]) if positive.size else w.size - 1
    out[out >= w.size] = last_positive
    return out.reshape(np.shape(u)) if np.ndim(u) else int(out[0])


def inverse_cdf_margin(w, u, tok):
    """How far u*W lies outside the CDF interval [C_{tok-1}, C_tok) of ``tok``, relative to W.

    0 means ``tok`` is exactly the inverse-CDF draw; a small positive value means ``tok`` would
    be the draw if u moved by that much (used to classify boundary flips).
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    W = C[-1]
    if not (0 <= tok < w.size) or W <= 0:
        return np.inf
    lo = C[tok - 1] if tok > 0 else 0.0
    hi = C[tok]
    target = float(u) * W
    if lo <= target < hi:
        return 0.0
    return float(min(abs(target - lo), abs(target - hi)) / W)


# ---------------------------------------------------------------------------------------------
# One verification step for one sequence (Chen et al. notes, A2 "改进的拒绝采样" and the bonus
# token paragraph; Leviathan blog, 基准设计 "草稿-验收-修正"):
#   for k = 0..K-1: a_k = accept probability of x~_k at position k; accept iff u_k < a_k;
#   n = first k that is not accepted (K if all are);
#   n < K: draw from the residual of position n with u_K;  n = K: draw the bonus token from the
#   target distribution of position K with u_K.
# Readings: one fresh uniform per accept test plus one for the final draw (u has K+1 entries);
#   strict comparison u < a, u in [0,1), so p == q always accepts; a draft token outside
#   [0, V) has p = q = 0 and is rejected.
# ---------------------------------------------------------------------------------------------
def _verify_core(q_rows, p_rows, drafts, u, lenience):
    K = len(drafts)
    V = q_rows[0].size
    q_x = np.zeros(K)
    p_x = np.zeros(K)
    for k in range(K):
        x = int(drafts[k])
        if 0 <= x < V:
            q_x[k] = q_rows[k][x]
            p_x[k] = p_rows[k][x]
    a = accept_probability(q_x, p_x, lenience) if K else np.zeros(0)
    a = np.atleast_1d(a)
    n = K
    for k in range(K):
        if not (float(u[k]) < a[k]):
            n = k
            break
    if n < K:
        w, fell_back = residual_weights(q_rows[n], p_rows[n])
    else:
        w, fell_back = np.asarray(q_rows[K], dtype=np.float64), False
    tok = inverse_cdf(w, float(u[K]))
    margin = inverse_cdf_margin(w, float(u[K]), tok)
    tokens = np.full(K + 1, -1, dtype=np.int64)
    tokens[:n] = np.asarray(drafts[:n], dtype=np.int64)
    tokens[n] = tok
    return {
        "tokens": tokens,
        "n": n,
        "a": a,
        "q_x": q_x,
        "p_x": p_x,
        "fallback": fell_back,
        "weights": w,
        "draw_margin": margin,
    }


def verify_sequence(q_rows, p_rows, drafts, u, lenience=1.0):
    """Verify one sequence given its processed distributions.

    q_rows: K+1 target probability vectors; p_rows: at least K draft probability vectors;
    drafts: K draft tokens; u: K+1 uniforms.  Returns a dict with tokens (K+1, -1 padded),
    n (accepted count), a, q_x, p_x (per position), fallback, weights of the final draw and
    draw_margin (0 unless the draw sits on a CDF boundary).
    """
    q_rows = [np.asarray(r, dtype=np.float64) for r in q_rows]
    p_rows = [np.asarray(r, dtype=np.float64) for r in p_rows]
    return _verify_core(q_rows, p_rows, list(drafts), list(u), lenience)


def verify_sequence_trials(q_rows, p_rows, drafts, u, lenience=1.0):
    """Many independent trials of one sequence with fixed rows (for statistical pins).

    drafts: [T, K] int, u: [T, K+1].  Same steps as ``verify_sequence``; each numpy call acts
    on all trials at once.  Returns (n [T], first emitted token [T], emitted tokens [T, K+1]).
    """
    q_rows = [np.asarray(r, dtype=np.float64) for r in q_rows]
    p_rows = [np.asarray(r, dtype=np.float64) for r in p_rows]
    drafts = np.asarray(drafts, dtype=np.int64)
    u = np.asarray(u, dtype=np.float64)
    trials, K = drafts.shape
    a = np.zeros((trials, K))
    for k in range(K):
        x = drafts[:, k]
        a[:, k] = accept_probability(q_rows[k][x], p_rows[k][x], lenience)
    accepted = u[:, :K] < a
    rejected_any = ~accepted
    n = np.where(rejected_any.any(axis=1), rejected_any.argmax(axis=1), K)
    final = np.empty(trials, dtype=np.int64)
    for pos in range(K + 1):
        sel = n == pos
        if not sel.any():
            continue
        if pos < K:
            w, _ = residual_weights(q_rows[pos], p_rows[pos])
        else:
            w = q_rows[K]
        final[sel] = inverse_cdf(w, u[sel, K])
    tokens = np.full((trials, K + 1), -1, dtype=np.int64)
    for pos in range(K + 1):
        sel = n == pos
        tokens[sel, :pos] = drafts[sel, :pos]
        tokens[sel, pos] = final[sel]
    return n, tokens[:, 0], tokens


def spec_verify(target_logits, draft_logits, drafts, uniforms, temperature=1.0, top_k=0,
                top_p=1.0, lenience=1.0):
    """Batch verification: target [B, K+1, V], draft [B, >=K, V], drafts [B, K], uniforms [B, K+1].

    Returns a dict of arrays: tokens [B, K+1], n [B], a / q_x / p_x [B, K], fallback [B],
    draw_margin [B], topp_margin_t [B, K+1], topp_margin_d [B, K].
    """
    target_logits = np.asarray(target_logits)
    draft_logits = np.asarray(draft_logits)
    drafts = np.asarray(drafts)
    uniforms = np.asarray(uniforms)
    B, K1, V = target_logits.shape
    K = K1 - 1
    out = {
        "tokens": np.full((B, K + 1), -1, dtype=np.int64),
        "n": np.zeros(B, dtype=np.int64),
        "a": np.zeros((B, K)),
        "q_x": np.zeros((B, K)),
        "p_x": np.zeros((B, K)),
        "fallback": np.zeros(B, dtype=bool),
        "draw_margin": np.zeros(B),
        "topp_margin_t": np.full((B, K + 1), np.inf),
        "topp_margin_d": np.full((B, K), np.inf),
    }
    for b in range(B):
        q_rows, p_rows = [], []
        for k in range(K + 1):
            d = {}
            q_rows.append(row_distribution(target_logits[b, k], temperature, top_k, top_p, d))
            out["topp_margin_t"][b, k] = d["topp_margin"]
        for k in range(K):
            d = {}
            p_rows.append(row_distribution(draft_logits[b, k], temperature, top_k, top_p, d))
            out["topp_margin_d"][b, k] = d["topp_margin"]
        r = _verify_core(q_rows, p_rows, list(drafts[b]), list(uniforms[b]), lenience)
        out["tokens"][b] = r["tokens"]
        out["n"][b] = r["n"]
        out["a"][b] = r["a"]
        out["q_x"][b] = r["q_x"]
        out["p_x"][b] = r["p_x"]
        out["fallback"][b] = r["fallback"]
        out["draw_margin"][b] = r["draw_margin"]
    return out


def sample_rows(logits, u, temperature=1.0, top_k=0, top_p=1.0):
    """Draw one token per row of ``logits`` [R, V] from its processed distribution (draft draw).

    This is the draft model's own sampling step (Chen et al. notes, A1: the draft model samples
    K tokens autoregressively), done with the same inverse-CDF rule as the final draw.
    """
    logits = np.asarray(logits)
    R = logits.shape[0]
    out = np.empty(R, dtype=np.int64)
    for r in range(R):
        prob = row_distribution(logits[r], temperature, top_k, top_p)
        out[r] = inverse_cdf(prob, float(u[r]))
    return out


# ---------------------------------------------------------------------------------------------
# Mentored decoding: the optimal lossy variant (page "推测解码的一种最优有损变体", sections 导师解码
# and 解决优化问题).  For one position with target q and draft p (the page's letters: p draft,
# q target, the same as here), choose the accept probabilities r and the replacement law s
# that maximise the chance of accepting the draft token, sum_i p_i r_i, subject to a bound D on
# the divergence of the emitted law pi_i = p_i r_i + s_i (1 - sum_j p_j r_j) from q.  The page
# states the optimum's form: r_i = min(1, q_i / (alpha p_i)) and
# s_i = max(0, q_i / beta - p_i) / (1 - sum_j p_j r_j), alpha in ]0, 1], beta fixed by alpha,
# the divergence decreasing in alpha, so alpha is found by bisection; and its speed-ups: the
# draft token is accepted without solving when u < min(1, q_x / p_x) (r_x is never smaller),
# and directly when the divergence of p itself is within D.
#
# Readings (the page's displays of the problem and of the algorithm are missing):
#   * the divergence is KL(q || pi) = sum_{q_i > 0} q_i ln(q_i / pi_i): the page's list of
#     precomputed sums (prefix sums of q_i ln(q_i / p_i) over tokens ordered by q_i / p_i)
#     evaluates exactly this, and with every draft accepted (pi = p) it is the KL(q, p) of the
#     page's direct-accept rule;
#   * trivial case KL(q || p) <= D: every draft token is accepted (r = 1, no replacement);
#   * otherwise alpha = the upper end after 50 bisection steps on [0, 1] of the condition
#     KL(q || pi_alpha) <= D (which holds at alpha = 1, where the rule is the lossless one);
#     D = 0 is the lossless rule, alpha = 1, without bisection and without the trivial-case
#     test (KL(q || p) <= 0 holds only for q = p, where the lossless rule accepts every draft
#     token anyway, so the test could only ever fire on rounding);
#   * beta solves sum_i max(0, q_i / beta - p_i) = 1 - sum_i min(p_i, q_i / alpha), so that pi
#     sums to 1; no replacement is needed when that residual mass is 0;
#   * the replacement token is drawn like the lossless one: inverse CDF in vocabulary index
#     order over the weights max(0, q_i / beta - p_i), with the final uniform.
# ---------------------------------------------------------------------------------------------
MENTORED_BISECTION_STEPS = 50


def kl_divergence(q, pi):
    """KL(q || pi) = sum over q_i > 0 of q_i ln(q_i / pi_i); +inf if pi_i = 0 < q_i."""
    q = np.asarray(q, dtype=np.float64)
    pi = np.asarray(pi, dtype=np.float64)
    sup = q > 0
    if np.any(pi[sup] <= 0):
        return np.inf
    return float(np.sum(q[sup] * np.log(q[sup] / pi[sup])))


def _mentored_beta(q, p, R):
    """beta with sum_i max(0, q_i / beta - p_i) = R > 0: tokens by q_i / p_i descending; with the
    m largest ratios in play, beta = (sum of their q) / (R + sum of their p), valid once it is
    at least the next ratio."""
    sup = np.nonzero(q > 0)[0]
    with np.errstate(divide="ignore"):
        ratio = np.where(p[sup] > 0, q[sup] / np.where(p[sup] > 0, p[sup], 1.0), np.inf)
    order = np.argsort(-ratio, kind="stable")
    Qm = 0.0
    Pm = 0.0
    beta = np.inf
    for pos, t in enumerate(order):
        Qm += q[sup[t]]
        Pm += p[sup[t]]
        beta = Qm / (R + Pm)
        nxt = ratio[order[pos + 1]] if pos + 1 < order.size else -np.inf
        if beta >= nxt:
            break
    return beta


def _mentored_pi(q, p, alpha):
    """(pi, beta, weights of the replacement) for r_i = min(1, q_i / (alpha p_i))."""
    acc = np.minimum(p, q / alpha)  # p_i r_i
    R = 1.0 - float(np.sum(acc))
    if R <= 0.0:
        return acc, np.inf, np.zeros_like(q)
    beta = _mentored_beta(q, p, R)
    w = np.maximum(0.0, q / beta - p)
    return acc + w, beta, w


def mentored_solve(q, p, D):
    """Optimum for one position.  Returns a dict: trivial (every draft accepted), alpha, beta,
    r (accept probabilities), w (replacement weights, unnormalised), kl (of the emitted law)."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    if D > 0 and kl_divergence(q, p) <= D:
        return {"trivial": True, "alpha": 0.0, "beta": np.inf, "r": np.ones_like(q),
                "w": np.zeros_like(q), "kl": kl_divergence(q, p)}
    lo, hi = 0.0, 1.0
    # D = 0 is the lossless rule itself (alpha = 1); no bisection, whose comparisons near
    # KL = 0 would only see rounding
    for _ in range(MENTORED_BISECTION_STEPS if D > 0 else 0):
        mid = 0.5 * (lo + hi)
        pi, _, _ = _mentored_pi(q, p, mid)
        if kl_divergence(q, pi) <= D:
            hi = mid
        else:
            lo = mid
    alpha = hi
    pi, beta, w = _mentored_pi(q, p, alpha)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(p > 0, np.minimum(1.0, q / (alpha * np.where(p > 0, p, 1.0))),
                     np.where(q > 0, 1.0, 0.0))
    return {"trivial": False, "alpha": alpha, "beta": beta, "r": r, "w": w,
            "kl": kl_divergence(q, pi)}


def mentored_verify_sequence(q_rows, p_rows, drafts, u, D):
    """One sequence under mentored decoding: position k accepts x~_k iff u_k < r_{x~_k};
    n = first rejection; the token at n < K is drawn from the replacement weights, the bonus at
    n = K from q_K.  Every position is solved here so that a = r at the draft token is reported
    for all of them (the page's speed-up, no solve when u_k < min(1, q/p), changes no
    decision).  Returns the same dict as verify_sequence plus alpha and beta per position."""
    q_rows = [np.asarray(r, dtype=np.float64) for r in q_rows]
    p_rows = [np.asarray(r, dtype=np.float64) for r in p_rows]
    K = len(drafts)
    V = q_rows[0].size
    q_x = np.zeros(K)
    p_x = np.zeros(K)
    a = np.zeros(K)
    sols = []
    for k in range(K):
        x = int(drafts[k])
        sol = mentored_solve(q_rows[k], p_rows[k], D)
        sols.append(sol)
        if 0 <= x < V:
            q_x[k] = q_rows[k][x]
            p_x[k] = p_rows[k][x]
            a[k] = sol["r"][x] if (q_x[k] > 0 or p_x[k] > 0) else 0.0
    n = K
    for k in range(K):
        if not (float(u[k]) < a[k]):
            n = k
            break
    fell_back = False
    if n < K:
        w = sols[n]["w"]
        if not np.sum(w) > 0:  # nothing to replace with (rounding): draw from q
            w, fell_back = q_rows[n], True
    else:
        w = q_rows[K]
    tok = inverse_cdf(w, float(u[K]))
    margin = inverse_cdf_margin(w, float(u[K]), tok)
    tokens = np.full(K + 1, -1, dtype=np.int64)
    tokens[:n] = np.asarray(drafts[:n], dtype=np.int64)
    tokens[n] = tok
    return {"tokens": tokens, "n": n, "a": a, "q_x": q_x, "p_x": p_x, "fallback": fell_back,
            "weights": w, "draw_margin": margin,
            "alpha": np.array([s["alpha"] for s in sols]),
            "beta": np.array([s["beta"] for s in sols])}


def mentored_spec_verify(target_logits, draft_logits, drafts, uniforms, temperature=1.0,
                         top_k=0, top_p=1.0, D=0.0):
    """Batch mentored verification; same inputs and outputs as spec_verify (plus alpha, beta
    [B, K])."""
    target_logits = np.asarray(target_logits)
    draft_logits = np.asarray(draft_logits)
    drafts = np.asarray(drafts)
    uniforms = np.asarray(uniforms)
    B, K1, V = target_logits.shape
    K = K1 - 1
    out = {
        "tokens": np.full((B, K + 1), -1, dtype=np.int64),
        "n": np.zeros(B, dtype=np.int64),
        "a": np.zeros((B, K)),
        "q_x": np.zeros((B, K)),
        "p_x": np.zeros((B, K)),
        "fallback": np.zeros(B, dtype=bool),
        "draw_margin": np.zeros(B),
        "alpha": np.zeros((B, K)),
        "beta": np.zeros((B, K)),
        "topp_margin_t": np.full((B, K + 1), np.inf),
        "topp_margin_d": np.full((B, K), np.inf),
    }
    for b in range(B):
        q_rows = [row_distribution(target_logits[b, k], temperature, top_k, top_p)
                  for k in range(K + 1)]
        p_rows = [row_distribution(draft_logits[b, k], temperature, top_k, top_p)
                  for k in range(K)]
        r = mentored_verify_sequence(q_rows, p_rows, list(drafts[b]), list(uniforms[b]), D)
        for key in ("tokens", "n", "a", "q_x", "p_x", "fallback", "draw_margin", "alpha",
                    "beta"):
            out[key][b] = r[key]
    return out


# ---------------------------------------------------------------------------------------------
# Greedy token-tree verification (REST article, section "REST: 基于检索的投机解码"): the drafts
# form a tree laid out as a BFS pseudo-sequence; one target forward scores every node; a draft
# token is accepted exactly when it equals the token the target model would emit greedily.
# Readings: node 0 is the root (the last committed token); parents precede children
# (0 <= parent[n] < n for n >= 1), anything else marks the node as not accepted; a node deeper
# than max_depth is not accepted; argmax ties go to the lowest vocabulary index; among the
# deepest accepted nodes the lowest node index wins.  Output: the tokens on the root->d path
# (root excluded), then the bonus argmax of node d's row.
# ---------------------------------------------------------------------------------------------
def tree_verify(target_logits, parent, node_tokens, max_depth):
    """target_logits [B, N, V]; parent, node_tokens [B, N]; returns tokens [B, max_depth+1],
    n [B] (depth of the deepest accepted node) and last_node [B]."""
    target_logits = np.asarray(target_logits)
    parent = np.asarray(parent, dtype=np.int64)
    node_tokens = np.asarray(node_tokens, dtype=np.int64)
    B, N, V = target_logits.shape
    tokens = np.full((B, max_depth + 1), -1, dtype=np.int64)
    n_acc = np.zeros(B, dtype=np.int64)
    last = np.zeros(B, dtype=np.int64)
    for b in range(B):
        g = [int(np.argmax(np.asarray(target_logits[b, i], dtype=np.float64))) for i in range(N)]
        accepted = [False] * N
        depth = [0] * N
        accepted[0] = True
        for i in range(1, N):
            par = int(parent[b, i])
            if not (0 <= par < i):
                continue
            depth[i] = depth[par] + 1
            accepted[i] = (accepted[par] and depth[i] <= max_depth
                           and int(node_tokens[b, i]) == g[par])
        best = 0
        for i in range(N):
            if accepted[i] and depth[i] > depth[best]:
                best = i
        path = []
        i = best
        while i != 0:
            path.append(int(node_tokens[b, i]))
            i = int(parent[b, i])
        path.reverse()
        tokens[b, : len(path)] = path
        tokens[b, len(path)] = g[best]
        n_acc[b] = len(path)
        last[b] = best
    return {"tokens": tokens, "n": n_acc, "last_node": last}


# ---------------------------------------------------------------------------------------------
# REST draft-tree construction (REST article, section "REST: 基于检索的投机解码"): the
# continuations retrieved for the context are the candidate sequences; every prefix of a
# candidate may follow the context, so the candidates are put in a trie (prefix tree) whose
# node weights are the number of candidates carrying that node's prefix; the draft is the
# subtree of the highest-weight nodes, and its breadth-first traversal is the pseudo-sequence
# fed to the target with a tree-attention mask that restores each token's own ancestry.
#
# Readings (the page gives no algorithm text and its figure is missing):
#   * candidates [M, L] of token ids; a candidate ends at its first negative entry; duplicate
#     candidates count once each;
#   * node 0 is the root (the context's last token, carried by the caller; written as -1);
#     every other node is a distinct non-empty prefix, its weight the number of candidates
#     that start with it, its "first candidate" the lowest candidate index that does;
#   * the subtree keeps the N - 1 non-root nodes that come first in the order (weight
#     descending, depth ascending, first candidate ascending) -- a parent always precedes its
#     children in that order, so the kept set is a subtree;
#   * breadth-first order: the root, then level by level, children of earlier nodes first and
#     siblings by (weight descending, first candidate ascending);
#   * outputs in that order: parent index (-1 for the root), token, depth, weight, and the
#     mask M[i, j] = 1 iff node j is node i or one of its ancestors; unused slots (fewer than
#     N nodes) hold -1 and zero mask rows.
# ---------------------------------------------------------------------------------------------
def rest_trie(candidates):
    """Trie of the candidate sequences: dict prefix (tuple of tokens) -> (weight, first
    candidate index), for every non-empty prefix of every candidate."""
    nodes = {}
    for c, cand in enumerate(np.asarray(candidates, dtype=np.int64)):
        prefix = ()
        for tok in cand:
            if tok < 0:
                break
            prefix = prefix + (int(tok),)
            w, first = nodes.get(prefix, (0, c))
            nodes[prefix] = (w + 1, first)
    return nodes


def rest_build_tree(candidates, N):
    """Draft tree of at most N nodes (root included) from candidates [M, L].  Returns a dict
    with parent, tokens, depth, weight [N] (int64), mask [N, N] (uint8) and n_nodes."""
    nodes = rest_trie(candidates)
    order = sorted(nodes, key=lambda pre: (-nodes[pre][0], len(pre), nodes[pre][1]))
    kept = set(order[: max(N - 1, 0)])
    # breadth-first traversal of the kept subtree
    children = {}
    for pre in kept:
        children.setdefault(pre[:-1], []).append(pre)
    for kids in children.values():
        kids.sort(key=lambda pre: (-nodes[pre][0], nodes[pre][1]))
    bfs = [()]
    head = 0
    while head < len(bfs):
        bfs.extend(children.get(bfs[head], []))
        head += 1
    index = {pre: i for i, pre in enumerate(bfs)}
    parent = np.full(N, -1, dtype=np.int64)
    tokens = np.full(N, -1, dtype=np.int64)
    depth = np.full(N, -1, dtype=np.int64)
    weight = np.full(N, -1, dtype=np.int64)
    mask = np.zeros((N, N), dtype=np.uint8)
    n_nodes = min(len(bfs), N)
    for i, pre in enumerate(bfs[:n_nodes]):
        depth[i] = len(pre)
        if i == 0:
            weight[i] = int(sum(1 for cand in np.asarray(candidates) if len(cand) and cand[0] >= 0))
        else:
            parent[i] = index[pre[:-1]]
            tokens[i] = pre[-1]
            weight[i] = nodes[pre][0]
        j = i
        while j >= 0:
            mask[i, j] = 1
            j = int(parent[j])
    return {"parent": parent, "tokens": tokens, "depth": depth, "weight": weight,
            "mask": mask, "n_nodes": n_nodes}


# ---------------------------------------------------------------------------------------------
# Counter-based uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
# as easy as 1, 2, 3", SC 2011), the generator the verify step's uniforms come from.  A block
# is a function of a 256-bit counter and a 128-bit key alone: ten rounds, each multiplying
# counter words 0 and 2 by two fixed 64-bit constants, xoring the high halves with the other
# two words and the round key, and permuting; the key advances by two Weyl constants per
# round.  The constants below are the published ones.
#
# Readings: word i of a stream (key, counter c) is word i mod 4 of the block at counter
# c + floor(i / 4) (the counter as a 256-bit little-endian integer); a word w becomes the
# float32 uniform (w >> 40) * 2^-24 in [0, 1 - 2^-24], exact in float32.
# ---------------------------------------------------------------------------------------------
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1


def philox4x64(counter, key, rounds=10):
    """One Philox4x64 block: counter = 4 ints (64-bit words), key = 2 ints; returns 4 ints."""
    x0, x1, x2, x3 = (int(v) & _MASK64 for v in counter)
    k0, k1 = (int(v) & _MASK64 for v in key)
    for _ in range(rounds):
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> 64, p0 & _MASK64
        hi1, lo1 = p1 >> 64, p1 & _MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & _MASK64
        k1 = (k1 + PHILOX_W1) & _MASK64
    return [x0, x1, x2, x3]


def philox_uniforms(key, counter, n):
    """n float32 uniforms of the stream (key = (k0, k1), counter = 256-bit start, an int)."""
    out = np.empty(int(n), dtype=np.float32)
    for blk in range((int(n) + 3) // 4):
        c = (int(counter) + blk) & ((1 << 256) - 1)
        words = philox4x64([(c >> (64 * j)) & _MASK64 for j in range(4)], key)
        for j, w in enumerate(words):
            i = 4 * blk + j
            if i < n:
                out[i] = np.float32((w >> 40) * 2.0 ** -24)
    return out


# ---------------------------------------------------------------------------------------------
# Analytics (Leviathan blog, section 方法细节: expected tokens per call, wall-clock factor and
# operation count; App. E figures).  With i.i.d. acceptance rate alpha and gamma = K drafts:
#   E[#tokens] = (1 - alpha^(K+1)) / (1 - alpha)
#   wall-clock factor = (1 - alpha^(K+1)) / ((1 - alpha) (K c + 1)), c = draft/target cost
#   operations factor = (1 - alpha) (K c_hat + K + 1) / (1 - alpha^(K+1))
# ---------------------------------------------------------------------------------------------
def expected_tokens_per_call(alpha, K):
    """Expected tokens emitted per target call (accepted drafts + the one drawn token)."""
    alpha = float(alpha)
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


def walltime_speedup(alpha, K, c):
    return expected_tokens_per_call(alpha, K) / (K * float(c) + 1.0)


def ops_factor(alpha, K, c_hat):
    return (K * float(c_hat) + K + 1.0) / expected_tokens_per_call(alpha, K)


def acceptance_rate(q, p, lenience=1.0):
    """beta = probability that a draft token x ~ p is accepted at one position:
    sum_x p(x) min(1, q(x) / (l p(x))) = sum_x min(p(x), q(x) / l); for l = 1 this is
    sum min(p, q) = 1 - D_LK(p, q), the total-variation distance the Leviathan blog calls D_LK
    (section 方法细节, the exact characterisation of the acceptance rate; alpha = E(beta))."""
    q = np.asarray(q, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    return float(np.sum(np.minimum(p, q / float(lenience))))


def optimal_gamma(alpha, c, max_gamma):
    """The number of draft tokens in 1..max_gamma with the largest wall-clock factor
    (Leviathan blog, FAQ on choosing gamma: maximise the factor numerically); the smallest
    such gamma on ties."""
    best, best_g = -np.inf, 1
    for g in range(1, int(max_gamma) + 1):
        v = walltime_speedup(alpha, g, c)
        if v > best:
            best, best_g = v, g
    return best_g
