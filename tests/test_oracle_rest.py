"""Pins of the oracle's REST draft-tree builder (REST article, section "REST: 基于检索的投机解码")
against a worked example written by hand from the prefixes the article names, and against
brute force over random candidate sets: prefix counts taken directly from the candidates,
the subtree and breadth-first properties, and the tree-attention mask as the ancestor
relation."""

import json
import os

import numpy as np
import pytest

import oracle.spec_verify_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rest_tree_example.json")


def _paths(r):
    """Token path (tuple) of every node, from the parent and token arrays."""
    paths = []
    for i in range(r["n_nodes"]):
        path = []
        j = i
        while j > 0:
            path.append(int(r["tokens"][j]))
            j = int(r["parent"][j])
        paths.append(tuple(reversed(path)))
    return paths


def _direct_counts(cands):
    """weight and first candidate of every distinct non-empty prefix, counted directly."""
    seqs = []
    for c in cands:
        c = [int(t) for t in c]
        seqs.append(c[: c.index(-1)] if -1 in c else c)
    allp = {tuple(c[:d]) for c in seqs for d in range(1, len(c) + 1)}
    out = {}
    for pre in allp:
        hits = [i for i, c in enumerate(seqs) if tuple(c[: len(pre)]) == pre]
        out[pre] = (len(hits), hits[0])
    return out


def _random_candidates(rng, M, L, alphabet):
    """Random candidates over a small alphabet, many sharing a start with an earlier one,
    of random lengths (-1 after the end)."""
    c = rng.integers(0, alphabet, size=(M, L))
    for i in range(1, M):
        if rng.random() < 0.6:
            j = int(rng.integers(0, i))
            d = int(rng.integers(0, L + 1))
            c[i, :d] = c[j, :d]
    lens = rng.integers(0, L + 1, size=M)
    for i in range(M):
        c[i, lens[i]:] = -1
    return c


def test_worked_example():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        r = O.rest_build_tree(g["candidates"], case["N"])
        for key in ("parent", "tokens", "depth", "weight"):
            assert r[key].tolist() == case[key], (case["N"], key)
        assert r["n_nodes"] == case["n_nodes"]


@pytest.mark.parametrize("seed", range(40))
def test_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    M, L = int(rng.integers(1, 24)), int(rng.integers(1, 7))
    N = int(rng.integers(1, 30))
    cands = _random_candidates(rng, M, L, int(rng.integers(2, 5)))
    r = O.rest_build_tree(cands, N)
    counts = _direct_counts(cands)
    paths = _paths(r)
    n = r["n_nodes"]
    assert n == min(N, 1 + len(counts))
    # weights and depths of the kept nodes, counted directly
    for i in range(1, n):
        assert paths[i] in counts
        assert r["weight"][i] == counts[paths[i]][0]
        assert r["depth"][i] == len(paths[i])
    assert len(set(paths)) == n  # distinct prefixes
    # the kept set: every kept prefix comes before every dropped one in the stated order
    key = {pre: (-w, len(pre), first) for pre, (w, first) in counts.items()}
    kept = set(paths[1:])
    if kept and len(kept) < len(counts):
        assert max(key[p] for p in kept) < min(key[p] for p in counts if p not in kept)
    # subtree: parents are kept and come first; breadth-first: depth never decreases, the
    # parents of consecutive nodes never go back, siblings by (weight desc, first asc)
    for i in range(1, n):
        par = int(r["parent"][i])
        assert 0 <= par < i and paths[par] == paths[i][:-1]
        if i > 1:
            assert r["depth"][i] >= r["depth"][i - 1]
            assert int(r["parent"][i]) >= int(r["parent"][i - 1])
            if r["parent"][i] == r["parent"][i - 1]:
                assert key[paths[i - 1]][::2] < key[paths[i]][::2]
    # unused slots
    assert (r["parent"][n:] == -1).all() and (r["tokens"][n:] == -1).all()
    assert (r["mask"][n:] == 0).all() and (r["mask"][:, n:] == 0).all()
    # mask: the ancestor-or-self relation, from the paths
    for i in range(n):
        for j in range(n):
            assert r["mask"][i, j] == (1 if paths[i][: len(paths[j])] == paths[j] else 0)
    # every kept prefix is a subsequence of the pseudo-sequence (the article's observation)
    seq = [int(t) for t in r["tokens"][1:n]]
    for p in paths[1:]:
        it = iter(seq)
        assert all(any(t == s for s in it) for t in p)


def test_degenerate_inputs():
    empty = O.rest_build_tree([[-1, -1], [-1, 5]], 4)  # a candidate ends at its first -1
    assert empty["n_nodes"] == 1 and empty["parent"].tolist() == [-1, -1, -1, -1]
    assert empty["weight"][0] == 0 and empty["mask"][0, 0] == 1
    root_only = O.rest_build_tree([[1, 2, 3]], 1)
    assert root_only["n_nodes"] == 1 and root_only["weight"].tolist() == [1]
    chain = O.rest_build_tree([[7, 8, 9]] * 3, 8)  # duplicates: each counts
    assert chain["n_nodes"] == 4 and chain["weight"][:4].tolist() == [3, 3, 3, 3]
    assert chain["parent"][:4].tolist() == [-1, 0, 1, 2]


def test_planted_mistakes_fail_a_pin(monkeypatch):
    """Kept nodes chosen by lowest weight, or a depth-first layout, break the worked example."""
    g = json.load(open(GOLDEN))
    case = g["cases"][1]
    orig = O.rest_trie
    monkeypatch.setattr(O, "rest_trie",
                        lambda c: {k: (-w, f) for k, (w, f) in orig(c).items()})
    r = O.rest_build_tree(g["candidates"], case["N"])
    assert r["tokens"].tolist() != case["tokens"] or r["weight"].tolist() != case["weight"]
