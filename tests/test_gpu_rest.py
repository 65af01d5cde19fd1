"""GPU parity of the REST draft-tree builder (spec_build_tree, through the C ABI) against the
oracle's rest_build_tree: parent, tokens, depth, weight, node count and the tree-attention
mask, bit-exact (integer work)."""

import numpy as np
import pytest
import torch

import oracle.spec_verify_oracle as O
from workloads import synthetic as S

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def svm():
    import speculative_sampling_verification_amd as m
    return m


def _check(svm, cands, N, want_mask=True):
    c = torch.from_numpy(np.ascontiguousarray(cands, dtype=np.int32)).cuda()
    g = svm.spec_build_tree(c, N, want_mask=want_mask)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    for b in range(cands.shape[0]):
        o = O.rest_build_tree(cands[b], N)
        assert int(g["num_nodes"][b]) == o["n_nodes"], b
        for key in ("parent", "tokens", "depth", "weight"):
            np.testing.assert_array_equal(g[key][b], o[key], err_msg=f"seq {b} {key}")
        if want_mask:
            np.testing.assert_array_equal(g["mask"][b], o["mask"], err_msg=f"seq {b} mask")
    return g


def test_workload_shape(svm):
    _announce("REST tree B=32 M=64 L=8 N=64 (the workload), every sequence")
    cands = S.workload_inputs("rest_B32_M64_L8_N64", seed=3).numpy()
    _check(svm, cands, 64)


@pytest.mark.parametrize("seed", range(6))
def test_random_small_alphabets(svm, seed):
    rng = np.random.default_rng(100 + seed)
    M = int(rng.integers(1, 129))
    L = int(rng.integers(1, 33))
    N = int(rng.integers(1, 257))
    _announce(f"REST tree random seed={seed} M={M} L={L} N={N}, alphabet of 3 (many ties)")
    B = 8
    cands = rng.integers(0, 3, size=(B, M, L)).astype(np.int32)
    lens = rng.integers(0, L + 1, size=(B, M))
    for b in range(B):
        for m in range(M):
            cands[b, m, lens[b, m]:] = -1
    _check(svm, cands, N)


def test_limits_and_degenerate_inputs(svm):
    _announce("REST tree limits: M=128 L=32 N=256; N=1; empty and duplicate candidates")
    rng = np.random.default_rng(7)
    big = rng.integers(0, 2, size=(2, 128, 32)).astype(np.int32)
    _check(svm, big, 256)
    _check(svm, big, 1)
    empty = np.full((2, 5, 4), -1, dtype=np.int32)
    empty[1, 2, 1] = 9  # after the end: ignored
    _check(svm, empty, 8)
    dup = np.tile(np.array([[4, 5, 6, 7]], dtype=np.int32), (3, 10, 1))
    _check(svm, dup, 16)
    # negative values other than -1 also end a candidate; large token ids pass through
    odd = np.array([[[2**31 - 1, 3, -5, 1], [2**31 - 1, 3, 4, -1]]], dtype=np.int32)
    _check(svm, odd, 6)
    _check(svm, big, 64, want_mask=False)


def test_build_then_verify(svm):
    _announce("REST tree then greedy tree verification of the built tree")
    B, M, L, N, V = 8, 48, 6, 40, 5000
    cands = S.rest_candidates(B, M, L, V, 4, 1.2, seed=5)
    c = torch.from_numpy(cands).cuda()
    tree = svm.spec_build_tree(c, N)
    g = torch.Generator().manual_seed(5)
    logits = torch.randn((B, N, V), generator=g)
    # make the target agree with the heaviest child of some nodes
    par = tree["parent"].cpu().numpy()
    tok = tree["tokens"].cpu().numpy()
    n_nodes = tree["num_nodes"].cpu().numpy()
    for b in range(B):
        for i in range(1, n_nodes[b]):
            p = par[b, i]
            if logits[b, p].max() < 50.0 and np.random.default_rng(b * 1000 + i).random() < 0.7:
                logits[b, p, tok[b, i]] = 60.0 + i * 1e-3
    lg = logits.to(torch.bfloat16)
    out = svm.spec_verify_tree(lg.cuda(), tree["parent"], tree["tokens"], L)
    torch.cuda.synchronize()
    o = O.tree_verify(lg.float().numpy(), par, tok, L)
    np.testing.assert_array_equal(out["num_accepted"].cpu().numpy(), o["n"])
    np.testing.assert_array_equal(out["tokens"].cpu().numpy(), o["tokens"])
    assert o["n"].max() >= 2


def test_invalid_arguments(svm):
    _announce("REST tree: out-of-range sizes return an error status")
    for shape, N in (((1, 129, 4), 8), ((1, 4, 33), 8), ((1, 4, 4), 0), ((1, 4, 4), 257)):
        c = torch.zeros(shape, dtype=torch.int32, device="cuda")
        with pytest.raises(svm.SpecVerifyError):
            svm.spec_build_tree(c, N)
