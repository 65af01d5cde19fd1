"""GPU parity on rows that do not start on a 16-byte boundary: vocabularies whose row length is
not a multiple of 16 bytes (e.g. V = 50257 in bf16) and logit tensors that begin a few
elements into their allocation.  The top-k stream loads the aligned interior of each row in
vectors and the few elements around it one by one; the chunked kernels count their chunks from
the 16-byte boundary before each row and mask what lies outside it.  These tests compare the
result, through the C ABI, with the oracle on the same logits (same bar as tests/parity.py).
"""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

from parity import check, make_inputs, verify_case

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def svm():
    import speculative_sampling_verification_amd as m
    return m


def _offset_copy(x, offset):
    """A contiguous device copy of x that starts `offset` elements into its allocation."""
    flat = torch.empty(x.numel() + offset, dtype=x.dtype, device="cuda")
    view = flat[offset:].view(x.shape)
    view.copy_(x.cuda())
    return view


def _run(svm, t, d, drafts, u, params):
    x = torch.from_numpy(np.ascontiguousarray(drafts)).cuda()
    uu = torch.from_numpy(np.ascontiguousarray(u)).cuda()
    out = svm.spec_verify(t, d, x, uu, temperature=params["temperature"],
                          top_k=params.get("top_k", 0), top_p=params.get("top_p", 1.0))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("V,dtype,k", [(50257, "bf16", 50), (32001, "bf16", 256),
                                       (40001, "f32", 40), (1003, "f32", 7)])
def test_odd_vocabulary(V, dtype, k):
    _announce(f"unaligned rows: V={V} {dtype} top-k {k}")
    t, d = S.zipf_logits(8, 3, V, 1.1, 1.0, dtype, seed=V % 97)
    verify_case(t, d, dict(temperature=0.8, top_k=k), seed=V % 89)


@pytest.mark.parametrize("offset", [1, 3, 7])
def test_tensor_offset_bf16(svm, offset):
    _announce(f"logit tensors starting {offset} elements into their allocation, bf16 top-k 30")
    t, d = S.zipf_logits(6, 4, 20000, 1.1, 1.0, "bf16", seed=60 + offset)
    params = dict(temperature=0.9, top_k=30)
    drafts, u = make_inputs(t, d, params, 60 + offset)
    g = _run(svm, _offset_copy(t, offset), _offset_copy(d, offset + 2), drafts, u, params)
    check(g, t, d, drafts, u, params)


@pytest.mark.parametrize("V,offset", [(5, 3), (9, 1), (17, 6)])
def test_tiny_rows_all_fringe(svm, V, offset):
    _announce(f"rows shorter than two vectors: V={V} bf16 offset {offset} top-k 3")
    t, d = S.normal_logits(5, 3, V, 2.0, 1.0, 0.5, "bf16", seed=70 + V)
    params = dict(temperature=1.0, top_k=3)
    drafts, u = make_inputs(t, d, params, 70 + V)
    g = _run(svm, _offset_copy(t, offset), _offset_copy(d, offset), drafts, u, params)
    check(g, t, d, drafts, u, params)


def test_tie_overflow_unaligned(svm):
    _announce("unaligned rows whose top-k ties overflow the lists (whole-row path), V=30001")
    gen = torch.Generator().manual_seed(80)
    t = torch.randint(0, 4, (3, 3, 30001), generator=gen).float().to(torch.bfloat16)
    d = torch.randint(0, 4, (3, 2, 30001), generator=gen).float().to(torch.bfloat16)
    verify_case(t, d, dict(temperature=1.0, top_k=50), seed=80)


def test_sample_matches_verify_bonus_draw_unaligned(svm):
    _announce("spec_sample on unaligned rows equals the oracle's draw")
    import oracle.spec_verify_oracle as O
    R, V = 40, 50257
    t, _ = S.zipf_logits(R, 0, V, 1.1, 1.0, "bf16", seed=81)
    rows = t[:, 0].contiguous()
    u = S.philox_uniforms(82, (R,))
    g = svm.spec_sample(_offset_copy(rows, 5), torch.from_numpy(u).cuda(), temperature=0.7,
                        top_k=50).cpu().numpy()
    o = O.sample_rows(rows.float().numpy(), u, np.float32(0.7), 50, np.float32(1.0))
    flips = 0
    for r in range(R):
        if g[r] != o[r]:
            q = O.row_distribution(rows[r].float().numpy(), np.float32(0.7), 50, np.float32(1.0))
            assert O.inverse_cdf_margin(q, float(u[r]), int(g[r])) < 1e-6, r
            flips += 1
    assert flips <= 1


DENSE_CASES = [
    ("dense T=1 bf16", dict(temperature=1.0), 50257, "bf16"),
    ("top-p 0.9 fp32", dict(temperature=1.0, top_p=0.9), 40001, "f32"),
    ("top-p 0.8 bf16", dict(temperature=0.9, top_p=0.8), 32769, "bf16"),
    ("top-k 300 + top-p 0.9 fp32", dict(temperature=1.0, top_k=300, top_p=0.9), 20003, "f32"),
    ("greedy bf16", dict(temperature=0.0), 32001, "bf16"),
]


@pytest.mark.parametrize("name,params,V,dtype", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_paths_odd_vocabulary(name, params, V, dtype):
    _announce(f"unaligned rows, {name}, V={V}")
    t, d = S.zipf_logits(6, 3, V, 1.1, 1.0, dtype, seed=V % 101)
    verify_case(t, d, params, seed=V % 83)


@pytest.mark.parametrize("name,params,V,dtype", DENSE_CASES, ids=[c[0] for c in DENSE_CASES])
def test_dense_paths_tensor_offset(svm, name, params, V, dtype):
    _announce(f"logit tensors starting inside their allocation, {name}, V={V}")
    t, d = S.zipf_logits(4, 3, V, 1.1, 1.0, dtype, seed=V % 103)
    drafts, u = make_inputs(t, d, params, V % 79)
    g = _run(svm, _offset_copy(t, 3), _offset_copy(d, 1), drafts, u, params)
    check(g, t, d, drafts, u, params)


def test_tree_unaligned(svm):
    _announce("greedy tree verify on unaligned rows, V=32001, offset 5")
    import oracle.spec_verify_oracle as O
    B, N, V = 4, 24, 32001
    t, _ = S.normal_logits(B, N - 1, V, 3.0, 0.8, 1.5, "bf16", seed=90)
    g = torch.Generator().manual_seed(90)
    parent = torch.full((B, N), -1, dtype=torch.int32)
    for i in range(1, N):
        parent[:, i] = torch.randint(0, i, (B,), generator=g, dtype=torch.int32)
    am = t.float().argmax(dim=2).to(torch.int32)
    tok = torch.randint(0, V, (B, N), generator=g, dtype=torch.int32)
    for i in range(1, N):
        p = parent[:, i].long()
        tok[:, i] = torch.where(torch.rand(B, generator=g) < 0.7, am[torch.arange(B), p],
                                tok[:, i])
    out = svm.spec_verify_tree(_offset_copy(t, 5), parent.cuda(), tok.cuda(), 10)
    torch.cuda.synchronize()
    o = O.tree_verify(t.float().numpy(), parent.numpy(), tok.numpy(), 10)
    np.testing.assert_array_equal(out["num_accepted"].cpu().numpy(), o["n"])
    np.testing.assert_array_equal(out["tokens"].cpu().numpy(), o["tokens"])
    np.testing.assert_array_equal(out["last_node"].cpu().numpy(), o["last_node"])


def test_acceptance_rate_unaligned(svm):
    _announce("acceptance rates on unaligned rows, dense fp32 V=40001 and top-k bf16 V=50257")
    import oracle.spec_verify_oracle as O
    for V, dtype, params in ((40001, "f32", dict(temperature=1.0)),
                             (50257, "bf16", dict(temperature=0.7, top_k=50))):
        t, d = S.zipf_logits(3, 3, V, 1.1, 1.0, dtype, seed=V % 71)
        beta = svm.spec_acceptance_rate(_offset_copy(t, 1), _offset_copy(d, 2),
                                        **params).cpu().numpy()
        tf, df = t.float().numpy(), d.float().numpy()
        T = np.float32(params["temperature"])
        k = params.get("top_k", 0)
        for b in range(3):
            for j in range(3):
                q = O.row_distribution(tf[b, j], T, k, np.float32(1.0))
                p = O.row_distribution(df[b, j], T, k, np.float32(1.0))
                assert abs(beta[b, j] - O.acceptance_rate(q, p, np.float32(1.0))) <= 1e-5


# The final draw runs one workgroup per (sequence, final chunk): a chunk of 256 threads x 16
# vectors split into quarters when B x chunks is in [1024, 16384), into its vector rows below
# that, and whole above it.
FINAL_GRAIN_CASES = [
    ("quarter chunks, unaligned fp32 B=256 V=49153", 256, 49153, "f32", 3),
    ("quarter chunks, unaligned bf16 B=256 V=98305", 256, 98305, "bf16", 1),
    ("vector rows, unaligned bf16 B=8 V=30001", 8, 30001, "bf16", 5),
    ("vector rows, unaligned fp32 B=3 V=5000", 3, 5000, "f32", 2),
]


@pytest.mark.parametrize("name,B,V,dtype,offset", FINAL_GRAIN_CASES,
                         ids=[c[0] for c in FINAL_GRAIN_CASES])
def test_final_draw_grain(svm, name, B, V, dtype, offset):
    _announce(f"dense final draw, {name}, offset {offset}")
    t, d = S.normal_logits(B, 1, V, 3.0, 0.8, 1.5, dtype, seed=V % 107)
    params = dict(temperature=1.0)
    drafts, u = make_inputs(t, d, params, V % 61)
    g = _run(svm, _offset_copy(t, offset), _offset_copy(d, offset + 1), drafts, u, params)
    check(g, t, d, drafts, u, params)


@pytest.mark.parametrize("offset", [0, 1])
def test_final_draw_whole_chunks_many_rows(svm, offset):
    # 8192 rows of two chunks each: B x chunks = 16384, so the final draw takes whole chunks
    _announce(f"dense spec_sample, whole final chunks: R=8192 V=16385 fp32, offset {offset}, "
              "64 sampled rows against the oracle")
    import oracle.spec_verify_oracle as O
    R, V = 8192, 16385
    t, _ = S.normal_logits(R, 0, V, 3.0, 0.8, 1.5, "f32", seed=91 + offset)
    rows = t[:, 0].contiguous()
    u = S.philox_uniforms(92 + offset, (R,))
    dev = _offset_copy(rows, offset) if offset else rows.cuda()
    g = svm.spec_sample(dev, torch.from_numpy(u).cuda(), temperature=1.0).cpu().numpy()
    pick = np.random.default_rng(93).choice(R, 64, replace=False)
    flips = 0
    for r in pick:
        o = O.sample_rows(rows[r:r + 1].numpy(), u[r:r + 1], np.float32(1.0), 0, np.float32(1.0))
        if g[r] != o[0]:
            q = O.row_distribution(rows[r].numpy(), np.float32(1.0), 0, np.float32(1.0))
            assert O.inverse_cdf_margin(q, float(u[r]), int(g[r])) < 1e-6, r
            flips += 1
    assert flips <= 1
