"""GPU parity: libspecverify.so (through its C ABI) against the CPU oracle.

Sizes are chosen so the oracle finishes in seconds while spanning several chunks (32768 bf16 /
16384 fp32 elements per chunk) and a ragged tail; the full-size workloads are checked on a
sample of sequences.  Every mismatch must be a counted boundary flip (see tests/parity.py).
"""

import numpy as np
import pytest
import torch

import oracle.spec_verify_oracle as O
from workloads import synthetic as S

from parity import check, make_inputs, run_gpu, run_oracle, verify_case

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import speculative_sampling_verification_amd as svm
    return svm


# ------------------------------------------------------------------ dense (no truncation)
def test_dense_fp32_small_vocab():
    _announce("normal fp32 B=32 K=4 V=1000 T=1")
    t, d = S.normal_logits(32, 4, 1000, 2.0, 1.0, 0.5, "f32", seed=1)
    verify_case(t, d, dict(temperature=1.0), seed=1)


def test_dense_bf16_multi_chunk():
    _announce("normal bf16 B=8 K=4 V=70000 T=1 (3 chunks, ragged)")
    t, d = S.normal_logits(8, 4, 70000, 3.0, 0.8, 1.5, "bf16", seed=2)
    verify_case(t, d, dict(temperature=1.0), seed=2)


def test_dense_bf16_config_shape():
    _announce("normal bf16 B=16 K=4 V=32000 T=1")
    t, d = S.normal_logits(16, 4, 32000, 3.0, 0.8, 1.5, "bf16", seed=3)
    verify_case(t, d, dict(temperature=1.0), seed=3)


# ------------------------------------------------------------------ top-k (compact path)
@pytest.mark.parametrize("V,K,B", [(128256, 7, 4), (70001 - 1, 3, 6), (5000, 2, 16)])
def test_topk_bf16(V, K, B):
    _announce(f"zipf bf16 top-k 50 T=0.7 B={B} K={K} V={V}")
    t, d = S.zipf_logits(B, K, V, 1.1, 1.0, "bf16", seed=V)
    verify_case(t, d, dict(temperature=0.7, top_k=50), seed=V)


def test_topk_fp32_with_topp():
    _announce("zipf fp32 top-k 40 + top-p 0.8 T=1 B=6 K=3 V=40000")
    t, d = S.zipf_logits(6, 3, 40000, 1.1, 2.0, "f32", seed=7)
    verify_case(t, d, dict(temperature=1.0, top_k=40, top_p=0.8), seed=7)


def test_topk_large_k_generic_path():
    _announce("zipf bf16 top-k 1000 (row-pass selection) B=4 K=3 V=20000")
    t, d = S.zipf_logits(4, 3, 20000, 1.1, 1.0, "bf16", seed=8)
    verify_case(t, d, dict(temperature=1.0, top_k=1000), seed=8)


def test_topk_heavy_ties_overflow_path():
    _announce("bf16 logits on 4 levels, top-k 50: candidate overflow -> row-pass selection")
    g = torch.Generator().manual_seed(9)
    t = torch.randint(0, 4, (3, 3, 40000), generator=g).float().to(torch.bfloat16)
    d = torch.randint(0, 4, (3, 2, 40000), generator=g).float().to(torch.bfloat16)
    verify_case(t, d, dict(temperature=1.0, top_k=50), seed=9)


# ------------------------------------------------------------------ top-p and lenience
@pytest.mark.parametrize("lenience", [1.0, 0.1])
def test_topp_fp32(lenience):
    _announce(f"zipf fp32 top-p 0.95 T=1 lenience {lenience} B=2 K=3 V=256000")
    t, d = S.zipf_logits(2, 3, 256000, 1.1, 2.0, "f32", seed=10)
    verify_case(t, d, dict(temperature=1.0, top_p=0.95, lenience=lenience), seed=10)


def test_topp_bf16_small():
    _announce("zipf bf16 top-p 0.9 T=0.8 B=8 K=2 V=9000")
    t, d = S.zipf_logits(8, 2, 9000, 1.1, 1.0, "bf16", seed=11)
    verify_case(t, d, dict(temperature=0.8, top_p=0.9), seed=11)


def test_topp_boundary_candidate_overflow():
    _announce("bf16 logits on 4 levels, top-p 0.9: boundary bin overflows -> row-pass selection")
    g = torch.Generator().manual_seed(23)
    t = torch.randint(0, 4, (3, 3, 40000), generator=g).float().to(torch.bfloat16)
    d = torch.randint(0, 4, (3, 2, 40000), generator=g).float().to(torch.bfloat16)
    verify_case(t, d, dict(temperature=1.0, top_p=0.9), seed=23)


@pytest.mark.parametrize("P,T", [(0.01, 1.0), (0.9999, 1.0), (0.95, 0.05), (0.5, 3.0)])
def test_topp_extremes(P, T):
    _announce(f"fp32 top-p {P} T={T}, rows with -inf entries and far outliers, V=70000")
    t, d = S.zipf_logits(3, 2, 70000, 1.1, 2.0, "f32", seed=24)
    t[:, :, ::97] = -float("inf")
    d[:, :, 5::89] = -float("inf")
    t[0, 0, 123] = 60.0
    t[1, 1, 17] = -1.0e4
    d[2, 0, 999] = 45.0
    verify_case(t, d, dict(temperature=T, top_p=P), seed=24)


@pytest.mark.parametrize("V", [9000, 16384, 16385, 49153])
def test_topp_fp32_chunk_edges(V):
    """fp32 top-p rows of one chunk, exactly one chunk, one element past it, and three chunks and
    a ragged tail (16 384 logits per chunk): the histogram pass writes the edge codes of every
    slot of each chunk frame, and slots outside the row must never become candidates."""
    _announce(f"zipf fp32 top-p 0.9 T=0.8 B=5 K=2 V={V}: chunk edges of the edge codes")
    t, d = S.zipf_logits(5, 2, V, 1.1, 2.0, "f32", seed=V + 7)
    verify_case(t, d, dict(temperature=0.8, top_p=0.9), seed=V + 7)


def test_topp_fp32_long_rows():
    """fp32 top-p rows of 68 chunks (V = 1.1 M): more chunks than the per-row kernel keeps in
    LDS, so their partials are read from memory."""
    _announce("zipf fp32 top-p 0.9 B=1 K=1 V=1100000: 68 chunks per row")
    t, d = S.zipf_logits(1, 1, 1100000, 1.1, 2.0, "f32", seed=71)
    verify_case(t, d, dict(temperature=1.0, top_p=0.9), seed=71)


def test_topp_fp32_sample_and_bonus(_lib):
    """spec_sample and the K = 0 bonus draw with fp32 top-p: the draw from a row's kept set found
    from its edge codes, against the oracle's sampler."""
    _announce("spec_sample fp32 top-p 0.95, R=24 V=70000, and K=0 verification")
    t, _ = S.zipf_logits(24, 0, 70000, 1.1, 2.0, "f32", seed=68)
    rows = t[:, 0].contiguous()
    u = S.philox_uniforms(69, (24,))
    got = _lib.spec_sample(rows.cuda(), torch.from_numpy(u.copy()).cuda(), temperature=1.0,
                           top_p=0.95).cpu().numpy()
    want = O.sample_rows(rows.numpy(), u, np.float32(1.0), 0, np.float32(0.95))
    np.testing.assert_array_equal(got, want)
    drafts, uu = make_inputs(t, t[:, :0], dict(temperature=1.0, top_p=0.95), 70)
    g = run_gpu(t, None, drafts, uu, dict(temperature=1.0, top_p=0.95))
    check(g, t, None, drafts, uu, dict(temperature=1.0, top_p=0.95))


def test_topp_fp32_boundary_candidate_overflow():
    _announce("fp32 logits on 4 levels, top-p 0.9: boundary bin overflows -> row-pass selection")
    g = torch.Generator().manual_seed(42)
    t = torch.randint(0, 4, (3, 3, 40000), generator=g).float()
    d = torch.randint(0, 4, (3, 2, 40000), generator=g).float()
    verify_case(t, d, dict(temperature=1.0, top_p=0.9), seed=42)


def test_topp_fp32_kept_segments_overflow():
    _announce("normal fp32 sd 0.5 top-p 0.95 V=40000: kept segments overflow -> dense final draw")
    t, d = S.normal_logits(6, 3, 40000, 0.5, 1.0, 0.2, "f32", seed=43)
    verify_case(t, d, dict(temperature=1.0, top_p=0.95), seed=43)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topp_crossing_near_bin_edge(dtype):
    """Top-p with P * S a hair (2e-6 relative) above the mass of every token at or above one edge
    of the 1/8-unit grid: the crossing lies in the next occupied bin but within the bin masses'
    rounding margin of its upper edge, so the candidate range takes that bin's neighbours too
    (a crossing clear of both edges takes the one bin); the tokens still equal the oracle's.
    P is tuned on target row (0, 0); the other rows take their own brackets."""
    _announce(f"zipf {dtype} top-p tuned to a bin edge, B=4 K=2 V=5000")
    t, d = S.zipf_logits(4, 2, 5000, 1.1, 2.0, dtype, seed=81)
    z = t[0, 0].float().numpy().astype(np.float64)
    w = np.exp(z - z.max())
    S_ = w.sum()
    edges = np.floor(8.0 * z)
    levels = np.unique(edges)[::-1]  # occupied edges, from the top
    mass = np.array([w[edges >= e].sum() for e in levels])
    j = int(np.argmax(mass / S_ >= 0.7))  # the first edge whose mass from the top reaches 0.7
    P = float(np.float32(mass[j] / S_ * (1.0 + 2e-6)))
    assert mass[j] < P * S_ < mass[j + 1]
    verify_case(t, d, dict(temperature=1.0, top_p=P), seed=81)


# ------------------------------------------------------------------ layouts and edge cases
def test_unaligned_vocab():
    _announce("unaligned rows: bf16 V=50001 top-k 50, fp32 V=1001 dense")
    t, d = S.zipf_logits(3, 2, 50001, 1.1, 1.0, "bf16", seed=12)
    verify_case(t, d, dict(temperature=0.7, top_k=50), seed=12)
    t, d = S.normal_logits(4, 3, 1001, 2.0, 1.0, 0.5, "f32", seed=13)
    verify_case(t, d, dict(temperature=1.0), seed=13)


def test_greedy_temperature_zero():
    _announce("T=0 greedy bf16 B=8 K=5 V=32000")
    t, d = S.normal_logits(8, 5, 32000, 3.0, 0.8, 1.5, "bf16", seed=14)
    drafts, u = make_inputs(t, d, dict(temperature=1.0), 14)
    g_arg = t.float().argmax(dim=2).numpy()
    drafts[:, :3] = g_arg[:, :3]  # make some drafts match the target argmax
    params = dict(temperature=0.0)
    g = run_gpu(t, d, drafts, u, params)
    check(g, t, d, drafts, u, params, max_flip_frac=0.0)


def test_p_equals_q_accepts_everything():
    _announce("draft == target: every draft accepted")
    t, _ = S.zipf_logits(8, 4, 30000, 1.1, 1.0, "bf16", seed=15)
    for params in (dict(temperature=1.0), dict(temperature=0.7, top_k=50),
                   dict(temperature=1.0, top_p=0.9)):
        drafts, u = make_inputs(t, t[:, :4].contiguous(), params, 15)
        g = run_gpu(t, t[:, :4].contiguous(), drafts, u, params)
        assert (g["num_accepted"] == 4).all(), params
        assert (g["accept_prob"] == 1.0).all(), params


def test_bonus_only_k0_and_spec_sample(_lib):
    _announce("K=0 (bonus draw) and spec_sample against the oracle sampler")
    t, _ = S.zipf_logits(16, 0, 20000, 1.1, 1.0, "bf16", seed=16)
    params = dict(temperature=0.7, top_k=50)
    drafts, u = make_inputs(t, t[:, :0], params, 16)
    g = run_gpu(t, None, drafts, u, params)
    o = run_oracle(t, None, drafts, u, params)
    np.testing.assert_array_equal(g["tokens"][:, 0], o["tokens"][:, 0])
    rows = t[:, 0].contiguous()
    uu = torch.from_numpy(u[:, 0].copy())
    got = _lib.spec_sample(rows.cuda(), uu.cuda(), temperature=0.7, top_k=50).cpu().numpy()
    want = O.sample_rows(rows.float().numpy(), u[:, 0], np.float32(0.7), 50)
    np.testing.assert_array_equal(got, want)


def test_out_of_range_drafts_rejected():
    _announce("draft tokens outside [0, V) are rejected")
    t, d = S.normal_logits(4, 3, 5000, 2.0, 1.0, 0.5, "f32", seed=17)
    drafts, u = make_inputs(t, d, dict(temperature=1.0), 17)
    drafts[:, 0] = np.array([-1, 5000, 10**6, -(10**6)])
    g = run_gpu(t, d, drafts, u, dict(temperature=1.0))
    assert (g["num_accepted"] == 0).all()
    assert (g["accept_prob"][:, 0] == 0.0).all()
    check(g, t, d, drafts, u, dict(temperature=1.0))


def test_masked_minus_inf_logits():
    _announce("-inf masked logits, top-k and dense")
    t, d = S.zipf_logits(4, 3, 33000, 1.1, 1.0, "f32", seed=18)
    g = torch.Generator().manual_seed(18)
    t[torch.rand(t.shape, generator=g) < 0.3] = -float("inf")
    d[torch.rand(d.shape, generator=g) < 0.3] = -float("inf")
    verify_case(t, d, dict(temperature=1.0, top_k=30), seed=18)
    verify_case(t, d, dict(temperature=1.0), seed=18)


def test_draft_rows_k_plus_one():
    _announce("draft tensor with K+1 rows (last one unused)")
    t, d = S.zipf_logits(4, 3, 9000, 1.1, 1.0, "bf16", seed=19)
    d4 = torch.cat([d, d[:, :1]], dim=1).contiguous()
    params = dict(temperature=0.7, top_k=50)
    drafts, u = make_inputs(t, d, params, 19)
    g3 = run_gpu(t, d, drafts, u, params)
    g4 = run_gpu(t, d4, drafts, u, params)
    for k in g3:
        np.testing.assert_array_equal(g3[k], g4[k])


def test_vocab_of_one():
    _announce("V=1: every token is 0")
    t = torch.zeros((3, 3, 1))
    d = torch.zeros((3, 2, 1))
    drafts = np.zeros((3, 2), dtype=np.int32)
    u = S.philox_uniforms(20, (3, 3))
    g = run_gpu(t, d, drafts, u, dict(temperature=1.0))
    assert (g["num_accepted"] == 2).all() and (g["tokens"] == 0).all()


def test_deterministic_bitwise():
    _announce("two runs give bitwise equal outputs")
    t, d = S.zipf_logits(8, 3, 60000, 1.1, 1.0, "bf16", seed=21)
    for params in (dict(temperature=0.7, top_k=50), dict(temperature=1.0),
                   dict(temperature=1.0, top_p=0.9)):
        drafts, u = make_inputs(t, d, params, 21)
        a = run_gpu(t, d, drafts, u, params)
        b = run_gpu(t, d, drafts, u, params)
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (params, k)


def test_invalid_arguments_raise(_lib):
    _announce("invalid arguments return an error status")
    t, d = S.normal_logits(2, 2, 100, 2.0, 1.0, 0.5, "f32", seed=22)
    t, d = t.cuda(), d.cuda()
    x = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    u = torch.zeros((2, 3), dtype=torch.float32, device="cuda")
    for bad in (dict(temperature=-1.0), dict(top_p=0.0), dict(top_p=1.5), dict(lenience=0.0),
                dict(top_k=-3)):
        with pytest.raises(_lib.SpecVerifyError):
            _lib.spec_verify(t, d, x, u, **bad)


# ------------------------------------------------------------------ full-size workloads
def _full_size_check(name, nseq, seed):
    cfg = S.WORKLOADS[name]
    params = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], top_p=cfg["top_p"],
                  lenience=cfg["lenience"])
    t, d = S.workload_inputs(name, device="cuda", seed=seed)
    B, K = cfg["B"], cfg["K"]
    # draft tokens and uniforms: the oracle's sampler on a sample of sequences, fixed values
    # elsewhere (their results are not compared)
    pick = np.random.default_rng(seed).choice(B, size=nseq, replace=False)
    pick.sort()
    tt, dd = t[pick].cpu(), d[pick].cpu()
    drafts_s, u_s = make_inputs(tt, dd, params, seed)
    drafts = np.zeros((B, K), dtype=np.int32)
    u = S.philox_uniforms(seed + 3, (B, K + 1))
    drafts[pick] = drafts_s
    u[pick] = u_s
    g = run_gpu(t, d, drafts, u, params)
    gs = {k: v[pick] for k, v in g.items()}
    return check(gs, tt, dd, drafts_s, u_s, params)[0]


def test_full_size_topk_metric_workload():
    _announce("full size B=256 K=7 V=128256 bf16 top-k 50 T=0.7, 12 sampled sequences")
    _full_size_check("zipf_B256_K7_V128256_bf16_topk50", 12, 31)


def test_full_size_topp_workload():
    _announce("full size B=128 K=3 V=256000 fp32 top-p 0.95, 3 sampled sequences")
    _full_size_check("zipf_B128_K3_V256000_f32_topp95", 3, 32)


def test_full_size_dense_workload():
    _announce("full size B=64 K=4 V=32000 bf16 T=1, 16 sampled sequences")
    _full_size_check("normal_B64_K4_V32000_bf16", 16, 33)


def test_full_size_topk_topp_workload():
    _announce("full size B=256 K=7 V=128256 bf16 top-k 256 + top-p 0.9 T=0.7, 8 sampled sequences")
    _full_size_check("zipf_B256_K7_V128256_bf16_topk256_topp90", 8, 34)


def test_topk256_topp_bf16_ties():
    _announce("top-k 256 + top-p 0.9 on bf16 rows with many tied logits, B=6 K=3 V=50000")
    t, d = S.zipf_logits(6, 3, 50000, 1.1, 1.0, "bf16", seed=35)
    t, d = (t * 4).round() / 4, (d * 4).round() / 4  # coarse values: ties at both boundaries
    verify_case(t, d, dict(temperature=0.7, top_k=256, top_p=0.9), seed=35)
