"""GPU parity of mentored decoding (the optimal lossy variant with a KL bound D) against the
oracle's mentored_spec_verify, through the C ABI.

The same bar as the lossless path (tests/parity.py): accepted counts and tokens bit-exact
except counted boundary flips, a_k = r at the draft token within 1e-5 absolute + 1e-4 relative.
Rows whose kept set exceeds the library's 1024-entry lists (ties at the top-k boundary) use the
lossless rule, which one test checks against the lossless oracle.
"""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

from parity import Lossless, check, make_inputs, run_gpu, verify_case, verify_mentored_case

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import speculative_sampling_verification_amd as svm
    return svm


@pytest.mark.parametrize("D", [0.02, 0.2])
def test_mentored_topk_bf16_full_vocab(D):
    _announce(f"mentored D={D} zipf bf16 top-k 50 T=0.7 B=4 K=7 V=128256")
    t, d = S.zipf_logits(4, 7, 128256, 1.1, 1.0, "bf16", seed=41)
    verify_mentored_case(t, d, dict(temperature=0.7, top_k=50, mentor_kl=D), seed=41)


@pytest.mark.parametrize("D", [1e-4, 0.01, 0.05, 0.5])
def test_mentored_many_sequences(D):
    _announce(f"mentored D={D} zipf bf16 top-k 64 T=1 B=48 K=4 V=3000")
    t, d = S.zipf_logits(48, 4, 3000, 1.1, 1.5, "bf16", seed=42)
    flips, g, o = verify_mentored_case(t, d, dict(temperature=1.0, top_k=64, mentor_kl=D),
                                       seed=42)
    # the case mixes solved, trivial and (at small D) nearly lossless positions
    assert o["n"].min() < 4


def test_mentored_fp32_topk_topp():
    _announce("mentored D=0.1 zipf fp32 top-k 40 + top-p 0.8 T=1 B=8 K=3 V=40000")
    t, d = S.zipf_logits(8, 3, 40000, 1.1, 2.0, "f32", seed=43)
    verify_mentored_case(t, d, dict(temperature=1.0, top_k=40, top_p=0.8, mentor_kl=0.1),
                         seed=43)


def test_mentored_topk_256_and_1():
    _announce("mentored D=0.05 with top-k 256 and top-k 1, bf16 B=6 K=3 V=20000")
    t, d = S.zipf_logits(6, 3, 20000, 1.1, 1.0, "bf16", seed=44)
    verify_mentored_case(t, d, dict(temperature=1.0, top_k=256, mentor_kl=0.05), seed=44)
    verify_mentored_case(t, d, dict(temperature=1.0, top_k=1, mentor_kl=0.05), seed=44)


def test_mentored_shortcut_changes_no_decision():
    _announce("mentored: the u < min(1, q/p) shortcut (no accept probabilities requested) "
              "gives the same tokens as solving every position")
    t, d = S.zipf_logits(32, 5, 8000, 1.1, 1.5, "bf16", seed=45)
    params = dict(temperature=0.9, top_k=50, mentor_kl=0.05)
    drafts, u = make_inputs(t, d, params, 45)
    full = run_gpu(t, d, drafts, u, params)
    short = run_gpu(t, d, drafts, u, dict(params, want_probs=False))
    np.testing.assert_array_equal(full["tokens"], short["tokens"])
    np.testing.assert_array_equal(full["num_accepted"], short["num_accepted"])


def test_mentored_accepts_at_least_as_often_as_lossless():
    _announce("mentored accept probabilities are >= the lossless ones, position by position")
    t, d = S.zipf_logits(16, 4, 6000, 1.1, 1.5, "bf16", seed=46)
    params = dict(temperature=1.0, top_k=50)
    drafts, u = make_inputs(t, d, params, 46)
    lossless = run_gpu(t, d, drafts, u, params)
    ment = run_gpu(t, d, drafts, u, dict(params, mentor_kl=0.1))
    assert (ment["accept_prob"] >= lossless["accept_prob"] - 1e-6).all()
    assert ment["accept_prob"].sum() > lossless["accept_prob"].sum()


def test_mentored_large_bound_accepts_every_draft():
    _announce("mentored D=50: KL(q || p) <= D everywhere, every draft accepted")
    t, d = S.zipf_logits(8, 4, 5000, 1.1, 1.0, "bf16", seed=47)
    # lift the same 20 tokens of each target row and its draft row far above the rest, so that
    # both top-20 sets coincide and KL(q || p) is finite
    gen = torch.Generator().manual_seed(47)
    for b in range(8):
        for k in range(5):
            top = torch.randperm(5000, generator=gen)[:20]
            t[b, k, top] += 30.0
            if k < 4:
                d[b, k, top] += 30.0
    params = dict(temperature=1.0, top_k=20, mentor_kl=50.0)
    flips, g, o = verify_mentored_case(t, d, params, seed=47)
    assert (g["num_accepted"] == 4).all()
    assert (g["accept_prob"] == 1.0).all()


def test_mentored_greedy_is_lossless():
    _announce("mentored at temperature 0 equals the lossless greedy rule")
    t, d = S.normal_logits(8, 5, 32000, 3.0, 0.8, 1.5, "bf16", seed=48)
    drafts, u = make_inputs(t, d, dict(temperature=1.0), 48)
    drafts[:, :3] = t.float().argmax(dim=2).numpy()[:, :3]
    g = run_gpu(t, d, drafts, u, dict(temperature=0.0, mentor_kl=0.3))
    check(g, t, d, drafts, u, dict(temperature=0.0), max_flip_frac=0.0)


def test_mentored_out_of_range_draft_tokens():
    _announce("mentored: draft tokens outside [0, V) are rejected, replacement drawn")
    t, d = S.zipf_logits(6, 3, 7000, 1.1, 1.0, "bf16", seed=49)
    params = dict(temperature=0.8, top_k=30, mentor_kl=0.1)
    drafts, u = make_inputs(t, d, params, 49)
    drafts[0, 0] = -1
    drafts[1, 1] = 7000
    drafts[2, 2] = 123456
    flips, g, o = verify_mentored_case(t, d, params, drafts=drafts, u=u)
    assert g["num_accepted"][0] == 0 and g["num_accepted"][1] <= 1
    assert g["accept_prob"][0, 0] == 0.0


def test_mentored_long_kept_lists():
    _announce("mentored: kept lists of 246-298 tokens (ties at top-k 230) take the second "
              "solve, fp32 B=6 K=3 V=20000")
    t, d = S.zipf_logits(6, 3, 20000, 1.1, 1.0, "f32", seed=53)
    t, d = (t * 2).round() / 2, (d * 2).round() / 2
    params = dict(temperature=1.0, top_k=230, mentor_kl=0.05)
    flips, g, o = verify_mentored_case(t, d, params, seed=53)
    drafts, u = make_inputs(t, d, params, 53)
    short = run_gpu(t, d, drafts, u, dict(params, want_probs=False))
    np.testing.assert_array_equal(g["tokens"], short["tokens"])


def test_mentored_tie_overflow_rows_use_lossless_rule():
    _announce("mentored: rows whose top-k ties overflow the kept lists use the lossless rule")
    g = torch.Generator().manual_seed(50)
    t = torch.randint(0, 4, (3, 3, 40000), generator=g).float().to(torch.bfloat16)
    d = torch.randint(0, 4, (3, 2, 40000), generator=g).float().to(torch.bfloat16)
    verify_case(t, d, dict(temperature=1.0, top_k=50, mentor_kl=0.2), seed=50,
                rule=Lossless(1.0))


def test_mentored_invalid_combinations(_lib):
    _announce("mentored: invalid parameter combinations return an error status")
    t, d = S.normal_logits(2, 2, 100, 2.0, 1.0, 0.5, "f32", seed=51)
    t, d = t.cuda(), d.cuda()
    x = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    u = torch.zeros((2, 3), dtype=torch.float32, device="cuda")
    for bad in (dict(mentor_kl=0.1), dict(mentor_kl=0.1, top_k=300),
                dict(mentor_kl=0.1, top_k=10, lenience=0.5), dict(mentor_kl=-1.0, top_k=10),
                dict(mentor_kl=float("nan"), top_k=10)):
        with pytest.raises(_lib.SpecVerifyError):
            _lib.spec_verify(t, d, x, u, **bad)


def test_mentored_full_size_sampled():
    _announce("mentored D=0.1 full size B=256 K=7 V=128256 bf16 top-k 50 T=0.7, "
              "6 sampled sequences")
    name = "zipf_B256_K7_V128256_bf16_topk50"
    cfg = S.WORKLOADS[name]
    params = dict(temperature=cfg["temperature"], top_k=cfg["top_k"], mentor_kl=0.1)
    t, d = S.workload_inputs(name, device="cuda", seed=52)
    B, K = cfg["B"], cfg["K"]
    pick = np.sort(np.random.default_rng(52).choice(B, size=6, replace=False))
    tt, dd = t[pick].cpu(), d[pick].cpu()
    drafts_s, u_s = make_inputs(tt, dd, params, 52)
    drafts = np.zeros((B, K), dtype=np.int32)
    u = S.philox_uniforms(55, (B, K + 1))
    drafts[pick] = drafts_s
    u[pick] = u_s
    g = run_gpu(t, d, drafts, u, params)
    gs = {k: v[pick] for k, v in g.items()}
    check(gs, tt, dd, drafts_s, u_s, params)
    assert ((g["num_accepted"] >= 0) & (g["num_accepted"] <= K)).all()
