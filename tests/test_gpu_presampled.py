"""spec_verify_presampled (binding: spec_verify(presampled=...)): verification that takes the
draft rows' summaries from the spec_sample call that drew the draft tokens, instead of
streaming the draft rows again.  Results must equal spec_verify's bit for bit (the summaries
are the same kernel's output on the same rows), and the tokens the oracle's."""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

from parity import check

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def svm():
    import speculative_sampling_verification_amd as m
    return m


def _pipeline(svm, t, d, params, seed):
    B, K1, V = t.shape
    K = K1 - 1
    tc, dc = t.cuda(), d.cuda()
    sp = {k: v for k, v in params.items() if k in ("temperature", "top_k", "top_p")}
    summary = svm.sample_summary(B * K, V, t.dtype, **sp)
    ud = torch.from_numpy(S.philox_uniforms(seed, (B * K,))).cuda()
    drafts = svm.spec_sample(dc.view(B * K, V), ud, summary=summary, **sp).view(B, K)
    u = torch.from_numpy(S.philox_uniforms(seed + 1, (B, K + 1))).cuda()
    pre = svm.spec_verify(tc, dc, drafts, u, presampled=summary, **params)
    plain = svm.spec_verify(tc, dc, drafts, u, **params)
    torch.cuda.synchronize()
    for k in plain:
        np.testing.assert_array_equal(pre[k].cpu().numpy(), plain[k].cpu().numpy(), err_msg=k)
    return drafts.cpu().numpy(), u.cpu().numpy(), {k: v.cpu().numpy() for k, v in pre.items()}


CASES = [
    ("bf16 top-k 50 T=0.7", dict(temperature=0.7, top_k=50), (32, 7), 128256, "bf16"),
    ("fp32 top-k 40 + top-p 0.9", dict(temperature=1.0, top_k=40, top_p=0.9), (8, 3), 40000,
     "f32"),
    ("bf16 top-k 256, unaligned V", dict(temperature=0.9, top_k=256), (6, 4), 50257, "bf16"),
    ("mentored D=0.1 top-k 40", dict(temperature=1.0, top_k=40, mentor_kl=0.1), (8, 4), 20000,
     "bf16"),
    ("lenience 0.5 top-k 20", dict(temperature=0.8, top_k=20, lenience=0.5), (8, 3), 30000,
     "bf16"),
]


@pytest.mark.parametrize("name,params,shape,V,dtype", CASES, ids=[c[0] for c in CASES])
def test_presampled_equals_spec_verify(svm, name, params, shape, V, dtype):
    _announce(f"presampled draft rows: {name}, B,K={shape} V={V}")
    B, K = shape
    t, d = S.zipf_logits(B, K, V, 1.1, 1.0, dtype, seed=V % 89)
    drafts, u, g = _pipeline(svm, t, d, params, V % 83)
    check(g, t, d, drafts, u, params)


def test_presampled_tie_overflow_rows(svm):
    _announce("presampled draft rows that took the whole-row path (ties overflow the lists)")
    gen = torch.Generator().manual_seed(91)
    t = torch.randint(0, 4, (3, 4, 30000), generator=gen).float().to(torch.bfloat16)
    d = torch.randint(0, 4, (3, 3, 30000), generator=gen).float().to(torch.bfloat16)
    _pipeline(svm, t, d, dict(temperature=1.0, top_k=50), 91)


def test_presampled_rejects_other_rows(svm):
    _announce("presampled needs draft rows [B, K, V] and compact sampling parameters")
    t, d = S.zipf_logits(2, 2, 1000, 1.1, 1.0, "bf16", seed=92)
    tc, dc = t.cuda(), d.cuda()
    summary = svm.sample_summary(4, 1000, torch.bfloat16, temperature=1.0, top_k=10)
    x = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    u = torch.zeros((2, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(svm.SpecVerifyError):
        svm.spec_verify(tc, dc, x, u, temperature=1.0, top_k=0, presampled=summary)
    with pytest.raises(svm.SpecVerifyError):
        svm.spec_verify(tc, dc, x, u, temperature=1.0, top_k=10,
                        presampled=summary[:16].contiguous())
