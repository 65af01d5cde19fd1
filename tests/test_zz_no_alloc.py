"""spec_verify_noalloc (the entry point without a workspace argument, for callers that cannot
allocate) against spec_verify, through the C ABI: two calls in a row on one GPU, the second on a
smaller problem than the first, each bitwise equal to spec_verify's results on the same inputs
(spec_verify is held to the oracle by the parity tests; these results are checked against it
too).  A problem whose workspace exceeds the scratch buffer is refused before any launch."""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

import parity

pytestmark = pytest.mark.gpu

KEYS = ("tokens", "num_accepted", "accept_prob", "q_draft", "p_draft")


@pytest.fixture(scope="module")
def svm():
    import speculative_sampling_verification_amd as m
    return m


def _prepare(name, params, B, K, V, dtype, seed):
    print(f"\n[case] noalloc {name}: B={B} K={K} V={V} {dtype} {params}", flush=True)
    t, d = S.zipf_logits(B, K, V, 1.1, 1.0 if dtype == "bf16" else 2.0, dtype, seed=seed)
    drafts, u = parity.make_inputs(t, d, params, seed)
    dev = torch.device("cuda")
    inp = (t.to(dev), d.to(dev), torch.from_numpy(drafts).to(dev), torch.from_numpy(u).to(dev))
    return t, d, drafts, u, inp


def _outs(B, K):
    dev = torch.device("cuda")
    o = {"tokens": torch.full((B, K + 1), -7, dtype=torch.int32, device=dev),
         "num_accepted": torch.full((B,), -7, dtype=torch.int32, device=dev)}
    for k in ("accept_prob", "q_draft", "p_draft"):
        o[k] = torch.full((B, K), -7.0, dtype=torch.float32, device=dev)
    return o


def test_noalloc_equals_spec_verify_on_two_calls_in_a_row(svm):
    cases = [
        ("larger", dict(temperature=0.7, top_k=50), 64, 7, 128256, "bf16", 3),
        ("smaller", dict(temperature=1.0, top_p=0.9), 4, 3, 40000, "f32", 4),
    ]
    prepared = [_prepare(*c) for c in cases]
    # spec_verify first (its own workspace), then the two no-allocation calls back to back
    want = []
    for (name, params, B, K, V, dtype, seed), (t, d, drafts, u, inp) in zip(cases, prepared):
        r = svm.spec_verify(*inp, **params)
        torch.cuda.synchronize()
        want.append({k: r[k].cpu().numpy() for k in KEYS})
    outs = []
    for (name, params, B, K, V, dtype, seed), (t, d, drafts, u, inp) in zip(cases, prepared):
        o = _outs(B, K)
        svm.spec_verify_noalloc(*inp, o, **params)
        outs.append(o)
    torch.cuda.synchronize()
    for (name, params, B, K, V, dtype, seed), (t, d, drafts, u, inp), o, w in zip(
            cases, prepared, outs, want):
        got = {k: o[k].cpu().numpy() for k in KEYS}
        for k in KEYS:
            assert np.array_equal(got[k].view(np.uint8), w[k].view(np.uint8)), (name, k)
        flips, _ = parity.check(got, t, d, drafts, u, params)
        print(f"[noalloc] {name}: equal to spec_verify, flips {flips}", flush=True)


def test_noalloc_refuses_a_problem_beyond_the_scratch(svm):
    # B=128 K=3 V=256000 fp32 top-p 0.95 needs about 253 MiB of workspace
    B, K, V = 128, 3, 256000
    from speculative_sampling_verification_amd import _lib
    import ctypes
    samp = _lib.sampling(temperature=1.0, top_p=0.95)
    need = _lib.lib().spec_verify_workspace_size(B, K, V, 0, ctypes.byref(samp))
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    t = torch.zeros((B, K + 1, V), dtype=torch.float32, device=dev)
    d = torch.zeros((B, K, V), dtype=torch.float32, device=dev)
    x = torch.zeros((B, K), dtype=torch.int32, device=dev)
    u = torch.zeros((B, K + 1), dtype=torch.float32, device=dev)
    o = _outs(B, K)
    with pytest.raises(svm.SpecVerifyError) as err:
        svm.spec_verify_noalloc(t, d, x, u, o, temperature=1.0, top_p=0.95)
    assert err.value.code == _lib.SV_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert (o["tokens"] == -7).all() and (o["num_accepted"] == -7).all()
