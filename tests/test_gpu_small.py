"""GPU parity of the single-launch path for small problems (every row of a sequence held by one
workgroup: 2K+1 rows of V logits, at most 64 values per thread; dense rows, T > 0), against the
CPU oracle.  The shapes sit on both sides of each of the path's limits (V = 256 L, 2K+1 = 64 / L
for L = 4, 8, 16), so that the multi-kernel path takes the cases just past them.
"""

import numpy as np
import pytest
import torch

import oracle.spec_verify_oracle as O
from workloads import synthetic as S

from parity import check, make_inputs, run_gpu, verify_case

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import speculative_sampling_verification_amd as svm
    return svm


@pytest.mark.parametrize("B,K,V,dtype", [
    (1, 4, 1000, "f32"),      # the small benchmark shape
    (7, 7, 1024, "f32"),      # L = 4 at both limits: V = 1024, 2K+1 = 15 <= 16
    (5, 8, 1000, "f32"),      # 2K+1 = 17: past L = 4's rows, too many for L = 8: multi-kernel
    (6, 3, 1025, "bf16"),     # L = 8: V just past 1024
    (4, 3, 2048, "f32"),      # L = 8 at both limits: V = 2048, 2K+1 = 7 <= 8
    (3, 1, 4096, "bf16"),     # L = 16: V = 4096, 2K+1 = 3
    (3, 1, 4097, "f32"),      # V past 4096: multi-kernel
    (64, 2, 333, "bf16"),     # many sequences, a ragged vocabulary
])
def test_small_dense(B, K, V, dtype):
    _announce(f"small dense B={B} K={K} V={V} {dtype}")
    t, d = S.normal_logits(B, K, V, 2.0, 1.0, 0.5, dtype, seed=B * 1000 + V)
    verify_case(t, d, dict(temperature=1.0), seed=B * 1000 + V)


@pytest.mark.parametrize("T,lenience", [(0.6, 1.0), (1.7, 0.3)])
def test_small_temperature_lenience(T, lenience):
    _announce(f"small dense T={T} lenience={lenience} B=16 K=4 V=1000 fp32")
    t, d = S.normal_logits(16, 4, 1000, 2.0, 1.0, 0.5, "f32", seed=61)
    verify_case(t, d, dict(temperature=T, lenience=lenience), seed=61)


def test_small_minus_inf_and_identical_rows():
    _announce("small dense: -inf entries; p = q accepts every draft exactly")
    t, d = S.normal_logits(8, 4, 700, 2.0, 1.0, 0.5, "f32", seed=62)
    g = torch.Generator().manual_seed(62)
    t[torch.rand(t.shape, generator=g) < 0.2] = -float("inf")
    d[torch.rand(d.shape, generator=g) < 0.2] = -float("inf")
    t[:, :, 5] = 1.0  # every row keeps a finite logit
    d[:, :, 5] = 1.0
    verify_case(t, d, dict(temperature=1.0), seed=62)
    same = t[:, :4].contiguous()
    drafts, u = make_inputs(t, same, dict(temperature=1.0), 63)
    out = run_gpu(t, same, drafts, u, dict(temperature=1.0))
    assert (out["num_accepted"] == 4).all()
    assert (out["accept_prob"] == 1.0).all()


def test_small_k0_sample(_lib):
    _announce("small dense K=0: spec_sample against the oracle sampler, B=32 V=900 fp32")
    t, _ = S.normal_logits(32, 0, 900, 2.0, 1.0, 0.5, "f32", seed=64)
    rows = t[:, 0].contiguous()
    u = S.philox_uniforms(65, (32,))
    got = _lib.spec_sample(rows.cuda(), torch.from_numpy(u.copy()).cuda(),
                           temperature=1.0).cpu().numpy()
    want = O.sample_rows(rows.numpy(), u, np.float32(1.0))
    np.testing.assert_array_equal(got, want)
    drafts, uu = make_inputs(t, t[:, :0], dict(temperature=1.0), 66)
    g = run_gpu(t, None, drafts, uu, dict(temperature=1.0))
    check(g, t, None, drafts, uu, dict(temperature=1.0))
