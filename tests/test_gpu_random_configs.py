"""Randomised parity sweep: many small configurations drawn at random (dtype, B, K, V with
ragged sizes, temperature, top-k, top-p, lenience, draft rows K or K+1, mentored bound),
each compared with the oracle to the same bar as the fixed cases (tests/parity.py)."""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

from parity import verify_case, verify_mentored_case

pytestmark = pytest.mark.gpu


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    B = int(rng.integers(1, 9))
    K = int(rng.integers(0, 9))
    V = int(rng.choice([1, 7, 64, 1000, 4097, 20000, 33000, 70001]))
    T = float(rng.choice([0.0, 0.3, 0.7, 1.0, 1.7]))
    top_k = int(rng.choice([0, 0, 1, 5, 50, 256, 300, 3000]))
    top_p = float(rng.choice([1.0, 1.0, 0.5, 0.9, 0.99]))
    lenience = float(rng.choice([1.0, 1.0, 1.0, 0.5, 0.1]))
    params = dict(temperature=T, top_k=top_k, top_p=top_p, lenience=lenience)
    gen = "zipf" if rng.random() < 0.6 else "normal"
    return dtype, B, K, V, params, gen, rng


@pytest.mark.parametrize("seed", range(30))
def test_random_config(seed):
    dtype, B, K, V, params, gen, rng = _config(seed)
    print(f"\n[case] seed={seed} {dtype} B={B} K={K} V={V} {gen} {params}", flush=True)
    if gen == "zipf":
        t, d = S.zipf_logits(B, K, V, 1.1, float(rng.choice([0.5, 1.0, 2.0])), dtype,
                             seed=seed)
    else:
        t, d = S.normal_logits(B, K, V, 3.0, 0.8, 1.5, dtype, seed=seed)
    if rng.random() < 0.3:  # some rows with -inf entries
        t[..., :: int(rng.integers(2, 50))] = -float("inf")
        t[..., 0] = 0.0
    if K > 0 and rng.random() < 0.3:  # a draft tensor with K+1 rows
        d = torch.cat([d, d[:, :1]], dim=1).contiguous()
    verify_case(t, d, params, seed=seed)


@pytest.mark.parametrize("seed", range(10))
def test_random_mentored_config(seed):
    rng = np.random.default_rng(2000 + seed)
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    B, K = int(rng.integers(1, 9)), int(rng.integers(1, 8))
    V = int(rng.choice([300, 5000, 40001]))
    params = dict(temperature=float(rng.choice([0.5, 1.0, 1.5])),
                  top_k=int(rng.choice([1, 10, 50, 200, 256])),
                  top_p=float(rng.choice([1.0, 0.9])),
                  mentor_kl=float(rng.choice([1e-3, 0.05, 0.3, 2.0])))
    print(f"\n[case] mentored seed={seed} {dtype} B={B} K={K} V={V} {params}", flush=True)
    t, d = S.zipf_logits(B, K, V, 1.1, float(rng.choice([0.5, 1.0, 2.0])), dtype, seed=seed)
    verify_mentored_case(t, d, params, seed=seed)
