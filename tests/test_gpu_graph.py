"""The library's launches inside a captured HIP graph (torch.cuda.CUDAGraph): every replay, with
new inputs copied into the captured buffers and eager work and synchronisations between the
replays, gives exactly what an eager call on the same inputs gives.

The entry points allocate nothing, query nothing from the device and issue no memset, so a
serving loop can capture a whole verify step once and replay it per decoding step.
"""

import numpy as np
import pytest
import torch

from workloads import synthetic as S

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def svm():
    import speculative_sampling_verification_amd as m
    return m


def _eager_noise():
    # unrelated eager work between replays, as a serving loop would have
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def _fresh(gen_seed, shape, V, dtype, kind):
    B, K1 = shape
    if kind == "zipf":
        t, d = S.zipf_logits(B, K1 - 1, V, 1.1, 1.0, dtype, seed=gen_seed)
    else:
        t, d = S.normal_logits(B, K1 - 1, V, 3.0, 0.8, 1.5, dtype, seed=gen_seed)
    g = torch.Generator().manual_seed(gen_seed)
    x = torch.randint(0, V, (B, K1 - 1), generator=g, dtype=torch.int32)
    u = torch.from_numpy(S.philox_uniforms(gen_seed + 7, (B, K1)))
    return t, d, x, u


def _copy_in(dst, src):
    for a, b in zip(dst, src):
        a.copy_(b.to(a.device))


VERIFY_CASES = [
    ("compact top-k 50 bf16", dict(temperature=0.7, top_k=50), (32, 6), 50000, "bf16", "zipf"),
    ("top-p 0.9 fp32", dict(temperature=1.0, top_p=0.9), (8, 4), 40000, "f32", "zipf"),
    ("dense T=1 bf16", dict(temperature=1.0), (8, 5), 32000, "bf16", "normal"),
    ("greedy T=0 bf16", dict(temperature=0.0), (8, 5), 32000, "bf16", "normal"),
    ("mentored D=0.1 top-k 40 bf16", dict(temperature=1.0, top_k=40, mentor_kl=0.1), (16, 5),
     20000, "bf16", "zipf"),
]


@pytest.mark.parametrize("name,params,shape,V,dtype,kind", VERIFY_CASES,
                         ids=[c[0] for c in VERIFY_CASES])
def test_spec_verify_graph_replays(svm, name, params, shape, V, dtype, kind):
    _announce(f"graph replay of spec_verify: {name}, B,K+1={shape} V={V}")
    host = _fresh(100, shape, V, dtype, kind)
    static = [h.cuda() for h in host]
    out = svm.spec_verify(*static, **params)  # eager warm-up: the workspace is allocated here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        svm.spec_verify(*static, out=out, **params)
    for rep in range(REPLAYS):
        _copy_in(static, _fresh(200 + rep, shape, V, dtype, kind))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        _eager_noise()
        ref = svm.spec_verify(*static, **params)
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(got[k].cpu().numpy(), ref[k].cpu().numpy(),
                                          err_msg=f"replay {rep}: {k}")


def test_spec_verify_tree_graph_replays(svm):
    _announce("graph replay of spec_verify_tree: B=8 N=16 V=32000 bf16")
    B, N, V = 8, 16, 32000

    def fresh(seed):
        t, _ = S.normal_logits(B, N - 1, V, 3.0, 0.8, 1.5, "bf16", seed=seed)
        g = torch.Generator().manual_seed(seed)
        parent = torch.full((B, N), -1, dtype=torch.int32)
        for i in range(1, N):
            parent[:, i] = torch.randint(0, i, (B,), generator=g, dtype=torch.int32)
        am = t.float().argmax(dim=2).to(torch.int32)
        tok = torch.randint(0, V, (B, N), generator=g, dtype=torch.int32)
        hit = torch.rand((B, N), generator=g) < 0.7  # most nodes carry their parent's argmax
        for i in range(1, N):
            p = parent[:, i].long()
            tok[:, i] = torch.where(hit[:, i], am[torch.arange(B), p], tok[:, i])
        return t, parent, tok

    static = [h.cuda() for h in fresh(300)]
    out = svm.spec_verify_tree(*static, 8)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        svm.spec_verify_tree(*static, 8, out=out)
    for rep in range(REPLAYS):
        _copy_in(static, fresh(400 + rep))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        _eager_noise()
        ref = svm.spec_verify_tree(*static, 8)
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(got[k].cpu().numpy(), ref[k].cpu().numpy(),
                                          err_msg=f"replay {rep}: {k}")


def test_spec_sample_graph_replays(svm):
    _announce("graph replay of spec_sample: R=64 V=50000 bf16 top-k 50")
    R, V = 64, 50000
    params = dict(temperature=0.8, top_k=50)

    def fresh(seed):
        t, _ = S.zipf_logits(R, 0, V, 1.1, 1.0, "bf16", seed=seed)
        return t[:, 0].contiguous(), torch.from_numpy(S.philox_uniforms(seed + 1, (R,)))

    static = [h.cuda() for h in fresh(500)]
    out = svm.spec_sample(*static, **params)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        svm.spec_sample(*static, out=out, **params)
    for rep in range(REPLAYS):
        _copy_in(static, fresh(600 + rep))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        _eager_noise()
        ref = svm.spec_sample(*static, **params)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy(),
                                      err_msg=f"replay {rep}")


def test_graph_replay_after_the_workspace_grew(svm):
    _announce("graph replay after a larger call replaced the stream's cached workspace")
    shape, V, params = (8, 5), 32000, dict(temperature=0.7, top_k=50)
    static = [h.cuda() for h in _fresh(700, shape, V, "bf16", "zipf")]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = svm.spec_verify(*static, **params)  # allocates side's workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        svm.spec_verify(*static, out=out, **params)
    # a larger call on the same stream replaces its cached workspace; the replaced buffer must
    # stay allocated for the graph
    big = [h.cuda() for h in _fresh(701, (64, 8), 128256, "bf16", "zipf")]
    with torch.cuda.stream(side):
        svm.spec_verify(*big, **params)
    torch.cuda.synchronize()
    for rep in range(2):
        _copy_in(static, _fresh(702 + rep, shape, V, "bf16", "zipf"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        ref = svm.spec_verify(*static, **params)
        torch.cuda.synchronize()
        for k in ref:
            np.testing.assert_array_equal(got[k].cpu().numpy(), ref[k].cpu().numpy(),
                                          err_msg=f"replay {rep}: {k}")


def test_two_streams_at_once(svm):
    _announce("spec_verify on two streams at once (one workspace per stream)")
    params = dict(temperature=0.8, top_k=40)
    a = [h.cuda() for h in _fresh(800, (32, 6), 50000, "bf16", "zipf")]
    b = [h.cuda() for h in _fresh(801, (32, 6), 50000, "bf16", "zipf")]
    ref_a = {k: v.cpu() for k, v in svm.spec_verify(*a, **params).items()}
    ref_b = {k: v.cpu() for k, v in svm.spec_verify(*b, **params).items()}
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = svm.spec_verify(*a, **params)
        with torch.cuda.stream(s2):
            ob = svm.spec_verify(*b, **params)
        torch.cuda.synchronize()
        for k in ref_a:
            np.testing.assert_array_equal(oa[k].cpu().numpy(), ref_a[k].numpy(), err_msg=k)
            np.testing.assert_array_equal(ob[k].cpu().numpy(), ref_b[k].numpy(), err_msg=k)


def test_release_workspaces_frees_the_cache(svm):
    _announce("release_workspaces frees the cached and outgrown workspaces; calls still work")
    from speculative_sampling_verification_amd import _lib
    params = dict(temperature=0.7, top_k=50)
    small = [h.cuda() for h in _fresh(900, (4, 3), 32000, "bf16", "zipf")]
    big = [h.cuda() for h in _fresh(901, (16, 5), 128256, "bf16", "zipf")]
    svm.release_workspaces()  # a clean cache, whatever ran before in this process
    assert not _lib._workspaces and not _lib._outgrown
    ref = {k: v.cpu() for k, v in svm.spec_verify(*small, **params).items()}
    svm.spec_verify(*big, **params)  # grows the stream's workspace: the small one is outgrown
    torch.cuda.synchronize()
    assert _lib._workspaces and _lib._outgrown
    held = sum(b.numel() for b in _lib._workspaces.values()) + sum(
        b.numel() for b in _lib._outgrown)
    assert svm.release_workspaces() == held
    assert not _lib._workspaces and not _lib._outgrown
    again = svm.spec_verify(*small, **params)  # allocates afresh
    torch.cuda.synchronize()
    for k in ref:
        np.testing.assert_array_equal(again[k].cpu().numpy(), ref[k].numpy(), err_msg=k)
