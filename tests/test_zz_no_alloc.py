"""proj_run_noalloc, the entry point that allocates nothing: its kernels'
workspace comes from the library's static device scratch instead of from the
plan.  Called through the C ABI and compared with proj_run_ex on the same
plan, bit for bit (same kernels, same order of operations), and with the
oracle at the projection tolerance, on two calls in a row with the second on a
smaller input (the scratch keeps the first call's contents).  Plans are built
with PROJ_FORCE so that the tuned choice is a kernel that uses the workspace:
split-K partials, split-tail partials, the normalised rows of the unfused
RMSNorm, the intermediate of the unfused SwiGLU.  A call whose kernel needs
more scratch than there is is rejected with nothing enqueued.
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _forced_plan(monkeypatch, N, K, dtype, pick, **kw):
    """A plan whose every applicable bucket runs the first candidate `pick` accepts."""
    from shape_specialised_bf16_amd import Plan
    names = G.plan(N, K, dtype, **kw).candidates()
    name = next(n for n in names if pick(n))
    monkeypatch.setenv("PROJ_FORCE", name)
    try:
        p = Plan(N, K, dtype, **kw)
    finally:
        monkeypatch.delenv("PROJ_FORCE")
    return p, name


def _both(plan, X, W, M, dtype, gamma=None):
    """Y from proj_run_ex and from proj_run_noalloc, after a sync."""
    import torch
    Ya = G.empty_out(M, plan.NO, dtype, extra_rows=1)
    Yb = G.empty_out(M, plan.NO, dtype, extra_rows=1)
    plan.run(X[:M], W, Ya, gamma=gamma)
    plan.run_noalloc(X[:M], W, Yb, gamma=gamma)
    torch.cuda.synchronize()
    a, b = G.host(Ya), G.host(Yb)
    view = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(a.view(view), b.view(view)), f"proj_run_noalloc differs from proj_run_ex at M={M}"
    return Yb


def test_split_k_partials_in_scratch_and_size_limit(monkeypatch):
    N, K = 7168, 1024
    plan, name = _forced_plan(monkeypatch, N, K, "f32", lambda n: n.endswith("_sk8"))
    Wh = synth.normal_bf16(130, 0, (N, K), 0.02)
    Xh = synth.normal_bf16(130, 1, (512, K), 1.0)
    W, X = G.dev(Wh), G.dev(Xh)
    for M in (128, 100):                                   # both in the {17..128} bucket: the split-K kernel
        assert plan.choice(M) == name
        Y = _both(plan, X, W, M, "f32")
        G.check_against_oracle(Y, Xh[:M], Wh, "f32", label=f"noalloc {name}")
    # 8 x 512 x 7168 f32 partials = 117 MiB > 64 MiB of scratch: rejected, nothing written
    from shape_specialised_bf16_amd import ProjError
    assert plan.choice(512) == name
    Y = G.empty_out(512, N, "f32")
    with pytest.raises(ProjError) as e:
        plan.run_noalloc(X, W, Y)
    assert "scratch" in str(e.value) and "PROJ_EINVAL" in str(e.value)
    import torch
    torch.cuda.synchronize()
    assert np.all(G.host(Y).view(np.uint32) == 0x7FC00001)
    plan.close()


def test_split_tail_partials_in_scratch(monkeypatch):
    N, K = 18432, 2560
    plan, name = _forced_plan(monkeypatch, N, K, "bf16", lambda n: "_tail2_" in n and n.startswith("gemm_256x128"))
    Wh = synth.normal_bf16(131, 0, (N, K), 0.02)
    Xh = synth.normal_bf16(131, 1, (2048, K), 1.0)
    W, X = G.dev(Wh), G.dev(Xh)
    for M in (2048, 1000):
        assert plan.choice(M) == name
        Y = _both(plan, X, W, M, "bf16")
        G.check_against_oracle(Y, Xh[:M], Wh, "bf16", rows=G.sample_rows(M, seed=M), label=f"noalloc {name}")
    plan.close()


def test_unfused_norm_rows_in_scratch():
    import torch
    N, K = 2048, 1024
    plan = G.plan(N, K, "f32", rmsnorm_eps=EPS)
    Wh = synth.normal_bf16(132, 0, (N, K), 0.02)
    Xh = synth.normal_bf16(132, 1, (64, K), 1.0)
    g = (1.0 + 0.25 * np.random.default_rng(132).standard_normal(K)).astype(np.float32)
    gd = torch.from_numpy(g).cuda()
    for M in (64, 16):                                     # M > 1: the norm runs unfused, into scratch
        Y = _both(plan, G.dev(Xh), G.dev(Wh), M, "f32", gamma=gd)
        ref = oracle.rmsnorm_matmul(Xh[:M], g, Wh, EPS)
        terms = oracle.rmsnorm_matmul(Xh[:M], g, Wh, EPS, absolute=True)
        rep = tolerance.check_norm_projection(G.host(Y)[:M], ref, terms, "f32")
        assert rep.ok, rep
        G.log(f"  noalloc norm plan M={M} ({plan.choice(M)}): {rep}")


def test_unfused_swiglu_intermediate_in_scratch(monkeypatch):
    N, K = 6144, 1024
    plan, name = _forced_plan(monkeypatch, N, K, "f32", lambda n: n.startswith("gemv_mfma") and n.endswith("_uf"),
                              epilogue="swiglu")
    Wh = synth.normal_bf16(133, 0, (N, K), 0.02)
    Xh = synth.normal_bf16(133, 1, (16, K), 1.0)
    for M in (16, 5):
        assert plan.choice(M) == name
        Y = _both(plan, G.dev(Xh), G.dev(Wh), M, "f32")
        gu = oracle.matmul(Xh[:M], Wh)
        rep = tolerance.check_swiglu(G.host(Y)[:M], gu[:, :N // 2], gu[:, N // 2:], "f32")
        assert rep.ok, rep
        G.log(f"  noalloc swiglu {name} M={M}: {rep}")
    plan.close()
