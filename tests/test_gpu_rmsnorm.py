"""The RMSNorm prologue folded into the projection (plans created with
rmsnorm_eps, through proj_plan_create_ex with PROJ_PRO_RMSNORM), on the GPU.

"#004 the same compiler on Apple's chips", section "Decode": running the norm
inside the next projection's kernel must reproduce the separate kernels bit for
bit, and the load-time measurement decides whether it is used.  So: each folded
("_nf") candidate equals its unfused twin (the separate norm kernel, then the
same kernel variant) bit for bit; both equal a plain plan's candidate run on
proj_rmsnorm's output; and every result is within the derived allowance of
the oracle (oracle.rmsnorm_matmul).
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _gamma(K, seed):
    import torch
    g = (1.0 + 0.25 * np.random.default_rng(seed).standard_normal(K)).astype(np.float32)
    return g, torch.from_numpy(g).cuda()


def _check(Y, X, g, W, dtype, rows=None, label="", refs=None):
    """Y against the oracle; refs (optional) caches the oracle's (ref, terms)
    per row count for callers that check many candidates on the same rows."""
    Xs = X if rows is None else X[rows]
    key = (Xs.shape[0], rows is None)
    if refs is not None and key in refs:
        ref, terms = refs[key]
    else:
        ref = oracle.rmsnorm_matmul(Xs, g, W, EPS)
        terms = oracle.rmsnorm_matmul(Xs, g, W, EPS, absolute=True)
        if refs is not None:
            refs[key] = (ref, terms)
    h = G.host(Y)
    h = h if rows is None else h[rows]
    rep = tolerance.check_norm_projection(h, ref, terms, dtype)
    assert rep.ok, f"{label}: {rep}"
    G.log(f"  {label}: {rep}")


@pytest.mark.parametrize("K", [1024, 5120])
def test_norm_kernel_against_oracle(K):
    import shape_specialised_bf16_amd as ssb
    X = synth.normal_bf16(97, K, (9, K), 1.0)
    g, gd = _gamma(K, K)
    Xn = ssb.rmsnorm(G.dev(X), gd, EPS)
    got = oracle.bf16_bits_to_f64(G.host(Xn))
    R = oracle.bf16_bits_to_f64(oracle.round_bf16(oracle.rmsnorm(X, g, EPS)))
    assert np.all(np.abs(got - R) <= tolerance.bf16_ulp(R)), np.max(np.abs(got - R) / tolerance.bf16_ulp(R))


@pytest.mark.parametrize("K", [520, 1024, 5120, 17408])
def test_norm_kernel_on_boundary_rows(K):
    """Rows whose normalised values sit next to bf16 rounding boundaries
    (synth.norm_boundary_case; the oracle's pins show that a mean over K - 1
    terms rounds row 0 the other way at every element, and that a misplaced or
    different epsilon moves row 1 by more than an ulp): row 0 must come out
    exactly as the oracle rounds it, row 1 within one bf16 ulp."""
    import shape_specialised_bf16_amd as ssb
    import torch
    X, g, lo, hi = synth.norm_boundary_case(K)
    Xn = G.host(ssb.rmsnorm(G.dev(X), torch.from_numpy(g).cuda(), EPS)).view(np.uint16)   # bits as uploaded
    R = oracle.round_bf16(oracle.rmsnorm(X, g, EPS))
    assert np.array_equal(R[0], hi)
    assert np.array_equal(Xn[0], R[0]), f"{int(np.sum(Xn[0] != R[0]))} of {K} elements of row 0 differ"
    got1, ref1 = oracle.bf16_bits_to_f64(Xn[1]), oracle.bf16_bits_to_f64(R[1])
    assert np.all(np.abs(got1 - ref1) <= tolerance.bf16_ulp(ref1))


def test_folded_norm_on_boundary_row():
    """The norm folded into the M = 1 decode kernels on the same row 0: every
    folded candidate equals the plain candidate run on the separate kernel's
    output, whose bits the test above fixes exactly."""
    import shape_specialised_bf16_amd as ssb
    import torch
    N, K = 2048, 1024
    X, g, lo, hi = synth.norm_boundary_case(K)
    gd = torch.from_numpy(g).cuda()
    W = synth.normal_bf16(98, 0, (N, K), 0.02)
    Wd = G.dev(W)
    pn, pp = G.plan(N, K, "f32", rmsnorm_eps=EPS), G.plan(N, K, "f32")
    Xd = G.dev(X[:1])
    Xn = ssb.rmsnorm(Xd, gd, EPS)
    assert np.array_equal(G.host(Xn).view(np.uint16)[0], hi)
    folded = [i for i, n in enumerate(pn.candidates()) if n.endswith("_nf")]
    assert folded, "no folded candidate"
    for i in folded:
        name = pn.candidates()[i]
        j = pp.candidates().index(name[: -len("_nf")])
        Yf = G.empty_out(1, N, "f32")
        pn.run_candidate(i, Xd, Wd, Yf, gamma=gd)
        Yp = G.empty_out(1, N, "f32")
        pp.run_candidate(j, Xn, Wd, Yp)
        assert np.array_equal(G.host(Yf).view(np.uint8), G.host(Yp).view(np.uint8)), name


@pytest.mark.parametrize("N,K,dtype", [(2048, 1024, "f32"), (10240, 5120, "bf16"), (1000, 520, "f32")])
def test_folded_norm_equals_unfused(N, K, dtype):
    import torch
    import shape_specialised_bf16_amd as ssb
    pn = G.plan(N, K, dtype, rmsnorm_eps=EPS)
    pp = G.plan(N, K, dtype)
    W = synth.normal_bf16(98, 0, (N, K), 0.02)
    X = synth.normal_bf16(98, 1, (130, K), 1.0)
    g, gd = _gamma(K, 7)
    Wd, Xd = G.dev(W), G.dev(X)
    Xn = ssb.rmsnorm(Xd, gd, EPS)
    names = pn.candidates()
    plain_names = pp.candidates()
    refs = {}
    for idx, name in enumerate(names):
        M = min(pn.candidate_max_m(idx), 130)
        Y = G.empty_out(M, N, dtype, extra_rows=1)
        pn.run_candidate(idx, Xd[:M], Wd, Y[:M], gamma=gd)
        base = name
        while base.endswith(("_nf", "_uf")):       # folded norm / unfused SwiGLU copies
            base = base[:-3]
        # the plain plan's same variant on the separately normalised rows
        Yp = pp.run_candidate(plain_names.index(base), Xn[:M], Wd)
        torch.cuda.synchronize()
        assert np.array_equal(G.host(Y)[:M].view(np.uint8), G.host(Yp).view(np.uint8)), \
            f"{name} M={M}: differs from {base} on proj_rmsnorm's output"
        pat = 0x7FC1 if dtype == "bf16" else 0x7FC00001
        assert np.all(G.host(Y)[M:].view(np.uint16 if dtype == "bf16" else np.uint32) == pat), f"{name} wrote past M"
        if name.endswith("_nf") or M == 130:
            _check(Y[:M], X[:M], g, W, dtype, label=f"{N}x{K} {dtype} {name} M={M} vs oracle", refs=refs)
    G.log(f"  {N}x{K} {dtype}: {len(names)} candidates equal to the unfused path")


def test_tuned_decode_projections_and_choice():
    """The 0.8B-like QKV and the head with the norm prologue, tuned, at M = 1;
    the plan records whether the folded or the unfused variant won."""
    cfg = synth.workload("decode_0.8b_layer_m1")
    for name in ("qkv", "head"):
        pi = [p.name for p in cfg.projections].index(name)
        p = cfg.projections[pi]
        W = synth.weights(cfg, pi)
        X = synth.activations(cfg, pi, 1)
        g, gd = _gamma(p.K, 11)
        plan = G.plan(p.N, p.K, "f32", rmsnorm_eps=EPS)
        Y = G.empty_out(1, p.N, "f32", extra_rows=1)
        plan.run(G.dev(X), G.dev(W), Y, gamma=gd)
        _check(Y[:1], X, g, W, "f32", label=f"0.8B {name} with the norm, tuned -> {plan.choice(1)}")
        assert np.all(G.host(Y)[1:].view(np.uint32) == 0x7FC00001)


def test_tuned_prefill_with_norm():
    cfg = synth.workload("prefill_4b_layer")
    pi = [p.name for p in cfg.projections].index("qkv")
    p = cfg.projections[pi]
    W = synth.weights(cfg, pi)
    M = 512
    X = synth.activations(cfg, pi, M)
    g, gd = _gamma(p.K, 12)
    plan = G.plan(p.N, p.K, "bf16", rmsnorm_eps=EPS)
    Y = G.empty_out(M, p.N, "bf16", extra_rows=1)
    plan.run(G.dev(X), G.dev(W), Y, gamma=gd)
    _check(Y, X, g, W, "bf16", rows=G.sample_rows(M, seed=3), label=f"4B qkv M={M} norm, {plan.choice(M)}")
    assert np.all(G.host(Y)[M].view(np.uint16) == 0x7FC1)


def test_norm_and_swiglu_together_equal_unfused_chain():
    """gate_up with both folded: equal to proj_rmsnorm -> the plain plan's same
    variant -> proj_swiglu, for every candidate."""
    import torch
    import shape_specialised_bf16_amd as ssb
    N, K = 6144, 1024
    pb = G.plan(N, K, "f32", epilogue="swiglu", rmsnorm_eps=EPS)
    pp = G.plan(N, K, "f32")
    W = synth.normal_bf16(99, 0, (N, K), 0.02)
    X = synth.normal_bf16(99, 1, (17, K), 1.0)
    g, gd = _gamma(K, 13)
    Wd, Xd = G.dev(W), G.dev(X)
    Xn = ssb.rmsnorm(Xd, gd, EPS)
    for idx, name in enumerate(pb.candidates()):
        M = min(pb.candidate_max_m(idx), 17)
        H = pb.run_candidate(idx, Xd[:M], Wd, gamma=gd)
        base = name
        while base.endswith(("_nf", "_uf")):       # folded norm / unfused SwiGLU copies
            base = base[:-3]
        Hu = ssb.swiglu(pp.run_candidate(pp.candidates().index(base), Xn[:M], Wd))
        torch.cuda.synchronize()
        assert np.array_equal(G.host(H).view(np.uint32), G.host(Hu).view(np.uint32)), name


def test_missing_gamma_is_rejected():
    import torch
    from shape_specialised_bf16_amd import ProjError
    plan = G.plan(2048, 1024, "f32", rmsnorm_eps=EPS)
    X = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((2048, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ProjError, match="gamma"):
        plan.run(X, W)
