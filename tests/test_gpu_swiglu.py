"""The SwiGLU epilogue folded into the gate_up projection (plans created with
epilogue="swiglu", through proj_plan_create_ex), on the GPU.  Such a plan holds
fused candidates and the plain candidates run unfused ("_uf"), the tuner
choosing between them.

"#004 the same compiler on Apple's chips", section "Decode": a fusion leaves
every output bit as the separate kernels produce it, and whether to use it is
decided by measurement at load time.  So: every fused candidate must equal, bit for bit, the plain plan's
candidate of the same name followed by the separate activation kernel
(proj_swiglu); and the fused result must be within the derived SwiGLU
allowance of the oracle (oracle.swiglu of the fp64 product).
"""
import numpy as np
import pytest

import oracle
from oracle import tolerance
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _oracle_gu(X, W, rows=None):
    ref = oracle.matmul(X, W) if rows is None else oracle.matmul_rows(X, rows, W)
    half = W.shape[0] // 2
    return ref[:, :half], ref[:, half:]


def _check_vs_oracle(H, X, W, dtype, rows=None, label="", refs=None):
    """H against the oracle; refs (optional) caches the oracle's gate and up
    sums per row count for callers that check many candidates on the same rows."""
    key = (X.shape[0], None if rows is None else tuple(rows))
    if refs is not None and key in refs:
        g, u = refs[key]
    else:
        g, u = _oracle_gu(X, W, rows)
        if refs is not None:
            refs[key] = (g, u)
    h = G.host(H)
    h = h if rows is None else h[rows]
    y = oracle.bf16_bits_to_f64(h) if dtype == "bf16" else h.astype(np.float64)
    rep = tolerance.check_swiglu(y, g, u, dtype)
    assert rep.ok, f"{label}: {rep}"
    G.log(f"  {label}: {rep}")


@pytest.mark.parametrize("N,K,dtype", [(6144, 1024, "f32"), (7168, 1024, "bf16"), (18432, 2560, "bf16"),
                                       (1000, 520, "f32")])
def test_every_fused_candidate_equals_unfused_path(N, K, dtype):
    import torch
    import shape_specialised_bf16_amd as ssb
    pf = G.plan(N, K, dtype, epilogue="swiglu")
    pu = G.plan(N, K, dtype)
    W = synth.normal_bf16(90, 0, (N, K), 0.02)
    Xall = synth.normal_bf16(90, 1, (600, K), 1.0)
    Wd = G.dev(W)
    unfused_names = pu.candidates()
    for idx, name in enumerate(pf.candidates()):
        # a fused candidate, or one of the plain plan's run unfused ("_uf"): both
        # must equal the plain plan's variant followed by proj_swiglu
        base = name[:-3] if name.endswith("_uf") else name
        assert base in unfused_names, name
        uidx = unfused_names.index(base)
        mmax = min(pf.candidate_max_m(idx), pu.candidate_max_m(uidx))
        Ms = [1, 5, 16] if mmax <= 16 else [1, 17, 130, 600]
        for M in [m for m in Ms if m <= mmax]:
            Xd = G.dev(Xall[:M])
            Hf = G.empty_out(M, N // 2, dtype, extra_rows=1)
            pf.run_candidate(idx, Xd, Wd, Hf)
            Y = G.empty_out(M, N, dtype)
            pu.run_candidate(uidx, Xd, Wd, Y)
            Hu = ssb.swiglu(Y)
            torch.cuda.synchronize()
            a = G.host(Hf)
            assert np.array_equal(a[:M].view(np.uint8), G.host(Hu).view(np.uint8)), f"{name} M={M}: fused != unfused"
            pat = 0x7FC1 if dtype == "bf16" else 0x7FC00001
            assert np.all(a[M:].view(np.uint16 if dtype == "bf16" else np.uint32) == pat), f"{name} wrote past M"
        G.log(f"  {N}x{K} {dtype} {name}: fused == unfused (bitwise)")
    # the fused results against the oracle, for the largest M each family ran
    refs = {}
    for idx, name in enumerate(pf.candidates()):
        M = min(pf.candidate_max_m(idx), 130)
        H = pf.run_candidate(idx, G.dev(Xall[:M]), Wd)
        _check_vs_oracle(H, Xall[:M], W, dtype, label=f"{N}x{K} {dtype} {name} M={M} vs oracle", refs=refs)


def test_integer_probe_bit_exact_through_the_epilogue():
    """With integer inputs the gate and up sums are exact in any order, so
    every fused candidate's output is the activation of exact integers: equal
    across candidates and to the oracle's sums pushed through the same f32
    evaluation on the GPU (the plain plan + proj_swiglu)."""
    import torch
    import shape_specialised_bf16_amd as ssb
    N, K = 2048, 1024
    pf = G.plan(N, K, "f32", epilogue="swiglu")
    W = synth.int_bf16(91, (N, K))
    X = synth.int_bf16(92, (130, K))
    exact = oracle.matmul(X, W)                       # integers, exact in f32
    Gd = torch.from_numpy(oracle.round_f32(exact)).cuda()
    want = G.host(ssb.swiglu(Gd))                     # the activation of the exact sums
    for idx, name in enumerate(pf.candidates()):
        M = min(pf.candidate_max_m(idx), 130)
        H = pf.run_candidate(idx, G.dev(X[:M]), G.dev(W))
        assert np.array_equal(G.host(H).view(np.uint32), want[:M].view(np.uint32)), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unfused_activation_kernel(dtype):
    """proj_swiglu against the fp64 activation of the very values it read."""
    import torch
    import shape_specialised_bf16_amd as ssb
    rng = np.random.default_rng(93)
    Gh = (rng.standard_normal((37, 2 * 1000)) * 4).astype(np.float32)
    Gd = torch.from_numpy(Gh).cuda()
    if dtype == "bf16":
        Gd = Gd.to(torch.bfloat16)
    H = ssb.swiglu(Gd)
    gv = Gd.float().cpu().numpy().astype(np.float64)
    g, u = gv[:, :1000], gv[:, 1000:]
    ref = g / (1.0 + np.exp(-g)) * u
    if dtype == "f32":
        got = H.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - ref) <= 2.0 ** -20 * np.abs(ref) + 1e-30)
    else:
        got = oracle.bf16_bits_to_f64(G.host(H))
        R = oracle.bf16_bits_to_f64(oracle.round_bf16(ref))
        assert np.all(np.abs(got - R) <= tolerance.bf16_ulp(R))


def test_decode_gate_up_08b_tuned():
    cfg = synth.workload("decode_0.8b_layer_m1")
    pi = [p.name for p in cfg.projections].index("gate_up")
    p = cfg.projections[pi]
    W = synth.weights(cfg, pi)
    X = synth.activations(cfg, pi, 1)
    plan = G.plan(p.N, p.K, "f32", epilogue="swiglu")
    H = G.empty_out(1, p.N // 2, "f32", extra_rows=1)
    plan.run(G.dev(X), G.dev(W), H)
    _check_vs_oracle(H[:1], X, W, "f32", label=f"0.8B gate_up fused {plan.choice(1)}")
    assert np.all(G.host(H)[1:].view(np.uint32) == 0x7FC00001)


@pytest.mark.parametrize("M", [512, 2048])
def test_prefill_gate_up_4b_tuned(M):
    cfg = synth.workload("prefill_4b_layer")
    pi = [p.name for p in cfg.projections].index("gate_up")
    p = cfg.projections[pi]
    W = synth.weights(cfg, pi)
    X = synth.activations(cfg, pi, M)
    plan = G.plan(p.N, p.K, "bf16", epilogue="swiglu")
    H = G.empty_out(M, p.N // 2, "bf16", extra_rows=1)
    plan.run(G.dev(X), G.dev(W), H)
    rows = G.sample_rows(M, seed=M)
    _check_vs_oracle(H, X, W, "bf16", rows=rows, label=f"4B gate_up fused M={M} {plan.choice(M)}")
    assert np.all(G.host(H)[M].view(np.uint16) == 0x7FC1)


def test_tuner_measures_fused_against_unfused():
    """The fusion is an option measured at load ("#004 the same compiler on
    Apple's chips", section "Decode"): in every row bucket the tuner times fused
    candidates and unfused ones ("_uf") side by side and picks from both."""
    plan = G.plan(6144, 1024, "f32", epilogue="swiglu")
    d = plan.describe()
    assert d["swiglu_intermediate_rows"] == 8192
    for b in d["buckets"]:
        t = b["timings_us"]
        fused = [n for n in t if not n.endswith("_uf")]
        unfused = [n for n in t if n.endswith("_uf")]
        assert fused and unfused, (b["lo"], b["hi"], sorted(t))
        assert b["choice"] in t
        G.log(f"  bucket {b['lo']}..{b['hi']}: best fused {min(fused, key=t.get)} {min(t[n] for n in fused):.2f} us, "
              f"best unfused {min(unfused, key=t.get)} {min(t[n] for n in unfused):.2f} us -> {b['choice']}")


@pytest.mark.parametrize("N,K,dtype", [(18432, 2560, "bf16"), (6144, 1024, "f32")])
def test_gate_rejects_no_candidate(N, K, dtype):
    """Every candidate computes the same SwiGLU up to the order of its sums, so
    the load-time gate must pass them all: a rejection here means the gate's
    allowance is tighter than the rounding the method permits (one bf16 ulp of
    a gate sum moves silu(g)*u by more than one ulp of the output), which
    would push whole row buckets onto the slow last-resort kernel."""
    plan = G.plan(N, K, dtype, epilogue="swiglu")
    d = plan.describe()
    for b in d["buckets"]:
        assert b["rejected"] == [], (b["lo"], b["hi"], b["rejected"])
        assert b["choice"] != "gemm_plain", (b["lo"], b["hi"])
        G.log(f"  {N}x{K} {dtype} bucket {b['lo']}..{b['hi']}: {len(b['timings_us'])} timed, -> {b['choice']}")
