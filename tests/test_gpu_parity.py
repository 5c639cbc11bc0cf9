"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Inputs follow the seeded recipe of ``synth``; tolerances are those of
``oracle.tolerance``.  Large shapes are compared on sampled rows (first, last,
tile boundaries, random), small ones in full.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ single projection
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [1, 16])
def test_single_projection_1024(M, dtype):
    cfg = synth.workload("single_1024x1024")
    W = synth.weights(cfg, 0)
    X = synth.activations(cfg, 0, M)
    p = G.plan(1024, 1024, dtype)
    Y = G.empty_out(M, 1024, dtype, extra_rows=2)
    p.run(G.dev(X), G.dev(W), Y)
    G.check_against_oracle(Y, X, W, dtype, label=f"1024x1024 {p.choice(M)}")
    tail = G.host(Y)[M:]
    pat = 0x7FC1 if dtype == "bf16" else 0x7FC00001
    assert np.all(tail.view(np.uint16 if dtype == "bf16" else np.uint32) == pat), "rows past M were written"


# ------------------------------------------------------------------ the pages' own decode shape
@pytest.mark.parametrize("M", [1, 3, 16, 100])
def test_pages_gate_up_shape_7168x1024(M):
    pr = synth.PAGES_GATE_UP_08B
    W = synth.normal_bf16(50, 0, (pr.N, pr.K), 0.02)
    X = synth.normal_bf16(50, 1 + M, (M, pr.K), 1.0)
    p = G.plan(pr.N, pr.K, "f32")
    Y = p.run(G.dev(X), G.dev(W))
    G.check_against_oracle(Y, X, W, "f32", label=f"7168x1024 {p.choice(M)}")


# ------------------------------------------------------------------ odd shape: no MFMA tile fits
@pytest.mark.parametrize("M", [1, 7, 16, 17, 300])
def test_odd_shape_1000x520(M):
    W = synth.normal_bf16(51, 0, (1000, 520), 0.02)
    X = synth.normal_bf16(51, 1 + M, (M, 520), 1.0)
    p = G.plan(1000, 520, "bf16")
    Y = p.run(G.dev(X), G.dev(W))
    G.check_against_oracle(Y, X, W, "bf16", label=f"1000x520 {p.choice(M)}")


# ------------------------------------------------------------------ every candidate, exact integers
# 3840 columns: a multiple of every tile width (64, 128, 160, 192, 256), so every GEMM
# kind the generator has is compiled for it
@pytest.mark.parametrize("N,K,dtype", [(7168, 1024, "f32"), (2560, 9216, "bf16"), (1000, 520, "f32"),
                                       (3840, 1024, "bf16")])
def test_every_candidate_bit_exact_on_integer_probe(N, K, dtype):
    """With integer inputs in [-4, 4] every summation order is exact, so every
    compiled candidate -- not only the tuned winners -- must reproduce the
    oracle bit for bit, at full, partial and odd row counts."""
    p = G.plan(N, K, dtype)
    W = synth.int_bf16(60, (N, K))
    Xall = synth.int_bf16(61, (600, K))
    Wd = G.dev(W)
    exact = oracle.matmul(Xall, W)
    want = oracle.round_bf16(exact) if dtype == "bf16" else oracle.round_f32(exact)
    for idx, name in enumerate(p.candidates()):
        mmax = p.candidate_max_m(idx)
        Ms = [1, 5, 16] if mmax <= 16 else [1, 17, 130, 600]
        for M in [m for m in Ms if m <= mmax]:
            Y = G.empty_out(M, N, dtype, extra_rows=1)
            p.run_candidate(idx, G.dev(Xall[:M]), Wd, Y)
            got = G.host(Y)
            assert np.array_equal(got[:M].view(np.uint8), want[:M].view(np.uint8)), f"{name} M={M}"
            assert np.all(got[M:].view(np.uint8) == G.host(G.empty_out(1, N, dtype))[0:1].view(np.uint8)), \
                f"{name} wrote past M={M}"
        G.log(f"  {N}x{K} {dtype} {name}: bit-exact")


@pytest.mark.parametrize("M", [2048 + 64, 4100])
def test_split_tail_candidates_with_whole_and_tail_tiles(M):
    """Split-tail GEMMs at row counts where some tiles run whole and the rest as
    K pieces: every output written (NaN-prefilled Y has no NaN left), the
    first and the last 600 rows bit-exact on the integer probe (the tail tiles
    are the last ones in tile order, i.e. the bottom tile-rows)."""
    import torch
    N, K, dtype = 7168, 1024, "f32"
    p = G.plan(N, K, dtype)
    W = synth.int_bf16(70, (N, K))
    X = synth.int_bf16(71, (M, K))
    rows = list(range(64)) + list(range(M - 600, M))
    want = oracle.round_f32(oracle.matmul_rows(X, rows, W))
    Xd, Wd = G.dev(X), G.dev(W)
    names = [n for n in p.candidates() if "_tail" in n and not n.endswith("_reduce")]
    assert names, "no split-tail candidate for this shape"
    for name in names:
        idx = p.candidates().index(name)
        if p.candidate_max_m(idx) < M:
            continue
        Y = G.empty_out(M, N, dtype, extra_rows=1)
        p.run_candidate(idx, Xd, Wd, Y)
        assert int(torch.isnan(Y[:M]).sum()) == 0, f"{name}: unwritten outputs"
        assert np.array_equal(G.host(Y)[rows], want), f"{name} M={M}"
        assert np.all(G.host(Y)[M:].view(np.uint32) == 0x7FC00001), f"{name} wrote past M"
        G.log(f"  {name} M={M}: bit-exact on sampled rows, all rows written")


@pytest.mark.parametrize("N,K,dtype", [(7168, 1024, "f32"), (2560, 9216, "bf16"), (3840, 1024, "bf16")])
def test_every_candidate_within_tolerance_on_random_inputs(N, K, dtype):
    p = G.plan(N, K, dtype)
    W = synth.normal_bf16(62, 0, (N, K), 0.02)
    X = synth.normal_bf16(62, 1, (300, K), 1.0)
    Wd = G.dev(W)
    ref = oracle.matmul(X, W)
    for idx, name in enumerate(p.candidates()):
        M = min(p.candidate_max_m(idx), 300)
        Y = p.run_candidate(idx, G.dev(X[:M]), Wd)
        rep = G.compare(G.host(Y), ref[:M], dtype)
        assert rep.ok, f"{name}: {rep}"


def test_plan_describe_and_no_rejections():
    """Every bucket has a choice; no candidate of a regular shape is rejected by
    the load-time gate (a rejection would mean a wrong kernel was compiled)."""
    p = G.plan(7168, 1024, "f32")
    d = p.describe()
    assert d["N"] == 7168 and d["K"] == 1024 and d["arch"].startswith("gfx9")
    assert len(d["buckets"]) == 7
    for b in d["buckets"]:
        assert b["choice"], b
        assert not b["rejected"], b
    assert any("[autotune]" in line for line in d["log"])


def test_determinism_and_nondefault_stream():
    import torch
    N, K = 6144, 1024
    W = synth.normal_bf16(63, 0, (N, K), 0.02)
    X = synth.normal_bf16(63, 1, (200, K), 1.0)
    p = G.plan(N, K, "f32")
    Wd, Xd = G.dev(W), G.dev(X)
    for M in (1, 16, 200):
        a = p.run(Xd[:M], Wd)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            b = p.run(Xd[:M], Wd, stream=s)
        s.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"M={M} not bitwise reproducible"


def test_large_m_is_processed_in_blocks():
    """M above 8192 runs as consecutive blocks of 8192 rows."""
    N, K = 1024, 1024
    W = synth.normal_bf16(64, 0, (N, K), 0.02)
    X = synth.normal_bf16(64, 1, (8192 + 300, K), 1.0)
    p = G.plan(N, K, "f32")
    Y = G.empty_out(X.shape[0], N, "f32", extra_rows=1)
    p.run(G.dev(X), G.dev(W), Y)
    rows = G.sample_rows(X.shape[0], extra=(8191, 8192, 8193, 8491))
    G.check_against_oracle(Y, X, W, "f32", rows=rows, label="1024x1024 M=8492")
    assert np.all(G.host(Y)[X.shape[0]:].view(np.uint32) == 0x7FC00001)


def test_m_zero_is_a_no_op():
    p = G.plan(1024, 1024, "f32")
    import torch
    X = torch.zeros((0, 1024), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((1024, 1024), dtype=torch.bfloat16, device="cuda")
    Y = p.run(X, W)
    assert Y.shape == (0, 1024)


def test_wrong_arguments_are_rejected():
    import torch
    from shape_specialised_bf16_amd import ProjError
    p = G.plan(1024, 1024, "f32")
    X = torch.zeros((4, 1024), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((1024, 1024), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((4, 1024), dtype=torch.float32, device="cuda")
    with pytest.raises(ProjError, match="aligned"):
        p.run_ptr(X.data_ptr() + 2, W.data_ptr(), Y.data_ptr(), 4, None)
    with pytest.raises(ProjError, match="negative"):
        p.run_ptr(X.data_ptr(), W.data_ptr(), Y.data_ptr(), -1, None)
    with pytest.raises(ProjError, match="2\\^48"):                 # sizes that would wrap: nothing enqueued
        p.run_ptr(X.data_ptr(), W.data_ptr(), Y.data_ptr(), 1 << 60, None)
    with pytest.raises(ProjError, match="null"):
        p.run_ptr(0, W.data_ptr(), Y.data_ptr(), 4, None)
    with pytest.raises(ProjError, match="overlaps"):               # Y on top of W's last rows
        p.run_ptr(X.data_ptr(), W.data_ptr(), W.data_ptr() + 1020 * 1024 * 2, 4, None)
    with pytest.raises(ProjError, match="overlaps"):               # Y on top of X
        p.run_ptr(X.data_ptr(), W.data_ptr(), X.data_ptr(), 4, None)
    with pytest.raises(ValueError):
        p.run(X, W[:512])


# ------------------------------------------------------------------ degenerate shapes
@pytest.mark.parametrize("N,K", [(1, 8), (3, 16), (17, 24), (64, 8)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_shapes(N, K, dtype):
    """The smallest shapes a plan accepts (one output row, one 16-byte chunk per
    weight row, counts no tile divides): only the families whose constraints
    they meet are compiled, and the tuned result matches the oracle at M = 1, 2
    and a ragged 17, every candidate bit-exact on the integer probe."""
    W = synth.normal_bf16(65, N * 100 + K, (N, K), 0.5)
    p = G.plan(N, K, dtype)
    assert "gemm_plain" in p.candidates()
    for M in (1, 2, 17):
        X = synth.normal_bf16(65, M, (M, K), 1.0)
        Y = G.empty_out(M, N, dtype, extra_rows=1)
        p.run(G.dev(X), G.dev(W), Y)
        G.check_against_oracle(Y, X, W, dtype, label=f"{N}x{K} {p.choice(M)}")
        pat = 0x7FC1 if dtype == "bf16" else 0x7FC00001
        assert np.all(G.host(Y)[M:].view(np.uint16 if dtype == "bf16" else np.uint32) == pat)
    Wi, Xi = synth.int_bf16(66, (N, K)), synth.int_bf16(67, (17, K))
    exact = oracle.matmul(Xi, Wi)
    want = oracle.round_bf16(exact) if dtype == "bf16" else oracle.round_f32(exact)
    for idx, name in enumerate(p.candidates()):
        M = min(p.candidate_max_m(idx), 17)
        got = G.host(p.run_candidate(idx, G.dev(Xi[:M]), G.dev(Wi)))
        assert np.array_equal(got.view(np.uint8), want[:M].view(np.uint8)), f"{N}x{K} {name}"


# ------------------------------------------------------------------ seeded random shapes
def _random_shapes(n=12, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 3001))
        K = 8 * int(rng.integers(1, 376))
        out.append((N, K, "bf16" if i % 2 else "f32", int(rng.integers(1, 301))))
    return out


@pytest.mark.parametrize("N,K,dtype,M", _random_shapes())
def test_random_shapes_against_oracle(N, K, dtype, M):
    """Shapes drawn from a seeded generator (N in [1, 3000], K any multiple of 8
    up to 3000, both output types, ragged M): plan creation succeeds, the tuned
    path matches the oracle at M = 1, 16 and the drawn M, and nothing is written
    past M."""
    W = synth.normal_bf16(68, N * 7 + K, (N, K), 0.05)
    p = G.plan(N, K, dtype)
    pat = 0x7FC1 if dtype == "bf16" else 0x7FC00001
    for m in sorted({1, 16, M}):
        X = synth.normal_bf16(69, m + N, (m, K), 1.0)
        Y = G.empty_out(m, N, dtype, extra_rows=1)
        p.run(G.dev(X), G.dev(W), Y)
        G.check_against_oracle(Y, X, W, dtype, label=f"random {N}x{K} {p.choice(m)}")
        assert np.all(G.host(Y)[m:].view(np.uint16 if dtype == "bf16" else np.uint32) == pat), "row M was written"
