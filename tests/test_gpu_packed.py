"""Load-time weight repacking (proj_pack_weights) and plans that read the
packed layout (PROJ_W_PACKED, run through proj_run_packed), on the GPU.

The pages pack weights in the order their kernels consume them ("#001 un
compilateur pour moteur de LLM", section "Lire le meme emetteur rempli deux
fois") and expect that to pay on GPUs as well, to be measured kernel by kernel
("#002 le meme compilateur sur un GPU", section "Les autres cartes").  Only the
addresses change, so: the pack kernel must reproduce the oracle's layout
exactly; every candidate of a packed plan must give the same bits as the
row-major plan's candidate of the same name; and the tuned packed path must be
within the usual tolerance of the oracle, fused epilogue and prologue included.
"""
import ctypes

import numpy as np
import pytest

import oracle
from oracle import tolerance
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _pack(W):
    import shape_specialised_bf16_amd as ssb
    return ssb.pack_weights(G.dev(W))


@pytest.mark.parametrize("N,K", [(128, 64), (256, 128), (7168, 1024), (2560, 9216), (384, 5120)])
def test_pack_kernel_equals_oracle_layout(N, K):
    import torch
    W = np.random.default_rng(N + K).integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    Wp = _pack(W)
    torch.cuda.synchronize()
    assert tuple(Wp.shape) == (N // 128, K // 64, 128, 64)
    got = Wp.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.pack_panels(W)), f"{N}x{K}: packed layout differs from the oracle's"
    G.log(f"  pack {N}x{K}: identical to oracle.pack_panels")


def test_pack_rejects_bad_arguments():
    import torch
    import shape_specialised_bf16_amd as ssb
    from shape_specialised_bf16_amd import ProjError, _lib
    W = torch.zeros((256, 128), dtype=torch.bfloat16, device="cuda")
    Wp = torch.zeros((2, 2, 128, 64), dtype=torch.bfloat16, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert _lib.proj_pack_weights(200, 128, W.data_ptr(), Wp.data_ptr(), s) == -1      # N % 128
    assert "N % 128" in _lib.proj_last_error().decode()
    assert _lib.proj_pack_weights(256, 96, W.data_ptr(), Wp.data_ptr(), s) == -1       # K % 64
    assert _lib.proj_pack_weights(256, 128, W.data_ptr() + 2, Wp.data_ptr(), s) == -1  # misaligned
    assert _lib.proj_pack_weights(256, 128, W.data_ptr(), W.data_ptr() + 4096, s) == -1  # overlap
    assert "overlap" in _lib.proj_last_error().decode()
    assert _lib.proj_pack_weights(256, 128, 0, Wp.data_ptr(), s) == -1                 # null
    assert _lib.proj_pack_weights(0, 128, 0, 0, s) == 0                                # empty: no-op
    with pytest.raises(ValueError):
        ssb.pack_weights(torch.zeros((200, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ProjError, match="N % 128"):
        ssb.Plan(1000, 520, "f32", packed=True)


@pytest.mark.parametrize("N,K,dtype", [(7168, 1024, "f32"), (2560, 9216, "bf16"), (1024, 3584, "f32"),
                                     (3840, 1024, "bf16")])
def test_every_packed_candidate_equals_row_major(N, K, dtype):
    """Same candidate, same inputs: the packed plan's output equals the
    row-major plan's bit for bit, at full, partial and odd row counts, and
    nothing is written past M.  (3840 columns are a multiple of every tile
    width, 64 to 256, so tiles that straddle the 128-row panels are among
    them.)"""
    import torch
    pk = G.plan(N, K, dtype, packed=True)
    pr = G.plan(N, K, dtype)
    W = synth.normal_bf16(110, 0, (N, K), 0.02)
    Xall = synth.normal_bf16(110, 1, (600, K), 1.0)
    Wd, Wpd = G.dev(W), _pack(W)
    names = pr.candidates()
    assert pk.candidates() == names, "packed and row-major plans compile different candidate lists"
    pat = G.host(G.empty_out(1, N, dtype))[0:1].view(np.uint8)
    for idx, name in enumerate(names):
        mmax = min(pk.candidate_max_m(idx), pr.candidate_max_m(idx))
        Ms = [1, 5, 16] if mmax <= 16 else [1, 17, 130, 600]
        for M in [m for m in Ms if m <= mmax]:
            Xd = G.dev(Xall[:M])
            Yp = G.empty_out(M, N, dtype, extra_rows=1)
            pk.run_candidate(idx, Xd, Wpd, Yp)
            Yr = G.empty_out(M, N, dtype, extra_rows=1)
            pr.run_candidate(idx, Xd, Wd, Yr)
            a, b = G.host(Yp), G.host(Yr)
            assert np.array_equal(a[:M].view(np.uint8), b[:M].view(np.uint8)), f"{name} M={M}: packed != rows"
            assert np.all(a[M:].view(np.uint8) == pat), f"{name} wrote past M={M}"
        G.log(f"  {N}x{K} {dtype} {name}: packed == row-major")
    # and the row-major results are right (so the comparison is not of two wrong values)
    Y = pk.run_packed(G.dev(Xall[:130]), Wpd)
    G.check_against_oracle(Y, Xall[:130], W, dtype, label=f"{N}x{K} packed {pk.choice(130)}")


@pytest.mark.parametrize("M", [1, 16, 300, 2112, 4100])
def test_tuned_packed_path_against_oracle(M):
    N, K, dtype = 7168, 1024, "f32"
    p = G.plan(N, K, dtype, packed=True)
    W = synth.normal_bf16(111, 0, (N, K), 0.02)
    X = synth.normal_bf16(111, M, (M, K), 1.0)
    Y = G.empty_out(M, N, dtype, extra_rows=1)
    p.run_packed(G.dev(X), _pack(W), Y)
    rows = None if M <= 300 else G.sample_rows(M, extra=(2047, 2048, M - 65))
    G.check_against_oracle(Y, X, W, dtype, rows=rows, label=f"7168x1024 packed {p.choice(M)}")
    assert np.all(G.host(Y)[M:].view(np.uint32) == 0x7FC00001), "rows past M were written"


@pytest.mark.parametrize("N,K,M", [(151936, 1024, 1), (34816, 5120, 8192)])
def test_packed_at_full_size(N, K, M):
    """The output head at decode and the large prefill shape, packed: sampled
    rows against the oracle."""
    import torch
    dtype = "bf16"
    p = G.plan(N, K, dtype, packed=True)
    W = synth.normal_bf16(112, 0, (N, K), 0.02)
    X = synth.normal_bf16(112, 1, (M, K), 1.0)
    Wp = _pack(W)
    Y = p.run_packed(G.dev(X), Wp)
    torch.cuda.synchronize()
    rows = None if M == 1 else G.sample_rows(M, extra=(4095, 4096, 8191))[:8]
    G.check_against_oracle(Y, X, W, dtype, rows=rows, label=f"{N}x{K} packed {p.choice(M)}")


def test_packed_swiglu_and_norm_equal_row_major():
    """The fused epilogue and prologue on packed weights: every candidate equals
    the row-major fused plan's candidate of the same name bit for bit."""
    N, K, dtype = 7168, 1024, "bf16"
    import torch
    g = (1.0 + 0.25 * np.random.default_rng(113).standard_normal(K)).astype(np.float32)
    gd = torch.from_numpy(g).cuda()
    W = synth.normal_bf16(113, 0, (N, K), 0.02)
    X = synth.normal_bf16(113, 1, (130, K), 1.0)
    Wd, Wpd, Xd = G.dev(W), _pack(W), G.dev(X)
    for kw in (dict(epilogue="swiglu"), dict(rmsnorm_eps=EPS), dict(epilogue="swiglu", rmsnorm_eps=EPS)):
        pk = G.plan(N, K, dtype, packed=True, **kw)
        pr = G.plan(N, K, dtype, **kw)
        gam = gd if "rmsnorm_eps" in kw else None
        assert pk.candidates() == pr.candidates()
        for idx, name in enumerate(pk.candidates()):
            mmax = min(pk.candidate_max_m(idx), pr.candidate_max_m(idx))
            for M in [m for m in (1, 16, 130) if m <= mmax]:
                a = pk.run_candidate(idx, Xd[:M], Wpd, gamma=gam)
                b = pr.run_candidate(idx, Xd[:M], Wd, gamma=gam)
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{kw} {name} M={M}"
        G.log(f"  7168x1024 bf16 packed {kw}: {len(pk.candidates())} candidates equal to row-major")
    # the tuned fused path against the oracle
    pk = G.plan(N, K, dtype, packed=True, epilogue="swiglu")
    H = pk.run_packed(Xd, Wpd)
    ref = oracle.matmul(X, W)
    y = oracle.bf16_bits_to_f64(G.host(H))
    rep = tolerance.check_swiglu(y, ref[:, :N // 2], ref[:, N // 2:], dtype)
    assert rep.ok, rep


def test_layout_mismatch_is_rejected():
    import torch
    from shape_specialised_bf16_amd import ProjError, _lib
    pk = G.plan(1024, 1024, "f32", packed=True)
    pr = G.plan(1024, 1024, "f32")
    X = torch.zeros((4, 1024), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((1024, 1024), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((4, 1024), dtype=torch.float32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert _lib.proj_run(pk._h, X.data_ptr(), W.data_ptr(), Y.data_ptr(), 4, s) == -1
    assert "proj_run_packed" in _lib.proj_last_error().decode()
    assert _lib.proj_run_packed(pr._h, X.data_ptr(), W.data_ptr(), Y.data_ptr(), 4, None, s) == -1
    assert "row-major" in _lib.proj_last_error().decode()
    with pytest.raises(ValueError):                 # a row-major matrix passed to a packed plan
        pk.run_packed(X, W)
    assert pk.describe()["layout"] == "packed" and pr.describe()["layout"] == "rows"
    with pytest.raises(ProjError):
        pk.run(X, W.view(8, 16, 128, 64))
