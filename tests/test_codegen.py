"""Emitted-source checks (no GPU): the shape appears as literals, every emitted
candidate tiles the shape exactly, and the source compiles for gfx950."""
import os
import re
import subprocess

import pytest

import shape_specialised_bf16_amd as ssb

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    gpu, cpu = [], []
    for line in open(os.path.join(HERE, "golden", "pages_emitted_constants.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "gpu":
            gpu.append(tuple(int(v) for v in line[1:]))
        else:
            cpu.append((int(line[1]), int(line[2], 16), None if line[3] == "-" else int(line[3], 16)))
    return gpu, cpu


@pytest.mark.parametrize("row", _golden()[0])
def test_pages_gpu_module_constants_appear_as_literals(row):
    """The pages' decode module for (N, K) carries N, K/8 and N-1 as constants;
    the emitted HIP source carries the same values as literals."""
    N, K, blocks16, last = row
    assert blocks16 == K // 8 and last == N - 1          # the fixture is self-consistent
    src = ssb.emit_source(N, K, "f32")
    assert re.search(rf"constexpr long N = {N};", src)
    assert re.search(rf"constexpr long K = {K};", src)
    assert re.search(rf"constexpr long K_BLOCKS16 = {blocks16};", src)
    assert re.search(rf"constexpr long N_LAST = {last};", src)
    assert re.search(rf"constexpr long ROW_BYTES = {2 * K};", src)


@pytest.mark.parametrize("row", _golden()[1])
def test_trip_counts_and_block_strides_are_literals(row):
    """The pages' x86 loop has its trip count (K/2) and the 16-row block stride
    (16*K*2 bytes) as immediates.  Here: each candidate's trip count is a
    literal checked by a static_assert, and the 16-row weight block stride
    appears in the MFMA GEMV candidates' description."""
    K, trips_x86, stride = row
    assert trips_x86 == K // 2
    src = ssb.emit_source(18432 if K == 2560 else 7168, K, "f32")
    # vector GEMV: K/8 blocks over 64 lanes
    assert f"static_assert(K_BLOCKS16 / 1 / 64 == {K // 8 // 64}, \"trip count\");" in src
    # MFMA GEMV: K / (32*U) batches
    assert f"static_assert(K / 1 / 128 == {K // 128}, \"trip count\");" in src
    assert f"next 16-row weight block at +{32 * K} B" in src
    if stride is not None:
        assert stride == 32 * K


def test_no_runtime_shape_arguments():
    """Every candidate wrapper takes only pointers and M: no run-time N or K
    (gamma, the norm weights of a plan with the RMSNorm prologue, is a pointer)."""
    src = ssb.emit_source(5120, 2560, "bf16")
    sigs = re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void (gemv_\w+|gemm_\w+)(\([^)]*\))', src)
    assert len(sigs) >= 10
    for name, sig in sigs:
        if name.endswith("_reduce") or name.startswith("splitk_reduce"):   # second pass: partials in, Y out
            assert sig == "(const float* __restrict__ ws, void* __restrict__ Y, int M)", name
            continue
        assert sig == ("(const u16* __restrict__ X, const u16* __restrict__ W, void* __restrict__ Y, "
                       "float* __restrict__ ws, const float* __restrict__ gamma, int M)"), name


@pytest.mark.parametrize("N,K", [(2048, 1024), (151936, 1024), (5120, 2560), (2560, 9216),
                                 (34816, 5120), (5120, 17408), (1000, 520), (24, 8)])
def test_candidates_tile_the_shape(N, K):
    src = ssb.emit_source(N, K, "f32")
    names = re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void ((?:gemv|gemm)_\w+)\(', src)
    assert "gemm_plain" in names
    for n in names:
        m = re.match(r"gemv_valu_r(\d+)_s(\d+)_m(\d+)_u(\d+)_nt(\d)(?:_p)?(?:_w(\d+))?(?:_x(\d+))?(?:_nf)?$", n)
        if m:
            R, S, MM, U, _ = map(int, m.groups()[:5])
            NW = int(m.group(6) or 4)          # waves per block
            KX = int(m.group(7) or 1)          # K split across workgroups
            assert (K // 8) % (S * KX) == 0 and N % (R * (NW // S)) == 0
            trips = K // 8 // (S * KX) // 64
            assert trips % U == 0 or trips == 0
            assert KX == 1 or (MM == 1 and trips >= 1)
            continue
        m = re.match(r"gemv_mfma_s(\d+)_u(\d+)_nt(\d)", n)
        if m:
            S, U, _ = map(int, m.groups())
            assert N % (16 * (4 // S)) == 0 and K % (32 * U * S) == 0
            continue
        m = re.match(r"gemm_(\d+)x(\d+)x(\d+)_st(\d+)_w(\d+)x(\d+)_sw(\d+)_g(\d+)_sk(\d+)(?:_reg)?", n)
        if m:
            BM, BN, BK, ST, WM, WN, SWZ, GM, SK = map(int, m.groups())
            assert N % BN == 0 and K % (BK * SK) == 0
            assert ST * (BM + BN) * BK * 2 <= 160 * 1024     # LDS of one workgroup
            continue
        assert n == "gemm_plain", n


def test_emitted_source_compiles_for_gfx950(tmp_path):
    """A device-code build check: the emitted unit for an odd shape (tails in K,
    few candidates) compiles with hipcc for gfx950."""
    src = ssb.emit_source(1000, 520, "bf16")
    f = tmp_path / "proj_1000x520.hip"
    f.write_text(src)
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-c", "-O3",
                        "-std=c++17", "-include", "hip/hip_runtime.h", str(f), "-o", str(f) + ".o"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_swiglu_module_constants_and_families():
    """A SwiGLU plan's module carries the epilogue and the halved output width
    as literals.  Its fused candidates (the activation in their epilogue, E = 1)
    come only from the families that have it: vector GEMVs with an even row
    count per wave, whole-tile GEMMs whose waves hold gate and up halves (no
    split-K, no split tail), and the plain kernel -- no MFMA GEMV.  Then every
    candidate of the plain plan except the plain kernel appears again run
    unfused ("_uf", E = 0: the N-column projection, then the activation kernel),
    so the tuner can measure the fusion against what it replaces."""
    src = ssb.emit_source(6144, 1024, "f32", epilogue="swiglu")
    assert "constexpr int EPI = 1;" in src
    assert "constexpr long NOUT = 3072;" in src
    wrappers = dict(re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void ((?:gemv|gemm)_\w+)\([^)]*\)\n\{ ([^;]*);',
                               src))
    names = [n for n in wrappers if not n.endswith("_reduce")]
    assert names[-1] == "gemm_plain" and any(n.startswith("gemv_valu") for n in names)
    fused = [n for n in names if not n.endswith("_uf")]
    unfused = [n[:-3] for n in names if n.endswith("_uf")]
    def epilogue_arg(call):
        """The E template argument of a wrapper's kernel call (gemv_valu<R, S, MMAX, U, NT, OUT, P, PRO, E>,
        gemm_mfma<BM, BN, BK, ST, WM, WN, SK, GM, SWZ, OUT, DMA, TAILS, ROUND, E, BST>, gemm_plain<OUT, E>)."""
        kernel, args = re.match(r"(\w+)<([^>]*)>", call).groups()
        args = [a.strip() for a in args.split(",")]
        return args[{"gemv_valu": 8, "gemm_mfma": 13, "gemm_plain": 1}[kernel]]

    for n in fused:
        assert epilogue_arg(wrappers[n]) == "1", (n, wrappers[n])
        assert not n.startswith("gemv_mfma"), n
        m = re.match(r"gemv_valu_r(\d+)_", n)
        if m:
            assert int(m.group(1)) % 2 == 0, n
        m = re.match(r"gemm_(\d+)x(\d+)x(\d+)_st(\d+)_w(\d+)x(\d+)_sw(\d+)_g(\d+)_sk(\d+)", n)
        if m:
            BM, BN, BK, ST, WM, WN, SWZ, GM, SK = map(int, m.groups())
            assert SK == 1 and "_tail" not in n and (BN // WN) % 64 == 0, n
    plain = ssb.emit_source(6144, 1024, "f32")
    assert "constexpr int EPI = 0;" in plain and "constexpr long NOUT = 6144;" in plain
    plain_names = [n for n in re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void ((?:gemv|gemm)_\w+)\(',
                                         plain) if not n.endswith("_reduce") and n != "gemm_plain"]
    assert unfused == plain_names
    for n in unfused:
        if not n.startswith("gemv_mfma"):
            assert epilogue_arg(wrappers[n + "_uf"]) == "0", (n, wrappers[n + "_uf"])


def test_swiglu_odd_n_rejected():
    with pytest.raises(ssb.ProjError, match="even"):
        ssb.emit_source(1001, 1024, "f32", epilogue="swiglu")


def test_swiglu_source_compiles_for_gfx950(tmp_path):
    src = ssb.emit_source(1000, 520, "bf16", epilogue="swiglu")
    f = tmp_path / "proj_1000x520_swiglu.hip"
    f.write_text(src)
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-c", "-O3",
                        "-std=c++17", "-include", "hip/hip_runtime.h", str(f), "-o", str(f) + ".o"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_rmsnorm_module_has_folded_and_unfused_candidates():
    """With the RMSNorm prologue the epsilon is a literal of the module, every
    ordinary candidate is kept (it runs after the separate norm kernel) and
    each M = 1 vector GEMV of four waves per block (the norm's block reduction
    takes 256 threads) comes a second time with the norm folded in."""
    src = ssb.emit_source(2048, 1024, "f32", rmsnorm_eps=1e-6)
    assert "constexpr float NORM_EPS = 0x1.0c6f7ap-20f;" in src        # 1e-6 as an f32, exactly
    names = re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void ((?:gemv|gemm)_\w+)\(', src)
    plain = set(re.findall(r'extern "C" __global__ __launch_bounds__\(\d+\) void ((?:gemv|gemm)_\w+)\(',
                           ssb.emit_source(2048, 1024, "f32")))
    assert plain <= set(names)
    folded = [n for n in names if n.endswith("_nf")]
    assert folded and all(n.startswith("gemv_valu") and "_m1_" in n for n in folded)
    assert {n[:-3] for n in folded} == {n for n in plain if n.startswith("gemv_valu") and "_m1_" in n
                                        and not re.search(r"_[wx]\d+$", n)}
    # the folded copies pass PRO = 1 (the template argument before the epilogue's), NW = 4, KX = 1
    assert "gemv_valu<" in src and ", 1, 0, 4, 1>(X, W, Y, gamma, M, ws)" in src


def test_rmsnorm_and_swiglu_module_compiles(tmp_path):
    src = ssb.emit_source(1000, 520, "bf16", epilogue="swiglu", rmsnorm_eps=1e-5)
    f = tmp_path / "proj_1000x520_both.hip"
    f.write_text(src)
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "--cuda-device-only", "-c", "-O3",
                        "-std=c++17", "-include", "hip/hip_runtime.h", str(f), "-o", str(f) + ".o"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


def test_k_order_variants_pass_kp_to_their_kernel():
    """Each "_kp4" GEMM is its row-ordered twin with KP = 4 as the last template
    argument of gemm_mfma (every other argument equal), and every other GEMM
    passes KP = 0; the fused-SwiGLU GEMMs have no K-order variant."""
    src = ssb.emit_source(18432, 2560, "bf16")
    calls = dict(re.findall(r'void (gemm_\w+)\([^)]*\)\n\{ gemm_mfma<([^>]*)>\(X, W, Y, ws, M\); \}', src))
    kp = [n for n in calls if "_kp4" in n]
    assert len(kp) >= 7
    for name, args in calls.items():
        a = [x.strip() for x in args.split(",")]
        assert len(a) == 16, (name, a)
        assert a[15] == ("4" if "_kp4" in name else "0"), (name, a)
    for name in kp:
        twin = name.replace("_kp4", "")
        assert twin in calls, name
        assert calls[name].rsplit(",", 1)[0] == calls[twin].rsplit(",", 1)[0], (name, twin)
    fused = ssb.emit_source(18432, 2560, "bf16", epilogue="swiglu")
    fused_calls = re.findall(r'void (gemm_\w+)\([^)]*\)\n\{ gemm_mfma<[^>]*>', fused)
    assert fused_calls and not [n for n in fused_calls if "_kp4" in n and not n.endswith("_uf")]
