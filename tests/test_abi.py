"""Host-side checks of the C ABI (no GPU needed): symbols, argument errors."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "proj.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(proj_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_core_abi():
    names = _declared_functions()
    for core in ("proj_plan_create", "proj_run", "proj_plan_destroy", "proj_last_error"):
        assert core in names


def test_library_exports_every_declared_symbol():
    import shape_specialised_bf16_amd as ssb

    lib = ctypes.CDLL(ssb.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in proj.h but not exported: {missing}"
    assert sorted(ssb.EXPORTED_SYMBOLS) == _declared_functions()


def test_invalid_arguments_fail_before_any_gpu_call():
    import shape_specialised_bf16_amd as ssb
    lib = ssb._lib
    # bad shapes / dtype: NULL plan with an explanatory message
    for N, K, dt in [(0, 64, 0), (16, 12, 0), (16, 0, 0), (-1, 64, 0), (16, 64, 7)]:
        assert not lib.proj_plan_create(N, K, dt)
        assert b"invalid" in lib.proj_last_error()
    # run on a NULL plan
    assert lib.proj_run(None, None, None, None, 1, None) == -1
    assert b"plan is NULL" in lib.proj_last_error()
    assert lib.proj_plan_describe(None, None, 0, None) == -1
    assert lib.proj_plan_num_candidates(None) == -1
    assert lib.proj_plan_choice(None, 1) == -1
    assert lib.proj_run_candidate(None, 0, None, None, None, 1, None) == -1
    assert lib.proj_probe_read(None, 16, 0, None, None) == -1
    assert lib.proj_probe_read(ctypes.c_void_p(16), 15, 0, ctypes.c_void_p(16), None) == -1
    assert lib.proj_round_bf16(None, None, -1, None) == -1
    assert lib.proj_round_bf16(None, None, 0, None) == 0
    lib.proj_plan_destroy(None)   # NULL-safe


def test_emit_source_size_protocol():
    import shape_specialised_bf16_amd as ssb
    lib = ssb._lib
    need = ctypes.c_size_t(0)
    assert lib.proj_emit_source(64, 64, 0, b"gfx950", None, 0, ctypes.byref(need)) == 0
    assert need.value > 1000
    small = ctypes.create_string_buffer(10)
    assert lib.proj_emit_source(64, 64, 0, b"gfx950", small, 10, None) == -1
    assert b"too small" in lib.proj_last_error()
    assert lib.proj_emit_source(64, 60, 0, b"gfx950", None, 0, ctypes.byref(need)) == -1


def test_python_binding_rejects_bad_dtype():
    import shape_specialised_bf16_amd as ssb
    with pytest.raises(ValueError):
        ssb.emit_source(64, 64, "f16")


def test_support_entry_points_check_alignment_and_overlap_before_any_gpu_call():
    """proj_swiglu, proj_rmsnorm and proj_round_bf16 reject misaligned and
    overlapping buffers (as include/proj.h states) before touching the device:
    the addresses below are never dereferenced."""
    import shape_specialised_bf16_amd as ssb
    lib = ssb._lib
    P = ctypes.c_void_p
    base = 1 << 32
    # SwiGLU: f32 G [4, 8] (128 B) and H [4, 4] (64 B)
    assert lib.proj_swiglu(P(base), P(base + 64), 4, 8, 0, None) == -1          # H inside G
    assert b"overlaps" in lib.proj_last_error()
    assert lib.proj_swiglu(P(base + 2), P(base + 4096), 4, 8, 0, None) == -1    # f32 G on a 2-byte boundary
    assert b"aligned" in lib.proj_last_error()
    assert lib.proj_swiglu(P(base), P(base + 4097), 4, 8, 1, None) == -1        # bf16 H on an odd address
    # RMSNorm: X [4, 64] bf16 (512 B), gamma 64 f32 (256 B)
    g = P(base + 8192)
    assert lib.proj_rmsnorm(P(base), g, P(base + 256), 4, 64, ctypes.c_float(1e-6), None) == -1   # Xn overlaps X
    assert b"overlaps" in lib.proj_last_error()
    assert lib.proj_rmsnorm(P(base), g, P(base + 8192 + 128), 4, 64, ctypes.c_float(1e-6), None) == -1  # Xn on gamma
    assert lib.proj_rmsnorm(P(base + 1), g, P(base + 4096), 4, 64, ctypes.c_float(1e-6), None) == -1   # odd X
    assert b"aligned" in lib.proj_last_error()
    assert lib.proj_rmsnorm(P(base), P(base + 8194), P(base + 4096), 4, 64, ctypes.c_float(1e-6), None) == -1
    # rounding: in 16 f32 (64 B), out 16 u16 (32 B)
    assert lib.proj_round_bf16(P(base), P(base + 32), 16, None) == -1
    assert b"overlaps" in lib.proj_last_error()
    assert lib.proj_round_bf16(P(base + 2), P(base + 4096), 16, None) == -1
    assert lib.proj_round_bf16(P(base), P(base + 4097), 16, None) == -1
    assert b"aligned" in lib.proj_last_error()
