"""Python binding of libproj: shape-specialised bf16 projections Y = X . W^T on gfx950.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libproj.so`` (built in-tree by ``shape_specialised_bf16_amd/build.py``);
torch supplies device memory and the current stream.  Importing this package
without the built library raises ImportError: there is no fallback.

    plan = Plan(N, K, "f32")          # emit, compile (hipRTC), validate and tune
    Y = plan.run(X, W)                # X [M,K] bf16, W [N,K] bf16 -> Y [M,N] f32

    Wp = pack_weights(W)              # once at load: the packed weight layout
    pp = Plan(N, K, "f32", packed=True)
    Y = pp.run_packed(X, Wp)          # same bits as plan.run(X, W) per kernel variant

C entry points and their semantics: ``include/proj.h``.
"""
from __future__ import annotations

import ctypes
import json
import os

__all__ = ["Plan", "ProjError", "emit_source", "compile_only", "probe_read", "round_bf16", "pack_weights", "swiglu", "rmsnorm",
           "LIB_PATH", "OUT_F32", "OUT_BF16", "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libproj.so")

OUT_F32 = 0
OUT_BF16 = 1
EPI_NONE = 0
EPI_SWIGLU = 1
PRO_RMSNORM = 2
W_PACKED = 4
PANEL_ROWS, PANEL_COLS = 128, 64   # blocks of the packed weight layout
_ERRORS = {-1: "PROJ_EINVAL", -2: "PROJ_EDEVICE", -3: "PROJ_ECOMPILE", -4: "PROJ_ENOCAND", -5: "PROJ_ENOMEM"}

# Every function declared in include/proj.h.
EXPORTED_SYMBOLS = (
    "proj_plan_create", "proj_run", "proj_plan_destroy", "proj_last_error", "proj_emit_source",
    "proj_plan_describe", "proj_plan_num_candidates", "proj_plan_candidate_name",
    "proj_plan_candidate_max_m", "proj_run_candidate", "proj_plan_choice", "proj_probe_read",
    "proj_round_bf16", "proj_plan_create_ex", "proj_emit_source_ex", "proj_swiglu", "proj_run_ex",
    "proj_run_candidate_ex", "proj_rmsnorm", "proj_pack_weights", "proj_run_packed", "proj_compile_only",
    "proj_run_noalloc",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python shape_specialised_bf16_amd/build.py` "
                      "(or __graft_entry__.build()) first")

# torch ships its own HIP runtime (SONAME libamdhip64.so.7, loaded by torch under
# another file name).  Importing torch first makes libproj.so bind to that same
# runtime instance, so torch's streams and allocations are valid in libproj;
# loading libproj first would bring up a second, separate HIP runtime.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib.proj_plan_create.argtypes = [_i64, _i64, ctypes.c_int]
_lib.proj_plan_create.restype = _p
_lib.proj_plan_create_ex.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_float]
_lib.proj_plan_create_ex.restype = _p
_lib.proj_run_ex.argtypes = [_p, _p, _p, _p, _i64, _p, _p]
_lib.proj_run_ex.restype = ctypes.c_int
_lib.proj_run_candidate_ex.argtypes = [_p, ctypes.c_int, _p, _p, _p, _i64, _p, _p]
_lib.proj_run_candidate_ex.restype = ctypes.c_int
_lib.proj_rmsnorm.argtypes = [_p, _p, _p, _i64, _i64, ctypes.c_float, _p]
_lib.proj_rmsnorm.restype = ctypes.c_int
_lib.proj_emit_source_ex.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_char_p,
                                     ctypes.c_char_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
_lib.proj_emit_source_ex.restype = ctypes.c_int
_lib.proj_swiglu.argtypes = [_p, _p, _i64, _i64, ctypes.c_int, _p]
_lib.proj_swiglu.restype = ctypes.c_int
_lib.proj_run.argtypes = [_p, _p, _p, _p, _i64, _p]
_lib.proj_run.restype = ctypes.c_int
_lib.proj_plan_destroy.argtypes = [_p]
_lib.proj_plan_destroy.restype = None
_lib.proj_last_error.argtypes = []
_lib.proj_last_error.restype = ctypes.c_char_p
_lib.proj_emit_source.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_char_p, ctypes.c_char_p,
                                  ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
_lib.proj_emit_source.restype = ctypes.c_int
_lib.proj_plan_describe.argtypes = [_p, ctypes.c_char_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
_lib.proj_plan_describe.restype = ctypes.c_int
_lib.proj_plan_num_candidates.argtypes = [_p]
_lib.proj_plan_num_candidates.restype = ctypes.c_int
_lib.proj_plan_candidate_name.argtypes = [_p, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]
_lib.proj_plan_candidate_name.restype = ctypes.c_int
_lib.proj_plan_candidate_max_m.argtypes = [_p, ctypes.c_int]
_lib.proj_plan_candidate_max_m.restype = _i64
_lib.proj_run_candidate.argtypes = [_p, ctypes.c_int, _p, _p, _p, _i64, _p]
_lib.proj_run_candidate.restype = ctypes.c_int
_lib.proj_plan_choice.argtypes = [_p, _i64]
_lib.proj_plan_choice.restype = ctypes.c_int
_lib.proj_probe_read.argtypes = [_p, _i64, ctypes.c_uint32, _p, _p]
_lib.proj_probe_read.restype = ctypes.c_int
_lib.proj_round_bf16.argtypes = [_p, _p, _i64, _p]
_lib.proj_round_bf16.restype = ctypes.c_int
_lib.proj_pack_weights.argtypes = [_i64, _i64, _p, _p, _p]
_lib.proj_pack_weights.restype = ctypes.c_int
_lib.proj_run_packed.argtypes = [_p, _p, _p, _p, _i64, _p, _p]
_lib.proj_run_packed.restype = ctypes.c_int
_lib.proj_run_noalloc.argtypes = [_p, _p, _p, _p, _i64, _p, _p]
_lib.proj_run_noalloc.restype = ctypes.c_int
_lib.proj_compile_only.argtypes = [_i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_char_p,
                                   ctypes.POINTER(ctypes.c_double)]
_lib.proj_compile_only.restype = ctypes.c_int


class ProjError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.proj_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_ERRORS.get(code, code)}: {msg}")


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise ProjError(rc, where)
    return rc


def _text(fn, *args) -> str:
    need = ctypes.c_size_t(0)
    _check(fn(*args, None, 0, ctypes.byref(need)), fn.__name__)
    buf = ctypes.create_string_buffer(need.value)
    _check(fn(*args, buf, need.value, None), fn.__name__)
    return buf.value.decode()


def _epi_code(epilogue) -> int:
    if epilogue in (None, "none", EPI_NONE):
        return EPI_NONE
    if epilogue in ("swiglu", EPI_SWIGLU):
        return EPI_SWIGLU
    raise ValueError(f"unsupported epilogue {epilogue!r} (None or 'swiglu')")


def emit_source(N: int, K: int, dtype: str = "f32", arch: str = "gfx950", epilogue=None, rmsnorm_eps=None,
                packed: bool = False) -> str:
    """The HIP source a plan for (N, K, dtype[, epilogue, RMSNorm prologue,
    packed weights]) compiles (no GPU needed)."""
    fusion = _epi_code(epilogue) | (PRO_RMSNORM if rmsnorm_eps is not None else 0) | (W_PACKED if packed else 0)
    return _text(_lib.proj_emit_source_ex, N, K, _dtype_code(dtype), fusion,
                 float(rmsnorm_eps or 0.0), arch.encode())


def compile_only(N: int, K: int, dtype: str = "f32", arch: str = "gfx950", epilogue=None, rmsnorm_eps=None,
                 packed: bool = False) -> float:
    """Compile every module of the plan (N, K, dtype[, ...]) for `arch` without
    a GPU (proj_compile_only); returns the seconds it took."""
    fusion = _epi_code(epilogue) | (PRO_RMSNORM if rmsnorm_eps is not None else 0) | (W_PACKED if packed else 0)
    sec = ctypes.c_double(0.0)
    _check(_lib.proj_compile_only(N, K, _dtype_code(dtype), fusion, float(rmsnorm_eps or 0.0), arch.encode(),
                                  ctypes.byref(sec)), "proj_compile_only")
    return sec.value


def _dtype_code(dtype) -> int:
    if dtype in ("f32", "float32", OUT_F32):
        return OUT_F32
    if dtype in ("bf16", "bfloat16", OUT_BF16):
        return OUT_BF16
    try:
        import torch
        if dtype is torch.float32:
            return OUT_F32
        if dtype is torch.bfloat16:
            return OUT_BF16
    except ImportError:
        pass
    raise ValueError(f"unsupported output dtype {dtype!r} (f32 or bf16)")


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bf16_2d(t, name: str, cols: int):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (bfloat16 or 16-bit bit patterns), got {t.dtype}")
    if t.dim() != 2 or t.shape[1] != cols or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [*, {cols}] matrix, got {tuple(t.shape)}")


class Plan:
    """A compiled, tuned projection plan for fixed (N, K) and output dtype.

    epilogue="swiglu": W is a gate_up matrix (gate rows then up rows) and the
    plan writes Y[M, N/2] = silu(gate) * up; rmsnorm_eps=<eps>: X is
    RMS-normalised first with the gamma given to run; packed=True: the plan
    reads weights in the packed layout of pack_weights and runs with
    run_packed (see proj_plan_create_ex)."""

    def __init__(self, N: int, K: int, dtype="f32", epilogue=None, rmsnorm_eps=None, packed: bool = False):
        self.N, self.K = int(N), int(K)
        self.dtype_code = _dtype_code(dtype)
        self.epi_code = _epi_code(epilogue)
        self.norm = rmsnorm_eps is not None
        self.packed = bool(packed)
        self.NO = self.N // 2 if self.epi_code == EPI_SWIGLU else self.N
        fusion = self.epi_code | (PRO_RMSNORM if self.norm else 0) | (W_PACKED if self.packed else 0)
        h = _lib.proj_plan_create_ex(self.N, self.K, self.dtype_code, fusion, float(rmsnorm_eps or 0.0))
        if not h:
            raise ProjError(-1, f"proj_plan_create_ex({N}, {K}, {dtype}, {epilogue}, {rmsnorm_eps}, packed={packed})")
        self._h = ctypes.c_void_p(h)

    @property
    def out_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype_code == OUT_BF16 else torch.float32

    def close(self):
        if getattr(self, "_h", None):
            _lib.proj_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _prep(self, X, W, Y):
        import torch
        _bf16_2d(X, "X", self.K)
        if self.packed:
            _bf16_packed(W, "Wp", self.N, self.K)
        else:
            _bf16_2d(W, "W", self.K)
            if W.shape[0] != self.N:
                raise ValueError(f"W must be [{self.N}, {self.K}], got {tuple(W.shape)}")
        M = X.shape[0]
        if Y is None:
            Y = torch.empty((M, self.NO), dtype=self.out_dtype, device=X.device)
        elif (Y.dtype != self.out_dtype or Y.dim() != 2 or Y.shape[1] != self.NO or Y.shape[0] < M
              or not Y.is_contiguous()):
            raise ValueError(f"Y must be a contiguous [>= {M}, {self.NO}] {self.out_dtype} matrix")
        return M, Y

    def _gamma(self, gamma):
        import torch
        if gamma is None:
            return None
        if not gamma.is_cuda or gamma.dtype != torch.float32 or gamma.numel() != self.K or not gamma.is_contiguous():
            raise ValueError(f"gamma must be a contiguous float32 device vector of {self.K} values")
        return gamma.data_ptr()

    def run(self, X, W, Y=None, stream=None, gamma=None):
        """Y[:M] = X . W^T for all M rows of X (RMS-normalised with gamma for a
        plan with the norm prologue), enqueued on `stream` (default: current)."""
        M, Y = self._prep(X, W, Y)
        _check(_lib.proj_run_ex(self._h, X.data_ptr(), W.data_ptr(), Y.data_ptr(), M, self._gamma(gamma),
                                _stream_handle(stream)), "proj_run_ex")
        return Y

    def run_noalloc(self, X, W, Y, stream=None, gamma=None):
        """run() through proj_run_noalloc: the kernels' workspace is the
        library's static scratch, and nothing is allocated (Y must be given)."""
        if Y is None:
            raise ValueError("run_noalloc: Y must be given (nothing is allocated)")
        M, Y = self._prep(X, W, Y)
        _check(_lib.proj_run_noalloc(self._h, X.data_ptr(), W.data_ptr(), Y.data_ptr(), M, self._gamma(gamma),
                                     _stream_handle(stream)), "proj_run_noalloc")
        return Y

    def run_packed(self, X, Wp, Y=None, stream=None, gamma=None):
        """run() for a packed plan: Wp is pack_weights(W)."""
        M, Y = self._prep(X, Wp, Y)
        _check(_lib.proj_run_packed(self._h, X.data_ptr(), Wp.data_ptr(), Y.data_ptr(), M, self._gamma(gamma),
                                    _stream_handle(stream)), "proj_run_packed")
        return Y

    def run_ptr(self, X_ptr: int, W_ptr: int, Y_ptr: int, M: int, stream_handle, gamma_ptr=None) -> None:
        """proj_run(_ex), or proj_run_packed for a packed plan, on raw device
        addresses (benchmark loops)."""
        if self.packed:
            _check(_lib.proj_run_packed(self._h, X_ptr, W_ptr, Y_ptr, M, gamma_ptr, stream_handle),
                   "proj_run_packed")
        elif gamma_ptr is None:
            _check(_lib.proj_run(self._h, X_ptr, W_ptr, Y_ptr, M, stream_handle), "proj_run")
        else:
            _check(_lib.proj_run_ex(self._h, X_ptr, W_ptr, Y_ptr, M, gamma_ptr, stream_handle), "proj_run_ex")

    def run_candidate(self, idx: int, X, W, Y=None, stream=None, gamma=None):
        M, Y = self._prep(X, W, Y)
        _check(_lib.proj_run_candidate_ex(self._h, idx, X.data_ptr(), W.data_ptr(), Y.data_ptr(), M,
                                          self._gamma(gamma), _stream_handle(stream)), "proj_run_candidate_ex")
        return Y

    def num_candidates(self) -> int:
        return _check(_lib.proj_plan_num_candidates(self._h), "proj_plan_num_candidates")

    def candidate_name(self, idx: int) -> str:
        buf = ctypes.create_string_buffer(128)
        _check(_lib.proj_plan_candidate_name(self._h, idx, buf, 128), "proj_plan_candidate_name")
        return buf.value.decode()

    def candidates(self):
        return [self.candidate_name(i) for i in range(self.num_candidates())]

    def candidate_max_m(self, idx: int) -> int:
        return _check(_lib.proj_plan_candidate_max_m(self._h, idx), "proj_plan_candidate_max_m")

    def choice(self, M: int) -> str:
        return self.candidate_name(_check(_lib.proj_plan_choice(self._h, M), "proj_plan_choice"))

    def describe(self) -> dict:
        return json.loads(_text(_lib.proj_plan_describe, self._h))


def _bf16_packed(t, name: str, N: int, K: int):
    import torch
    shape = (N // PANEL_ROWS, K // PANEL_COLS, PANEL_ROWS, PANEL_COLS)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (bfloat16 or 16-bit bit patterns), got {t.dtype}")
    if tuple(t.shape) != shape or not t.is_contiguous():
        raise ValueError(f"{name} must be packed weights, a contiguous {shape} tensor (pack_weights), "
                         f"got {tuple(t.shape)}")


def pack_weights(W, Wp=None, stream=None):
    """W [N, K] (bf16, row-major, on the device) in the packed layout of
    proj_pack_weights, as a (N/128, K/64, 128, 64) tensor whose memory order is
    that layout: element [p, b, r, q] = W[128 p + r, 64 b + q]."""
    import torch
    if W.dim() != 2 or not W.is_contiguous() or W.element_size() != 2 or not W.is_cuda:
        raise ValueError("pack_weights: W must be a contiguous 16-bit [N, K] device matrix")
    N, K = W.shape
    if N % PANEL_ROWS or K % PANEL_COLS:
        raise ValueError(f"pack_weights: N % 128 == 0 and K % 64 == 0 needed, got {N}x{K}")
    if Wp is None:
        Wp = torch.empty((N // PANEL_ROWS, K // PANEL_COLS, PANEL_ROWS, PANEL_COLS), dtype=W.dtype, device=W.device)
    else:
        _bf16_packed(Wp, "Wp", N, K)
    _check(_lib.proj_pack_weights(N, K, W.data_ptr(), Wp.data_ptr(), _stream_handle(stream)), "proj_pack_weights")
    return Wp


def probe_read(buf, sink, never: int = 0x9E3779B9, stream=None) -> None:
    """Enqueue one streaming read of the whole device tensor `buf` (see proj.h)."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.proj_probe_read(buf.data_ptr(), nbytes, never, sink.data_ptr(), _stream_handle(stream)),
           "proj_probe_read")


def swiglu(G, H=None, stream=None):
    """H = silu(G[:, :N/2]) * G[:, N/2:] with the library's kernel (the unfused
    path of the SwiGLU epilogue); G is f32 or bf16 [M, N] on the device."""
    import torch
    if G.dim() != 2 or G.shape[1] % 2 or not G.is_contiguous() or G.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("swiglu: G must be a contiguous f32 or bf16 [M, N] matrix with N even")
    M, N = G.shape
    if H is None:
        H = torch.empty((M, N // 2), dtype=G.dtype, device=G.device)
    elif H.dtype != G.dtype or tuple(H.shape) != (M, N // 2) or not H.is_contiguous():
        raise ValueError(f"swiglu: H must be a contiguous [{M}, {N // 2}] {G.dtype} matrix")
    _check(_lib.proj_swiglu(G.data_ptr(), H.data_ptr(), M, N, _dtype_code(G.dtype), _stream_handle(stream)),
           "proj_swiglu")
    return H


def rmsnorm(X, gamma, eps: float, Xn=None, stream=None):
    """Xn = RMSNorm(X) * gamma row by row with the library's kernel (the
    unfused path of the norm prologue): X bf16 [M, K], gamma float32 [K]."""
    import torch
    if X.dim() != 2 or not X.is_contiguous() or X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("rmsnorm: X must be a contiguous bf16 [M, K] matrix")
    M, K = X.shape
    if not gamma.is_cuda or gamma.dtype != torch.float32 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError(f"rmsnorm: gamma must be a contiguous float32 device vector of {K} values")
    if Xn is None:
        Xn = torch.empty_like(X)
    elif tuple(Xn.shape) != (M, K) or Xn.element_size() != 2 or not Xn.is_contiguous():
        raise ValueError(f"rmsnorm: Xn must be a contiguous 16-bit [{M}, {K}] matrix")
    _check(_lib.proj_rmsnorm(X.data_ptr(), gamma.data_ptr(), Xn.data_ptr(), M, K, float(eps), _stream_handle(stream)),
           "proj_rmsnorm")
    return Xn


def round_bf16(inp, out, stream=None) -> None:
    """out[i] = bf16_rne(inp[i]) with the epilogue's device conversion."""
    import torch
    if inp.dtype != torch.float32 or out.dtype not in (torch.int16, torch.uint16, torch.bfloat16):
        raise TypeError("round_bf16: float32 in, 16-bit out")
    if out.numel() < inp.numel():
        raise ValueError("round_bf16: out too small")
    _check(_lib.proj_round_bf16(inp.data_ptr(), out.data_ptr(), inp.numel(), _stream_handle(stream)),
           "proj_round_bf16")
