"""Helpers for GPU parity tests: plan cache, transfers, oracle comparison."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from oracle import tolerance

_plans = {}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def plan(N: int, K: int, dtype: str = "f32", epilogue=None, rmsnorm_eps=None, packed: bool = False):
    from shape_specialised_bf16_amd import Plan

    key = (N, K, dtype, epilogue, rmsnorm_eps, packed)
    if key not in _plans:
        log(f"[plan] creating {N}x{K} {dtype}" + (f" epilogue {epilogue}" if epilogue else "")
            + (f" rmsnorm eps {rmsnorm_eps}" if rmsnorm_eps is not None else "") + (" packed" if packed else ""))
        _plans[key] = Plan(N, K, dtype, epilogue=epilogue, rmsnorm_eps=rmsnorm_eps, packed=packed)
    return _plans[key]


def dev(a: np.ndarray):
    import torch
    assert a.dtype == np.uint16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host(Y) -> np.ndarray:
    import torch
    if Y.dtype == torch.bfloat16:
        return Y.view(torch.int16).cpu().numpy().view(np.uint16)
    return Y.cpu().numpy()


def empty_out(M: int, N: int, dtype: str, extra_rows: int = 0, fill_nan: bool = True):
    """Output buffer with `extra_rows` guard rows, pre-filled with a NaN pattern."""
    import torch
    t = torch.empty((M + extra_rows, N), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device="cuda")
    if fill_nan:
        t.view(torch.int16 if dtype == "bf16" else torch.int32).fill_(0x7FC1 if dtype == "bf16" else 0x7FC00001)
    return t


def compare(Yh: np.ndarray, ref: np.ndarray, dtype: str):
    if dtype == "bf16":
        return tolerance.check_bf16(Yh, ref)
    return tolerance.check_f32(Yh, ref)


def sample_rows(M: int, seed: int = 0, extra=()):
    """First, last, tile-boundary and a few random rows below M."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, M // 2}
    for b in (15, 16, 31, 32, 63, 64, 127, 128, 255, 256, 1023, 1024, 4095, 4096):
        if b < M:
            rows.add(b)
    rows.update(int(v) for v in rng.integers(0, M, size=3))
    rows.update(r for r in extra if r < M)
    return sorted(rows)


def check_against_oracle(Y, X: np.ndarray, W: np.ndarray, dtype: str, rows=None, label: str = ""):
    """Compare device output Y[:M] with the oracle, on all rows or on `rows`."""
    M = X.shape[0]
    Yh = host(Y)[:M]
    if rows is None:
        ref = oracle.matmul(X, W)
        got = Yh
    else:
        ref = oracle.matmul_rows(X, rows, W)
        got = Yh[rows]
    rep = compare(got, ref, dtype)
    log(f"  {label} M={M} {dtype}: {rep}")
    assert rep.ok, f"{label}: {rep}"
    if dtype == "bf16":
        # the near-zero clause may only rescue tiny |ref| elements
        assert rep.n_second_clause <= max(8, rep.n // 1000), rep
    return rep
