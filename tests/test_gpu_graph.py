"""proj_run recorded into a HIP graph and replayed.

A decode step (the GEMV path) and prefill launches that use the plan's
workspace (a split-K GEMM and a split-tail GEMM, both with their second pass)
are captured once, then the graph is replayed several times with the program's
own eager work -- the same plans run eagerly on other buffers, which reuses the
same workspace, torch ops, synchronisations -- between the replays.  Every
replay is compared with the oracle element by element at the projection
tolerance (all rows of the decode and split-K outputs, sampled rows -- first,
last, tile edges, random -- of the 2112-row split-tail output), and must also
reproduce the eager result bit for bit.
"""
import pytest

import oracle
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _pick(p, pattern, M):
    for idx, name in enumerate(p.candidates()):
        if pattern(name) and p.candidate_max_m(idx) >= M:
            return idx, name
    pytest.skip(f"no candidate for {pattern} at M={M}")


def test_graph_replay_matches_eager():
    import torch

    # decode: two GEMV projections at M=1 through the tuned choice
    dec, host = [], []
    for i, (N, K) in enumerate([(2048, 1024), (1024, 3072)]):
        p = G.plan(N, K, "f32")
        Wh = synth.normal_bf16(80, 2 * i, (N, K), 0.02)
        Xh = synth.normal_bf16(80, 2 * i + 1, (1, K), 1.0)
        dec.append((p, G.dev(Xh), G.dev(Wh), N))
        host.append((Xh, Wh, None))
    # prefill: a split-K and a split-tail candidate of one plan (both use the workspace)
    N, K = 7168, 1024
    pg = G.plan(N, K, "f32")
    Wgh = synth.normal_bf16(81, 0, (N, K), 0.02)
    Xgh = synth.normal_bf16(81, 1, (2112, K), 1.0)
    Wg, Xg = G.dev(Wgh), G.dev(Xgh)
    host.append((Xgh[:300], Wgh, None))
    host.append((Xgh, Wgh, G.sample_rows(2112, seed=81, extra=(255, 256, 1791, 1792, 2047, 2048))))
    # the oracle's results, computed once
    refs = [oracle.matmul(X, W) if rows is None else oracle.matmul_rows(X, rows, W) for X, W, rows in host]

    def check_oracle(outs, what):
        for k, (Y, (X, W, rows), ref) in enumerate(zip(outs, host, refs)):
            got = G.host(Y)[:X.shape[0]]
            if rows is not None:
                got = got[rows]
            rep = G.compare(got, ref, "f32")
            assert rep.ok, f"{what}: output {k} against the oracle: {rep}"
    sk_idx, sk_name = _pick(pg, lambda n: "_sk2" in n or "_sk4" in n, 300)
    tl_idx, tl_name = _pick(pg, lambda n: "_tail" in n and not n.endswith("_reduce"), 2112)

    def launch(outs):
        for (p, X, W, _), Y in zip(dec, outs[:2]):
            p.run(X, W, Y)
        pg.run_candidate(sk_idx, Xg[:300], Wg, outs[2])
        pg.run_candidate(tl_idx, Xg, Wg, outs[3])

    def fresh():
        return [G.empty_out(1, n, "f32") for (_, _, _, n) in dec] + \
               [G.empty_out(300, N, "f32"), G.empty_out(2112, N, "f32")]

    ref = fresh()
    launch(ref)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ref]

    outs = fresh()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    launch(outs)                          # warm-up on the eager stream before capture
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            launch(outs)
    torch.cuda.synchronize()

    scratch = fresh()
    for rep in range(4):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_oracle(outs, f"replay {rep}")
        for k, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), \
                f"replay {rep}: output {k} ({sk_name if k == 2 else tl_name if k == 3 else 'decode'}) differs"
        # eager work between replays: same plans, other buffers, same workspace
        launch(scratch)
        torch.cuda.synchronize()
        check_oracle(scratch, f"eager run {rep}")
        for k, (a, b) in enumerate(zip(scratch, ref)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"eager run {rep}: output {k} differs"
        for y in scratch:
            y.zero_()
    G.log(f"  graph of 2 GEMVs + {sk_name} + {tl_name}: 4 replays within the oracle's tolerance and "
          f"bit-identical to eager")
