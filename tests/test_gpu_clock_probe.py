"""The clock probe on the GPU: the probe copy of a tuned GEMM computes the
same bits as the plan's own launch of that candidate, and every workgroup
reports a clock within the part's range."""
import pytest

import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_probe_copy_matches_the_candidate_and_reads_sane_clocks():
    import torch

    from shape_specialised_bf16_amd import clock_probe

    N, K, M = 5120, 2560, 512
    p = G.plan(N, K, "bf16")
    idx = next(i for i, n in enumerate(p.candidates())
               if clock_probe.geometry(n, N, M) is not None and p.candidate_max_m(i) >= M)
    name = p.candidates()[idx]
    G.log(f"  clock probe of {name} at M={M}")
    Xh = synth.normal_bf16(90, 0, (M, K), 1.0)
    Wh = synth.normal_bf16(90, 1, (N, K), 0.02)
    X, W = G.dev(Xh), G.dev(Wh)
    Yp = G.empty_out(M, N, "bf16")
    Yr = G.empty_out(M, N, "bf16")
    p.run_candidate(idx, X, W, Yr)
    r = clock_probe.measure(N, K, "bf16", name, X.view(torch.bfloat16), [W.view(torch.bfloat16)],
                            Yp.view(torch.bfloat16), M, launches=5, warm_s=0.02)
    torch.cuda.synchronize()
    assert torch.equal(Yp.view(torch.int16), Yr.view(torch.int16)), "probe copy differs from the candidate"
    assert 100.0 <= r["mhz_p10"] <= r["mhz_weighted"] * 1.5 and r["mhz_p90"] <= 2600.0, r
    G.log(f"  {name}: {r['mhz_weighted']} MHz (p10 {r['mhz_p10']}, p90 {r['mhz_p90']})")
