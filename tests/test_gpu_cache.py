"""The persistent tuning cache (PROJ_CACHE_DIR): a tuned plan's choices are
kept per key, a later plan of the same key re-validates them through the
load-time gate instead of timing, and a cached choice that is unknown or fails
the gate sends its bucket back to full tuning."""
import os

import pytest

from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _choices(d):
    return [b["choice"] for b in d["buckets"]]


def test_cache_miss_hit_and_stale(tmp_path, monkeypatch):
    from shape_specialised_bf16_amd import Plan
    N, K = 2048, 1024
    monkeypatch.delenv("PROJ_CACHE_DIR", raising=False)
    assert Plan(N, K, "f32").describe()["cache"] == "off"

    monkeypatch.setenv("PROJ_CACHE_DIR", str(tmp_path))
    first = Plan(N, K, "f32").describe()
    assert first["cache"] == "miss"
    path = first["cache_path"]
    assert os.path.exists(path), path
    text = open(path).read().splitlines()
    assert text[0] == "libproj tuning cache 1"

    second = Plan(N, K, "f32").describe()
    assert second["cache"] == "hit" and second["cache_path"] == path
    assert _choices(second) == _choices(first)
    assert sum("cached, re-validated" in line for line in second["log"]) == len(second["buckets"])
    assert not any(b["timings_us"] for b in second["buckets"]), "a hit must not time candidates"
    G.log(f"  tune {first['tune_s']:.2f} s on a miss, {second['tune_s']:.2f} s on a hit")

    # an unknown name for bucket 0: that bucket is tuned again, the file is rewritten
    lines = [("bucket 0 gemv_no_such_kernel 1.0" if ln.startswith("bucket 0 ") else ln) for ln in text]
    open(path, "w").write("\n".join(lines) + "\n")
    third = Plan(N, K, "f32").describe()
    assert third["cache"] == "stale"
    assert third["buckets"][0]["timings_us"], "bucket 0 was not re-tuned"
    assert all(not b["timings_us"] for b in third["buckets"][1:])
    assert "gemv_no_such_kernel" not in open(path).read()

    # a different output type is a different key
    other = Plan(N, K, "bf16").describe()
    assert other["cache"] == "miss" and other["cache_path"] != path


def test_compiled_module_cache(tmp_path, monkeypatch):
    """With PROJ_CACHE_DIR the compiled modules are kept under the plan's key
    (one file per module): the next plan of that key loads them instead of
    compiling; a file that is not a loadable module makes the set stale, so it
    is compiled afresh and replaced; the plan computes the same result either
    way."""
    import numpy as np
    import oracle
    import synth
    from shape_specialised_bf16_amd import Plan
    N, K = 1024, 2048
    W = synth.normal_bf16(120, 0, (N, K), 0.02)
    X = synth.normal_bf16(120, 1, (37, K), 1.0)

    def run(p):
        Y = p.run(G.dev(X), G.dev(W))
        G.check_against_oracle(Y, X, W, "f32", label=f"cached module {p.choice(37)}")
        return G.host(Y)

    monkeypatch.delenv("PROJ_CACHE_DIR", raising=False)
    assert Plan(N, K, "f32").describe()["code_cache"] == "off"
    monkeypatch.setenv("PROJ_CACHE_DIR", str(tmp_path))
    p1 = Plan(N, K, "f32")
    d1 = p1.describe()
    assert d1["code_cache"] == "miss"
    base = d1["cache_path"][:-len(".txt")]
    files = [f"{base}.m{g}.co" for g in range(d1["modules"])]
    assert d1["modules"] > 1
    assert sum(os.path.getsize(f) for f in files) == d1["code_bytes"]
    co = files[-1]
    size_last = os.path.getsize(co)
    y1 = run(p1)
    p2 = Plan(N, K, "f32")
    assert p2.describe()["code_cache"] == "hit"
    assert np.array_equal(run(p2).view(np.uint32), y1.view(np.uint32))
    open(co, "wb").write(b"not a code object")
    p3 = Plan(N, K, "f32")
    assert p3.describe()["code_cache"] == "stale"
    assert os.path.getsize(co) == size_last, "the stale file was not replaced"
    assert np.array_equal(run(p3).view(np.uint32), y1.view(np.uint32))
    G.log(f"  code cache: miss {d1['compile_s']:.2f} s, then hit and stale handled")
