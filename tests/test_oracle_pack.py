"""Pins of the oracle's packed weight layout (oracle.pack_panels).

The layout is the library's own choice (declared with proj_pack_weights); the
oracle is pinned to its written definition by positions worked out by hand
(``tests/golden/packed_layout_256x128.txt``), which tell apart the plausible
mistakes -- column-major blocks (index 64), panel-major instead of block-major
order inside a panel (index 8192), a wrong panel stride (index 16384) -- and by
the fact that packing only moves values.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packed_layout_256x128.txt")


def _codes(N, K):
    """W whose every value is its own position code n * K + k (unique below 2^16)."""
    assert N * K <= 1 << 16
    return np.arange(N * K, dtype=np.uint32).astype(np.uint16).reshape(N, K)


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            rows.append(tuple(int(v) for v in line))
    return rows


def test_hand_derived_positions():
    N, K = 256, 128
    flat = oracle.pack_panels(_codes(N, K)).ravel()
    rows = _golden()
    assert len(rows) >= 10
    for i, n, k in rows:
        assert int(flat[i]) == n * K + k, f"packed index {i}: holds W[{int(flat[i]) // K}, {int(flat[i]) % K}], " \
                                          f"expected W[{n}, {k}]"


def test_shape_and_block_contiguity():
    N, K = 384, 192
    W = np.random.default_rng(5).integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    P = oracle.pack_panels(W)
    assert P.shape == (3, 3, 128, 64) and P.dtype == np.uint16
    flat = P.ravel()
    # block (p, b) is 8192 consecutive values holding rows 128p.., columns 64b..
    for p in range(3):
        for b in range(3):
            blk = flat[(p * 3 + b) * 8192:(p * 3 + b + 1) * 8192].reshape(128, 64)
            assert np.array_equal(blk, W[128 * p:128 * p + 128, 64 * b:64 * b + 64])


def test_packing_only_moves_values():
    N, K = 256, 256
    W = _codes(N, K)
    flat = oracle.pack_panels(W).ravel()
    assert np.array_equal(np.sort(flat), np.sort(W.ravel())), "a value was lost or duplicated"
    # and as a projection weight the packed matrix gives the same product once
    # its blocks are put back (brute force over the small matrix)
    back = np.empty_like(W)
    for i, v in enumerate(flat.tolist()):
        back[v // K, v % K] = v
    assert np.array_equal(back, W)


@pytest.mark.parametrize("N,K", [(100, 128), (128, 100), (128, 8)])
def test_shapes_without_whole_blocks_are_rejected(N, K):
    with pytest.raises(ValueError):
        oracle.pack_panels(np.zeros((N, K), dtype=np.uint16))
