"""The MFMA GEMM's global->LDS copy ring, checked on the CPU (no GPU).

gemm_mfma (csrc/gemm.hip) keeps k-tiles of X and W in rings of LDS buffers and
waits for its copies with explicit vmcnt counts (s_waitcnt) followed by a
workgroup barrier, instead of draining every copy.  This test replays the
kernel's issue order -- prologue, then per k-tile: copies, operand reads, wait,
barrier, first reads of the next tile, early copies -- in a model of one wave's
in-order copy queue, for every GEMM configuration the code generator emits and
every k-tile count up to a few ring periods, and checks:

  * every operand read finds its own k-tile fully landed in the buffer it reads
    (all of that copy's instructions completed at the last barrier), and
  * no copy is issued into a buffer that some wave may still read: the buffer's
    last read happened before the last barrier (each wave's wait also drains
    its LDS reads, so a barrier ends every earlier read).

Each wave issues the same sequence and waits only for its own copies, so one
wave's queue with the barrier as the point where all waves' copies older than
the wait count have landed is the whole workgroup.  The wait counts are the
kernel's constants; the test also checks that gemm.hip still defines them as
modelled here.
"""
import math
import os
import re

import pytest

import shape_specialised_bf16_amd as ssb

GEMM_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "shape_specialised_bf16_amd", "csrc", "gemm.hip")

# the ring constants as gemm_mfma defines them (checked against the source below)
KERNEL_LINES = [
    "constexpr bool EARLY = DMA && STAGES == 2;",
    "constexpr int LEAD = EARLY ? STAGES : STAGES - 1;",
    "constexpr bool SPLIT = BST != 0;",
    "constexpr int NB = SPLIT ? BST : STAGES;",
    "constexpr int LEAD_B = SPLIT ? LEAD + BST - STAGES : LEAD;",
    "constexpr int PERIOD = SPLIT ? STAGES * BST / gcd(STAGES, BST) : STAGES;",
    "constexpr int WAIT0 = (LEAD - 1) * IA + (LEAD_B - 1) * IB;",
    "constexpr int WAITK = (SPLIT ? IB : 0) + (DMA && !EARLY ? (STAGES - 2) * PER_TILE : 0);",
]


def ring_constants(STAGES, DMA, BST, IA, IB):
    EARLY = bool(DMA) and STAGES == 2
    LEAD = STAGES if EARLY else STAGES - 1
    SPLIT = BST != 0
    NB = BST if SPLIT else STAGES
    LEAD_B = LEAD + BST - STAGES if SPLIT else LEAD
    PERIOD = STAGES * BST // math.gcd(STAGES, BST) if SPLIT else STAGES
    WAIT0 = (LEAD - 1) * IA + (LEAD_B - 1) * IB
    WAITK = (IB if SPLIT else 0) + ((STAGES - 2) * (IA + IB) if DMA and not EARLY else 0)
    return dict(EARLY=EARLY, LEAD=LEAD, SPLIT=SPLIT, NB=NB, LEAD_B=LEAD_B, PERIOD=PERIOD,
                WAIT0=WAIT0, WAITK=WAITK)


class RingError(AssertionError):
    pass


def replay(NKT, STAGES, DMA, BST, IA, IB, KK, wait0=None, waitk=None, early_before_barrier=False):
    """Replay the k loop over NKT k-tiles; raise RingError on a violation.
    wait0 / waitk replace the kernel's wait counts, and early_before_barrier
    moves the two-buffer ring's copies ahead of the barrier (both planted
    mistakes, for the tests that show the model catches them)."""
    c = ring_constants(STAGES, DMA, BST, IA, IB)
    W0 = c["WAIT0"] if wait0 is None else wait0
    WK = c["WAITK"] if waitk is None else waitk
    EARLY, LEAD, LEAD_B, NB, PERIOD, SPLIT = (c[k] for k in ("EARLY", "LEAD", "LEAD_B", "NB", "PERIOD", "SPLIT"))

    def bufA(s):
        return ("A", s % STAGES)

    def bufB(s):
        return ("B", s % NB) if SPLIT else ("B", s % STAGES)   # without SPLIT: W's half of buffer s

    def clamp(t):
        return min(t, NKT - 1)

    queue = []           # one wave's outstanding copy instructions, oldest first: (buffer, serial)
    content = {}         # buffer -> [tile, landed instructions, instructions, serial]
    last_read = {}       # buffer -> epoch of its last read
    state = dict(epoch=0, serial=0, landed_at_barrier={})

    def issue(buf, tile, n):
        if last_read.get(buf, -1) >= state["epoch"]:
            raise RingError(f"NKT={NKT}: copy of tile {tile} into {buf} while it may still be read")
        state["serial"] += 1
        content[buf] = [tile, 0, n, state["serial"]]
        if DMA:
            queue.extend([(buf, state["serial"])] * n)
        else:
            content[buf][1] = n            # LDS stores from registers: complete by the next wait

    def wait(n):
        while len(queue) > n:
            buf, serial = queue.pop(0)
            if content[buf][3] == serial:
                content[buf][1] += 1

    def barrier():
        state["epoch"] += 1
        state["landed_at_barrier"] = {b: (v[0], v[3]) for b, v in content.items() if v[1] == v[2]}

    def read(buf, tile, check=True):
        last_read[buf] = state["epoch"]
        if not check:
            return
        landed = state["landed_at_barrier"].get(buf)
        cur = content.get(buf)
        if landed is None or landed[0] != tile or cur is None or cur[3] != landed[1]:
            raise RingError(f"NKT={NKT}: read of tile {tile} from {buf} finds "
                            f"{'nothing landed' if landed is None else f'tile {landed[0]}'}"
                            f"{' (overwritten since)' if landed and cur and cur[3] != landed[1] else ''}")

    # prologue
    if DMA:
        for s in range(LEAD_B):
            if s < LEAD:
                issue(bufA(s), clamp(s), IA)
            issue(bufB(s), clamp(s), IB)
    else:
        issue(bufA(0), 0, IA)
        issue(bufB(0), 0, IB)
    wait(W0 if DMA else 0)
    barrier()
    read(bufA(0), 0)
    read(bufB(0), 0)
    for kt in range(NKT):
        R = kt % PERIOD
        if DMA and not EARLY:
            issue(bufA(R + STAGES - 1), clamp(kt + LEAD), IA)
            issue(bufB(R + NB - 1), clamp(kt + LEAD_B), IB)
        for _ in range(KK - 1):
            read(bufA(R), kt)
            read(bufB(R), kt)
        if not DMA:
            issue(bufA(R + 1), clamp(kt + 1), IA)
            issue(bufB(R + 1), clamp(kt + 1), IB)
        if EARLY and early_before_barrier:
            issue(bufA(R), clamp(kt + LEAD), IA)
            issue(bufB(R), clamp(kt + LEAD_B), IB)
        wait(WK)
        barrier()
        # the next tile's first fragments (past the last tile: a re-read whose values go unused)
        read(bufA(R + 1), kt + 1, check=kt + 1 < NKT)
        read(bufB(R + 1), kt + 1, check=kt + 1 < NKT)
        if EARLY and not early_before_barrier:
            issue(bufA(R), clamp(kt + LEAD), IA)
            issue(bufB(R), clamp(kt + LEAD_B), IB)
    wait(0)


def emitted_configs():
    """(BM, BN, BK, STAGES, WM, WN, SK, DMA, TAILS, BST) and K of every gemm_mfma
    instantiation the generator emits for a spread of shapes."""
    shapes = [(7168, 1024, "f32", {}), (2560, 9216, "bf16", {}), (34816, 5120, "bf16", {}),
              (5120, 17408, "bf16", {}), (18432, 2560, "bf16", {}), (18432, 2560, "bf16", dict(epilogue="swiglu")),
              (7168, 1024, "bf16", dict(packed=True))]
    out = set()
    for N, K, dt, kw in shapes:
        src = ssb.emit_source(N, K, dt, **kw)
        for args in re.findall(r"gemm_mfma<([^>]*)>\(X, W, Y, ws, M\)", src):
            a = [x.strip() for x in args.split(",")]
            BM, BN, BK, ST, WM, WN, SK, GM, SWZ = (int(v) for v in a[:9])
            DMA, TAILS, ROUND, E, BST = (int(v) for v in a[10:15])
            out.add((BM, BN, BK, ST, WM, WN, SK, DMA, TAILS, BST, K))
    return sorted(out)


CONFIGS = emitted_configs()


def test_kernel_defines_the_modelled_constants():
    src = open(GEMM_SRC).read()
    for line in KERNEL_LINES:
        assert line in src, f"gemm.hip no longer has: {line}"


def test_configurations_cover_every_ring_kind():
    kinds = {(ST, DMA, BST > 0) for (_, _, _, ST, _, _, _, DMA, _, BST, _) in CONFIGS}
    assert {(2, 1, False), (2, 1, True), (3, 1, False), (3, 1, True), (2, 0, False)} <= kinds, kinds
    # W rings deeper than X's by more than one buffer, on both ring kinds
    deep = {(ST, BST - ST) for (_, _, _, ST, _, _, _, DMA, _, BST, _) in CONFIGS if BST > ST + 1}
    assert any(st == 2 for st, _ in deep) and any(st == 3 for st, _ in deep), deep


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: "{}x{}x{}_st{}_w{}x{}_sk{}_dma{}_t{}_b{}_K{}".format(*c))
def test_ring_waits_are_exact_for_every_tile_count(cfg):
    BM, BN, BK, ST, WM, WN, SK, DMA, TAILS, BST, K = cfg
    nthr = WM * WN * 64
    IA, IB = BM * (BK // 8) // nthr, BN * (BK // 8) // nthr
    c = ring_constants(ST, DMA, BST, IA, IB)
    assert c["WAIT0"] <= 63 and c["WAITK"] <= 63, "wait counts fit the vmcnt field"
    KT = K // SK // BK
    counts = set(range(1, min(KT, 3 * c["PERIOD"] + 2) + 1)) | {KT}
    if TAILS > 1:                                 # a tail piece: KT // TAILS k-tiles or one more
        counts |= {KT // TAILS, -(-KT // TAILS)}
    for nkt in sorted(counts):
        replay(nkt, ST, DMA, BST, IA, IB, BK // 16)


@pytest.mark.parametrize("ST,BST", [(2, 0), (2, 3), (2, 4), (2, 6), (3, 0), (3, 4), (3, 6), (4, 7)])
def test_model_rejects_a_wait_one_copy_short(ST, BST):
    """A wait that leaves one more copy instruction outstanding than the kernel's
    count lets a read find its tile partly landed: the model must see it."""
    IA, IB = 4, 4
    c = ring_constants(ST, 1, BST, IA, IB)
    replay(40, ST, 1, BST, IA, IB, 4)                                   # the kernel's counts pass
    with pytest.raises(RingError):
        replay(40, ST, 1, BST, IA, IB, 4, waitk=c["WAITK"] + 1)
    with pytest.raises(RingError):
        replay(40, ST, 1, BST, IA, IB, 4, wait0=c["WAIT0"] + 1)


@pytest.mark.parametrize("BST", [0, 3])
def test_model_rejects_a_copy_into_a_buffer_still_read(BST):
    """The two-buffer ring issues the copy of tile kt+2 into tile kt's buffer
    right after the barrier that ends tile kt's reads; issued before that
    barrier it races with other waves still reading tile kt."""
    replay(40, 2, 1, BST, 4, 4, 4)
    with pytest.raises(RingError, match="may still be read"):
        replay(40, 2, 1, BST, 4, 4, 4, early_before_barrier=True)
