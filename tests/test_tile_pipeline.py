"""Host model of the copy pipeline of the tiled GEMM kernel (the prefill and
256 x 16 tilings): every copy a wave issues, in the kernel's order, and the
waits and barriers between steps.  The model checks, for every format and
tiling the library builds, that when a step reads the x tile of its group and
the code stage of the next group, every wave's copies of them are among the
operations its wait at the step's barrier has retired (loads retire in order,
so a wait for "at most n outstanding" retires all but the n youngest), and
that no copy overwrites a buffer a step may still read.  The configuration
values restate the kernel's tile shapes and LDS budget; nothing here runs on
the GPU.
"""
import math

import pytest

GROUP = 128            # weights per group: k advances one group per step
LDS_BYTES = 160 * 1024
UNROLL = 12            # steps per loop iteration of the kernel
CODE_SLOTS = 3
DEPTH_CAP = 3          # the kernel's x ring depth cap

# format: groups per code stage P, 16-byte head chunks per row HC, tail words
FORMATS = {"sherry": dict(P=2, HC=2, tail=True), "tern2": dict(P=1, HC=2, tail=False)}
# tiling: waves along rows WR, along tokens WC, 16-token tiles per wave UT,
# rows per wave, workgroups per CU
TILINGS = {"large": dict(WR=4, WC=1, UT=8, rows=64, wgcu=2),
           "small": dict(WR=2, WC=2, UT=4, rows=64, wgcu=2),
           "skinny": dict(WR=4, WC=1, UT=1, rows=64, wgcu=2)}


def config(fmt, tiling):
    f, t = FORMATS[fmt], TILINGS[tiling]
    W = t["WR"] * t["WC"]
    R = t["rows"] * t["WR"]
    tok = 16 * t["UT"] * t["WC"]
    xbytes = tok * GROUP
    TX = xbytes // (16 * 64)
    P, HC = f["P"], f["HC"]
    stage = R * (16 * HC + (4 * P if f["tail"] else 0))
    fit = (LDS_BYTES // t["wgcu"] - 1024 - CODE_SLOTS * stage) // xbytes
    D = min(fit, DEPTH_CAP, P + 1)
    TH = R * HC // 64
    TT = R * P // 64 if f["tail"] else 0
    CPW = (TH + TT) // (P * W)
    assert CPW * P * W == TH + TT and CPW >= 1
    assert D >= 2 and UNROLL % D == 0 and UNROLL % (CODE_SLOTS * P) == 0 and D <= P + 1
    lds = 1024 + D * xbytes + CODE_SLOTS * stage
    assert lds <= LDS_BYTES // t["wgcu"], "the tiling's LDS fits its workgroups per CU"
    return dict(W=W, TX=TX, NX=math.ceil(TX / W), P=P, D=D, CPW=CPW, ops=TX // W + CPW)


def simulate(cfg, G):
    """Issue order of every wave; returns the checks' failures (empty: safe)."""
    W, TX, NX, P, D, CPW, ops = (cfg[k] for k in ("W", "TX", "NX", "P", "D", "CPW", "ops"))
    PC = P * CPW
    late = (D - 1) * CPW
    assert late <= PC
    issued = [[] for _ in range(W)]   # per wave: (kind, index) in issue order
    retired = [0] * W                 # per wave: number of its oldest ops retired

    def copy_x(w, step):
        for j in range(NX):
            if NX * w + j < TX:
                issued[w].append(("x", step))

    def wait(w, n):
        retired[w] = max(retired[w], len(issued[w]) - n)

    def done(kind, idx):
        """Every wave's copies of (kind, idx) are retired."""
        return all((kind, idx) not in issued[w][retired[w]:] for w in range(W))

    failures = []
    # prologue: code stages 0 and 1, x steps 0 .. D - 2
    for w in range(W):
        issued[w] += [("code", 0)] * PC + [("code", 1)] * (PC - late)
        for b in range(D - 1):
            copy_x(w, b)
            issued[w] += [("code", 1)] * CPW
        wait(w, PC - late + (D - 1) * ops)
    # barrier, then every wave decodes step 0 from stage 0
    if not done("code", 0):
        failures.append("prologue: stage 0 not landed")
    # which buffers are being read: step s reads x slot s % D and (decoding
    # step s + 1) code slot ((s + 1) // P) % 3
    steps = -(-G // UNROLL) * UNROLL
    for s in range(steps):
        for w in range(W):
            wait(w, ops * (D - 2))
        # barrier: every wave has retired what its wait covers
        if s < G:
            if not done("x", s):
                failures.append(f"step {s}: x not landed")
            if s + 1 < G and not done("code", (s + 1) // P):
                failures.append(f"step {s}: code stage {(s + 1) // P} not landed")
        # copies issued after the barrier: x of step s + D - 1 into the slot
        # of step s - 1, and part of stage s // P + 2 into the slot of stage
        # s // P - 1
        xs_slot, cs_slot = (s + D - 1) % D, (s // P + 2) % CODE_SLOTS
        if s < G and xs_slot == s % D:
            failures.append(f"step {s}: x copy into the slot being read")
        if s + 1 < G and cs_slot == ((s + 1) // P) % CODE_SLOTS:
            failures.append(f"step {s}: code copy into the stage being decoded")
        for w in range(W):
            copy_x(w, s + D - 1)
            issued[w] += [("code", s // P + 2)] * CPW
    return failures


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("tiling", sorted(TILINGS))
@pytest.mark.parametrize("G", [1, 2, 3, 5, 16, 24, 64, 65])
def test_tile_pipeline_is_safe(fmt, tiling, G):
    cfg = config(fmt, tiling)
    assert simulate(cfg, G) == []


def test_tile_pipeline_model_catches_a_short_wait():
    """The model is not vacuous: one outstanding copy more at the barrier than
    the kernel allows leaves a step reading a tile still in flight."""
    cfg = dict(config("sherry", "large"))
    cfg["ops"] += 1
    assert simulate(cfg, 16) != []


def test_tile_configs():
    """The ring depths and copy counts of the kept tilings."""
    big = config("sherry", "large")
    assert (big["D"], big["TX"], big["CPW"], big["ops"]) == (3, 16, 2, 6)
    t2 = config("tern2", "large")
    assert (t2["D"], t2["TX"], t2["CPW"], t2["ops"]) == (2, 16, 2, 6)
