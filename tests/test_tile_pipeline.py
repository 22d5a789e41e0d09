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
UNROLL = 8             # steps per loop iteration of the kernel
CODE_SLOTS = 2
DEPTH = 2              # x ring

# format: groups per code stage P, 16-byte head chunks per row HC, tail words
FORMATS = {"sherry": dict(P=4, HC=4, tail=True), "tern2": dict(P=2, HC=4, tail=False)}
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
    TH = R * HC // 64
    TT = R * P // 64 if f["tail"] else 0
    CPW = (TH + TT) // ((P // 2) * W)
    assert CPW * (P // 2) * W == TH + TT and CPW >= 1
    assert P % 2 == 0 and UNROLL % (CODE_SLOTS * P) == 0 and UNROLL % DEPTH == 0
    lds = 1024 + DEPTH * xbytes + CODE_SLOTS * stage
    assert lds <= LDS_BYTES // t["wgcu"], "the tiling's LDS fits its workgroups per CU"
    return dict(W=W, TX=TX, NX=math.ceil(TX / W), P=P, CPW=CPW, rows=R, stage_rows=TH + TT, wait=0)


def simulate(cfg, G):
    """Issue order of every wave; returns the checks' failures (empty: safe).
    cfg["wait"]: the outstanding copies the barrier wait allows (the kernel: 0)."""
    W, TX, NX, P, CPW = (cfg[k] for k in ("W", "TX", "NX", "P", "CPW"))
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
    # prologue: code stage 0 and the x tile of step 0, then the wait and the
    # barrier; every wave then decodes step 0 from stage 0
    for w in range(W):
        issued[w] += [("code", 0)] * ((P // 2) * CPW)
        copy_x(w, 0)
        wait(w, cfg["wait"])
    if not done("code", 0) or not done("x", 0):
        failures.append("prologue: stage 0 or step 0 not landed")
    # step s reads x slot s % 2 and (decoding step s + 1) code slot
    # ((s + 1) // P) % 2
    steps = -(-G // UNROLL) * UNROLL
    for s in range(steps):
        for w in range(W):
            wait(w, cfg["wait"])
        # barrier: every wave has retired what its wait covers
        if s < G:
            if not done("x", s):
                failures.append(f"step {s}: x not landed")
            if s + 1 < G and not done("code", (s + 1) // P):
                failures.append(f"step {s}: code stage {(s + 1) // P} not landed")
        # copies issued after the barrier: x of step s + 1 into the slot of
        # step s - 1, and (first P / 2 steps of a stage) part of stage
        # s // P + 1 into the slot of stage s // P - 1
        if s < G and (s + 1) % 2 == s % 2:
            failures.append(f"step {s}: x copy into the slot being read")
        code_copy = s % P < P // 2
        if code_copy and s + 1 < G and (s // P + 1) % 2 == ((s + 1) // P) % 2:
            failures.append(f"step {s}: code copy into the stage being decoded")
        if code_copy and s < G and s % P != 0 and (s // P + 1) % 2 == (s // P) % 2:
            failures.append(f"step {s}: code copy into the stage in use")
        for w in range(W):
            copy_x(w, s + 1)
            if code_copy:
                issued[w] += [("code", s // P + 1)] * CPW
    return failures


@pytest.mark.parametrize("fmt", sorted(FORMATS))
@pytest.mark.parametrize("tiling", sorted(TILINGS))
@pytest.mark.parametrize("G", [1, 2, 3, 5, 16, 24, 64, 65])
def test_tile_pipeline_is_safe(fmt, tiling, G):
    cfg = config(fmt, tiling)
    assert simulate(cfg, G) == []


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_tile_pipeline_model_catches_a_short_wait(fmt):
    """The model is not vacuous: a barrier that leaves the wave's youngest
    copies in flight lets a step read a tile or a stage still in flight."""
    cfg = dict(config(fmt, "large"))
    cfg["wait"] = cfg["NX"]
    assert simulate(cfg, 16) != []


def test_tile_configs():
    """Copy counts of the kept tilings: per wave and step, 4 x-tile copies and
    (in the first half of a stage) 4 code copies."""
    big = config("sherry", "large")
    assert (big["TX"], big["CPW"]) == (16, 4)
    t2 = config("tern2", "large")
    assert (t2["TX"], t2["CPW"]) == (16, 4)
