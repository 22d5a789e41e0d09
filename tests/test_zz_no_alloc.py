"""sherry_gemv_grouped_noalloc (the grouped GEMV launch that takes no device
copy of its plan and allocates nothing) against sherry_gemv_grouped on the
same plans, through the C ABI: bit-exact outputs on consecutive calls whose
second plan is smaller, and on two plans queued back to back on one stream."""
import numpy as np
import pytest
import torch

import synth
from oracle import sherry_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def say(*a):
    print(*a, flush=True)


def make_problems(shapes, seed):
    """Random codes, fp16 row scales and absmax-int8 tokens; fp16 outputs and
    int32 accumulators pre-filled with a pattern no product writes."""
    g = synth.rng(seed)
    probs, refs = [], []
    for n, k in shapes:
        words = synth.random_words(n * (k // 128) * 5, g)
        sw = synth.row_scales(n, g, np.float16)
        xq, sx, _ = synth.act_absmax_int8(1, k, g)
        refs.append(sherry_ref.gemv_i8(words, sw, n, k, xq[0], sx[0], np.float16))
        probs.append(dict(codes=dev(np.asarray(words, np.uint32).view(np.int32)), scales=dev(sw), x=dev(xq[0]),
                          x_scale=dev(sx), acc=torch.full((n,), -7, dtype=torch.int32, device=DEV),
                          y=torch.full((n,), float("nan"), dtype=torch.float16, device=DEV)))
    return probs, refs


def outputs(probs):
    return [(p["acc"].cpu().numpy().copy(), p["y"].cpu().numpy().view(np.uint16).copy()) for p in probs]


def reset(probs):
    for p in probs:
        p["acc"].fill_(-7)
        p["y"].fill_(float("nan"))


def check_same(probs, expect, refs, shapes):
    got = outputs(probs)
    for i, ((ga, gy), (ea, ey), (ra, ry)) in enumerate(zip(got, expect, refs)):
        assert np.array_equal(ga, ea), ("acc", i, shapes[i])
        assert np.array_equal(gy, ey), ("y", i, shapes[i])
        assert np.array_equal(ga, ra) and np.array_equal(gy, ry.view(np.uint16)), ("oracle", i, shapes[i])


BIG = [(2048, 2048), (512, 2048), (700, 8192), (256, 1024), (300, 384), (65, 3072), (17, 4096)] * 6
SMALL = [(33, 1024), (130, 2048), (5, 8192)]


def test_noalloc_matches_grouped_two_calls(gpu_lib):
    """Two calls in a row, the second with a smaller plan (fewer problems,
    fewer tiles): each call's outputs equal those of sherry_gemv_grouped on
    the same plan, and the oracle's, bit for bit."""
    for shapes, seed in ((BIG, 71), (SMALL, 72)):
        say(f"noalloc: {len(shapes)} problems, seed {seed}")
        probs, refs = make_problems(shapes, seed)
        grouped = gpu_lib.GroupedGemv(probs)
        grouped()
        torch.cuda.synchronize()
        expect = outputs(probs)
        reset(probs)
        grouped.call_noalloc()
        torch.cuda.synchronize()
        check_same(probs, expect, refs, shapes)


def test_noalloc_plans_queued_on_one_stream(gpu_lib):
    """Two different plans launched through the static plan memory back to
    back on one stream with no host wait between them: the second plan's copy
    is ordered after the first launch, so both give their own results."""
    say("noalloc: two plans queued back to back")
    pa, ra = make_problems(BIG[:7], 73)
    pb, rb = make_problems(SMALL, 74)
    ga, gb = gpu_lib.GroupedGemv(pa), gpu_lib.GroupedGemv(pb)
    ga()
    gb()
    torch.cuda.synchronize()
    ea, eb = outputs(pa), outputs(pb)
    reset(pa)
    reset(pb)
    ga.call_noalloc()
    gb.call_noalloc()
    torch.cuda.synchronize()
    check_same(pa, ea, ra, BIG[:7])
    check_same(pb, eb, rb, SMALL)
