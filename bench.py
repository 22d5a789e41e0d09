#!/usr/bin/env python3
"""Benchmark of the Sherry 1.25-bit ternary GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one batch-1 decode pass of the GEMV over every matrix of a
LLaMA-3.2-1B decoder layer (q, k, v, o, gate, up, down; int8 activations with
a per-token scale, fp16 row scales, fp16 outputs), repeated over R distinct
replicas of the layer (default 112, 1.06 GB of codes, four times the 256 MB
last-level cache) in one grouped launch, so the codes stream from HBM.  All
inputs are seeded synthetic data already resident in device memory.

Prints one JSON line (the metric), with the dominant kernel's roofline and
the CPU oracle's throughput on a bounded sample; secondary measurements go
under "extras".
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
METRIC = "1.25-bit ternary GEMV weights/s + % of HBM peak (LLaMA-3.2-1B shapes, batch 1)"
KERNEL_SOURCES = ["ultra_bit_weight_amd/csrc/gemv.hip", "ultra_bit_weight_amd/csrc/formats.h",
                  "ultra_bit_weight_amd/csrc/common.h", "ultra_bit_weight_amd/csrc/launch.h"]
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemv_grouped_llama1b_b1_counters.md")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=112)
    p.add_argument("--seed", type=int, default=2)
    p.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                   help="sustained-load time before each timed region (lets the clocks settle)")
    p.add_argument("--no-extras", action="store_true", help="only the metric line (no secondary measurements)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--probes", action="store_true",
                   help="only the ceiling probes (streaming read, matrix-core and v_dot4 rates): one JSON line")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one plain 1 GiB device copy (calibrates HBM byte counters)")
    p.add_argument("--gemm-profile", action="store_true",
                   help="only the grouped GEMM launches on the 1B layer (M = 2048 prefill and M = 16 few-token), "
                        "a few of each, for a profiler; prints their timing and exits")
    p.add_argument("--f4-profile", action="store_true",
                   help="only the decode pipeline (a 1B token's fused products over min(16, replicas) layers, "
                        "eager and graph replay); prints its timing and exits")
    p.add_argument("--bf16-gemm-profile", action="store_true",
                   help="only the grouped bf16 few-token GEMM on the 3B layer (M = 2, 4, 8, 16) over 72 replicas; "
                        "prints their rates and exits")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) and exit")
    p.add_argument("--summarize-pmc", nargs="+", metavar="PMC_DIR",
                   help="summarise rocprofv3 --pmc runs of `bench.py --no-extras` (grouped GEMV counters per "
                        "dispatch and per 128-weight group) and exit")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="summarise a rocprofv3 --kernel-trace run of `bench.py --no-extras` (the last --steps "
                        "dispatches of the grouped GEMV are its timed launches) and exit")
    return p.parse_args(argv)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------- workloads ---

def layer_bytes(shapes, x_bytes_per_elem=1, y_bytes=2, scale_bytes=2, with_sx=True):
    """Algorithmic bytes of one batch-1 pass over a layer: codes (5/32 B per
    weight), row scales, x, y and the per-token scale, each read/written once."""
    total = 0
    for _, n, k in shapes:
        total += n * k * 5 // 32 + n * scale_bytes + k * x_bytes_per_elem + n * y_bytes + (4 if with_sx else 0)
    return total


def build_layer_replicas(torch, sherry, synth, shapes, replicas, seed, x_kind="i8", tern2=False):
    """R replicas of a decoder layer, all distinct: codes from a seeded device
    RNG (uniform words are uniform 3:4 ternary matrices), fp16 row scales
    U[0.01, 0.1], activations per matrix from the host generator."""
    import numpy as np

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    words_per_layer = sum(n * (k // 128) * 5 for _, n, k in shapes)
    codes = torch.randint(-2 ** 31, 2 ** 31, (replicas * words_per_layer,), dtype=torch.int32, device=dev,
                          generator=gen)
    rows_per_layer = sum(n for _, n, _ in shapes)
    scales = (torch.rand(replicas * rows_per_layer, generator=gen, device=dev, dtype=torch.float64) * 0.09
              + 0.01).to(torch.float16)
    g = synth.rng(seed)
    probs = []
    wo = so = 0
    for r in range(replicas):
        for name, n, k in shapes:
            nw = n * (k // 128) * 5
            c = codes[wo:wo + nw]
            s = scales[so:so + n]
            wo += nw
            so += n
            if x_kind == "i8":
                xq, sx, _ = synth.act_absmax_int8(1, k, g)
                x = torch.from_numpy(xq[0]).to(dev)
                xs = torch.from_numpy(sx).to(dev)
                y = torch.empty(n, dtype=torch.float16, device=dev)
            else:
                xb = synth.x_bf16_normal(k, g)
                x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
                xs = None
                y = torch.empty(n, dtype=torch.float32, device=dev)
            probs.append(dict(codes=c, scales=s, x=x, x_scale=xs, acc=None, y=y, n=n, k=k, name=name, replica=r))
    return codes, probs


SETTLE_MS = 80.0


def time_launches(torch, fn, steps, warmup, settle_ms=None):
    """Time `steps` back-to-back calls of fn on the current stream: one HIP event
    pair brackets the whole timed region (events between launches would add
    their own overhead to every launch), plus a wall clock around it with a
    synchronize on both sides.  Returns (mean ms per call from the events,
    wall ms per call).

    Before timing, fn runs `warmup` times and then keeps running until
    `settle_ms` of wall time have passed: after an idle period the GPU's power
    management first lowers the shader clock under this load and needs some
    tens of milliseconds of sustained work to settle (measured with a clock
    probe on MI355X: ~1.6 GHz after the first launches, ~2.3 GHz after
    ~40 ms), so a short warmup would time the transient."""
    stream = torch.cuda.current_stream()
    if settle_ms is None:
        settle_ms = SETTLE_MS
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return a.elapsed_time(b) / steps, wall_ms


def per_launch_us(torch, fn, steps=200):
    """Each of `steps` calls of fn between its own HIP event pair on the
    current stream (call right after time_launches, so the clock has
    settled): p10 / median / p90 of the per-call times in microseconds.  The
    events add a little to each call, so these are upper bounds beside the
    mean that time_launches gives."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return {"p10": round(t[steps // 10], 2), "median": round(t[steps // 2], 2), "p90": round(t[(9 * steps) // 10], 2)}


def per_call_table(torch, probs, shapes, call, x_bytes=1, y_bytes=2, with_sx=True):
    """Per-call latency of each matrix of a layer, rotating over the layer
    replicas in `probs` so that the codes come from HBM, not the last-level
    cache: the mean over 200 back-to-back calls and the per-call
    percentiles."""
    lat = {}
    for name, n, k in shapes:
        sel = [p for p in probs if p["name"] == name]
        it = [0]

        def one():
            p = sel[it[0] % len(sel)]
            it[0] += 1
            call(p)
        mean_ms, _ = time_launches(torch, one, 200, 20)
        us = mean_ms * 1e3
        byts = n * k * 5 / 32 + 2 * n + x_bytes * k + y_bytes * n + (4 if with_sx else 0)
        lat[f"{name}_{n}x{k}"] = {"us_per_call": round(us, 2), "GBps": round(byts / (us * 1e-6) / 1e9, 1),
                                  "per_call_us": per_launch_us(torch, one)}
    return lat


def traffic_from_summary():
    """HBM bytes per launch of the grouped kernel from the committed counter
    summary, or None if absent or taken on a different version of the kernel."""
    if not os.path.exists(COUNTER_SUMMARY):
        return None
    vals = {}
    for line in open(COUNTER_SUMMARY):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_hash") != kernel_hash():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------ cpu oracle ---

def cpu_baseline(torch, probs, shapes, min_seconds=10.0, max_layers=16):
    """The oracle as it stands, one thread, on whole 1B layers (7 matrices
    each, replicas 0, 1, ...) until at least min_seconds of CPU work:
    unpack + exact product + epilogue, per matrix.  The oracle's outputs are
    then compared, bit for bit, with what the timed grouped launch wrote for
    the same problems (`checked`)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import sherry_ref

    per_layer = sum(n * k for _, n, k in shapes)
    done = 0
    dt = 0.0
    checked = {"problems": 0, "rows": 0, "mismatched_rows": 0}
    with threadpool_limits(limits=1):
        for r in range(max_layers):
            layer = [p for p in probs if p["replica"] == r]
            if not layer:
                break
            host = [(p["codes"].cpu().numpy().view(np.uint32), p["scales"].cpu().numpy(), p["n"], p["k"],
                     p["x"].cpu().numpy(), p["x_scale"].cpu().numpy()[0]) for p in layer]
            t0 = time.perf_counter()
            outs = [sherry_ref.gemv_i8(words, sw, n, k, x, sx, np.float16) for words, sw, n, k, x, sx in host]
            dt += time.perf_counter() - t0
            for p, (_, y_ref) in zip(layer, outs):
                y_gpu = p["y"].cpu().numpy()
                checked["problems"] += 1
                checked["rows"] += p["n"]
                checked["mismatched_rows"] += int(np.count_nonzero(y_gpu.view(np.uint16) != y_ref.view(np.uint16)))
            done += 1
            if dt >= min_seconds:
                break
    line = {"value": done * per_layer / dt, "unit": "weights/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} LLaMA-3.2-1B decoder layer(s) (7 matrices, {per_layer} weights each), batch 1, "
                      f"numpy oracle limited to 1 thread, {dt:.1f} s"}
    line["checked"] = dict(checked, what="fp16 outputs of the timed grouped launch against the oracle, bit for bit")
    # the same oracle with the BLAS pool at its default size, on fewer layers
    with threadpool_limits(limits=None):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        done_all, dt_all = 0, 0.0
        for r in range(max_layers):
            layer = [p for p in probs if p["replica"] == r]
            if not layer:
                break
            host = [(p["codes"].cpu().numpy().view(np.uint32), p["scales"].cpu().numpy(), p["n"], p["k"],
                     p["x"].cpu().numpy(), p["x_scale"].cpu().numpy()[0]) for p in layer]
            t0 = time.perf_counter()
            for words, sw, n, k, x, sx in host:
                sherry_ref.gemv_i8(words, sw, n, k, x, sx, np.float16)
            dt_all += time.perf_counter() - t0
            done_all += 1
            if dt_all >= min_seconds / 4:
                break
    line["all_threads"] = {"value": done_all * per_layer / dt_all, "blas_threads": threads,
                           "sample": f"{done_all} layer(s), {dt_all:.1f} s"}
    line["host"] = {"cpus_in_affinity": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    return line


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_per_row(synth, max_seconds=2.0):
    """The oracle of each measured row as it stands, one thread, on a bounded
    synthetic sample of that row's workload (a few seconds in all): the CPU
    rate beside each GPU figure.  Rates are per unit of the row's work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import act_ref, sherry_ref, tern2_ref, tern3_ref

    g = synth.rng(97)
    out = {}

    def timed(fn, reps_max=50):
        t0 = time.perf_counter()
        reps = 0
        while reps < reps_max:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= max_seconds:
                break
        return (time.perf_counter() - t0) / reps

    with threadpool_limits(limits=1):
        words = {k: (synth.random_words(n * k // 128 * 5, g), synth.row_scales(n, g, np.float16), n)
                 for name, n, k in synth.LLAMA32_1B_LAYER if name in ("q", "down")}
        n, k = 2048, 2048
        w, sw, _ = words[2048]
        xq, sx, _ = synth.act_absmax_int8(16, k, g)
        s16 = timed(lambda: sherry_ref.gemm_i8(w, sw, n, k, xq, sx, np.float16))
        out["a7_gemm_m16_q_2048x2048"] = {"s": round(s16, 4), "weights_per_s": n * k / s16}
        xp, sxp, _ = synth.act_absmax_int8(2048, k, g)
        s2048 = timed(lambda: sherry_ref.gemm_i8(w, sw, n, k, xp, sxp, np.float16), reps_max=2)
        out["a8_gemm_m2048_q_2048x2048"] = {"s": round(s2048, 3), "TOPS": 2 * 2048 * n * k / s2048 / 1e12}
        t = synth.ternary_dense(n, k, g)
        w2 = tern2_ref.pack(t)
        x1, s1, _ = synth.act_absmax_int8(1, k, g)
        st = timed(lambda: tern2_ref.gemv_i8(w2, sw, n, k, x1[0], s1[0], np.float16))
        out["a9_tern2_gemv_q_2048x2048"] = {"s": round(st, 4), "weights_per_s": n * k / st}
        t3 = t[:256]
        w3t = tern3_ref.pack(t3)
        st3 = timed(lambda: tern3_ref.gemv_i8(w3t, sw[:256], 256, k, x1[0], s1[0], np.float16), reps_max=5)
        out["f2_tern3_gemv_q_256x2048"] = {"s": round(st3, 4), "weights_per_s": 256 * k / st3}
        n3 = k3 = 3072
        w3 = synth.random_words(n3 * k3 // 128 * 5, g)
        sw3 = synth.row_scales(n3, g, np.float32)
        xb = synth.x_bf16_normal(k3, g)
        sb = timed(lambda: sherry_ref.gemv_bf16(w3, sw3, n3, k3, xb))
        out["a2_a6_bf16_gemv_q_3072x3072"] = {"s": round(sb, 4), "weights_per_s": n3 * k3 / sb}
        xa = synth.x_bf16_normal((16, 2048), g)
        sa = timed(lambda: act_ref.quantize(xa, "bf16"))
        out["f1_act_quant_16x2048_bf16"] = {"s": round(sa, 5), "values_per_s": 16 * 2048 / sa}
        wp = (g.standard_normal((512, 2048)) * 0.02).astype(np.float16)
        spk = timed(lambda: sherry_ref.pack(wp, np.float16), reps_max=2)
        out["a1_pack_512x2048_fp16"] = {"s": round(spk, 3), "weights_per_s": 512 * 2048 / spk}
    out["cores"] = 1
    return out


# ----------------------------------------------------------------- extras ---

def peak_probes(torch, sherry):
    """Measured ceilings beside the published peaks: a 1 GiB streaming read
    (HBM), the int8 matrix-core and v_dot4 rates, and both kinds of work in
    the same wave and in alternate waves.  overlap = t(both) / (t(mfma) +
    t(dot4)): 1.0 when they do not overlap, max / sum when they fully do."""
    dev = torch.device("cuda:0")
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    buf = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    buf.fill_(1)
    mean_ms, _ = time_launches(torch, lambda: sherry.probe_read(buf, sink), 20, 3)
    out = {"read_1GiB_TBps": round((1 << 30) / (mean_ms * 1e-3) / 1e12, 3)}
    del buf
    blocks, iters = 1024, 8192
    t = {}
    ticks = torch.zeros(blocks, 4, dtype=torch.int64, device=dev)
    clock = {}
    for name, mode in (("mfma", sherry.PROBE_MFMA), ("dot4", sherry.PROBE_DOT4), ("same_wave", sherry.PROBE_SAME_WAVE),
                       ("alt_waves", sherry.PROBE_ALT_WAVES), ("mfma32", sherry.PROBE_MFMA32), ("alu", sherry.PROBE_ALU),
                       ("same_wave_alu", sherry.PROBE_SAME_ALU)):
        mean_ms, _ = time_launches(torch, lambda: sherry.probe_rates(mode, iters, blocks, sink), 10, 2, settle_ms=20)
        t[name] = mean_ms
        if name in ("mfma", "dot4", "mfma32"):  # one more launch, recording the shader clock (s_memtime / 100 MHz)
            sherry.probe_clock(mode, iters, blocks, sink, ticks)
            torch.cuda.synchronize()
            tk = ticks.cpu().double()
            ghz = ((tk[:, 1] - tk[:, 0]) / (tk[:, 3] - tk[:, 2]) * 0.1).median().item()
            clock[name] = round(ghz, 3)
    waves = 4 * blocks * iters
    out["mfma_i8_TOPS"] = round(waves * sherry.PROBE_MFMA_OPS / (t["mfma"] * 1e-3) / 1e12, 1)
    out["mfma32_i8_TOPS"] = round(waves * sherry.PROBE_MFMA_OPS / (t["mfma32"] * 1e-3) / 1e12, 1)
    out["dot4_i8_TOPS"] = round(waves * sherry.PROBE_DOT4_OPS / (t["dot4"] * 1e-3) / 1e12, 1)
    # the shader clock while each probe ran, and the rate it implies per clock against the peak's 2.4 GHz: a rate
    # below the spec at full per-clock efficiency is the clock, not the kernel
    out["clock_GHz"] = clock
    if clock.get("mfma"):
        out["mfma_i8_TOPS_at_2p4GHz"] = round(out["mfma_i8_TOPS"] * 2.4 / clock["mfma"], 1)
    if clock.get("mfma32"):
        out["mfma32_i8_TOPS_at_2p4GHz"] = round(out["mfma32_i8_TOPS"] * 2.4 / clock["mfma32"], 1)
    if clock.get("dot4"):
        out["dot4_i8_TOPS_at_2p4GHz"] = round(out["dot4_i8_TOPS"] * 2.4 / clock["dot4"], 1)
    out["ms"] = {k: round(v, 4) for k, v in t.items()}
    out["overlap_same_wave"] = round(t["same_wave"] / (t["mfma"] + t["dot4"]), 3)  # 16 x 16 x 64 products
    out["overlap_alt_waves"] = round(2 * t["alt_waves"] / (t["mfma"] + t["dot4"]), 3)
    # matrix-core products beside plain 32-bit VALU operations (shift, mask, add) in the same wave
    out["overlap_same_wave_alu"] = round(t["same_wave_alu"] / (t["mfma"] + t["alu"]), 3)
    return out


def library_beside(torch, synth, args):
    """Dense products of the installed libraries (through torch) on the same
    shapes, as context: batch 1 with fp16 weights over the 112 replicas
    (seven batched products per step, one per matrix shape, operands
    contiguous), and M = 2048 with int8 (torch._int_mm) and bf16 weights,
    seven calls per layer.  Random data; nothing here is checked."""
    dev = torch.device("cuda:0")
    shapes = synth.LLAMA32_1B_LAYER
    R = args.replicas
    out = {}
    ws = {name: torch.randn(R, n, k, device=dev, dtype=torch.float16) for name, n, k in shapes}
    xs = {name: torch.randn(R, k, 1, device=dev, dtype=torch.float16) for name, n, k in shapes}

    def gemv_step():
        for name, _, _ in shapes:
            torch.bmm(ws[name], xs[name])
    mean_ms, _ = time_launches(torch, gemv_step, 20, 3)
    wbytes = R * sum(2 * n * k for _, n, k in shapes)
    out["dense_fp16_gemv_1b_x%d" % R] = {"ms_per_step": round(mean_ms, 4),
                                         "weights_per_s": R * sum(n * k for _, n, k in shapes) / (mean_ms * 1e-3),
                                         "weight_GBps": round(wbytes / (mean_ms * 1e-3) / 1e9, 1)}
    del ws, xs
    torch.cuda.empty_cache()
    M = 2048
    ops = 2 * M * sum(n * k for _, n, k in shapes)
    for dt in ("int8", "bf16"):
        calls = []
        for name, n, k in shapes:
            if dt == "int8":
                a = torch.randint(-127, 128, (M, k), dtype=torch.int8, device=dev)
                b = torch.randint(-1, 2, (n, k), dtype=torch.int8, device=dev).t()
                calls.append(lambda a=a, b=b: torch._int_mm(a, b))
            else:
                a = torch.randn(M, k, device=dev).to(torch.bfloat16)
                b = torch.randn(k, n, device=dev).to(torch.bfloat16)
                calls.append(lambda a=a, b=b: torch.matmul(a, b))
        try:
            mean_ms, _ = time_launches(torch, lambda: [c() for c in calls], 20, 3)
        except RuntimeError as ex:
            out[f"dense_{dt}_gemm_1b_M2048"] = {"error": str(ex)[:200]}
            continue
        out[f"dense_{dt}_gemm_1b_M2048"] = {"us_per_layer": round(mean_ms * 1e3, 1),
                                            "TOPS": round(ops / (mean_ms * 1e-3) / 1e12, 1)}
        del calls
    return out


def gemm_profile(torch, sherry, synth, probs, args):
    """The grouped GEMM launches alone: one 1B layer at M = 2048 (tiled int8
    MFMA kernel) and every replica at M = 16 (few-token kernel), a few
    launches of each after the clocks settle; one JSON line of their mean
    times."""
    dev = torch.device("cuda:0")
    g = synth.rng(args.seed + 7)
    shapes = synth.LLAMA32_1B_LAYER
    res = {}
    for m, sel, steps in ((2048, [p for p in probs if p["replica"] == 0], 10), (16, probs, 20)):
        xs = {}
        for _, n, k in shapes:
            if k not in xs:
                xq, sx, _ = synth.act_absmax_int8(m, k, g)
                xs[k] = (torch.from_numpy(xq).to(dev), torch.from_numpy(sx).to(dev))
        gp = [dict(codes=p["codes"], scales=p["scales"], x=xs[p["k"]][0], x_scales=xs[p["k"]][1],
                   y=torch.empty(m, p["n"], dtype=torch.float16, device=dev)) for p in sel]
        grouped = sherry.GroupedGemm(gp)
        mean_ms, _ = time_launches(torch, grouped, steps, 3)
        layers = len(sel) // len(shapes)
        ops = 2 * m * layers * sum(n * k for _, n, k in shapes)
        code_bytes = layers * sum(n * k * 5 // 32 for _, n, k in shapes)
        res[f"M{m}"] = {"us_per_launch": round(mean_ms * 1e3, 2), "layers": layers, "tiles": grouped.n_tiles,
                        "TOPS": round(ops / (mean_ms * 1e-3) / 1e12, 1),
                        "code_TBps": round(code_bytes / (mean_ms * 1e-3) / 1e12, 3)}
        if m == 2048:  # the other large-tile kernels on the same launch
            for name, kind in (("decode_once", sherry.PREFILL_DECODE_ONCE), ("tiled32", sherry.PREFILL_TILED32)):
                sherry.set_prefill_kernel(kind)
                mean1, _ = time_launches(torch, grouped, steps, 3)
                sherry.set_prefill_kernel(sherry.PREFILL_TILED)
                res[f"M2048_{name}"] = {"us_per_launch": round(mean1 * 1e3, 2),
                                        "TOPS": round(ops / (mean1 * 1e-3) / 1e12, 1)}
        if m == 2048:  # the 2-bit comparator on the same ternary matrices, same launch shape
            g2 = [dict(q, codes=sherry.tern2_encode(sherry.decode(p["codes"], p["n"], p["k"])))
                  for q, p in zip(gp, sel)]
            grouped2 = sherry.GroupedGemm(g2, tern2=True)
            mean2, _ = time_launches(torch, grouped2, steps, 3)
            res["M2048_tern2"] = {"us_per_launch": round(mean2 * 1e3, 2), "TOPS": round(ops / (mean2 * 1e-3) / 1e12, 1)}
            res["M2048_sherry_over_tern2"] = round(mean2 / mean_ms, 3)
            sherry.set_prefill_kernel(sherry.PREFILL_TILED32)
            mean3, _ = time_launches(torch, grouped2, steps, 3)
            sherry.set_prefill_kernel(sherry.PREFILL_TILED)
            res["M2048_tern2_tiled32"] = {"us_per_launch": round(mean3 * 1e3, 2),
                                          "TOPS": round(ops / (mean3 * 1e-3) / 1e12, 1)}
            del g2, grouped2
        del gp, grouped
    print(json.dumps(res), flush=True)
    return 0


def bf16_gemm_rates(torch, sherry, synth, probs_3b, replicas, seed, ms=(2, 4, 8, 16), steps=20):
    """The bf16 few-token GEMM (matrix cores, fp32 outputs) over every matrix
    of the 3B-layer replicas in `probs_3b`, one grouped launch per token
    count; algorithmic bytes per layer = codes + fp16 row scales + X (2 m k)
    + Y (4 m n)."""
    import numpy as np

    dev = torch.device("cuda:0")
    g = synth.rng(seed)
    shapes = synth.LLAMA32_3B_LAYER
    res = {}
    for m in ms:
        xs = {}
        for _, n, k in shapes:
            if k not in xs:
                xb = synth.x_bf16_normal((m, k), g)
                xs[k] = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        ys = {p["name"]: torch.empty(m, p["n"], dtype=torch.float32, device=dev) for p in probs_3b if p["replica"] == 0}
        gp = [dict(codes=p["codes"], scales=p["scales"], x=xs[p["k"]], y=ys[p["name"]]) for p in probs_3b]
        grouped = sherry.GroupedGemm(gp)
        mean_ms, _ = time_launches(torch, grouped, steps, 3)
        per_layer_ms = mean_ms / replicas
        byts = sum(n * k * 5 // 32 + 2 * n + 2 * m * k + 4 * m * n for _, n, k in shapes)
        flops = 2 * m * sum(n * k for _, n, k in shapes)
        res[f"M{m}"] = {"grouped_us_per_layer": round(per_layer_ms * 1e3, 3), "replicas": replicas,
                        "workgroups": grouped.n_tiles, "GBps": round(byts / (per_layer_ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(byts / (per_layer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "TFLOPs": round(flops / (per_layer_ms * 1e-3) / 1e12, 1)}
        del gp, grouped
    return res


def f4_decode_token(torch, sherry, probs, layers):
    """A 1B token's weight pass as decode runs it: per decoder layer the four
    products in dependency order, x quantized inside each -- q|k|v,
    (attention not run) o, gate|up, down -- over `layers` layers with weights
    of their own (replica l is layer l).  Timed eager as prepared calls, eager
    as plain binding calls (argument checks every call), and replayed from
    one HIP graph holding the whole token (checked against eager first)."""
    dev = torch.device("cuda:0")
    steps, outs, plain = [], [], []
    code_bytes = 0
    for l in range(layers):
        by = {p["name"]: p for p in probs if p["replica"] == l}
        code_bytes += sum(p["n"] * p["k"] * 5 // 32 for p in by.values())
        qkv = (torch.cat([by[nm]["codes"] for nm in ("q", "k", "v")]),
               torch.cat([by[nm]["scales"] for nm in ("q", "k", "v")]))
        gu = (torch.cat([by[nm]["codes"] for nm in ("gate", "up")]),
              torch.cat([by[nm]["scales"] for nm in ("gate", "up")]))
        mats = [qkv, (by["o"]["codes"], by["o"]["scales"]), gu, (by["down"]["codes"], by["down"]["scales"])]
        for (c, sc), k in zip(mats, (2048, 2048, 2048, 8192)):
            x = torch.randn(k, device=dev).to(torch.bfloat16)
            y = torch.empty(sc.numel(), dtype=torch.float16, device=dev)
            steps.append(sherry.PreparedGemvQuant(c, sc, x, out=y))
            plain.append((c, sc, x, y))
            outs.append(y)
    stream = torch.cuda.current_stream().cuda_stream

    def token_prepared():
        for c in steps:
            c(stream)

    def token_prepared_current():  # torch's current stream, for capture
        for c in steps:
            c()

    def token_plain():
        for c, sc, x, y in plain:
            sherry.gemv_quant(c, sc, x, out=y)
    res = {"layers": layers, "launches_per_token": len(steps), "code_bytes_per_token": code_bytes}
    mean_ms, _ = time_launches(torch, token_prepared, 50, 5)
    res["eager_us_per_token"] = round(mean_ms * 1e3, 1)
    mean_ms, _ = time_launches(torch, token_plain, 50, 5)
    res["eager_unprepared_us_per_token"] = round(mean_ms * 1e3, 1)
    gus = graph_time(torch, token_prepared_current, outs, replays=50)
    res["graph_us_per_token"] = gus
    for key in ("eager_us_per_token", "eager_unprepared_us_per_token", "graph_us_per_token"):
        if isinstance(res[key], float):
            res[key.replace("per_token", "per_layer")] = round(res[key] / layers, 2)
    if isinstance(gus, float):
        res["graph_GBps"] = round(code_bytes / (gus * 1e-6) / 1e9, 1)
    return res


def graph_time(torch, fn, outs, replays=200):
    """Mean us per replay of fn captured in a HIP graph, after checking three
    replays (outputs cleared before each) against one eager run; a string
    when capture or the check fails."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            fn()
        for _ in range(3):
            for o in outs:
                o.zero_()
            graph.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(o, r) for o, r in zip(outs, ref)):
                return "replay mismatch"
        mean_ms, _ = time_launches(torch, graph.replay, replays, 20)
        return round(mean_ms * 1e3, 2)
    except RuntimeError as e:  # capture not available: report, do not fail the run
        return f"capture failed: {e}"[:120]


def extras(torch, sherry, synth, probs_1b, codes_1b, args):
    import numpy as np

    out = {}
    dev = torch.device("cuda:0")
    shapes_1b = synth.LLAMA32_1B_LAYER
    R = args.replicas

    # per-call latency of single matrices, rotating over replicas
    out["per_call_gemv_1b"] = per_call_table(
        torch, probs_1b, shapes_1b, lambda p: sherry.gemv(p["codes"], p["scales"], p["x"], p["x_scale"], out=p["y"]))

    # the same grouped launch over 4x the replicas: time per launch grows by
    # the marginal cost per replica, so the fixed per-launch cost (start-up
    # and drain, a few microseconds) weighs 4x less
    R4 = 4 * R
    codes4, probs4 = build_layer_replicas(torch, sherry, synth, shapes_1b, R4, args.seed + 11)
    g4 = sherry.GroupedGemv(probs4)
    mean_ms, _ = time_launches(torch, g4, max(20, args.steps // 4), args.warmup)
    b4 = R4 * layer_bytes(shapes_1b)
    out[f"gemv_grouped_1b_x{R4}"] = {"ms_per_launch": round(mean_ms, 4), "GBps": round(b4 / (mean_ms * 1e-3) / 1e9, 1),
                                     "frac_hbm": round(b4 / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del g4, probs4, codes4
    torch.cuda.empty_cache()

    # 2-bit dense-ternary comparator on the same ternary matrices
    t2_codes = []
    probs_t2 = []
    for p in probs_1b:
        t = sherry.decode(p["codes"], p["n"], p["k"])
        c2 = sherry.tern2_encode(t)
        del t
        t2_codes.append(c2)
        q = dict(p)
        q["codes"] = c2
        probs_t2.append(q)
    torch.cuda.synchronize()
    g2 = sherry.GroupedGemv(probs_t2, tern2=True)
    mean_ms, wall_ms = time_launches(torch, g2, args.steps, args.warmup)
    weights = R * sum(n * k for _, n, k in shapes_1b)
    bytes2 = R * (sum(n * k // 4 + 2 * n + k + 2 * n + 4 for _, n, k in shapes_1b))
    out["tern2_grouped_1b"] = {"ms_per_launch": round(mean_ms, 4), "weights_per_s": weights / (mean_ms * 1e-3),
                               "GBps": round(bytes2 / (mean_ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(bytes2 / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # per call; GBps on the 2-bit bytes (8/5 of the 3:4 codes)
    t2lat = per_call_table(
        torch, probs_t2, shapes_1b, lambda p: sherry.tern2_gemv(p["codes"], p["scales"], p["x"], p["x_scale"], out=p["y"]))
    for (name, n, k), v in zip(shapes_1b, t2lat.values()):
        v["GBps"] = round((n * k / 4 + 2 * n + k + 2 * n + 4) / (v["us_per_call"] * 1e-6) / 1e9, 1)
    out["per_call_tern2_gemv_1b"] = t2lat
    # same grouped launch on the 1.25-bit codes, for the ratio
    del g2, probs_t2, t2_codes
    torch.cuda.empty_cache()

    # 1.67-bit comparator (three weights in five bits) on the same matrices
    t3_codes = []
    probs_t3 = []
    for p in probs_1b:
        t = sherry.decode(p["codes"], p["n"], p["k"])
        c3 = sherry.tern3_encode(t)
        del t
        t3_codes.append(c3)
        q = dict(p)
        q["codes"] = c3
        probs_t3.append(q)
    torch.cuda.synchronize()
    g3 = sherry.GroupedGemv(probs_t3, tern3=True)
    mean_ms, wall_ms = time_launches(torch, g3, args.steps, args.warmup)
    bytes3 = R * (sum(sherry.tern3_packed_bytes(n, k) + 2 * n + k + 2 * n + 4 for _, n, k in shapes_1b))
    out["tern3_grouped_1b"] = {"ms_per_launch": round(mean_ms, 4), "weights_per_s": weights / (mean_ms * 1e-3),
                               "GBps": round(bytes3 / (mean_ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(bytes3 / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del g3, probs_t3, t3_codes
    torch.cuda.empty_cache()

    # bf16 activations on the 3B layer (fp32 accumulation), 72 replicas
    shapes_3b = synth.LLAMA32_3B_LAYER
    R3 = max(1, int(round(R * 72 / 112)))
    codes_3b, probs_3b = build_layer_replicas(torch, sherry, synth, shapes_3b, R3, args.seed + 1, x_kind="bf16")
    g3 = sherry.GroupedGemv(probs_3b)
    mean_ms, _ = time_launches(torch, g3, args.steps, args.warmup)
    b3 = R3 * layer_bytes(shapes_3b, x_bytes_per_elem=2, y_bytes=4, with_sx=False)
    w3 = R3 * sum(n * k for _, n, k in shapes_3b)
    out["bf16_grouped_3b"] = {"replicas": R3, "ms_per_launch": round(mean_ms, 4),
                              "weights_per_s": w3 / (mean_ms * 1e-3),
                              "GBps": round(b3 / (mean_ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(b3 / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    out["per_call_gemv_bf16_3b"] = per_call_table(
        torch, probs_3b, shapes_3b, lambda p: sherry.gemv(p["codes"], p["scales"], p["x"], None, out_dtype=torch.float32,
                                                          out=p["y"]),
        x_bytes=2, y_bytes=4, with_sx=False)
    # the same launch on the matrix cores (sherry_gemv_plan_mfma)
    g3m = sherry.GroupedGemv(probs_3b, mfma=True)
    mean_ms, _ = time_launches(torch, g3m, args.steps, args.warmup)
    out["bf16_grouped_3b_mfma"] = {"replicas": R3, "ms_per_launch": round(mean_ms, 4),
                                   "weights_per_s": w3 / (mean_ms * 1e-3),
                                   "GBps": round(b3 / (mean_ms * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(b3 / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # bf16 x for a few tokens on the matrix cores: every matrix of the 72
    # replicas in one grouped launch per token count
    out["gemm_bf16_3b_layer"] = bf16_gemm_rates(torch, sherry, synth, probs_3b, R3, args.seed + 5)
    del g3, g3m, probs_3b, codes_3b
    torch.cuda.empty_cache()

    # M-token GEMM on the 1B layer: small batch (HBM-bound) and prefill (MFMA-bound)
    g = synth.rng(args.seed + 7)
    gemm = {}
    layer0 = [p for p in probs_1b if p["replica"] < 16]

    # prefill, 2048 tokens: the layer's seven matrices in one grouped launch,
    # and the 2-bit comparator on the same ternary matrices
    m = 2048
    xs = {}
    for _, n, k in shapes_1b:
        if k not in xs:
            xq, sx, _ = synth.act_absmax_int8(m, k, g)
            xs[k] = (torch.from_numpy(xq).to(dev), torch.from_numpy(sx).to(dev))
    rep0 = [p for p in probs_1b if p["replica"] == 0]
    ops = 2 * m * sum(n * k for _, n, k in shapes_1b)
    for label, tern2 in (("M2048_grouped", False), ("M2048_grouped_tern2", True)):
        gp = []
        for p in rep0:
            codes = p["codes"]
            if tern2:
                codes = sherry.tern2_encode(sherry.decode(p["codes"], p["n"], p["k"]))
            x, sx = xs[p["k"]]
            gp.append(dict(codes=codes, scales=p["scales"], x=x, x_scales=sx,
                           y=torch.empty(m, p["n"], dtype=torch.float16, device=dev)))
        grouped = sherry.GroupedGemm(gp, tern2=tern2)
        mean_ms, _ = time_launches(torch, grouped, 20, 3)
        gemm[label] = {"us_per_layer": round(mean_ms * 1e3, 2), "workgroups": grouped.n_tiles,
                       "TOPS": round(ops / (mean_ms * 1e-3) / 1e12, 2),
                       "frac_int8_peak": round(ops / (mean_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
        del gp, grouped
    gemm["M2048_sherry_over_tern2"] = round(gemm["M2048_grouped_tern2"]["us_per_layer"] /
                                            gemm["M2048_grouped"]["us_per_layer"], 3)
    torch.cuda.empty_cache()

    # a few tokens (small-batch decode): every matrix of all R replicas in one
    # grouped launch (few-token kernel, HBM-bound), and, for latency, one
    # layer's seven matrices as separate calls
    for m in (2, 4, 8, 16):
        xs = {}
        for _, n, k in shapes_1b:
            if k not in xs:
                xq, sx, _ = synth.act_absmax_int8(m, k, g)
                xs[k] = (torch.from_numpy(xq).to(dev), torch.from_numpy(sx).to(dev))
        ys = {p["name"]: torch.empty(m, p["n"], dtype=torch.float16, device=dev) for p in rep0}
        gp = [dict(codes=p["codes"], scales=p["scales"], x=xs[p["k"]][0], x_scales=xs[p["k"]][1], y=ys[p["name"]])
              for p in probs_1b]
        grouped = sherry.GroupedGemm(gp)
        mean_ms, _ = time_launches(torch, grouped, 50, 5)
        per_layer_ms = mean_ms / R
        ops = 2 * m * sum(n * k for _, n, k in shapes_1b)
        byts = sum(n * k * 5 // 32 + 2 * n + m * k + 2 * m * n + 4 * m for _, n, k in shapes_1b)

        def layer_pass():
            for p in rep0:
                x, sx = xs[p["k"]]
                sherry.gemm(p["codes"], p["scales"], x, sx, out=ys[p["name"]])
        call_ms, _ = time_launches(torch, layer_pass, 20, 2)
        gemm[f"M{m}"] = {"grouped_us_per_layer": round(per_layer_ms * 1e3, 3), "replicas": R,
                         "GBps": round(byts / (per_layer_ms * 1e-3) / 1e9, 1),
                         "frac_hbm": round(byts / (per_layer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "TOPS": round(ops / (per_layer_ms * 1e-3) / 1e12, 2),
                         "us_per_layer_7_calls": round(call_ms * 1e3, 2)}
        del gp, grouped
    out["gemm_1b_layer"] = gemm

    # activation quantization, and the decode step it feeds for one 1B layer:
    # bf16 x -> int8 on the GPU, one product over the concatenated q | k | v
    # rows (shared x), then again for gate | up -- as four launches
    # (quantize, product, quantize, product) and as two products that
    # quantize x themselves; eager, and replayed from a HIP graph (checked
    # against eager first)
    act = {}
    for label, m in (("x_1x2048_bf16", 1), ("x_2048x2048_bf16", 2048), ("x_1x8192_bf16", 1)):
        k = 8192 if "8192" in label else 2048
        xb = torch.randn(m, k, device=dev).to(torch.bfloat16)
        mean_ms, _ = time_launches(torch, lambda: sherry.act_quant(xb), 100, 10)
        act[label] = {"us": round(mean_ms * 1e3, 2), "GBps": round(3 * m * k / (mean_ms * 1e-3) / 1e9, 1)}
    by = {p["name"]: p for p in rep0}
    qkv = (torch.cat([by[nm]["codes"] for nm in ("q", "k", "v")]), torch.cat([by[nm]["scales"] for nm in ("q", "k", "v")]))
    gu = (torch.cat([by[nm]["codes"] for nm in ("gate", "up")]), torch.cat([by[nm]["scales"] for nm in ("gate", "up")]))
    x1 = torch.randn(2048, device=dev).to(torch.bfloat16)
    x2 = torch.randn(2048, device=dev).to(torch.bfloat16)
    y_qkv = torch.empty(qkv[1].numel(), dtype=torch.float16, device=dev)
    y_gu = torch.empty(gu[1].numel(), dtype=torch.float16, device=dev)

    def decode_step():
        q1, s1 = sherry.act_quant(x1)
        sherry.gemv(qkv[0], qkv[1], q1, s1, out=y_qkv)
        q2, s2 = sherry.act_quant(x2)
        sherry.gemv(gu[0], gu[1], q2, s2, out=y_gu)

    def decode_step_fused():  # x quantized inside the products: two launches
        sherry.gemv_quant(qkv[0], qkv[1], x1, out=y_qkv)
        sherry.gemv_quant(gu[0], gu[1], x2, out=y_gu)

    for label, fn in (("decode_step", decode_step), ("decode_step_fused_quant", decode_step_fused)):
        mean_ms, _ = time_launches(torch, fn, 200, 20)
        act[f"{label}_us"] = round(mean_ms * 1e3, 2)
        act[f"{label}_graph_us"] = graph_time(torch, fn, (y_qkv, y_gu))
    act["decode_step_code_bytes"] = int(qkv[0].numel() * 4 + gu[0].numel() * 4)
    out["act_quant_and_fused_projections"] = act

    out["f4_decode_token_1b"] = f4_decode_token(torch, sherry, probs_1b, min(16, R))
    out["library_beside"] = library_beside(torch, synth, args)
    out["peak_probes"] = peak_probes(torch, sherry)

    # packer: fp16 weights of one 1B layer -> codes + fp16 scales
    wts = {}
    for name, n, k in shapes_1b:
        wts[name] = (torch.randn(n, k, device=dev, dtype=torch.float32) * 0.02).to(torch.float16)
    def pack_all():
        for name, _, _ in shapes_1b:
            sherry.pack(wts[name], torch.float16)
    mean_ms, _ = time_launches(torch, pack_all, 3, 1)
    wl = sum(n * k for _, n, k in shapes_1b)
    out["pack_1b_layer_fp16"] = {"ms": round(mean_ms, 3), "weights_per_s": wl / (mean_ms * 1e-3)}
    return out


# ------------------------------------------------------------ counters ---

def summarize_counters(fetch_dir, write_dir):
    """rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of `bench.py --copy-probe`:
    per-dispatch KiB of the grouped GEMV and of the 1 GiB negation (reads
    1 GiB, writes 1 GiB), the factor bytes / counter that calibrates each
    counter, and the scaled HBM bytes per grouped launch."""
    import csv

    def read(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row.get("Kernel_Name", "")
                    rows.setdefault(name, []).append(float(row["Counter_Value"]))
        return rows

    fetch, write = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")

    def pick(rows, pat):
        vals = [v for k, vs in rows.items() if pat in k for v in vs]
        return statistics.median(vals) if vals else None

    g_f, g_w = pick(fetch, GEMV_KERNEL_PATTERNS[0]), pick(write, GEMV_KERNEL_PATTERNS[0])
    c_f, c_w = pick(fetch, "neg_kernel"), pick(write, "neg_kernel")
    gib = float(1 << 30)
    f_fac = gib / (c_f * 1024) if c_f else None
    w_fac = gib / (c_w * 1024) if c_w else None
    res = {"grouped_fetch_kib": g_f, "grouped_write_kib": g_w, "copy_fetch_kib": c_f, "copy_write_kib": c_w,
           "fetch_factor": f_fac, "write_factor": w_fac}
    if g_f and f_fac and g_w is not None and w_fac:
        res["hbm_bytes_per_launch"] = int(g_f * 1024 * f_fac + g_w * 1024 * w_fac)
    print(json.dumps(res))
    return res


# the grouped GEMV's kernel
GEMV_KERNEL_PATTERNS = ("gemv_i8_grouped_kernel",)


def summarize_pmc(dirs, replicas):
    """rocprofv3 --pmc runs of `bench.py --no-extras` (one counter set per
    directory): the median per dispatch of every counter the grouped GEMV
    dispatches carry, and the instruction counters per 128-weight group per
    lane (wave instructions x 64 lanes / groups of the launch: each lane walks
    one group per row)."""
    import csv

    layer_groups = sum(n * k // 128 for n, k in
                       ((2048, 2048), (512, 2048), (512, 2048), (2048, 2048), (8192, 2048), (8192, 2048), (2048, 8192)))
    groups = replicas * layer_groups
    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if not any(p in row.get("Kernel_Name", "") for p in GEMV_KERNEL_PATTERNS):
                        continue
                    vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    res = {"groups_per_launch": groups, "per_dispatch_median": {}, "per_group_lane": {}}
    for name, v in sorted(vals.items()):
        med = statistics.median(v)
        res["per_dispatch_median"][name] = med
        if name.startswith("SQ_INSTS") or name in ("SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_VALU"):
            res["per_group_lane"][name] = round(med * 64 / groups, 2)
    print(json.dumps(res))
    return res


def summarize_trace(trace_dir, timed):
    """A rocprofv3 --kernel-trace run of the default benchmark: the grouped
    GEMV's duration over all its dispatches (warm-up and clock settling
    included) and over the last `timed` dispatches, which are the timed
    launches when the run had no extras (--no-extras)."""
    import csv

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name", "")
                if any(p in name for p in GEMV_KERNEL_PATTERNS):
                    rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]) - int(row["Start_Timestamp"]),
                                 name))
    rows.sort()
    durs = [d / 1e3 for _, d, _ in rows]
    tail = durs[-timed:]
    res = {"kernel": rows[-1][2] if rows else None, "dispatches": len(durs),
           "all_mean_us": round(statistics.mean(durs), 2) if durs else None,
           "timed": len(tail), "timed_mean_us": round(statistics.mean(tail), 2) if tail else None,
           "timed_min_us": round(min(tail), 2) if tail else None, "timed_max_us": round(max(tail), 2) if tail else None}
    if tail:
        layer = sum(n * k * 5 // 32 + 2 * n + k + 2 * n + 4 for n, k in
                    ((2048, 2048), (512, 2048), (512, 2048), (2048, 2048), (8192, 2048), (8192, 2048), (2048, 8192)))
        res["timed_frac_hbm_112_layers"] = round(112 * layer / (res["timed_mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    print(json.dumps(res))
    return res


# ------------------------------------------------------------------- main ---

def main(argv=None):
    global SETTLE_MS
    args = parse_args(argv)
    SETTLE_MS = args.settle_ms
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.replicas)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps)
        return 0
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is described in the design notes but not measured.", file=sys.stderr)
        return 2
    import torch

    import synth
    from ultra_bit_weight_amd import sherry

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sherry.load()
    torch.cuda.set_device(0)
    if args.probes:
        print(json.dumps(peak_probes(torch, sherry)), flush=True)
        return 0
    if args.bf16_gemm_profile:
        R3 = max(1, int(round(args.replicas * 72 / 112)))
        _, probs_3b = build_layer_replicas(torch, sherry, synth, synth.LLAMA32_3B_LAYER, R3, args.seed + 1,
                                           x_kind="bf16")
        print(json.dumps(bf16_gemm_rates(torch, sherry, synth, probs_3b, R3, args.seed + 5)), flush=True)
        return 0
    shapes = synth.LLAMA32_1B_LAYER
    R = args.replicas
    codes, probs = build_layer_replicas(torch, sherry, synth, shapes, R, args.seed)
    if args.gemm_profile:
        return gemm_profile(torch, sherry, synth, probs, args)
    if args.f4_profile:
        print(json.dumps(f4_decode_token(torch, sherry, probs, min(16, R))), flush=True)
        return 0
    grouped = sherry.GroupedGemv(probs)
    torch.cuda.synchronize()
    print(f"# built {R} replicas of the 1B layer: {codes.numel() * 4 / 1e9:.3f} GB of codes, "
          f"{grouped.n_tiles} workgroup tiles",
          file=sys.stderr, flush=True)

    if args.copy_probe:
        # plain streaming kernel of known traffic: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    mean_ms, wall_ms = time_launches(torch, grouped, args.steps, args.warmup)
    weights_per_step = R * sum(n * k for _, n, k in shapes)
    alg_bytes = R * layer_bytes(shapes)
    value = weights_per_step / (wall_ms * 1e-3)
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    print(f"# grouped GEMV: {mean_ms:.4f} ms per launch (events), {wall_ms:.4f} ms per step (wall)",
          file=sys.stderr, flush=True)

    traffic = traffic_from_summary()
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "LLaMA-3.2-1B decoder-layer GEMVs (q 2048x2048, k/v 512x2048, o 2048x2048, "
                        "gate/up 8192x2048, down 2048x8192), batch 1, int8 activations with per-token scale, "
                        f"fp16 row scales and outputs; {R} distinct layer replicas per step in one grouped launch",
            "replicas": R,
            "weights_per_step": weights_per_step,
            "code_bytes_per_step": R * sum(n * k * 5 // 32 for _, n, k in shapes),
            "bits_per_weight": 1.25,
            "kernel": "gemv_i8_grouped_kernel<Sherry3of4>",
            "workgroups": grouped.n_tiles,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "launch_ms": round(mean_ms, 4),
        },
    }
    mismatch = False
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, probs, shapes)
        chk = line["cpu_baseline"]["checked"]
        line["checked"] = {k: chk[k] for k in ("problems", "rows", "mismatched_rows")}
        mismatch = chk["mismatched_rows"] != 0
        if not args.no_extras:
            line["cpu_baseline"]["per_row"] = cpu_baseline_per_row(synth)
        print(f"# cpu oracle: {line['cpu_baseline']['value']:.3e} weights/s; timed launch vs oracle: "
              f"{chk['problems']} problems, {chk['rows']} rows, {chk['mismatched_rows']} mismatched",
              file=sys.stderr, flush=True)
    if not args.no_extras:
        ex = extras(torch, sherry, synth, probs, codes, args)
        t2 = ex.get("tern2_grouped_1b")
        if t2:
            ex["sherry_over_tern2_speedup"] = round(t2["ms_per_launch"] / mean_ms, 3)
        t3 = ex.get("tern3_grouped_1b")
        if t3:
            ex["sherry_over_tern3_speedup"] = round(t3["ms_per_launch"] / mean_ms, 3)
        dense = ex.get("library_beside", {}).get("dense_fp16_gemv_1b_x%d" % args.replicas)
        if dense:
            ex["sherry_over_dense_fp16_gemv_speedup"] = round(dense["ms_per_step"] / mean_ms, 2)
        line["extras"] = ex
    print(json.dumps(line), flush=True)
    if mismatch:
        print("bench.py: the timed launch's outputs differ from the oracle", file=sys.stderr, flush=True)
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
