"""Benchmark of the few-row draft-head vocabulary projection on one MI355X.

One step = one pass of the whole projection over one batch: dh_draft on the FP8 E4M3 head
with E8M0 32x32 block scales (H=5120, V=129280, one activation row; --rows 5, 10, 15 or 16
takes the row-sweep workload's head and rows instead): the GEMV (fp32 logits kept) then the
top-64 and argmax.  Inputs are resident in HBM before timing;
three copies of the FP8 head are rotated so that no step finds the head in the 256 MB
Infinity Cache.  The head is stored tiled for the GEMV (dh_tile_head, once at load: the same
bytes re-arranged so that each wave load reads 1 KiB of whole lines); the row-major head's
GEMV time is reported beside it.

Printed: one JSON line.  value = algorithmic HBM bytes of a step (head codes + scales +
activations + fp32 logits written) / time per step, in GB/s.  Extra fields give the row
sweep (1/5/10/15/16 rows) per entry point (per-call events and back-to-back means), the
bf16 head, the two-stage head (FP8 row scale + dense bf16 rescore of 512 candidates), the
roofline of the GEMV kernel (HIP events around K back-to-back launches on the launching
stream, a timed region of its own) and the CPU oracle timed on the host's cores.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
NCOPY = 3
# HBM traffic of the GEMV launch, from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE)
# calibrated on a plain copy kernel; valid only for the kernel source it was taken on.
def traffic_file(rows):
    return os.path.join(ROOT, "profiles", f"gemv_fp8_block32_R{rows}_H5120_V129280_traffic.txt")



KERNEL_SOURCES = [os.path.join(ROOT, "few_row_vocab_amd", "csrc", f)
                  for f in ("gemv.hip", "dh_internal.h", "launch.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats_us(times_ms):
    t = np.sort(np.asarray(times_ms)) * 1e3
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)),
            "p90": float(np.percentile(t, 90)), "n": int(t.size)}


def gemv_source_hash():
    """Hash of the GEMV kernel's code: its sources with comments and whitespace removed, so
    that a comment edit does not void counters taken on the same code."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(rows):
    """Bytes per GEMV launch from the committed counter summary for this row count, or None
    when there is none or when the kernel's source has changed since the counters were
    taken."""
    try:
        text = open(traffic_file(rows)).read()
    except OSError:
        return None
    src = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    if not src or not val or src.group(1) != gemv_source_hash():
        return None
    return int(val.group(1))


def gemv_kernel_name(fmt_code, H, tiled=True):
    """The template instance the library launches for this head width (up to 8192) and up to
    16 rows (its rule for the per-wave K blocks and the unguarded tile loop; one K chunk, not
    split), as rocprofv3 names it."""
    nkb = (H + 63) // 64
    kbw = -(-nkb // 16)
    vw = 2 if fmt_code == 0 and kbw == 5 else 1        # bf16 tiles of 5 blocks: 8 waves
    full = H % 64 == 0 and nkb % (vw * kbw) == 0
    tf = lambda b: "true" if b else "false"
    return f"gemv_kernel<{fmt_code}, {kbw}, {tf(full)}, 1, 1, {vw}, {tf(tiled)}, false, false>"


def copy_calibration():
    """A plain device-to-device copy of known size, run under the same counters as the
    GEMV to turn FETCH_SIZE / WRITE_SIZE into bytes."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes 3 times")


def copy_ceiling(torch):
    """Practical bandwidth figures for the same device from library kernels: torch's 1 GiB
    device copy (read + write bytes) and a 2 GiB float32 sum (a streaming read), each over
    back-to-back calls."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    tc = back_to_back_us(lambda i: dst.copy_(src), 20)
    del src, dst
    big = torch.ones(2 * n // 4, dtype=torch.float32, device="cuda")
    ts = back_to_back_us(lambda i: big.sum(), 20)
    del big
    return {"copy_bytes": 2 * n, "copy_us": tc, "copy_GBps": round(2 * n / (tc * 1e-6) / 1e9, 1),
            "sum_read_bytes": 2 * n, "sum_us": ts,
            "sum_read_GBps": round(2 * n / (ts * 1e-6) / 1e9, 1)}


def algorithmic_bytes(fmt, V, H, R):
    w = V * H * (2 if fmt == "bf16" else 1)
    s = ((V + 31) // 32) * (H // 32) if fmt == "fp8_block32" else (V * 4 if fmt == "fp8_row" else 0)
    return w + s + R * H * 2 + R * V * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calls", type=int, default=50, help="timed calls per sweep entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="main step only (for profiling)")
    ap.add_argument("--rows", type=int, default=1, choices=[1, 5, 10, 15, 16],
                    help="activation rows of the timed step: 1 is the one-row FP8 block "
                         "workload, the others the row-sweep workload's first rows")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--only", choices=["subset", "lowrank", "twostage", "widelinear", "topk"],
                    help="only the draft-vocabulary subset comparison, the low-rank "
                         "two-stage head, the two-stage head, the wide linear or the "
                         "standalone top-k (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the projection "
              "shards by vocabulary rows across GPUs, which is a design note here, not "
              "something this benchmark runs.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import synth
    from few_row_vocab_amd import dh

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only == "subset":
        print(json.dumps({"subset_head": subset_sweep(dh, torch, args.calls)}), flush=True)
        return
    if args.only == "lowrank":
        print(json.dumps({"lowrank_two_stage": lowrank_sweep(dh, torch, args.calls)}),
              flush=True)
        return
    if args.only == "topk":
        print(json.dumps({"topk": topk_sweep(dh, torch, args.calls)}), flush=True)
        return
    if args.only == "widelinear":
        print(json.dumps({"wide_linear": wide_linear(dh, torch, args.calls)}), flush=True)
        return
    if args.only == "twostage":
        c = synth.CONFIGS["row_sweep"]
        wd = torch.from_numpy(synth.head_bf16("row_sweep").view(np.int16)).to(dev)
        xd = torch.from_numpy(synth.activations("row_sweep", 16).view(np.int16)).to(dev)
        print(json.dumps({"two_stage": two_stage_sweep(dh, torch, wd, xd, c["V"], c["H"],
                                                       args.calls)}), flush=True)
        return
    R = args.rows
    name = "fp8_block_1row" if R == 1 else "row_sweep"
    c = synth.CONFIGS[name]
    V, H, K = c["V"], c["H"], 64

    t0 = time.time()
    w = synth.head_bf16(name)
    x = synth.activations(name, R)
    log(f"generated {V}x{H} head in {time.time() - t0:.1f}s")
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    rm_heads = []
    for i in range(NCOPY):
        codes, scale = dh.quantize(wd, dh.FP8_BLOCK32)
        rm_heads.append(dh.Head(dh.FP8_BLOCK32, codes, scale))
    heads = [dh.tile(h) for h in rm_heads]             # load time: the tiled copies
    torch.cuda.synchronize()
    te = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    te[0].record()
    dh.tile(rm_heads[0])
    te[1].record()
    torch.cuda.synchronize()
    tile_ms = te[0].elapsed_time(te[1])
    # quantization time (load-time prep; the pages quote 0.2 s on 16 CPU workers)
    qe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    qe[0].record()
    dh.quantize(wd, dh.FP8_BLOCK32)
    qe[1].record()
    torch.cuda.synchronize()
    quant_ms = qe[0].elapsed_time(qe[1])
    # the same quantization written straight into the tiled layout
    qe[0].record()
    dh.quantize(wd, dh.FP8_BLOCK32 | dh.TILED)
    qe[1].record()
    torch.cuda.synchronize()
    quant_tiled_ms = qe[0].elapsed_time(qe[1])

    logits = torch.empty((R, V), dtype=torch.float32, device=dev)
    ids = torch.empty((R, K), dtype=torch.int32, device=dev)
    vals = torch.empty((R, K), dtype=torch.float32, device=dev)
    am = torch.empty((R,), dtype=torch.int32, device=dev)
    ws = dh.workspace(R, V, K)

    out_bufs = {"ids": ids, "vals": vals, "draft": am, "logits": logits}

    def step(i):
        # one pass of the whole projection: dh_draft = the GEMV (logits kept) + the top-k
        dh.draft(heads[i % NCOPY], xd, K, ws=ws, out=out_bufs)

    # Device warm-up before the W warm-up steps: the first ~50 steps after start-up run about
    # 30% slower while the clocks ramp, so ~20 ms of steps go first, untimed.
    t_end = time.time() + 0.02
    i = 0
    while time.time() < t_end or i < 100:
        step(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed region: K steps back to back, nothing else on the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    step_bytes = algorithmic_bytes("fp8_block32", V, H, R)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # The GEMV's own duration, in a second timed region: K launches of it back to back on
    # the same stream between two HIP events (an event between kernels costs the stream a
    # few microseconds, so none sits between launches or inside the headline region).
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record()
    for i in range(args.steps):
        dh.gemv(heads[i % NCOPY], xd, logits)
    g1.record()
    torch.cuda.synchronize()
    gemv_avg_ms = g0.elapsed_time(g1) / args.steps
    achieved = step_bytes / (gemv_avg_ms * 1e-3) / 1e9
    # the same GEMV from the row-major head (not the benchmarked layout), for comparison
    rm_us = back_to_back_us(lambda i: dh.gemv(rm_heads[i % NCOPY], xd, logits), args.steps)
    # the device's practical streaming-read bandwidth: dh_stream_read over the same tiled head
    # bytes (the three copies rotated), read the way the GEMV reads them
    sink = torch.empty((dh.STREAM_SINK_WORDS,), dtype=torch.int32, device=dev)
    sr_bytes = heads[0].weight.numel()
    sr_us = back_to_back_us(lambda i: dh.stream_read(heads[i % NCOPY].weight, sink),
                            args.steps)
    sr_gbps = sr_bytes / (sr_us * 1e-6) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us, gemv {gemv_avg_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s); row-major head gemv {rm_us:.1f} us; stream read "
        f"{sr_gbps:.0f} GB/s")

    out = {
        "metric": "draft-head µs/call and achieved HBM GB/s (FP8 head, 1/5/10/16 rows)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2), "rows_per_s": round(R / (ms_per_step * 1e-3), 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) head quantized to FP8 on the GPU, N(0,1) rows)",
        "config": {"workload": f"FP8 E4M3 head with E8M0 32x32 block scales, H={H}, V={V}, "
                               f"{R} activation row{'s' if R > 1 else ''}, dh_draft: GEMV (fp32 logits kept) + "
                               f"top-{K} and argmax",
                   "H": H, "V": V, "rows": R, "k": K, "format": "fp8_block32",
                   "layout": "tiled (dh_tile_head at load)",
                   "head_copies_rotated": NCOPY, "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(R),
                     "kernel": gemv_kernel_name(dh.FP8_BLOCK32, H),
                     "kernel_us": round(gemv_avg_ms * 1e3, 2),
                     "algorithmic_bytes": step_bytes, "kernel_source": gemv_source_hash()},
        "stream_read": {"bytes": sr_bytes, "us": sr_us, "GBps": round(sr_gbps, 1),
                        "frac_of_8TBps": round(sr_gbps / PEAK_HBM_GBPS, 4),
                        "gemv_frac_of_stream_read": round(achieved / sr_gbps, 4),
                        "kernel": "dh_stream_read (1 KiB non-temporal loads, 32 KiB in "
                                  "flight per CU)"},
        "row_major_head_gemv": {"us": rm_us,
                                "GBps": round(step_bytes / (rm_us * 1e-6) / 1e9, 1),
                                "kernel": gemv_kernel_name(dh.FP8_BLOCK32, H, tiled=False)},
        "quantize_fp8_block32_ms": round(quant_ms, 3),
        "tile_head_ms": round(tile_ms, 3),
        "quantize_fp8_block32_tiled_ms": round(quant_tiled_ms, 3),
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, V, H, R, K)
    if not args.quick:
        # the row sweep has a workload of its own (its head and 16 activation rows)
        del heads, rm_heads, logits, ids, vals, am, ws, out_bufs, wd, xd
        torch.cuda.empty_cache()
        sw = "row_sweep"
        wd = torch.from_numpy(synth.head_bf16(sw).view(np.int16)).to(dev)
        xd = torch.from_numpy(synth.activations(sw, 16).view(np.int16)).to(dev)
        heads = [dh.Head(dh.FP8_BLOCK32, *dh.quantize(wd, dh.FP8_BLOCK32)) for _ in range(NCOPY)]
        out["sweep"] = sweep(dh, torch, heads, wd, xd, V, H, K, args.calls)
        del heads, wd, xd
        torch.cuda.empty_cache()
        out["edge_shape"] = edge_shape(dh, torch, args.calls)
        out["subset_head"] = subset_sweep(dh, torch, args.calls)
        out["wide_linear"] = wide_linear(dh, torch, args.calls)
        out["lowrank_two_stage"] = lowrank_sweep(dh, torch, args.calls)
        out["topk_standalone"] = topk_sweep(dh, torch, args.calls)
        out["device_ceiling"] = copy_ceiling(torch)
    print(json.dumps(out), flush=True)


def back_to_back_us(fn, n, warm=3):
    """Mean time of one call when n calls run back to back between two events."""
    import torch
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / n, 2)


def graph_us(fn, n, replays=5):
    """Mean time of one call inside a HIP graph of n captured calls (no host launch cost):
    for kernels shorter than the binding's own per-call host time."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    g, side = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) * 1e3 / (n * replays), 2)


def timed(fn, n, warm=3):
    import torch
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def sweep(dh, torch, rm_heads, wd, xd, V, H, K, n):
    """The row sweep on tiled heads (FP8 and bf16), with the row-major heads' GEMV at 1 and
    16 rows beside it; then the two-stage head, the softmax statistics and the keyed pick."""
    res = {"layout": "tiled", "fp8_block32": [], "bf16": [], "row_major_gemv_us": {}}
    dense = [dh.Head(dh.BF16, wd)] + [dh.Head(dh.BF16, wd.clone()) for _ in range(1)]
    heads = [dh.tile(h) for h in rm_heads]
    dense_t = [dh.tile(h) for h in dense]
    torch.cuda.synchronize()
    for fmt, hs in (("fp8_block32", rm_heads), ("bf16", dense)):
        res["row_major_gemv_us"][fmt] = {}
        for R in (1, 16):
            x = xd[:R].contiguous()
            lg = torch.empty((R, V), dtype=torch.float32, device=xd.device)
            res["row_major_gemv_us"][fmt][str(R)] = back_to_back_us(
                lambda i: dh.gemv(hs[i % len(hs)], x, lg), n)
    log(f"row-major heads, gemv back to back: {res['row_major_gemv_us']}")
    for fmt, hs in (("fp8_block32", heads), ("bf16", dense_t)):
        for R in (1, 5, 10, 15, 16):
            x = xd[:R].contiguous()
            lg = torch.empty((R, V), dtype=torch.float32, device=xd.device)
            ws = dh.workspace(R, V, K)
            o = {"ids": torch.empty((R, K), dtype=torch.int32, device=xd.device),
                 "vals": torch.empty((R, K), dtype=torch.float32, device=xd.device),
                 "draft": torch.empty((R,), dtype=torch.int32, device=xd.device)}
            fg = lambda i: dh.gemv(hs[i % len(hs)], x, lg)
            ft = lambda i: dh.topk(lg, K, ws=ws, ids=o["ids"], vals=o["vals"], argmax=o["draft"])
            fd = lambda i: dh.draft(hs[i % len(hs)], x, K, ws=ws, out=o)
            g, t, d = stats_us(timed(fg, n)), stats_us(timed(ft, n)), stats_us(timed(fd, n))
            bb = {"dh_gemv": back_to_back_us(fg, n), "dh_topk": back_to_back_us(ft, n),
                  "dh_draft": back_to_back_us(fd, n)}
            b = algorithmic_bytes(fmt, V, H, R)
            res[fmt].append({"rows": R, "dh_gemv_us": g, "dh_topk_us": t, "dh_draft_us": d,
                             "back_to_back_us": bb,
                             "gemv_GBps": round(b / (g["median"] * 1e-6) / 1e9, 1),
                             "draft_GBps": round(b / (bb["dh_draft"] * 1e-6) / 1e9, 1),
                             "rows_per_s": round(R / (bb["dh_draft"] * 1e-6), 1),
                             "frac_of_8TBps": round(b / (g["median"] * 1e-6) / 8e12, 4)})
            log(f"{fmt} R={R}: gemv {g['median']:.1f} us, topk {t['median']:.1f} us, "
                f"draft {d['median']:.1f} us (per-call events); back to back: "
                f"gemv {bb['dh_gemv']:.1f}, topk {bb['dh_topk']:.1f}, draft {bb['dh_draft']:.1f}")
    res["two_stage"] = two_stage_sweep(dh, torch, wd, xd, V, H, n, dense[0])
    # the top-k with the softmax statistics (probabilities of the kept entries, each row's
    # log-sum-exp) against the plain top-k, on the FP8 head's 16-row logits, top-64
    lg16 = torch.empty((16, V), dtype=torch.float32, device=xd.device)
    dh.gemv(heads[0], xd, lg16)
    ws64 = dh.workspace(16, V, K)
    res["topk_softmax"] = {
        "rows": 16, "k": K,
        "dh_topk_us": back_to_back_us(lambda i: dh.topk(lg16, K, ws=ws64), n),
        "dh_topk_softmax_us": back_to_back_us(lambda i: dh.topk_softmax(lg16, K, ws=ws64), n)}
    log(f"top-64 of 16 rows: {res['topk_softmax']['dh_topk_us']:.1f} us, with softmax "
        f"statistics {res['topk_softmax']['dh_topk_softmax_us']:.1f} us")
    # the keyed pick from the top-k lists (temperature 0.8, top-p 0.95), 16 rows
    pos16 = torch.arange(16, dtype=torch.int64, device=xd.device)
    i64, v64, _ = dh.topk(lg16, K, ws=ws64)
    i512, v512, _ = dh.topk(lg16, 512)
    tok16 = torch.empty((16,), dtype=torch.int32, device=xd.device)
    kept16 = torch.empty((16,), dtype=torch.int32, device=xd.device)
    f64 = lambda i: dh.sample(i64, v64, pos16, 0.8, 0.95, seed=i, token=tok16, kept=kept16)
    f512 = lambda i: dh.sample(i512, v512, pos16, 0.8, 0.95, seed=i, token=tok16, kept=kept16)
    res["sample"] = {
        "rows": 16, "temperature": 0.8, "top_p": 0.95,
        "dh_sample_k64_us": back_to_back_us(f64, n),
        "dh_sample_k512_us": back_to_back_us(f512, n),
        "dh_sample_k64_graph_us": graph_us(f64, n),
        "dh_sample_k512_graph_us": graph_us(f512, n)}
    sm = res["sample"]
    log(f"keyed pick of 16 rows: {sm['dh_sample_k64_us']:.1f} us from 64 candidates, "
        f"{sm['dh_sample_k512_us']:.1f} us from 512 (host-launched back to back); in a graph "
        f"{sm['dh_sample_k64_graph_us']:.1f} and {sm['dh_sample_k512_graph_us']:.1f} us")
    return res


def two_stage_sweep(dh, torch, wd, xd, V, H, n, dense=None):
    """The two-stage head of 16 rows: an FP8 row-scaled stage 1 (three tiled copies rotated,
    as in the step), its top 512 candidates rescored from the dense bf16 head (wd), and each
    part alone; the rescore also over rotated sets of random candidates (a cold gather)."""
    dense = dense if dense is not None else dh.Head(dh.BF16, wd)
    h1s = [dh.tile(dh.Head(dh.FP8_ROW, *dh.quantize(wd, dh.FP8_ROW))) for _ in range(NCOPY)]
    R, k = 16, 512
    ws = dh.workspace(R, V, k)
    o = {"ids": torch.empty((R, k), dtype=torch.int32, device=xd.device),
         "vals": torch.empty((R, k), dtype=torch.float32, device=xd.device),
         "draft": torch.empty((R,), dtype=torch.int32, device=xd.device),
         "exact": torch.empty((R, k), dtype=torch.float32, device=xd.device)}
    fd = lambda i: dh.draft(h1s[i % NCOPY], xd, k, dense=dense, ws=ws, out=o)
    d = stats_us(timed(fd, n))
    dbb = back_to_back_us(fd, n)
    lg = torch.empty((R, V), dtype=torch.float32, device=xd.device)
    g = stats_us(timed(lambda i: dh.gemv(h1s[i % NCOPY], xd, lg), n))
    t = stats_us(timed(lambda i: dh.topk(lg, k, ws=ws, ids=o["ids"], vals=o["vals"]), n))
    s = stats_us(timed(lambda i: dh.rescore(dense, xd, o["ids"], exact=o["exact"],
                                            draft=o["draft"]), n))
    # the same ids every call stay in the Infinity Cache; a cold gather rotates four sets of
    # uniformly random candidate ids (4 x 84 MB of rows)
    gen = torch.Generator(device=xd.device).manual_seed(404)
    sets = [torch.randint(0, V, (R, k), dtype=torch.int32, device=xd.device, generator=gen)
            for _ in range(4)]
    # dh_rescore_sync (one launch: the candidates' workgroups pick the drafts), and
    # dh_rescore (a second, small kernel picks them)
    sync = dh.rescore_sync_buffer(xd.device)
    s_cold = back_to_back_us(lambda i: dh.rescore(dense, xd, sets[i % 4], exact=o["exact"],
                                                   draft=o["draft"], sync=sync), n)
    s_cold2 = back_to_back_us(lambda i: dh.rescore(dense, xd, sets[i % 4], exact=o["exact"],
                                                    draft=o["draft"]), n)
    b = algorithmic_bytes("fp8_row", V, H, R) + R * k * H * 2
    log(f"two-stage: draft {d['median']:.1f} us per-call, {dbb:.1f} us back to back (gemv "
        f"{g['median']:.1f}, topk {t['median']:.1f}, rescore {s['median']:.1f}); rescore over "
        f"rotated random candidates {s_cold:.1f} us (two launches {s_cold2:.1f})")
    return {"rows": R, "cand_k": k, "stage1_copies_rotated": NCOPY, "dh_draft_us": d,
            "dh_gemv_us": g, "dh_topk_us": t, "dh_rescore_us": s,
            "dh_draft_back_to_back_us": dbb, "dh_rescore_rotated_ids_us": s_cold,
            "rescore_rotated_entry": "dh_rescore_sync (one launch)",
            "dh_rescore_two_launch_rotated_ids_us": s_cold2,
            "rescore_rotated_GBps": round(R * k * H * 2 / (s_cold * 1e-6) / 1e9, 1),
            "draft_GBps_upper_bytes": round(b / (dbb * 1e-6) / 1e9, 1)}


def edge_shape(dh, torch, n):
    """The GEMV at a second shape, the edge-case workload's H=7168, V=163840 (7 blocks a wave):
    FP8 E4M3 with E8M0 32x32 blocks quantized straight into the tiled layout from seeded
    N(0, 0.02) weights made on the device (timing only; its parity is a test), three rotated
    copies, 1 and 16 rows, dh_gemv and dh_draft (top-512) back to back."""
    V, H = 163840, 7168
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(505)
    heads = []
    for _ in range(NCOPY):
        w = (torch.randn((V, H), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        codes, scale = dh.quantize(w, dh.FP8_BLOCK32 | dh.TILED)
        del w
        heads.append(dh.Head(dh.FP8_BLOCK32 | dh.TILED, codes, scale, (V, H)))
    res = {"workload": f"FP8 E4M3 head with E8M0 32x32 block scales, tiled, H={H}, V={V}",
           "kernel": gemv_kernel_name(dh.FP8_BLOCK32, H), "rows": []}
    for R in (1, 16):
        x = torch.randn((R, H), device=dev, generator=g).to(torch.bfloat16)
        lg = torch.empty((R, V), dtype=torch.float32, device=dev)
        ws = dh.workspace(R, V, 512)
        o = {}
        tg = back_to_back_us(lambda i: dh.gemv(heads[i % NCOPY], x, lg), n)
        td = back_to_back_us(lambda i: dh.draft(heads[i % NCOPY], x, 512, ws=ws, out=o), n)
        b = algorithmic_bytes("fp8_block32", V, H, R)
        res["rows"].append({"rows": R, "dh_gemv_us": tg, "gemv_GBps": round(b / (tg * 1e-6) / 1e9, 1),
                            "frac_of_8TBps": round(b / (tg * 1e-6) / 8e12, 4),
                            "dh_draft_top512_us": td})
        log(f"edge shape R={R}: gemv {tg:.1f} us ({b / (tg * 1e-6) / 1e9:.0f} GB/s), "
            f"draft top-512 {td:.1f} us")
    del heads
    torch.cuda.empty_cache()
    return res


def wide_linear(dh, torch, n):
    """One of the head's own linears with a wide input, like a w2 whose input is the FFN width:
    N=5120 outputs, K=18432 inputs, FP8 E4M3 with a row scale (tiled), fp32 and bf16-add
    outputs, 1 and 16 rows, back to back over three rotated weight copies (device-generated
    N(0, 0.02) weights; timing only, its parity is a test).  The GEMV streams the 18432 columns
    in chunks of 8192: dh_linear one chunk after another, dh_linear_ws (with a workspace) every
    (tile, chunk) at once."""
    N, K = 5120, 18432
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(808)
    ws = []
    for _ in range(NCOPY):
        w = (torch.randn((N, K), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        ws.append(dh.tile(dh.Head(dh.FP8_ROW, *dh.quantize(w, dh.FP8_ROW))))
        del w
    res = {"workload": f"linear N={N} K={K}, FP8 E4M3 with a row scale, tiled", "rows": []}
    for R in (1, 16):
        x = torch.randn((R, K), device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty((R, N), dtype=torch.float32, device=dev)
        r16 = torch.zeros((R, N), dtype=torch.bfloat16, device=dev)
        lws = dh.linear_workspace(R, N, K)
        tf = back_to_back_us(lambda i: dh.linear(ws[i % NCOPY], x, dh.OUT_F32, out=out), n)
        ta = back_to_back_us(lambda i: dh.linear(ws[i % NCOPY], x, dh.OUT_ADD_BF16,
                                                 residual=r16, out=r16), n)
        wf = back_to_back_us(lambda i: dh.linear(ws[i % NCOPY], x, dh.OUT_F32, out=out,
                                                 ws=lws), n)
        wa = back_to_back_us(lambda i: dh.linear(ws[i % NCOPY], x, dh.OUT_ADD_BF16,
                                                 residual=r16, out=r16, ws=lws), n)
        b = N * K + N * 4 + R * K * 2 + R * N * 4
        res["rows"].append({"rows": R, "f32_us": tf, "f32_GBps": round(b / (tf * 1e-6) / 1e9, 1),
                            "add_bf16_us": ta, "frac_of_8TBps": round(b / (tf * 1e-6) / 8e12, 4),
                            "ws_f32_us": wf, "ws_f32_GBps": round(b / (wf * 1e-6) / 1e9, 1),
                            "ws_add_bf16_us": wa,
                            "ws_frac_of_8TBps": round(b / (wf * 1e-6) / 8e12, 4)})
        log(f"wide linear R={R}: f32 {tf:.1f} us ({b / (tf * 1e-6) / 1e9:.0f} GB/s), "
            f"bf16 add {ta:.1f} us; with a workspace {wf:.1f} us "
            f"({b / (wf * 1e-6) / 1e9:.0f} GB/s), bf16 add {wa:.1f} us")
    del ws
    torch.cuda.empty_cache()
    return res


def topk_sweep(dh, torch, n):
    """dh_topk alone (the cut pass over each row's chunks, then the merge) on the row-sweep
    workload's own logits (FP8 E4M3 + E8M0 32x32 head, H=5120, V=129280): 1 and 16 rows,
    k = 64 and 512; back to back, and inside a HIP graph (no host launch cost); then
    dh_topk_softmax (the same two kernels with the softmax statistics) the same way."""
    import synth
    c = synth.CONFIGS["row_sweep"]
    V, H = c["V"], c["H"]
    dev = torch.device("cuda:0")
    wd = torch.from_numpy(synth.head_bf16("row_sweep").view(np.int16)).to(dev)
    head = dh.tile(dh.Head(dh.FP8_BLOCK32, *dh.quantize(wd, dh.FP8_BLOCK32)))
    del wd
    xd = torch.from_numpy(synth.activations("row_sweep", 16).view(np.int16)).to(dev)
    lg16 = dh.gemv(head, xd)
    res = {}
    for R in (1, 16):
        lg = lg16[:R].contiguous()
        for k in (64, 512):
            ws = dh.workspace(R, V, k)
            o = [torch.empty((R, k), dtype=torch.int32, device=dev),
                 torch.empty((R, k), dtype=torch.float32, device=dev),
                 torch.empty((R,), dtype=torch.int32, device=dev)]
            f = lambda i: dh.topk(lg, k, ws=ws, ids=o[0], vals=o[1], argmax=o[2])
            res[f"rows{R}_k{k}"] = {"back_to_back_us": back_to_back_us(f, n),
                                    "graph_us": graph_us(f, n)}
    for R in (1, 16):
        lg = lg16[:R].contiguous()
        for k in (64, 512):
            ws = dh.workspace(R, V, k)
            o = {"ids": torch.empty((R, k), dtype=torch.int32, device=dev),
                 "vals": torch.empty((R, k), dtype=torch.float32, device=dev),
                 "probs": torch.empty((R, k), dtype=torch.float32, device=dev),
                 "lse": torch.empty((R,), dtype=torch.float32, device=dev),
                 "argmax": torch.empty((R,), dtype=torch.int32, device=dev)}
            f = lambda i: dh.topk_softmax(lg, k, ws=ws, out=o)
            res[f"rows{R}_k{k}"]["softmax_back_to_back_us"] = back_to_back_us(f, n)
            res[f"rows{R}_k{k}"]["softmax_graph_us"] = graph_us(f, n)
    log("dh_topk: " + ", ".join(f"{key} {v['graph_us']:.1f} us (graph)" for key, v in res.items()))
    log("dh_topk_softmax: " + ", ".join(f"{key} {v['softmax_graph_us']:.1f} us (graph)"
                                         for key, v in res.items()))
    return {"workload": f"logits of the FP8 block head H={H} V={V}", **res}


def subset_sweep(dh, torch, n):
    """The draft-vocabulary subset head against the whole head it is gathered from: an FP8
    head with a row scale, H=4096, V=131072, and 49,152 of its rows with their token ids;
    dh_draft on the whole head and dh_draft_mapped on the subset, top-64, 1, 16 and 32 rows,
    back to back over rotated copies (each subset copy is 201 MB, so three of them do not
    fit the 256 MB Infinity Cache), plus the gather itself."""
    import synth
    name = "subset_head"
    c = synth.CONFIGS[name]
    V, H, nd, K = c["V"], c["H"], c["n_draft"], 64
    dev = torch.device("cuda:0")
    wd = torch.from_numpy(synth.head_bf16(name).view(np.int16)).to(dev)
    x32 = torch.from_numpy(synth.activations(name, 32).view(np.int16)).to(dev)
    im = torch.from_numpy(synth.draft_ids(name)).to(dev)
    fulls, subs = [], []
    for i in range(NCOPY):
        codes, scale = dh.quantize(wd, dh.FP8_ROW)
        fulls.append(dh.Head(dh.FP8_ROW, codes, scale))
        subs.append(dh.gather_rows(fulls[-1], im))
    del wd
    torch.cuda.synchronize()
    fg = lambda i: dh.gather_rows(fulls[i % NCOPY], im, out=subs[i % NCOPY])
    gat = back_to_back_us(fg, n)
    gbytes = 2 * nd * H + 2 * nd * 4 + nd * 4
    # both heads are projected from their tiled copies (the subset tiled after the gather)
    fulls_t, subs_t = [dh.tile(h) for h in fulls], [dh.tile(h) for h in subs]
    res = {"workload": f"FP8 E4M3 head with a row scale, H={H}, V={V}; subset of {nd} "
                       f"sorted token ids; top-{K}; both heads tiled",
           "gather_us": gat, "gather_bytes": gbytes,
           "gather_GBps": round(gbytes / (gat * 1e-6) / 1e9, 1), "rows": []}
    for R in (1, 16, 32):
        x = x32[:R].contiguous()
        ws_f, ws_s = dh.workspace(R, V, K), dh.workspace(R, nd, K)
        mk = lambda: {"ids": torch.empty((R, K), dtype=torch.int32, device=dev),
                      "vals": torch.empty((R, K), dtype=torch.float32, device=dev),
                      "draft": torch.empty((R,), dtype=torch.int32, device=dev)}
        of, os_ = mk(), mk()
        ff = lambda i: dh.draft(fulls_t[i % NCOPY], x, K, ws=ws_f, out=of)
        fs = lambda i: dh.draft_mapped(subs_t[i % NCOPY], im, x, K, ws=ws_s, out=os_)
        tf, ts = back_to_back_us(ff, n), back_to_back_us(fs, n)
        bf = algorithmic_bytes("fp8_row", V, H, R)
        bs = algorithmic_bytes("fp8_row", nd, H, R)
        res["rows"].append({"rows": R, "whole_head_dh_draft_us": tf,
                            "subset_dh_draft_mapped_us": ts,
                            "speedup": round(tf / ts, 3),
                            "whole_head_GBps": round(bf / (tf * 1e-6) / 1e9, 1),
                            "subset_GBps": round(bs / (ts * 1e-6) / 1e9, 1)})
        log(f"subset head R={R}: whole head {tf:.1f} us, subset {ts:.1f} us "
            f"({tf / ts:.2f}x)")
    log(f"subset gather: {gat:.1f} us ({gbytes / (gat * 1e-6) / 1e9:.0f} GB/s)")
    return res


def lowrank_sweep(dh, torch, n):
    """The two-stage head with a low-rank stage 1: bf16 factors of rank 512 (H=5120,
    V=129280), 16 rows, the top 512 candidates rescored from the dense bf16 head; each
    launch of dh_draft_lowrank and of its parts, back to back, over rotated factor copies."""
    import synth
    name = "lowrank"
    c = synth.CONFIGS[name]
    V, H, rk, k = c["V"], c["H"], c["rank"], c["ks"][0]
    R = max(c["rows"])
    dev = torch.device("cuda:0")
    down, up = synth.lowrank_factors(name)
    dn = torch.from_numpy(down.view(np.int16)).to(dev)
    ups = [torch.from_numpy(up.view(np.int16)).to(dev) for _ in range(NCOPY)]
    dense = dh.Head(dh.BF16, torch.from_numpy(synth.head_bf16(name).view(np.int16)).to(dev))
    x = torch.from_numpy(synth.activations(name, R).view(np.int16)).to(dev)
    hd = dh.tile(dh.Head(dh.BF16, dn))                 # both factors tiled at load
    hu = [dh.tile(dh.Head(dh.BF16, u)) for u in ups]
    ws = dh.workspace(R, V, k)
    o = {"ids": torch.empty((R, k), dtype=torch.int32, device=dev),
         "vals": torch.empty((R, k), dtype=torch.float32, device=dev),
         "draft": torch.empty((R,), dtype=torch.int32, device=dev),
         "exact": torch.empty((R, k), dtype=torch.float32, device=dev),
         "t": torch.empty((R, rk), dtype=torch.int16, device=dev)}
    lg = torch.empty((R, V), dtype=torch.float32, device=dev)
    fd = lambda i: dh.draft_lowrank(hd, hu[i % NCOPY], x, k, dense=dense, ws=ws, out=o)
    ft = lambda i: dh.linear(hd, x, dh.OUT_BF16, out=o["t"])
    fu = lambda i: dh.gemv(hu[i % NCOPY], o["t"], lg)
    d, td, tu = back_to_back_us(fd, n), back_to_back_us(ft, n), back_to_back_us(fu, n)
    b = (rk * H * 2 + R * H * 2 + R * rk * 2) + (V * rk * 2 + R * V * 4) + R * k * H * 2
    log(f"low-rank two-stage: draft {d:.1f} us back to back (down {td:.1f}, up {tu:.1f})")
    return {"workload": f"rank {rk} bf16 factors, H={H}, V={V}, {R} rows, top {k} rescored "
                        f"from the dense bf16 head",
            "dh_draft_lowrank_us": d, "down_linear_us": td, "up_gemv_us": tu,
            "up_gemv_GBps": round((V * rk * 2 + R * rk * 2 + R * V * 4) / (tu * 1e-6) / 1e9, 1),
            "draft_GBps_upper_bytes": round(b / (d * 1e-6) / 1e9, 1)}


def cpu_baseline(w, x, V, H, R, K):
    """The oracle as it stands (C, double precision, OpenMP over vocabulary rows) on the
    host's cores: the whole step (GEMV of the step's rows over the full FP8 head, then the
    top-k) repeated until about 10 s have passed, plus one GEMV on a single thread over
    the first 8192 vocabulary rows.  The FP8 codes come from the oracle's own quantizer
    (not timed)."""
    import oracle
    t0 = time.time()
    codes, scales = oracle.quant_block32(w)
    tq = time.time() - t0
    times = []
    while not times or (sum(times) < 10.0 and len(times) < 400):
        t0 = time.time()
        lg = oracle.gemv(oracle.FMT_FP8_BLOCK32, codes, scales, x)
        oracle.topk(lg, K)
        times.append(time.time() - t0)
    dt = float(np.median(times))
    b = algorithmic_bytes("fp8_block32", V, H, R)
    nt = oracle.threads()
    S = 8192
    oracle.threads(1)
    t0 = time.time()
    oracle.gemv(oracle.FMT_FP8_BLOCK32, codes[:S], scales[:S // 32], x)
    d1 = time.time() - t0
    oracle.threads(nt)
    b1 = algorithmic_bytes("fp8_block32", S, H, R)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    log(f"cpu oracle: full step {dt:.2f}s median of {len(times)} on {nt} threads; "
        f"1 thread: {S} vocab rows in {d1:.2f}s ({cpu})")
    wider = cpu_baseline_wider(oracle, nt)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": nt, "cpu": cpu,
            "rows16": wider["rows16"], "two_stage": wider["two_stage"],
            "kind": "oracle", "seconds_per_step": round(dt, 3), "steps": len(times),
            "quantize_seconds": round(tq, 3),
            "single_thread": {"value": round(b1 / d1 / 1e9, 4), "unit": "GB/s",
                              "seconds": round(d1, 3),
                              "sample": f"GEMV only, first {S} vocabulary rows, {R} activation row(s)"},
            "sample": f"the full step (GEMV over all {V} vocabulary rows of the FP8 block "
                      f"head for {R} activation row(s), then top-{K}), {len(times)} times, median; GB/s "
                      f"over the step's algorithmic bytes"}


def cpu_baseline_wider(oracle, nt):
    """The oracle once each on the row-sweep workload's head (H=5120, V=129280) at 16 rows:
    the 16-row step (FP8 32x32 block head, GEMV then top-64 and argmax) and the two-stage
    draft (FP8 row-scaled stage 1, top 512, rescore from the dense bf16 head).  Quantization
    is the oracle's own and is not timed."""
    import synth
    name = "row_sweep"
    c = synth.CONFIGS[name]
    V, H, R = c["V"], c["H"], 16
    w = synth.head_bf16(name)
    x = synth.activations(name, R)
    codes, scales = oracle.quant_block32(w)
    t0 = time.time()
    oracle.draft(oracle.FMT_FP8_BLOCK32, codes, scales, x, 64)
    d16 = time.time() - t0
    del codes, scales
    rc, rs = oracle.quant_row(w)
    t0 = time.time()
    oracle.draft(oracle.FMT_FP8_ROW, rc, rs, x, 512, dense_w=w)
    d2 = time.time() - t0
    b16 = algorithmic_bytes("fp8_block32", V, H, R)
    b2 = algorithmic_bytes("fp8_row", V, H, R) + R * 512 * H * 2
    log(f"cpu oracle: 16-row step {d16:.2f}s, two-stage draft {d2:.2f}s on {nt} threads")
    return {"rows16": {"seconds": round(d16, 3), "value": round(b16 / d16 / 1e9, 4),
                       "unit": "GB/s", "cores": nt, "kind": "oracle",
                       "sample": f"one dh_draft-equivalent call: {R} activation rows, FP8 "
                                 f"32x32 block head H={H} V={V}, GEMV then top-64 and argmax"},
            "two_stage": {"seconds": round(d2, 3), "value": round(b2 / d2 / 1e9, 4),
                          "unit": "GB/s", "cores": nt, "kind": "oracle",
                          "sample": f"one two-stage draft: {R} rows, FP8 row-scaled stage 1 "
                                    f"H={H} V={V}, top 512, rescore from the dense bf16 head "
                                    f"(GB/s over the upper-bound bytes)"}}


if __name__ == "__main__":
    main()
