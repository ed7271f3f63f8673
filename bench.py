#!/usr/bin/env python3
"""Benchmark of the MXFP4 dequantize-and-multiply path on one MI355X.

Headline step (the metric's workload: a 4096 x 4096 MXFP4 weight, fp32
activations): one decode matvec (b = 1) and one small-batch GEMM (b = 8),
each on a different copy of the weight taken from a rotating pool of more
than 512 MiB, so every launch streams its weight from HBM rather than from
the 256 MB Infinity Cache.  ``value`` is weight bytes streamed per second
over exactly --steps steps, inputs resident in HBM: the steps are bracketed
by device synchronisations, and their time is taken by HIP events recorded
on the launch stream right before the first and after the last step (so a
fixed host-side launch and synchronisation cost does not enter a short run;
the wall-clock figure is reported beside it).  Launches are replayed from
HIP graphs captured on torch's stream (the library is stream-ordered and
allocation-free), so host launch overhead does not hide the kernels.

Also reported (``extra``): each workload's kernel time, weight GB/s and
fraction of the 8 TB/s peak (256 x 512; 4096 x 4096 at b = 1, 8;
14336 x 4096 at b = 1..32), the two expert-bank layers in tokens/s (64
experts decode, 256 experts Zipf prefill), the roofline of the dominant
kernel, the read ceiling (a plain streaming-read kernel timed on the same
cold pools at the same sizes, so each figure can also be read against what
one launch of that size can stream on this GPU), and the CPU oracle timed
on bounded samples of every workload.

One GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 expert matvec weight GB/s (% of HBM peak) at 1/8 tokens; MoE layer tok/s"
PEAK_HBM = 8.0e12  # bytes/s, MI355X HBM3E
POOL_BYTES = 512 * 2 ** 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Sources that decide what the headline GEMM launches run (kernel code and
# launch-shape choice); the committed HBM-traffic figures are valid while
# these and the compiler flags are unchanged.
KERNEL_SOURCES = ["device.h", "launch.h", "skinny.hip", "api.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    from gemm_mxfp4_dequant_amd import build as hb
    h = hashlib.sha256()
    h.update(" ".join(hb.FLAGS).encode())
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gemm_mxfp4_dequant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def tensor_bytes(rows, cols):
    return rows * cols // 2 + rows * cols // 32


def spread_us(timer, n):
    """p10 / median / p90 of the per-launch time over ``n`` separately timed
    graph replays, in us (empty in eager mode)."""
    sp = timer.spread(n)
    if sp is None:
        return {}
    return {"p10_us": round(sp[0] * 1e3, 3), "p50_us": round(sp[1] * 1e3, 3),
            "p90_us": round(sp[2] * 1e3, 3)}


class Timer:
    """Graph-replayed launches timed with HIP events on torch's stream."""

    def __init__(self, torch, launches, eager=False, passes=None):
        self.torch = torch
        self.launches = launches  # list of zero-arg callables (one launch each)
        self.eager = eager
        self.graph = None
        self.passes = 1
        for f in launches:  # warm: attributes set, code loaded
            f()
        torch.cuda.synchronize()
        if not eager:
            # enough passes over the launch list in one graph that replay
            # boundaries are a small part of the timed span
            self.passes = passes if passes else max(1, 256 // len(launches))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(self.passes):
                    for f in launches:
                        f()
            self.graph = g
            g.replay()
            torch.cuda.synchronize()

    def run(self, reps):
        """``reps`` passes over the launch list."""
        if self.graph is not None:
            for _ in range((reps + self.passes - 1) // self.passes):
                self.graph.replay()
        else:
            for _ in range(reps):
                for f in self.launches:
                    f()

    def launches_run(self, reps):
        if self.graph is not None:
            return (reps + self.passes - 1) // self.passes * self.passes * len(self.launches)
        return reps * len(self.launches)

    def spread(self, n):
        """Per-launch GPU ms of ``n`` separately timed graph replays (each one
        pass count over the launch list): (p10, median, p90)."""
        torch = self.torch
        if self.graph is None:
            return None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            self.graph.replay()
            e1.record()
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) / (self.passes * len(self.launches)) for e0, e1 in ev)
        q = lambda f: per[min(len(per) - 1, int(f * len(per)))]
        return q(0.1), q(0.5), q(0.9)

    def time(self, reps):
        """Average GPU ms per launch over ``reps`` passes."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        self.run(1)  # one warm pass (a replay right after capture runs slower)
        torch.cuda.synchronize()
        e0.record()
        self.run(reps)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / self.launches_run(reps)


def gemm_setup(torch, mx, inputs, rows, cols, b, seed, pool_bytes=POOL_BYTES):
    nb = tensor_bytes(rows, cols)
    n = max(2, math.ceil(pool_bytes / nb) + 1)
    pool = inputs.draw_weights_device(seed, rows, cols, 118, 132, n)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1000)
    x = torch.randn((b, cols), generator=g, device="cuda", dtype=torch.float32)
    y = torch.empty((b, rows), device="cuda", dtype=torch.float32)
    launches = [lambda i=i: mx.mxfp4_gemm(pool[i], rows, cols, x, b=b, y=y) for i in range(n)]
    return dict(pool=pool, x=x, y=y, n=n, nb=nb, launches=launches,
                alg_bytes=nb + b * cols * 4 + b * rows * 4)


def moe_setup(torch, mx, inputs, wl, banks, extra_experts=0):
    import numpy as np
    cfg = inputs.WORKLOADS[wl]
    E, H, I, T, K = (cfg["n_experts"], cfg["hidden"], cfg["inter"], cfg["n_tokens"],
                     cfg["top_k"])
    rng = inputs.rng_for(wl)
    if cfg["routing"] == "softmax":
        ids, w = inputs.route_softmax(rng, T, E, K)
    else:
        ids, w = inputs.route_zipf(rng, T, E, K, cfg["zipf_s"])
    tb = tensor_bytes(I, H)
    bank = []
    for j in range(banks):
        s = 100 * wl + 10 * j
        bank.append([inputs.draw_weights_device(s + r, I if r < 2 else H, H if r < 2 else I,
                                                cfg["scale_lo"], cfg["scale_hi"],
                                                E + extra_experts)
                     for r in range(3)])
    g = torch.Generator(device="cuda")
    g.manual_seed(wl)
    xdt = torch.float32 if cfg["x_dtype"] == "f32" else torch.bfloat16
    x = torch.randn((T, H), generator=g, device="cuda", dtype=torch.float32).to(xdt)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.moe_experts_mxfp4_workspace_size(T, K, E, H, I, xdt), dtype=torch.uint8,
                     device="cuda")
    active = int(np.unique(ids).size)
    launches = [lambda bk=bk: mx.moe_experts_mxfp4(bk[0], bk[1], bk[2], E, H, I, x, ids_d, w_d,
                                                   out=out, workspace=ws) for bk in bank]
    return dict(launches=launches, T=T, touched=active * 3 * tb, active=active, bank=bank,
                x=x, ids=ids_d, w=w_d, out=out, ws=ws)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds):
    """The oracle, as it stands, on the host cores of this machine.

    ``value``: the headline step (4096 x 4096, b = 1 and b = 8) repeated until
    ``seconds`` have elapsed, in weight GB/s.  ``workloads``: every other
    workload timed once or as the minimum of three runs, each with the
    throughput it implies; the 256-expert prefill layer on a sample of 8 of
    its 512 tokens (all 64 of their pairs; the whole layer would take
    minutes), scaled to tokens per second."""
    import oracle
    from gemm_mxfp4_dequant_amd import inputs
    threads = oracle.default_threads()

    def best(f, n):
        t = 1e30
        for _ in range(n):
            t0 = time.perf_counter()
            f()
            t = min(t, time.perf_counter() - t0)
        return t

    w, x = inputs.gemm_case(2, 4096, 4096, 9)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemm(w, 4096, 4096, x[:1], threads)
        oracle.gemm(w, 4096, 4096, x[1:9], threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    gbs = reps * 2 * tensor_bytes(4096, 4096) / el / 1e9
    wl = {}
    w1, x1 = inputs.workload_case(1)
    t = best(lambda: oracle.gemm(w1, 256, 512, x1, threads), 3)
    wl["gemm_256x512_b1"] = {"s": round(t, 6), "weight_GBps": round(tensor_bytes(256, 512) / t
                                                                    / 1e9, 4)}
    for b in (1, 8):
        t = best(lambda: oracle.gemm(w, 4096, 4096, x[:b], threads), 3)
        wl[f"gemm_4096x4096_b{b}"] = {"s": round(t, 5),
                                      "weight_GBps": round(tensor_bytes(4096, 4096) / t / 1e9, 4)}
    w3, x3 = inputs.gemm_case(3, 14336, 4096, 32)
    for b in (1, 2, 4, 8, 16, 32):
        t = best(lambda: oracle.gemm(w3, 14336, 4096, x3[:b], threads), 3 if b in (1, 32) else 1)
        wl[f"gemm_14336x4096_b{b}"] = {"s": round(t, 4),
                                       "weight_GBps": round(tensor_bytes(14336, 4096) / t / 1e9,
                                                            4)}
    c = inputs.workload_case(4)
    cfg = inputs.WORKLOADS[4]
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
    t = best(lambda: oracle.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"], c["ids"],
                                c["w"], False, threads), 3)
    wl["moe_decode_e64"] = {"s": round(t, 3), "tok_per_s": round(cfg["n_tokens"] / t, 3)}
    del c
    cfg = inputs.WORKLOADS[5]
    c = inputs.workload_case(5)
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
    toks = np.arange(8)
    t = best(lambda: oracle.moe(c["gate"], c["up"], c["down"], E, H, I, c["x"][toks],
                                c["ids"][toks], c["w"][toks], True, threads), 1)
    wl["moe_prefill_e256"] = {"s": round(t, 3), "sample": "tokens 0-7 of 512 (64 pairs)",
                              "tok_per_s": round(len(toks) / t, 3)}
    del c
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{reps} headline steps (4096x4096 fp64 oracle, b=1 and b=8) in "
                      f"{el:.1f} s; other workloads: min of 3 runs (one run for 14336x4096 "
                      f"b=2..16 and for the prefill sample)",
            "seconds": round(el, 2), "workloads": wl}


def load_traffic(key, launches_bytes):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or key not in t.get("per_launch", {}):
        return None
    e = t["per_launch"][key]
    return e.get("fetch_bytes", 0) + e.get("write_bytes", 0)


def read_ceiling(torch, mx, bufs, nbytes, eager, reps):
    """Best per-launch rate of the plain streaming-read kernel over ``bufs``
    (one launch per buffer, in rotation, cold as the GEMM pools are), over
    4, 8 and 16 loads per thread: GB/s and us per launch."""
    sink = torch.empty(1, dtype=torch.int32, device="cuda")
    best = None
    for u in (4, 8, 16):
        L = [lambda b=b, u=u: mx.mxfp4_probe_read(b, nbytes, u, sink) for b in bufs]
        t = Timer(torch, L, eager)
        ms = t.time(reps)
        if best is None or ms < best[1]:
            best = (u, ms)
        del t
    u, ms = best
    return {"GBps": round(nbytes / ms / 1e6, 1), "us": round(ms * 1e3, 3), "bytes": nbytes,
            "loads_per_thread": u}


def gemm_line(s, ms, timer, ceil=None):
    gb = s["nb"] / ms / 1e6
    d = {"us": round(ms * 1e3, 3), "weight_GBps": round(gb, 1),
         "pct_peak": round(100 * gb / 8000, 1)}
    if ceil:
        d["pct_of_read_ceiling"] = round(100 * ceil["us"] / (ms * 1e3), 1)
    d.update(spread_us(timer, 50 if s["n"] > 20 else 30))
    return d


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true",
                    help="headline step only (no extra workloads, no CPU baseline)")
    ap.add_argument("--eager", action="store_true",
                    help="launch eagerly instead of replaying graphs (counter runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run plain 1 GiB device copies (counter calibration)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--sections", default="gemm,decode,prefill,cpu",
                    help="extra sections to run: gemm, decode, prefill, cpu")
    args = ap.parse_args()
    sections = set(args.sections.split(",")) if not args.quick else set()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_mxfp4_dequant_amd import inputs
    from gemm_mxfp4_dequant_amd import mxfp4 as mx

    if not os.path.exists(mx.LIB_PATH):
        from gemm_mxfp4_dequant_amd import build as hb
        hb.build()
    torch.cuda.set_device(0)
    mx.lib()

    # ---------------- headline step: 4096^2 at b = 1 and b = 8 -------------
    rows = cols = 4096
    s1 = gemm_setup(torch, mx, inputs, rows, cols, 1, 21)
    s8 = gemm_setup(torch, mx, inputs, rows, cols, 8, 22)
    n = min(s1["n"], s8["n"])
    step_launches = []
    for i in range(n):
        step_launches += [s1["launches"][i], s8["launches"][i]]
    # exactly --steps steps: whole replays of the multi-pass graph, then one
    # replay of a graph holding the remaining steps
    main_t = Timer(torch, step_launches, args.eager)
    per_replay = n * main_t.passes if not args.eager else n
    full, rem = divmod(args.steps, per_replay)
    rem_launches = [step_launches[i % (2 * n)] for i in range(2 * rem)]
    rem_t = Timer(torch, rem_launches, args.eager, passes=1) if rem else None
    main_t.run(max(1, math.ceil(args.warmup / n)))
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    evs = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # a GPU spin ahead of the start event keeps the device busy while the
    # host submits the first replay, so the events bracket the steps alone
    # (at --steps 20 the submission gap was ~10 % of the window); the spin's
    # own time is taken off the wall clock below
    evs.record()
    if not args.eager:
        torch.cuda._sleep(2_000_000)
    ev0.record()
    for _ in range(full):
        main_t.run(per_replay // n)
    if rem_t:
        rem_t.run(1)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0 - evs.elapsed_time(ev0) * 1e-3
    gpu_s = ev0.elapsed_time(ev1) * 1e-3
    step_bytes = s1["nb"] + s8["nb"]
    value = args.steps * step_bytes / gpu_s / 1e9
    wall_value = args.steps * step_bytes / wall / 1e9
    log(f"headline: {args.steps} steps in {gpu_s * 1e3:.3f} ms (events; wall {wall * 1e3:.3f} ms)"
        f" -> {value:.1f} GB/s weight ({value / 80:.1f}% of 8 TB/s; wall-clock rate "
        f"{wall_value:.1f})")

    # per-kernel launch times (HIP events on the launch stream)
    k1 = Timer(torch, s1["launches"], args.eager)
    k8 = Timer(torch, s8["launches"], args.eager)
    reps = max(3, 4000 // n)
    ms1, ms8 = k1.time(reps), k8.time(reps)
    # the read ceiling at this size, on the same cold pool
    ceil_2 = read_ceiling(torch, mx, [s1["pool"][i] for i in range(s1["n"])], s1["nb"],
                          args.eager, reps)
    log(f"read ceiling, {s1['nb']} bytes per launch: {ceil_2}")
    extra = {
        "gemm_4096x4096_b1": gemm_line(s1, ms1, k1, ceil_2),
        "gemm_4096x4096_b8": gemm_line(s8, ms8, k8, ceil_2),
        "read_ceiling_8.9MB": ceil_2,
    }
    for k, v in extra.items():
        log(f"{k}: {v}")
    dom, dms, dset = ("gemm_4096x4096_b8", ms8, s8) if ms8 >= ms1 else ("gemm_4096x4096_b1", ms1, s1)
    achieved = dset["alg_bytes"] / (dms * 1e-3) / 1e9
    traffic = load_traffic(dom, dset["alg_bytes"])
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": 8000.0,
                "unit": "GB/s", "frac": round(achieved / 8000.0, 4), "traffic": traffic,
                "alg_bytes_per_launch": dset["alg_bytes"], "avg_launch_us": round(dms * 1e3, 3),
                "ceiling_GBps": ceil_2["GBps"],
                "frac_of_ceiling": round(ceil_2["us"] / (dms * 1e3), 4)}

    if args.calib_copy:
        # a plain elementwise kernel of known traffic for counter calibration:
        # reads 1 GiB (cold: written before the 1 GiB destination) and
        # writes 1 GiB
        src = torch.ones(2 ** 28, dtype=torch.float32, device="cuda")
        dst = torch.zeros_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    del main_t, rem_t, k1, k8, s1, s8
    if "gemm" in sections:
        # 256 x 512 (latency-bound; reported in us)
        s = gemm_setup(torch, mx, inputs, 256, 512, 1, 1, pool_bytes=0)
        t = Timer(torch, s["launches"] * 50, args.eager)
        ms = t.time(20)
        extra["gemm_256x512_b1"] = {"us": round(ms * 1e3, 3)}
        log(f"gemm_256x512_b1: {extra['gemm_256x512_b1']}")
        del s, t
        ceil_3 = None
        for b in (1, 2, 4, 8, 16, 32):
            s = gemm_setup(torch, mx, inputs, 14336, 4096, b, 30 + b)
            if ceil_3 is None:
                ceil_3 = read_ceiling(torch, mx, [s["pool"][i] for i in range(s["n"])], s["nb"],
                                      args.eager, max(3, 1000 // s["n"]))
                extra["read_ceiling_31.2MB"] = ceil_3
                log(f"read ceiling, {s['nb']} bytes per launch: {ceil_3}")
            t = Timer(torch, s["launches"], args.eager)
            ms = t.time(max(3, 1000 // s["n"]))
            extra[f"gemm_14336x4096_b{b}"] = gemm_line(s, ms, t, ceil_3)
            log(f"gemm_14336x4096_b{b}: {extra[f'gemm_14336x4096_b{b}']}")
            del s, t
        # the opt-in block-scaled FP4 x FP8 product (activations quantized to
        # MXFP8 in the call; its own accuracy contract) beside the exact path,
        # at 64 tokens
        for xname, xdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
            rows_, cols_, b = 14336, 4096, 64
            s = gemm_setup(torch, mx, inputs, rows_, cols_, b, 90)
            x = s["x"].to(xdt)
            ws = torch.empty(mx.mxfp4_gemm_a8_workspace_size(b, cols_), dtype=torch.uint8,
                             device="cuda")
            for name, fn in (("a8", lambda i: mx.mxfp4_gemm_a8(s["pool"][i], rows_, cols_, x,
                                                               b=b, y=s["y"], workspace=ws)),
                             ("exact", lambda i: mx.mxfp4_gemm(s["pool"][i], rows_, cols_, x,
                                                               b=b, y=s["y"]))):
                t = Timer(torch, [lambda i=i: fn(i) for i in range(s["n"])], args.eager)
                ms = t.time(max(3, 1000 // s["n"]))
                key = f"gemm_{name}_14336x4096_b64_{xname}"
                extra[key] = gemm_line(s, ms, t, ceil_3)
                log(f"{key}: {extra[key]}")
                del t
            del s, ws, x
        torch.cuda.empty_cache()
    if "decode" in sections:
        # expert bank, decode layer (2 banks alternate: 466 MB touched per step)
        s = moe_setup(torch, mx, inputs, 4, 2)
        t = Timer(torch, s["launches"], args.eager)
        ms = t.time(100)
        # read ceiling for the layer's touched bytes, read contiguously from
        # the two banks in turn
        tb = s["touched"]
        bufs = []
        for bk in s["bank"]:
            flat = torch.cat([r.reshape(-1) for r in bk])
            bufs.append(flat[:tb])
        ceil_4 = read_ceiling(torch, mx, bufs, tb, args.eager, 20)
        del bufs, flat
        extra["read_ceiling_decode_touched"] = ceil_4
        extra["moe_decode_e64"] = {"us_per_layer": round(ms * 1e3, 2),
                                   "tok_per_s": round(s["T"] / (ms * 1e-3), 1),
                                   "touched_GB": round(s["touched"] / 1e9, 4),
                                   "active_experts": s["active"],
                                   "touched_GBps": round(s["touched"] / ms / 1e6, 1),
                                   "pct_peak": round(100 * s["touched"] / ms / 1e6 / 8000, 1),
                                   "pct_of_read_ceiling": round(100 * ceil_4["us"] / (ms * 1e3),
                                                                1),
                                   **spread_us(t, 30)}
        log(f"moe_decode_e64: {extra['moe_decode_e64']}")
        # the same layer with its four most-routed experts in pinned host
        # memory (moe_experts_mxfp4_ptrs: their weights cross the host link
        # on every step; the other experts stay in device memory)
        import numpy as np
        cfg = inputs.WORKLOADS[4]
        E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
        ids_h = s["ids"].cpu().numpy()
        hot = set(int(e) for e in np.argsort(-np.bincount(ids_h.reshape(-1), minlength=E),
                                             kind="stable")[:4])
        bk = s["bank"][0]
        tabs = []
        keep = []
        for r, (rows_, cols_) in enumerate(((I, H), (I, H), (H, I))):
            ts = []
            for e in range(E):
                if e in hot:
                    tp = torch.empty(bk[r][e].numel(), dtype=torch.uint8, pin_memory=True)
                    tp.copy_(bk[r][e])
                    ts.append(tp)
                else:
                    ts.append(bk[r][e])
            keep.append(ts)
            tabs.append(mx.expert_table(ts, rows_, cols_))
        hb = sum(3 * tensor_bytes(I, H) for e in hot if e in set(ids_h.reshape(-1).tolist()))
        L = [lambda: mx.moe_experts_mxfp4_ptrs(tabs[0], tabs[1], tabs[2], E, H, I, s["x"],
                                               s["ids"], s["w"], out=s["out"], workspace=s["ws"])]
        t2 = Timer(torch, L, args.eager, passes=8)
        ms2 = t2.time(16)
        extra["moe_decode_e64_host4"] = {"us_per_layer": round(ms2 * 1e3, 2),
                                         "tok_per_s": round(s["T"] / (ms2 * 1e-3), 1),
                                         "host_experts": sorted(hot),
                                         "host_bytes": hb,
                                         "host_GBps": round(hb / ms2 / 1e6, 2)}
        log(f"moe_decode_e64_host4: {extra['moe_decode_e64_host4']}")
        del s, t, t2, L, tabs, keep
        # the device router on the routing sizes of both layers (outside the
        # layer's own timing: the layer takes its routing as input)
        for name, (T, E, K) in (("route_topk_8x64_k6", (8, 64, 6)),
                                ("route_topk_512x256_k8", (512, 256, 8))):
            L = torch.from_numpy(inputs.gating_logits(inputs.rng_for(T + E), T, E)).cuda()
            ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
            w = torch.empty((T, K), dtype=torch.float32, device="cuda")
            t = Timer(torch, [lambda: mx.moe_route_topk(L, K, ids, w)] * 50, args.eager)
            ms = t.time(20)
            extra[name] = {"us": round(ms * 1e3, 3)}
            log(f"{name}: {extra[name]}")
            del L, ids, w, t
        torch.cuda.empty_cache()
    if "prefill" in sections:
        s = moe_setup(torch, mx, inputs, 5, 1)
        t = Timer(torch, s["launches"], args.eager, passes=4)
        ms = t.time(8)
        extra["moe_prefill_e256"] = {"us_per_layer": round(ms * 1e3, 2),
                                     "tok_per_s": round(s["T"] / (ms * 1e-3), 1),
                                     "touched_GB": round(s["touched"] / 1e9, 4),
                                     "active_experts": s["active"],
                                     "touched_GBps": round(s["touched"] / ms / 1e6, 1),
                                     "pct_peak": round(100 * s["touched"] / ms / 1e6 / 8000, 1),
                                     **spread_us(t, 10)}
        log(f"moe_prefill_e256: {extra['moe_prefill_e256']}")
        del t
        # the same layer on the opt-in FP4 x FP8 bank (x and h quantized to
        # MXFP8), on the same weights and routing
        cfg = inputs.WORKLOADS[5]
        E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
        ws8 = torch.empty(mx.moe_experts_mxfp4_a8_workspace_size(s["T"], cfg["top_k"], E, H, I),
                          dtype=torch.uint8, device="cuda")
        bk = s["bank"][0]
        L = [lambda: mx.moe_experts_mxfp4_a8(bk[0], bk[1], bk[2], E, H, I, s["x"], s["ids"],
                                             s["w"], out=s["out"], workspace=ws8)]
        t = Timer(torch, L, args.eager, passes=4)
        ms = t.time(8)
        extra["moe_prefill_e256_a8"] = {"us_per_layer": round(ms * 1e3, 2),
                                        "tok_per_s": round(s["T"] / (ms * 1e-3), 1),
                                        "touched_GBps": round(s["touched"] / ms / 1e6, 1),
                                        **spread_us(t, 10)}
        log(f"moe_prefill_e256_a8: {extra['moe_prefill_e256_a8']}")
        del s, t, L, ws8
        torch.cuda.empty_cache()
        # the same layer in V4.1 form: bf16 gate/up, SwiGLU limit 10, route
        # weight folded into h, plus a shared expert on every token
        s = moe_setup(torch, mx, inputs, 5, 1, extra_experts=1)
        cfg = inputs.WORKLOADS[5]
        E, H, I = cfg["n_experts"], cfg["hidden"], cfg["inter"]
        ws = torch.empty(mx.moe_experts_mxfp4_v41_workspace_size(s["T"], cfg["top_k"], E, H, I,
                                                                 True),
                         dtype=torch.uint8, device="cuda")
        bk = s["bank"][0]
        L = [lambda: mx.moe_experts_mxfp4_v41(bk[0], bk[1], bk[2], E, H, I, s["x"], s["ids"],
                                              s["w"], swiglu_limit=10.0, has_shared=True,
                                              out=s["out"], workspace=ws)]
        t = Timer(torch, L, args.eager, passes=4)
        ms = t.time(8)
        touched = s["touched"] + 3 * tensor_bytes(I, H)
        extra["moe_prefill_e256_v41_shared"] = {
            "us_per_layer": round(ms * 1e3, 2), "tok_per_s": round(s["T"] / (ms * 1e-3), 1),
            "touched_GB": round(touched / 1e9, 4),
            "touched_GBps": round(touched / ms / 1e6, 1),
            "pct_peak": round(100 * touched / ms / 1e6 / 8000, 1), **spread_us(t, 10)}
        log(f"moe_prefill_e256_v41_shared: {extra['moe_prefill_e256_v41_shared']}")
        del s, t, L, ws
        torch.cuda.empty_cache()
    if "cpu" in sections:
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"cpu_baseline: {cpu}")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gpu_s * 1e3 / args.steps, 6),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mxfp4 4096x4096 decode matvec b=1 + GEMM b=8, fp32 in/out, "
                               "cold HBM (rotating >512 MiB weight pool)",
                   "rows": rows, "cols": cols, "batches": [1, 8], "pool_copies": n,
                   "launch": "hip graph replay", "timing": "hip events on the launch stream"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
