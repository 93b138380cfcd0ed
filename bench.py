"""Benchmark of the fused W4A16 decode GEMV (and the prefill GEMM) on one MI355X.

A step is one decode layer's weight matmuls of Llama-3-8B at M=1: the four
projections qkv [6144,4096], o [4096,4096], gate_up [28672,4096] and down
[4096,14336], INT4 asymmetric, group 128, fp16 scale + zero, bf16 activations.
Each step reads a different copy of the packed weights (copies rotate over at
least 1 GiB, four times the 256 MB Infinity Cache), so the weights stream
from HBM as they do in a real decode over 32 layers.  Inputs are resident in
HBM before the timed region starts.

value = algorithmic bytes of a step / step time (GB/s), where the algorithmic
bytes per [N, K] projection are N*K/2 + 4*N*K/G + 2*K + 2*N (packed codes,
fp16 scale and zero per group, bf16 x in, bf16 y out).  Before timing, every
projection's output is checked against the CPU oracle on sampled rows.

The roofline object describes the step's only kernel (every projection runs
the same streaming GEMV kernel): algorithmic bytes per launch over the
average launch duration, both from the timed region, against 8 TB/s.  Its
`traffic` comes from rocprofv3 FETCH_SIZE / WRITE_SIZE passes (see
--profile-pass and --summarize-traffic), scaled by what the same counters
read for a copy of known size; it is reported only while the GEMV source is
the one the counters were taken on, else null.

Also reported: the prefill GEMM (M=2048, same shapes) in TFLOP/s against the
dense bf16 MFMA peak, the small-batch and super-block GEMVs, a bf16 GEMV
comparator (torch linear, hipBLASLt) for the effective-bytes speedup, and the
CPU oracle timed on a bounded sample on this host.

Prints ONE JSON line.  python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "W4A16 dequant-GEMV HBM GB/s & % peak (M=1); MFMA TFLOP/s at M=2048"
# the streaming kernel's sources: traffic counters taken before a change to
# either no longer describe the kernel
GEMV_SOURCES = [os.path.join(ROOT, "w4a16_dequant_gemm_group_amd", "csrc", f)
                for f in ("gemv.hip", "stream_util.h")]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "w4a16_gemv_stream_traffic.json")
GEMV_KERNEL = "gemv_stream_kernel"
GEMV_KERNEL_M1 = "gemv_stream_kernel<1,"  # the one-row instantiation (trace names)
CALIB_BYTES = 256 << 20          # calibration copy: reads and writes this many bytes
G = 128
# which kernel serves each small-batch M on the four projections (sym g32)
SMALL_BATCH_KERNELS = {
    1: "gemv_stream_kernel (dot products, one activation row)",
    2: "gemv_stream_kernel (dot products, 2 activation rows in LDS)",
    3: "gemv_stream_kernel (dot products, 3 activation rows in LDS)",
    4: "gemv_mfma_xreg_kernel (matrix cores, x in registers) on qkv/o/gate_up; "
       "gemv_stream_kernel (dot products, 4 activation rows in LDS) on down",
    5: "gemv_mfma_xreg_kernel (matrix cores, x in registers) on qkv/o/gate_up; "
       "gemv_mfma_xs_kernel (matrix cores, x streamed per item) on down; no scratch",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(n, k, g, m=1, sym=False):
    meta = 2 if sym else 4
    return n * k // 2 + n * (k // g) * meta + 2 * m * k + 2 * m * n


def source_digest() -> str:
    h = hashlib.sha256()
    for p in GEMV_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# rocprofv3 counter passes -> per-launch HBM traffic
# ----------------------------------------------------------------------------

def _counter_rows(d):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    yield from csv.DictReader(f)


def summarize_traffic(fetch_dir, write_dir):
    """Reduce the FETCH_SIZE and WRITE_SIZE passes of `--profile-pass` to
    per-launch HBM bytes of the GEMV, calibrated against the copy kernel."""
    import synth
    shapes = [(nm,) + synth.LLAMA3_8B_SHAPES[nm] for nm in synth.SHAPE_ORDER]
    out = {"source_sha256_16": source_digest(), "kernel": GEMV_KERNEL, "calibration_bytes": CALIB_BYTES}
    for cname, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == cname]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        calib = [float(r["Counter_Value"]) for r in rows if "neg" in r["Kernel_Name"]]
        gemv = [float(r["Counter_Value"]) for r in rows if GEMV_KERNEL_M1 in r["Kernel_Name"]]
        if not calib or not gemv or len(gemv) % len(shapes):
            raise SystemExit(f"{cname}: expected calibration and {len(shapes)}*k GEMV dispatches, "
                             f"found {len(calib)} / {len(gemv)}")
        factor = CALIB_BYTES / (max(calib) * 1024.0)        # bytes per counted KiB
        per = {}
        for i, (nm, _, _) in enumerate(shapes):
            vals = gemv[i::len(shapes)]
            per[nm] = float(np.median(vals)) * 1024.0 * factor
        out[cname] = {"scale_bytes_per_KiB": round(factor * 1024.0, 4), "per_launch_bytes": per}
    tot = {nm: out["FETCH_SIZE"]["per_launch_bytes"][nm] + out["WRITE_SIZE"]["per_launch_bytes"][nm]
           for nm, _, _ in shapes}
    out["hbm_bytes_per_launch"] = tot
    out["mean_hbm_bytes_per_launch"] = float(np.mean(list(tot.values())))
    out["algorithmic_bytes_per_launch"] = {nm: gemv_bytes(n, k, G) for nm, n, k in shapes}
    print(json.dumps(out, indent=1))


def load_traffic():
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256_16") != source_digest():
        return None
    return t


# ----------------------------------------------------------------------------
# issue-rate probes: the GPU facts behind the kernels' instruction scheduling
# ----------------------------------------------------------------------------

def run_probes(torch, B, iters=2000):
    """Per-wave loop cycles of the two probes in libgq (include/gq_bench.h), one
    workgroup per compute unit: cycles per iteration of 8 independent
    v_mfma_f32_32x32x16_bf16 with 0/32/64/128 fp32 FMAs behind them (two waves
    per SIMD), and LDS bytes per clock of a compute unit for 16-byte reads with
    4, 8 and 16 waves (the slowest wave of each workgroup sets its time)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"compute_units": cus, "iterations": iters,
           "mfma_valu": {"what": "s_memtime cycles per iteration of one wave (8 MFMAs + n FMAs), median over waves"},
           "lds_read": {"what": "LDS bytes per clock of a compute unit, median over workgroups"}}
    for valu in (0, 32, 64, 128):
        c = B.gq_probe_mfma_valu(valu, iters, cus).cpu().numpy()
        out["mfma_valu"][f"fma_{valu}"] = round(float(np.median(c)) / iters, 1)
    for waves in (4, 8, 16):
        c = B.gq_probe_lds_read(waves, iters, cus).cpu().numpy().reshape(cus, waves)
        bpc = waves * iters * 16 * 1024 / c.max(axis=1)
        out["lds_read"][f"waves_{waves}"] = round(float(np.median(bpc)), 1)
    return out


# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--reps", type=int, default=7,
                    help="timed replays of the step graph; the median is reported")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the decode step (used for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--profile-pass", action="store_true",
                    help="run a few decode steps and one calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--probes", action="store_true",
                    help="run the issue-rate probes (MFMA with vector work, LDS reads) and print their JSON")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="reduce two rocprofv3 --pmc passes of --profile-pass to per-launch bytes")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported here "
              "(the kernels shard by output rows with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a16_dequant_gemm_group_amd import binding as B
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def bits16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    shapes = [(name,) + synth.LLAMA3_8B_SHAPES[name] for name in synth.SHAPE_ORDER]

    # ---------------- inputs, quantized on the GPU -------------------------------
    W, X, host = {}, {}, {}
    for name, n, k in shapes:
        w, x = synth.decode_case(name)
        host[name] = (w, x)
        codes, s, z = B.gq_quantize_groups(to_dev(w), 4, G, False)
        W[name] = (B.gq_pack_int4(codes), s, z)
        X[name] = to_dev(x)
        del codes
    torch.cuda.synchronize()
    Y = {nm: torch.empty((1, n), dtype=torch.bfloat16, device=dev) for nm, n, _ in shapes}

    if args.probes:
        print(json.dumps(run_probes(torch, B)), flush=True)
        return
    if args.profile_pass:
        for _ in range(3):
            for nm, _, _ in shapes:
                qw, s, z = W[nm]
                B.gq_w4a16_gemv(X[nm], qw, s, z, G, False, y=Y[nm])
        for nm, n, k in shapes:   # one prefill GEMM per projection (M = 2048)
            _, xb = synth.prefill_case(nm)
            qw, s, z = W[nm]
            B.gq_w4a16_gemm(to_dev(xb), qw, s, z, G, False)
        # one small-batch GEMV per projection and row count: M = 2, 3 (and 4 on
        # down) run the multi-row streaming kernel, M = 4, 8 and 16 the
        # matrix-core kernels
        for m in (2, 3, 4, 8, 16):
            for nm, n, k in shapes:
                qw, s, z = W[nm]
                xm, _ = synth.activations(m, k, seed=2000 + 10 * m + synth.SHAPE_ORDER.index(nm))
                B.gq_w4a16_gemv(to_dev(xm), qw, s, z, G, False)
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        log("profile pass done")
        return

    from oracle import gq_oracle as O

    def gate(name, w, x, qw, s, z, g, sym):
        """Correctness before timing: 64 sampled rows of the packed weights equal
        the oracle's bytes and the GEMV output on them meets the parity bar."""
        n = qw.shape[0]
        y = B.gq_w4a16_gemv(to_dev(x), qw, s, z, g, sym)
        rows = np.sort(np.random.default_rng(0).choice(n, min(64, n), replace=False))
        c_ref, s_ref, z_ref = O.quantize_to_storage(w[rows], 4, g, sym)
        qref = O.pack_int4(c_ref, sym)
        if not np.array_equal(qw.cpu().numpy()[rows], qref):
            raise SystemExit(f"parity gate: packed weights of {name} differ from the oracle")
        ref = O.w4a16_reference(x, qref, s_ref, z_ref, g, sym)
        wh = O.dequantize_packed(qref, s_ref, z_ref, g, sym)
        ok, rel, ratio = O.within_parity(O.bf16_to_f64(bits16(y))[:, rows], ref, O.bf16_to_f64(x), wh)
        if not ok:
            raise SystemExit(f"parity gate: {name} relF {rel:.2e} max/allowed {ratio:.2f}")

    log("inputs ready; parity gate")
    for name, n, k in shapes:
        w, x = host[name]
        gate(name, w, x, *W[name], G, False)
    log("parity gate passed")

    # ---------------- rotation copies ------------------------------------------------
    step_weight_bytes = sum(W[nm][0].numel() + 2 * W[nm][1].numel() + 2 * W[nm][2].numel()
                            for nm, _, _ in shapes)
    R = max(2, int(np.ceil(args.rotate_gib * 2 ** 30 / step_weight_bytes)))
    copies = [W] + [{nm: tuple(t.clone() for t in W[nm]) for nm, _, _ in shapes} for _ in range(R - 1)]
    torch.cuda.synchronize()
    log(f"{R} rotating weight copies of {step_weight_bytes / 1e6:.1f} MB")
    step_bytes = sum(gemv_bytes(n, k, G) for _, n, k in shapes)

    def run_step(i):
        # launches go to the current stream (the capture stream inside a graph)
        c = copies[i % R]
        for nm, n, k in shapes:
            qw, s, z = c[nm]
            B.gq_w4a16_gemv(X[nm], qw, s, z, G, False, y=Y[nm])

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    # The timed region replays a HIP graph holding exactly `steps` steps (4 launches
    # each, rotating weight copies), so host launch overhead does not leak into the
    # measurement.  The graph holds only this library's kernels.
    # Each repetition replays the whole graph (exactly `steps` steps) between two
    # events; the reported step time is the median over the repetitions.
    g = capture(torch, stream, lambda: [run_step(i) for i in range(args.steps)])
    g.replay()
    torch.cuda.synchronize()
    rep_ms = []
    for _ in range(args.reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(t0.elapsed_time(t1) / args.steps)
    ms_per_step = float(np.median(rep_ms))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"decode step {ms_per_step * 1e3:.2f} us, {value:.0f} GB/s (median of {args.reps})")
    # the graph's outputs match eager launches of the same step
    yg = {nm: Y[nm].clone() for nm, _, _ in shapes}
    run_step(args.steps - 1)
    torch.cuda.synchronize()
    for nm, _, _ in shapes:
        if not torch.equal(yg[nm], Y[nm]):
            raise SystemExit(f"graph replay of {nm} differs from the eager launch")
    del g

    # per-launch durations: one graph per projection, `nrep` launches over the copies
    nrep = max(20, min(args.steps, 200))
    per_us = {}
    for nm, n, k in shapes:
        def one(i, nm=nm):
            qw, s, z = copies[i % R][nm]
            B.gq_w4a16_gemv(X[nm], qw, s, z, G, False, y=Y[nm], stream=torch.cuda.current_stream())
        per_us[nm] = graph_time(torch, stream, one, nrep)
        # (graph_time is the median over repeated replays)
    per_gbps = {nm: gemv_bytes(n, k, G) / (per_us[nm] * 1e-6) / 1e9 for nm, n, k in shapes}
    log(f"per-shape us {per_us}")
    ceiling = stream_ceiling(torch, B, dev, stream, {nm: gemv_bytes(n, k, G) for nm, n, k in shapes})
    log(f"stream read ceiling {ceiling['GB/s']:.0f} GB/s; same-size pure reads {ceiling['per_shape_us']}")

    # Every launch of the step is the same streaming GEMV kernel: its algorithmic
    # bytes per launch over its average launch duration in the timed region,
    # i.e. the event-timed region divided by its launches (gaps between the
    # back-to-back launches of the graph included; the kernel trace of the same
    # command gives the durations alone).
    bytes_per_launch = step_bytes / len(shapes)
    avg_launch_us = ms_per_step * 1e3 / len(shapes)
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    tr = load_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": None if tr is None else round(tr["mean_hbm_bytes_per_launch"]),
                "kernel": f"{GEMV_KERNEL}<1,2,NT,false,false,false> (M = 1, asym; all four projections; NT = 256 threads at K = 4096, 512 on down)",
                "bytes_per_launch": bytes_per_launch,
                "event_us_per_launch": round(avg_launch_us, 3),
                "event_us_per_launch_is": "HIP-event time of the timed graph replays / launches "
                                          "(launch gaps included)",
                "frac_of_measured_read_ceiling": round(achieved / ceiling["GB/s"], 4),
                # time of pure reads of the same byte counts over the time of the GEMVs
                "frac_of_same_size_reads": round(sum(ceiling["per_shape_us"].values())
                                                 / (ms_per_step * 1e3), 4)}
    # per projection (each in its own graph): its rate against the 8 TB/s peak,
    # and the time a plain read of its byte count takes over its GEMV time
    roofline["per_shape"] = {
        nm: {"us": round(per_us[nm], 3), "frac": round(per_gbps[nm] / HBM_PEAK_GBPS, 4),
             "same_size_read_us": ceiling["per_shape_us"][nm],
             "frac_of_same_size_read": round(ceiling["per_shape_us"][nm] / per_us[nm], 4)}
        for nm, _, _ in shapes}
    if tr is not None:
        roofline["traffic_per_shape"] = {k: round(v) for k, v in tr["hbm_bytes_per_launch"].items()}

    extras = {}
    if not args.skip_extras:
        extras = run_extras(torch, B, synth, to_dev, dev, stream, shapes, W, X, gate,
                            ms_per_step * 1e3, ceiling, copies)

    cpu = cpu_baseline(args, O, host, shapes)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights with 0.1% input channels x20, N(0,1) bf16 activations)",
        "config": {"workload": "Llama-3-8B decode layer GEMVs, M=1, INT4 asym g128 fp16 scale+zero: "
                               "qkv[6144,4096] o[4096,4096] gate_up[28672,4096] down[4096,14336]",
                   "M": 1, "group_size": G, "rotating_copies": R,
                   "step_algorithmic_bytes": step_bytes,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "per_shape_us": {k: round(v, 3) for k, v in per_us.items()},
                   "per_shape_GBps": {k: round(v, 1) for k, v in per_gbps.items()}},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timing": {"us_per_step": spread([v * 1e3 for v in rep_ms]),
                   "method": f"median of {args.reps} replays of one HIP graph of {args.steps} steps, "
                             "HIP events on the launch stream"},
        "stream_read_ceiling": ceiling,
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


def capture(torch, stream, body):
    """Capture body() (launches on the current stream) into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            body()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    return g


def graph_times(torch, stream, fn, launches, reps=5):
    """Microseconds per fn(i) call in each of `reps` timed replays of one graph
    holding fn(0) .. fn(launches - 1), after one untimed replay."""
    g = capture(torch, stream, lambda: [fn(i) for i in range(launches)])
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1) / launches * 1e3)
    del g
    return out


def graph_time(torch, stream, fn, launches, reps=5):
    """Median of graph_times."""
    return float(np.median(graph_times(torch, stream, fn, launches, reps)))


def spread(v):
    """median, p10, p90 of a list of times."""
    v = np.asarray(v, dtype=np.float64)
    return {"median": round(float(np.median(v)), 3), "p10": round(float(np.percentile(v, 10)), 3),
            "p90": round(float(np.percentile(v, 90)), 3), "n": int(v.size)}


def time_launches(torch, stream, fn, reps):
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(reps):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps * 1e3  # us


def stream_ceiling(torch, B, dev, stream, sizes):
    """Read bandwidth one kernel reaches: gq_stream_read over a 2 GiB buffer (8x
    the Infinity Cache), and the time of a pure read of each size in `sizes`,
    rotating through the same buffer so every read comes from HBM."""
    total = 1 << 31
    buf = torch.zeros(total // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    B.gq_stream_read(buf, sink)
    t = graph_times(torch, stream, lambda i: B.gq_stream_read(buf, sink), 4)
    gbps = total / (np.median(t) * 1e-6) / 1e9
    raw = buf.view(torch.uint8)
    per_us = {}
    for nm, nb in sizes.items():
        nb = nb // 16 * 16
        chunks = total // nb
        per_us[nm] = round(graph_time(torch, stream, lambda i, nb=nb, c=chunks:
                                      B.gq_stream_read(raw[(i % c) * nb:(i % c + 1) * nb], sink),
                                      2 * chunks), 3)
    del buf, raw
    torch.cuda.empty_cache()
    return {"GB/s": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "us_2GiB": spread(t), "per_shape_us": per_us,
            "kernel": "stream_read_kernel (16-byte nontemporal loads, 2048 per workgroup)"}


def run_extras(torch, B, synth, to_dev, dev, stream, shapes, W, X, gate, fused_step_us, ceiling,
               W_copies):
    ex = {}
    # ---- prefill GEMM, M = 2048 -------------------------------------------------
    gemm = {}
    tot_flop, tot_us = 0.0, 0.0
    for name, n, k in shapes:
        _, xb = synth.prefill_case(name)
        xd = to_dev(xb)
        qw, s, z = W[name]
        y = torch.empty((2048, n), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(B.gq_w4a16_gemm_workspace_size(2048, k, n, G), dtype=torch.uint8, device=dev)
        for _ in range(3):
            B.gq_w4a16_gemm(xd, qw, s, z, G, False, y=y, stream=stream, workspace=ws)
        torch.cuda.synchronize()
        # a graph of 10 launches replayed 3 times: GPU time only (an eager loop
        # would add the host's per-call time whenever it exceeds the kernel's)
        us = graph_time(torch, stream, lambda i: B.gq_w4a16_gemm(xd, qw, s, z, G, False, y=y,
                                                                  workspace=ws), 10, reps=3)
        fl = 2.0 * 2048 * n * k
        gemm[name] = {"us": round(us, 2), "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1)}
        tot_flop += fl
        tot_us += us
        del xd, y, ws
    agg = tot_flop / (tot_us * 1e-6) / 1e12
    ex["gemm_m2048"] = {"per_shape": gemm, "aggregate_TFLOPs": round(agg, 1),
                        "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS, "frac": round(agg / MFMA_BF16_PEAK_TFLOPS, 4)}
    log(f"gemm M=2048: {agg:.0f} TFLOP/s")

    # ---- bf16 GEMV comparator: the faster of hipBLASLt (torch) and gq_bf16_gemv --------
    import torch.nn.functional as F
    wb = {}
    for name, n, k in shapes:
        wb[name] = torch.randn((n, k), dtype=torch.bfloat16, device=dev) * 0.02
    bf16_bytes = sum(2 * n * k + 2 * k + 2 * n for _, n, k in shapes)
    Rb = max(2, int(np.ceil(2 ** 30 / bf16_bytes)))
    wcopies = [wb] + [{nm: t.clone() for nm, t in wb.items()} for _ in range(Rb - 1)]
    Yb = {nm: torch.empty((1, n), dtype=torch.bfloat16, device=dev) for nm, n, _ in shapes}

    def bf16_step_torch(i):
        c = wcopies[i % Rb]
        for nm, _, _ in shapes:
            torch.matmul(X[nm], c[nm].t(), out=Yb[nm])

    def bf16_step_own(i):
        c = wcopies[i % Rb]
        for nm, _, _ in shapes:
            B.gq_bf16_gemv(X[nm], c[nm], y=Yb[nm])

    for i in range(3):
        bf16_step_torch(i)
        bf16_step_own(i)
    torch.cuda.synchronize()
    t_own = graph_times(torch, stream, bf16_step_own, 2 * Rb)
    try:
        t_torch = graph_times(torch, stream, bf16_step_torch, 2 * Rb)
        torch_how = "HIP graph"
    except Exception as e:  # a library call that cannot be captured is timed eagerly
        log(f"hipBLASLt GEMV not capturable ({type(e).__name__}); timing eager launches")
        torch.cuda.synchronize()
        t_torch = [time_launches(torch, stream, bf16_step_torch, 2 * Rb) for _ in range(5)]
        torch_how = "eager launches"
    u_own, u_torch = float(np.median(t_own)), float(np.median(t_torch))
    t_bf16 = min(u_own, u_torch)
    bf16_per_shape = {}
    for nm, n, k in shapes:
        def one_own(i, nm=nm):
            B.gq_bf16_gemv(X[nm], wcopies[i % Rb][nm], y=Yb[nm])
        bf16_per_shape[nm] = round(graph_time(torch, stream, one_own, 2 * Rb), 3)
    ex["bf16_gemv_comparator"] = {
        "us_per_step": round(t_bf16, 2), "GB/s": round(bf16_bytes / (t_bf16 * 1e-6) / 1e9, 1),
        "hipblaslt_us_per_step": spread(t_torch), "hipblaslt_timing": torch_how,
        "gq_bf16_gemv_us_per_step": spread(t_own), "gq_bf16_gemv_per_shape_us": bf16_per_shape,
        "faster": "gq_bf16_gemv" if u_own <= u_torch else "hipBLASLt",
        "byte_ratio": round(bf16_bytes / sum(gemv_bytes(n, k, G) for _, n, k in shapes), 3),
        "speedup_w4a16_vs_bf16": round(t_bf16 / fused_step_us, 3)}
    log(f"bf16 GEMV step: own {u_own:.1f} us, hipBLASLt {u_torch:.1f} us; "
        f"W4A16 speedup {t_bf16 / fused_step_us:.2f}x")

    # ---- unfused comparator: gq_dequantize -> bf16 W^ in HBM -> bf16 product ----------
    # M = 1: the decode step with every weight first expanded into a bf16 buffer.
    Rq = len(W_copies)
    wh = {nm: torch.empty((n, k), dtype=torch.bfloat16, device=dev) for nm, n, k in shapes}

    def unfused_step(i):
        c = W_copies[i % Rq]
        for nm, _, _ in shapes:
            qw, s_, z_ = c[nm]
            B.gq_dequantize(qw, s_, z_, G, False, out=wh[nm])
            B.gq_bf16_gemv(X[nm], wh[nm], y=Yb[nm])
    unfused_step(0)
    t_unf = graph_times(torch, stream, unfused_step, Rq)
    unf_bytes = sum(gemv_bytes(n, k, G) + 4 * n * k for _, n, k in shapes)
    u_unf = float(np.median(t_unf))
    ex["unfused_m1"] = {
        "us_per_step": spread(t_unf), "bytes_per_step": unf_bytes,
        "bytes_vs_fused": round(unf_bytes / sum(gemv_bytes(n, k, G) for _, n, k in shapes), 3),
        "bytes_vs_bf16": round(unf_bytes / bf16_bytes, 3),
        "time_vs_fused": round(u_unf / fused_step_us, 3), "time_vs_bf16": round(u_unf / t_bf16, 3),
        "path": "gq_dequantize (bf16 out) then gq_bf16_gemv, per projection, rotating weight copies"}
    log(f"unfused decode step {u_unf:.1f} us ({u_unf / fused_step_us:.2f}x fused, "
        f"{u_unf / t_bf16:.2f}x bf16)")
    del wcopies, wb
    torch.cuda.empty_cache()

    # M = 2048: dequantize then hipBLASLt, against the fused GEMM and a plain bf16 GEMM.
    unf_pf = {}
    for name, n, k in shapes:
        _, xb = synth.prefill_case(name)
        xd = to_dev(xb)
        qw, s_, z_ = W[name]
        wb1 = torch.randn((n, k), dtype=torch.bfloat16, device=dev) * 0.02
        yp = torch.empty((2048, n), dtype=torch.bfloat16, device=dev)

        def unf(i):
            B.gq_dequantize(qw, s_, z_, G, False, out=wh[name])
            torch.matmul(xd, wh[name].t(), out=yp)

        def plain(i):
            torch.matmul(xd, wb1.t(), out=yp)
        for i in range(3):
            unf(i)
            plain(i)
        torch.cuda.synchronize()
        try:   # graphs, as for the fused GEMM: GPU time only
            t_u = graph_time(torch, stream, unf, 5, reps=3)
            t_p = graph_time(torch, stream, plain, 5, reps=3)
            how = "HIP graph"
        except Exception as e:  # a library call that cannot be captured is timed eagerly
            log(f"M=2048 comparator not capturable ({type(e).__name__}); timing eager launches")
            torch.cuda.synchronize()
            t_u = float(np.median([time_launches(torch, stream, unf, 5) for _ in range(3)]))
            t_p = float(np.median([time_launches(torch, stream, plain, 5) for _ in range(3)]))
            how = "eager launches"
        fl = 2.0 * 2048 * n * k
        unf_pf[name] = {"unfused_us": round(t_u, 2), "bf16_gemm_us": round(t_p, 2),
                        "fused_us": gemm[name]["us"], "timing": how,
                        "bf16_gemm_TFLOP/s": round(fl / (t_p * 1e-6) / 1e12, 1)}
        del xd, wb1, yp
    ex["unfused_and_bf16_m2048"] = unf_pf
    log(f"M=2048 unfused / bf16 / fused: {unf_pf}")
    del wh
    torch.cuda.empty_cache()

    # ---- group-size sweep on down [4096, 14336], M = 1, symmetric and asymmetric --------
    name = "down"
    n, k = synth.LLAMA3_8B_SHAPES[name]
    w, x = synth.decode_case(name)
    wd, xd = to_dev(w), to_dev(x)
    yd = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
    sweep = {}
    for sym in (True, False):
        for g in (32, 64, 128):
            codes, s_, z_ = B.gq_quantize_groups(wd, 4, g, sym)
            qw = B.gq_pack_int4(codes, sym)
            del codes
            gate(f"{name} g{g} {'sym' if sym else 'asym'}", w, x, qw, s_, z_, g, sym)
            one = (qw, s_, z_)
            byt = gemv_bytes(n, k, g, 1, sym)
            R = max(2, int(np.ceil(2 ** 30 / byt)))
            cp = [one] + [tuple(None if t is None else t.clone() for t in one) for _ in range(R - 1)]

            def fn(i, cp=cp, g=g, sym=sym):
                a, b, c = cp[i % len(cp)]
                B.gq_w4a16_gemv(xd, a, b, c, g, sym, y=yd)
            t = graph_times(torch, stream, fn, 2 * R)
            us = float(np.median(t))
            gbps = byt / (us * 1e-6) / 1e9
            sweep[f"{'sym' if sym else 'asym'}_g{g}"] = {
                "us": spread(t), "bytes": byt, "GB/s": round(gbps, 1),
                "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                "frac_of_read_ceiling": round(gbps / ceiling["GB/s"], 4)}
            del cp, one, qw, s_, z_
    ex["group_sweep_down_m1"] = sweep
    log(f"group sweep down M=1: { {k_: v['us']['median'] for k_, v in sweep.items()} }")
    del wd, xd, yd

    # ---- small batch M in {1,2,3,4,8,16}, symmetric g32, rotating weight copies -----
    sym_w, gate_w = {}, {}
    for name, n, k in shapes:
        w, _ = synth.decode_case(name)
        if name in ("o", "down"):  # K = 4096 and K = 14336: both kernels of each M
            gate_w[name] = w
        codes, s, _ = B.gq_quantize_groups(to_dev(w), 4, 32, True)
        sym_w[name] = (B.gq_pack_int4(codes, True), s)
        del codes
    sym_bytes = sum(sym_w[nm][0].numel() + 2 * sym_w[nm][1].numel() for nm, _, _ in shapes)
    Rs = max(2, int(np.ceil(2 ** 30 / sym_bytes)))
    sym_copies = [sym_w] + [{nm: tuple(t.clone() for t in sym_w[nm]) for nm, _, _ in shapes}
                            for _ in range(Rs - 1)]
    sb = {}
    for m in (1, 2, 3, 4, 8, 16):
        xs = {nm: to_dev(synth.activations(m, k, seed=2000 + synth.SHAPE_ORDER.index(nm))[0])
              for nm, _, k in shapes}
        ys = {nm: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for nm, n, _ in shapes}
        for nm, w in gate_w.items():
            xb = xs[nm].view(torch.int16).cpu().numpy().view(np.uint16)
            gate(f"{nm} M={m} sym g32", w, xb, *sym_w[nm], None, 32, True)

        def sb_step(i):
            c = sym_copies[i % Rs]
            for nm, _, _ in shapes:
                B.gq_w4a16_gemv(xs[nm], c[nm][0], c[nm][1], None, 32, True, y=ys[nm])
        sb_step(0)
        us = graph_time(torch, stream, sb_step, 4 * Rs)
        tot_b = sum(gemv_bytes(n, k, 32, m, True) for _, n, k in shapes)
        gbps = tot_b / (us * 1e-6) / 1e9
        sb[f"M={m}"] = {"us_per_step": round(us, 2), "GB/s": round(gbps, 1),
                        "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                        "TFLOP/s": round(2.0 * m * sum(n * k for _, n, k in shapes) / (us * 1e-6) / 1e12, 2),
                        "kernels": SMALL_BATCH_KERNELS[min(m, 5)]}
    del sym_copies, sym_w, gate_w
    ex["small_batch_sym_g32"] = sb
    log(f"small batch {sb}")

    # ---- super-block format GEMV, M = 1, 2, 4, 8, 16, rotating copies -------------------
    from oracle import gq_oracle as O

    def bits16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    q4 = {}
    for name in ("down", "gate_up"):
        n, k = synth.LLAMA3_8B_SHAPES[name]
        w, _ = synth.q4k_case(name)
        blocks = B.gq_q4k_quantize(to_dev(w))
        # parity gate: 256 sampled rows' blocks equal the oracle's bytes and the
        # GEMV on them meets the parity bar, at every M timed below
        rows = np.sort(np.random.default_rng(1).choice(n, 256, replace=False))
        bref = O.q4k_encode(O.q4k_quantize(O.bf16_to_f64(w[rows])))
        if not np.array_equal(blocks.cpu().numpy()[rows], bref):
            raise SystemExit(f"parity gate: super-block bytes of {name} differ from the oracle")
        wh = O.q4k_dequantize_fields(O.q4k_decode(bref))
        reps = max(2, int(np.ceil(2 ** 30 / blocks.numel())))
        bl = [blocks] + [blocks.clone() for _ in range(reps - 1)]
        for m in (1, 2, 4, 8, 16):
            _, x = synth.q4k_case(name, m)
            xd = to_dev(x)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            B.gq_q4k_gemv(xd, bl[0], y=y)
            ref = O.q4k_reference(x, bref)
            ok, rel, ratio = O.within_parity(O.bf16_to_f64(bits16(y))[:, rows], ref, O.bf16_to_f64(x), wh)
            if not ok:
                raise SystemExit(f"parity gate: super-block {name} M={m} relF {rel:.2e} max/allowed {ratio:.2f}")
            us = graph_time(torch, stream, lambda i: B.gq_q4k_gemv(xd, bl[i % reps], y=y), 4 * reps)
            byt = 144 * n * k // 256 + 2 * m * k + 2 * m * n
            q4[name if m == 1 else f"{name}_M{m}"] = {"us": round(us, 3), "GB/s": round(byt / (us * 1e-6) / 1e9, 1)}
        del bl, blocks
    ex["q4k_gemv_m1"] = {k_: v for k_, v in q4.items() if "_M" not in k_}
    ex["q4k_gemv_small_batch"] = {k_: v for k_, v in q4.items() if "_M" in k_}
    log(f"super-block GEMV {q4}")
    return ex


def cpu_baseline(args, O, host, shapes):
    """The oracle's W4A16 product (dequantize + float64 group-by-group matmul, as
    it stands) on a bounded sample of the decode workload: the first `rows`
    output rows of each projection, repeated until about `cpu_seconds` of work."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rows = 512
    packed = {}
    for name, n, k in shapes:
        w, x = host[name]
        codes, s, z = O.quantize_to_storage(w[:rows], 4, G, False)
        packed[name] = (x, O.pack_int4(codes, False), s, z)
    done_bytes, t_total, passes = 0, 0.0, 0
    while t_total < args.cpu_seconds:
        for name, n, k in shapes:
            x, qw, s, z = packed[name]
            t = time.perf_counter()
            O.w4a16_reference(x, qw, s, z, G, False)
            t_total += time.perf_counter() - t
            done_bytes += gemv_bytes(rows, k, G)
        passes += 1
    gbps = done_bytes / t_total / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} output rows of each of the 4 decode projections (M=1, asym g128), "
                      f"{passes} passes, {t_total:.1f} s of oracle W4A16 product (dequantize + float64 "
                      f"group-by-group matmul); host has {os.cpu_count()} logical CPUs"}


if __name__ == "__main__":
    main()
