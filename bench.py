"""Benchmark: quantized GEMV weight GB/s and fraction of MI355X HBM peak.

One step = one pass of the hot path over one synthetic input: qk_quantize_act of
the activation (once per distinct activation) followed by the workload's
qk_gemv launch(es).  Inputs are resident in HBM before timing starts.  Weight
matrices rotate over >= 512 MB of distinct copies (twice the 256 MB Infinity
Cache) so every step streams its weights from HBM.

Prints ONE JSON line on stdout (details on stderr):
  value      whole-job weight GB/s = steps * weight bytes per step / elapsed
  roofline   the GEMV kernels: algorithmic bytes per launch / mean kernel duration
             (HIP events recorded by the kernel launches themselves, on the
             launch stream; the quantize launches of the step record theirs too,
             reported as detail.quantize_kernel_us) against the 8 TB/s HBM peak
  cpu_baseline  the scalar C oracle on the host, single thread, on a bounded
             sample of the same workload (all_cores: the same sample on every
             usable host core at once)
  detail.read_stream_ceiling  qk_read_probe_ex over the same weight tensors: the
             bandwidth a launch that only reads those bytes reaches on the machine
Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]

Profiling helpers (no GPU use; they read rocprofv3 CSV output):
  --summarize-trace DIR         per-kernel durations of a --kernel-trace --stats run
  --summarize-pmc FDIR WDIR     HBM bytes per step from a FETCH_SIZE run and a
                                WRITE_SIZE run, scaled by the copy kernel that
                                --calibrate-copy adds to the profiled run
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix-core peak (5.0 POP/s)
ROTATE_BYTES = 512 * 1024 * 1024
CALIB_BYTES = 256 * 1024 * 1024  # the copy kernel reads and writes this much per dispatch
CSRC = os.path.join(ROOT, "quantized_gemv_quantize_amd", "csrc")
# sources of each kernel family; a recorded HBM traffic figure is used only while
# these files are unchanged since the counters were taken
KERNEL_SOURCES = {"gemv": ["qk_gemv.hip", "qk_device.h", "qk_internal.h"],
                  "gemm": ["qk_gemm.hip", "qk_device.h", "qk_internal.h"],
                  "dequant": ["qk_dequant.hip", "qk_device.h", "qk_internal.h"],
                  "quantize_row": ["qk_quantize.hip", "qk_device.h", "qk_internal.h"]}
METRIC = "quantized GEMV weight GB/s and % of HBM peak (Q4_K/Q6_K/Q8_0, batch 1)"
# The pages' own figures for these dot products (candle formats page, "实测：一次点积"):
# one 4096-element row against one activation row on one M2 Max CPU core, the row
# cache-resident, fastest of 9 batches; weight GB/s = row bytes / time.  Context for
# the bench line only: another machine, another memory level, another workload.
PAGES_CONTEXT = {
    "Q4_K": "Q4K x Q8K vec_dot 99.9 ns per 4096-element row (2304 B): 23.1 GB/s, one M2 Max core, cache-resident",
    "Q6_K": "Q6K x Q8K vec_dot 152.3 ns per 4096-element row (3360 B): 22.1 GB/s, one M2 Max core, cache-resident",
    "Q8_0": "Q8_0 x Q8_0 vec_dot 121.9 ns per 4096-element row (4352 B): 35.7 GB/s, one M2 Max core, cache-resident",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Workloads: a list of GEMVs sharing activations.  Each GEMV: (name, w_type,
# n_out, n_in, activation key).  Activations: key -> (act_type, n, ncols).
# ---------------------------------------------------------------------------

def workloads(qk):
    T4K, T6K, T40, T80 = qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q6_K, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q8_0
    T50, T5K = qk.QK_TYPE_Q5_0, qk.QK_TYPE_Q5_K
    T41, T51, T81 = qk.QK_TYPE_Q4_1, qk.QK_TYPE_Q5_1, qk.QK_TYPE_Q8_1
    T2K, T3K = qk.QK_TYPE_Q2_K, qk.QK_TYPE_Q3_K
    T8K = qk.QK_TYPE_Q8_K
    return {
        "q4_K_decode_4096x11008": {
            "gemvs": [("W", T4K, 4096, 11008, "x")], "acts": {"x": (T8K, 11008, 1)}},
        "q5_K_decode_4096x11008": {
            "gemvs": [("W", T5K, 4096, 11008, "x")], "acts": {"x": (T8K, 11008, 1)}},
        # the _1 weight formats against Q8_1 activations (candle VecDotType table)
        "q4_1_decode_4096x11008": {
            "gemvs": [("W", T41, 4096, 11008, "x")], "acts": {"x": (T81, 11008, 1)}},
        "q5_1_decode_4096x11008": {
            "gemvs": [("W", T51, 4096, 11008, "x")], "acts": {"x": (T81, 11008, 1)}},
        # the 2- and 3-bit K-quants (GGUF arrangement) against Q8_K
        "q2_K_decode_4096x11008": {
            "gemvs": [("W", T2K, 4096, 11008, "x")], "acts": {"x": (T8K, 11008, 1)}},
        "q3_K_decode_4096x11008": {
            "gemvs": [("W", T3K, 4096, 11008, "x")], "acts": {"x": (T8K, 11008, 1)}},
        "q4_K_4096x4096": {
            "gemvs": [("W_q4_K", T4K, 4096, 4096, "x")], "acts": {"x": (T8K, 4096, 1)}},
        "q4_0_4096x4096": {
            "gemvs": [("W_q4_0", T40, 4096, 4096, "x")], "acts": {"x": (T80, 4096, 1)}},
        "q5_0_4096x4096": {
            "gemvs": [("W", T50, 4096, 4096, "x")], "acts": {"x": (T80, 4096, 1)}},
        "ffn_7b_q4_K_q6_K": {
            "gemvs": [("gate", T4K, 11008, 4096, "x"), ("up", T4K, 11008, 4096, "x"),
                      ("down", T6K, 4096, 11008, "x2")],
            "acts": {"x": (T8K, 4096, 1), "x2": (T8K, 11008, 1)}},
        # the FFN decode step as one layer runs it: quantize x, gate + up in one
        # qk_gemv_pair launch with the SwiGLU epilogue (h), quantize h, down
        "ffn_7b_swiglu": {
            "gemvs": [("gate", T4K, 11008, 4096, "x"), ("up", T4K, 11008, 4096, "x"),
                      ("down", T6K, 4096, 11008, "h")],
            "acts": {"x": (T8K, 4096, 1), "h": (T8K, 11008, 1)}, "swiglu_pair": True},
        # the same step with Q5_K gate / up (the Q5_K_M layout of these layers)
        "ffn_7b_q5_K_swiglu": {
            "gemvs": [("gate", T5K, 11008, 4096, "x"), ("up", T5K, 11008, 4096, "x"),
                      ("down", T6K, 4096, 11008, "h")],
            "acts": {"x": (T8K, 4096, 1), "h": (T8K, 11008, 1)}, "swiglu_pair": True},
        "q6_K_head_32000x4096": {
            "gemvs": [("W", T6K, 32000, 4096, "x")], "acts": {"x": (T8K, 4096, 1)}},
        "q8_0_256x1024": {
            "gemvs": [("W", T80, 256, 1024, "x")], "acts": {"x": (T80, 1024, 1)}},
        "q4_K_batched_14336x4096_n16": {
            "gemvs": [("W", T4K, 14336, 4096, "X")], "acts": {"X": (T8K, 4096, 16)}},
        "q4_K_batched_14336x4096_n64": {
            "gemvs": [("W", T4K, 14336, 4096, "X")], "acts": {"X": (T8K, 4096, 64)}},
        # qk_dequantize_row of the whole Q6_K head matrix to f32 (no activations)
        "q6_K_dequantize_32000x4096": {
            "gemvs": [("W", T6K, 32000, 4096, None)], "acts": {}, "dequant": True},
        # qk_quantize_row of an f32 weight matrix to Q4_0 blocks (no activations)
        "q4_0_quantize_row_4096x11008": {
            "gemvs": [("W_f32", T40, 4096, 11008, None)], "acts": {}, "quantize_row": True},
    }


def host_inputs(name, qk):
    """Seeded synthetic inputs (numpy) of a workload: weights and f32 activations."""
    from quantized_gemv_quantize_amd import synth
    if name == "q4_K_decode_4096x11008":
        return synth.q4_K_decode_4096x11008()
    if name == "q5_K_decode_4096x11008":
        return synth.q5_K_decode_4096x11008()
    if name == "q2_K_decode_4096x11008":
        return synth.q2_K_decode_4096x11008()
    if name == "q3_K_decode_4096x11008":
        return synth.q3_K_decode_4096x11008()
    if name == "q4_1_decode_4096x11008":
        return synth.q4_1_decode_4096x11008()
    if name == "q5_1_decode_4096x11008":
        return synth.q5_1_decode_4096x11008()
    if name in ("q4_K_4096x4096", "q4_0_4096x4096"):
        return synth.q4_gemv_4096x4096()
    if name in ("ffn_7b_q4_K_q6_K", "ffn_7b_swiglu", "ffn_7b_q5_K_swiglu"):
        d = synth.ffn_7b_q5_K() if name == "ffn_7b_q5_K_swiglu" else synth.ffn_7b()
        d["h"] = d["x2"]  # initial contents of the gated activation buffer
        return d
    if name in ("q6_K_head_32000x4096", "q6_K_dequantize_32000x4096"):
        return synth.q6_K_head_32000x4096()
    if name.startswith("q4_K_batched"):
        d = synth.q4_K_batched_14336x4096()
        return {"W": d["W"], "X": d["X"]}
    if name == "q8_0_256x1024":
        return synth.q8_0_gemv_256x1024()
    if name == "q5_0_4096x4096":
        return synth.q5_0_gemv_4096x4096()
    if name == "q4_0_quantize_row_4096x11008":
        return synth.f32_weights_4096x11008()
    raise KeyError(name)


def gpu_copy_like(torch, w_type, n_out, n_in, gen):
    """One more weight matrix with the generator recipe of synth.py, drawn on the
    GPU from a seeded torch generator (uniform bytes; f16 scales uniform in the
    recipe's range; Q6_K int8 scales uniform in -64..63)."""
    from quantized_gemv_quantize_amd import synth
    bb = synth.BLOCK_BYTES[w_type]
    nb = n_in // synth.BLOCK_ELEMS[w_type]
    w = torch.randint(0, 256, (n_out, nb, bb), dtype=torch.uint8, device="cuda", generator=gen)

    def f16(lo, hi):
        v = torch.rand((n_out, nb), device="cuda", generator=gen, dtype=torch.float64) * (hi - lo) + lo
        return v.to(torch.float16).view(torch.uint8).reshape(n_out, nb, 2)

    if w_type in (synth.Q4_K, synth.Q5_K):
        w[:, :, 0:2] = f16(1e-4, 1e-3)
        w[:, :, 2:4] = f16(1e-4, 1e-3)
    elif w_type == synth.Q6_K:
        sc = torch.randint(-64, 64, (n_out, nb, 16), dtype=torch.int8, device="cuda", generator=gen)
        w[:, :, 192:208] = sc.view(torch.uint8)
        w[:, :, 208:210] = f16(1e-4, 1e-3)
    elif w_type == synth.Q4_0:
        w[:, :, 0:2] = f16(1e-3, 4e-3)
    elif w_type == synth.Q5_0:
        w[:, :, 0:2] = f16(5e-4, 2e-3)
    elif w_type == synth.Q2_K:
        w[:, :, 80:82] = f16(1e-4, 1e-3)
        w[:, :, 82:84] = f16(1e-4, 1e-3)
    elif w_type == synth.Q3_K:
        w[:, :, 108:110] = f16(1e-4, 1e-3)
    elif w_type in (synth.Q4_1, synth.Q5_1):
        w[:, :, 0:2] = f16(1e-3, 4e-3) if w_type == synth.Q4_1 else f16(5e-4, 2e-3)
        w[:, :, 2:4] = f16(-0.03, -0.005)
    else:
        raise ValueError("GPU copies are drawn for block-byte weight formats only")
    return w.reshape(n_out, nb * bb)


def cpu_baseline(name, wl, inputs, seconds, seconds_all=5.0):
    """The scalar C oracle on a bounded sample of the workload: the first rows of
    each GEMV, repeated until `seconds` have passed on one thread; then the same
    sample on every usable host core at once (one thread each, the C calls release
    the GIL) for `seconds_all`, reported beside it."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc
    sample_rows = {}

    def one_rep():
        """One pass over the sample; returns the bytes it covers."""
        done = 0
        if wl.get("dequant"):
            for wname, wt, n_out, n_in, _ in wl["gemvs"]:
                W = inputs[wname]
                rows = min(n_out, max(1, int(4e6 // n_in)))
                sample_rows[wname] = rows
                orc.dequantize(wt, W[:rows], rows * n_in)
                done += rows * W.shape[1] + 4 * rows * n_in
            return done
        if wl.get("quantize_row"):
            for wname, wt, n_out, n_in, _ in wl["gemvs"]:
                W = inputs[wname]
                rows = min(n_out, max(1, int(4e6 // n_in)))
                sample_rows[wname] = rows
                b = orc.quantize(wt, W[:rows])
                done += 4 * rows * n_in + b.size
            return done
        if wl.get("swiglu_pair"):
            # gate / up rows with the SwiGLU epilogue; down rows against the
            # quantized stand-in activation (the full h needs every gate row)
            (gn, gt, g_out, g_in, _), (un, _, _, _, _), (dn, dt, d_out, d_in, _) = wl["gemvs"]
            xq = orc.quantize(orc.Q8_K, inputs["x"][None, :])
            rows = min(g_out, max(1, int(4e6 // g_in)))
            g, _ = orc.gemv(gt, inputs[gn][:rows], rows, g_in, xq, 1)
            u, _ = orc.gemv(gt, inputs[un][:rows], rows, g_in, xq, 1)
            orc.swiglu(g, u)
            hq = orc.quantize(orc.Q8_K, inputs["h"][None, :])
            rows_d = min(d_out, max(1, int(4e6 // d_in)))
            orc.gemv(dt, inputs[dn][:rows_d], rows_d, d_in, hq, 1)
            sample_rows.update({gn: rows, un: rows, dn: rows_d})
            return 2 * rows * inputs[gn].shape[1] + rows_d * inputs[dn].shape[1]
        for key, (at, n, ncols) in wl["acts"].items():
            x = inputs[key] if inputs[key].ndim == 2 else inputs[key][None, :]
            xq = orc.quantize(at, x[:ncols])
            for wname, wt, n_out, n_in, akey in wl["gemvs"]:
                if akey != key:
                    continue
                W = inputs[wname]
                rows = min(n_out, max(1, int(4e6 // n_in)))  # about 4 M weights per GEMV
                sample_rows[wname] = rows
                orc.gemv(wt, W[:rows], rows, n_in, xq, ncols)
                done += rows * W.shape[1]
        return done

    def run_for(budget):
        t_end = time.perf_counter() + budget
        done, reps = 0, 0
        while True:
            done += one_rep()
            reps += 1
            if time.perf_counter() >= t_end:
                return done, reps

    t0 = time.perf_counter()
    done_bytes, reps = run_for(seconds)
    dt = time.perf_counter() - t0
    desc = ", ".join(f"{k}: first {r} rows" for k, r in sample_rows.items())
    out = {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{desc}; {_kind(wl)} repeated "
                     f"{reps}x in {dt:.1f} s, single thread on {_host_cpu()}"}
    if seconds_all > 0:
        nthreads = min(len(os.sched_getaffinity(0)), 16)  # the host share of one GPU
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            res = list(ex.map(lambda _: run_for(seconds_all), range(nthreads)))
        dt_all = time.perf_counter() - t0
        out["all_cores"] = {"value": round(sum(r[0] for r in res) / dt_all / 1e9, 4), "cores": nthreads,
                            "sample": f"the same sample on {nthreads} threads at once, "
                                      f"{sum(r[1] for r in res)} passes in {dt_all:.1f} s"}
    return out


def _host_cpu():
    """CPU model and logical CPU count of the host running the oracle."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model} ({os.cpu_count()} logical CPUs visible)"


def _kind(wl):
    if wl.get("dequant"):
        return "dequantize"
    if wl.get("swiglu_pair"):
        return "quantize x + gate/up + SwiGLU + quantize h + down"
    return "weight quantize" if wl.get("quantize_row") else "quantize + GEMV"


def kernel_family(workload):
    if workload.startswith("q4_K_batched"):
        return "gemm"
    if "quantize_row" in workload:
        return "quantize_row"
    return "dequant" if "dequantize" in workload else "gemv"


def source_hash(family):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"{kernel_family(workload)}_{workload}_pmc_traffic.txt")


def recorded_traffic(workload):
    """HBM bytes per step of the GEMV kernels from the committed counter summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash(kernel_family(workload)):
        return None
    try:
        return int(kv["traffic_bytes_per_step"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(wl, qk):
    """Weights + activation blocks + f32 outputs of the GEMV launches of one step
    (for a dequantize workload: the blocks read plus the f32 values written; for a
    weight-quantize workload: the f32 values read plus the blocks written; the
    gate / up pair reads its activation row once and writes one f32 per row)."""
    total = 0
    if wl.get("swiglu_pair"):
        (_, gt, g_out, g_in, gk), _, (_, dt, d_out, d_in, dk) = wl["gemvs"]
        return (2 * qk.qk_row_bytes(gt, g_in) * g_out + qk.qk_row_bytes(wl["acts"][gk][0], g_in)
                + 4 * g_out + qk.qk_row_bytes(dt, d_in) * d_out
                + qk.qk_row_bytes(wl["acts"][dk][0], d_in) + 4 * d_out)
    for _, wt, n_out, n_in, akey in wl["gemvs"]:
        if wl.get("dequant") or wl.get("quantize_row"):
            total += qk.qk_row_bytes(wt, n_in) * n_out + 4 * n_out * n_in
            continue
        at, n, ncols = wl["acts"][akey]
        total += qk.qk_row_bytes(wt, n_in) * n_out + qk.qk_row_bytes(at, n) * ncols + 4 * n_out * ncols
    return total


def _short(name):
    if _is_calib(name):
        return f"copy kernel (torch.neg, {CALIB_BYTES >> 20} MiB read + write)"
    name = name.replace("qk::(anonymous namespace)::", "")
    return name.split("(")[0] if name.startswith(("void gemv", "void gemm", "gemv", "gemm", "quantize",
                                                      "void quantize", "dequant", "void dequant")) else name[:90]


def _is_calib(name):
    """The --calibrate-copy kernel (torch.neg over CALIB_BYTES of f32)."""
    return "qk::" not in name and "neg" in name.lower()


def _is_family(name, family):
    """Library kernels of one family: gemv_*, gemm_*, dequant_* or quantize_row_*."""
    return "qk::" in name and f"{family}_" in name


def summarize_trace(d):
    """Per-kernel durations from a rocprofv3 --kernel-trace --stats output directory."""
    stats = glob.glob(os.path.join(d, "*kernel_stats.csv"))
    trace = glob.glob(os.path.join(d, "*kernel_trace.csv"))
    if stats:
        print("rocprofv3 --stats (library kernels):")
        print(f"  {'kernel':60s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s}")
        for r in csv.DictReader(open(stats[0])):
            if "qk::" in r["Name"] or _is_calib(r["Name"]):
                print(f"  {_short(r['Name']):60s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:9.3f} "
                      f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f}")
    if trace:
        rows = [r for r in csv.DictReader(open(trace[0]))
                if "qk::" in r["Kernel_Name"] or _is_calib(r["Kernel_Name"])]
        names = sorted({r["Kernel_Name"] for r in rows})
        print("per-dispatch trace, split into back-to-back runs (gaps > 1 ms):")
        for nm in names:
            rr = sorted((r for r in rows if r["Kernel_Name"] == nm), key=lambda r: int(r["Start_Timestamp"]))
            dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rr]
            runs, cur = [], [dur[0]]
            for i in range(1, len(rr)):
                if int(rr[i]["Start_Timestamp"]) - int(rr[i - 1]["End_Timestamp"]) > 1_000_000:
                    runs.append(cur)
                    cur = []
                cur.append(dur[i])
            runs.append(cur)
            print(f"  {_short(nm)}")
            for r in runs:
                print(f"    {len(r):5d} dispatches: mean {np.mean(r):8.3f} us  median {np.median(r):8.3f}"
                      f"  p10 {np.percentile(r, 10):8.3f}  p90 {np.percentile(r, 90):8.3f}")


def _counter_means(d):
    """Kernel name -> (dispatches, mean counter value per dispatch) of a --pmc run."""
    files = glob.glob(os.path.join(d, "*counter_collection.csv"))
    if not files:
        sys.exit(f"no counter_collection.csv under {d}")
    acc = {}
    for r in csv.DictReader(open(files[0])):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (nm, _), v in acc.items():
        per.setdefault(nm, []).append(v)
    return {nm: (len(v), float(np.mean(v)), float(np.sum(v))) for nm, v in per.items()}


def summarize_pmc(fdir, wdir, workload):
    """HBM bytes per step of the workload's GEMV kernels, from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for
    the calibration copy kernel (CALIB_BYTES read + CALIB_BYTES written)."""
    import quantized_gemv_quantize_amd as qk  # constants only; the library is not loaded
    wl = workloads(qk)[workload]
    n_g = 2 if wl.get("swiglu_pair") else len(wl["gemvs"])  # library kernel launches per step
    out = {}
    for tag, d in (("FETCH_SIZE", fdir), ("WRITE_SIZE", wdir)):
        m = _counter_means(d)
        calib = [v for nm, v in m.items() if _is_calib(nm)]
        if not calib:
            sys.exit(f"{tag}: no calibration copy kernel in {d} (run bench.py with --calibrate-copy)")
        c_n, c_mean, _ = calib[0]
        factor = CALIB_BYTES / (c_mean * 1024.0)
        g = {nm: v for nm, v in m.items() if _is_family(nm, kernel_family(workload))}
        disp = sum(v[0] for v in g.values())
        steps = disp / n_g
        per_step_kib = sum(v[2] for v in g.values()) / steps
        out[tag] = (factor, per_step_kib, c_mean, c_n, g)
    alg = algorithmic_bytes(wl, qk)
    fetch = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][1] * 1024.0
    write = out["WRITE_SIZE"][0] * out["WRITE_SIZE"][1] * 1024.0
    print(f"workload: {workload}")
    print(f"kernel_family: {kernel_family(workload)}")
    print(f"source_sha256: {source_hash(kernel_family(workload))}")
    for tag in ("FETCH_SIZE", "WRITE_SIZE"):
        factor, per_step, c_mean, c_n, g = out[tag]
        print(f"{tag.lower()}_calibration: copy kernel {c_mean:.1f} KiB per dispatch over {c_n} dispatches "
              f"for {CALIB_BYTES} bytes -> factor {factor:.4f}")
        for nm, (n, mean, _) in sorted(g.items()):
            print(f"  {_short(nm)}: {n} dispatches, mean {mean:.1f} KiB (raw)")
        print(f"{tag.lower()}_bytes_per_step: {int(round(factor * per_step * 1024.0))}")
    print(f"traffic_bytes_per_step: {int(round(fetch + write))}")
    print(f"algorithmic_bytes_per_step: {alg}")
    print(f"traffic_over_algorithmic: {(fetch + write) / alg:.4f}")


# Read-probe variants of the sweep: (kilobytes per wavefront, persistent grid
# workgroups or 0 for one wavefront per group, non-temporal loads)
SWEEP_VARIANTS = [(2, 0, 0), (1, 0, 0), (4, 0, 0), (8, 0, 0), (16, 0, 0), (2, 0, 1), (8, 0, 1),
                  (2, 256, 0), (2, 512, 0), (2, 1024, 0), (2, 2048, 0), (8, 256, 0), (8, 1024, 0),
                  (16, 256, 0), (16, 512, 0)]
SWEEP_SIZES = [4_194_304, 8_388_608, 16_777_216, 25_362_432, 33_030_144, 67_108_864, 134_217_728,
               268_435_456, 536_870_912]


def read_sweep(steps, warmup):
    """Read-only launches of growing size and every probe load pattern: per launch
    the kernel time from events the launch records itself (launches back to back
    behind a stream hold, each reading a different copy out of a 2 GiB pool, so no
    launch finds its bytes in the 256 MB Infinity Cache), then a least-squares fit
    t = t0 + bytes / BW per pattern over the sizes of 8 MB and up."""
    import torch

    import quantized_gemv_quantize_amd as qk
    torch.cuda.set_device(0)
    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for off in range(0, pool_bytes, 256 << 20):
        pool[off:off + (256 << 20)].random_(0, 256, generator=gen)
    outs = torch.empty((pool_bytes // 1024,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    torch.cuda._sleep(1_000_000)
    s1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(s0.elapsed_time(s1), 1e-3)
    results = {}
    for size in SWEEP_SIZES:
        copies = pool_bytes // size
        for var in SWEEP_VARIANTS:
            kb, grid, nt = var
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for e0, e1 in ev:
                e0.record(stream)
                e1.record(stream)
            for k in range(warmup):
                src = pool[(k % copies) * size:]
                qk.qk_read_probe_ex(src, size, kb, grid, nt, out=outs)
            torch.cuda.synchronize()
            hold = torch.cuda.Event()
            torch.cuda._sleep(int(cycles_per_ms * (0.05 * steps + 20.0)))
            hold.record(stream)
            for k in range(steps):
                src = pool[((warmup + k) % copies) * size:]
                qk.qk_read_probe_ex(src, size, kb, grid, nt, out=outs, ev_start=ev[k][0], ev_stop=ev[k][1])
            held = not hold.query()
            torch.cuda.synchronize()
            us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
            results[(size, var)] = (float(np.median(us)), float(np.mean(us)), held)
        best = min(SWEEP_VARIANTS, key=lambda v: results[(size, v)][0])
        log(f"[sweep] {size / 1e6:8.2f} MB: best {best} {results[(size, best)][0]:.3f} us "
            f"({size / results[(size, best)][0] / 1e3 / HBM_PEAK_GBS:.3f} of peak)")

    def name(v):
        kb, grid, nt = v
        return f"{kb:2d} KB/wave, " + (f"grid {grid:4d}" if grid else "grid all ") + (", nt" if nt else "    ")

    print("read-only probe launches: median kernel time (us) / fraction of the 8 TB/s HBM peak")
    print(f"  {'pattern':28s}" + "".join(f"{s / 1e6:>13.1f}" for s in SWEEP_SIZES) + "   fit t0 (us)  BW (GB/s)")
    fits = {}
    for v in SWEEP_VARIANTS:
        xs = np.array([s for s in SWEEP_SIZES if s >= 8_000_000], dtype=np.float64)
        ts = np.array([results[(s, v)][0] for s in xs.astype(np.int64)])
        A = np.stack([np.ones_like(xs), xs], axis=1)
        (t0, inv_bw), *_ = np.linalg.lstsq(A, ts, rcond=None)
        fits[v] = (float(t0), float(1e-3 / inv_bw))  # GB/s
        cells = "".join(f"{results[(s, v)][0]:7.2f}/{s / results[(s, v)][0] / 1e3 / HBM_PEAK_GBS:.2f}"
                        for s in SWEEP_SIZES)
        print(f"  {name(v):28s}{cells}   {fits[v][0]:8.3f}  {fits[v][1]:9.1f}")
    held_all = all(r[2] for r in results.values())
    print(f"all timed launches queued behind the stream hold: {held_all}")
    print("best pattern per size, and the fitted line's time and fraction at that size:")
    for s in SWEEP_SIZES:
        best = min(SWEEP_VARIANTS, key=lambda v: results[(s, v)][0])
        t_best = results[(s, best)][0]
        bfit = min(SWEEP_VARIANTS, key=lambda v: fits[v][0] + s / (fits[v][1] * 1e3))
        t_fit = fits[bfit][0] + s / (fits[bfit][1] * 1e3)
        print(f"  {s:>11d} B: {name(best)} {t_best:8.3f} us = {s / t_best / 1e3 / HBM_PEAK_GBS:.3f} of peak; "
              f"fitted line {t_fit:8.3f} us = {s / t_fit / 1e3 / HBM_PEAK_GBS:.3f} ({name(bfit)})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="q4_K_decode_4096x11008")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB read + write kernel (counter calibration)")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--read-sweep", action="store_true",
                    help="time read-only probe launches over sizes and load patterns (no workload)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return
    if args.read_sweep:
        read_sweep(args.steps, args.warmup)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the GEMV library runs on a single MI355X, "
              "so --gpus must be 1 (multi-GPU sharding is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_gemv_quantize_amd as qk

    torch.cuda.set_device(0)
    wls = workloads(qk)
    if args.workload not in wls:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(wls)}")
    wl = wls[args.workload]
    log(f"[bench] workload {args.workload}: generating inputs")
    inputs = host_inputs(args.workload, qk)
    if args.workload == "q8_0_256x1024":
        # Q8_0 weights are made by the library's own quantizer from the f32 draw
        Wf = torch.from_numpy(inputs["W_f32"]).cuda()
        inputs["W"] = qk.qk_quantize_act(qk.QK_TYPE_Q8_0, Wf).cpu().numpy()

    step_w_bytes = sum(qk.qk_row_bytes(t, n_in) * n_out for _, t, n_out, n_in, _ in wl["gemvs"])
    quant_row = bool(wl.get("quantize_row"))
    # the rotated inputs: weight blocks, or the f32 weights a weight-quantize step reads
    resident = (sum(4 * n_out * n_in for _, _, n_out, n_in, _ in wl["gemvs"]) if quant_row
                else step_w_bytes)
    copies = max(1, -(-ROTATE_BYTES // resident))
    dev_w = []  # per copy: list of weight tensors, one per GEMV
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    for c in range(copies):
        mats = []
        for wname, wt, n_out, n_in, _ in wl["gemvs"]:
            if quant_row and c > 0:
                # f32 weights N(0, 0.02), as synth's draw, from the seeded generator
                mats.append(torch.randn((n_out, n_in), device="cuda", generator=gen) * 0.02)
            elif c == 0 or wt == qk.QK_TYPE_Q8_0:
                src = torch.from_numpy(np.ascontiguousarray(inputs[wname])).cuda()
                mats.append(src if c == 0 else src.clone())
            else:
                mats.append(gpu_copy_like(torch, wt, n_out, n_in, gen))
        dev_w.append(mats)
    acts = {}
    for key, (at, n, ncols) in wl["acts"].items():
        x = inputs[key] if inputs[key].ndim == 2 else inputs[key][None, :]
        xf = torch.from_numpy(np.ascontiguousarray(x[:ncols])).cuda()
        xq = torch.empty((ncols, qk.qk_row_bytes(at, n)), dtype=torch.uint8, device="cuda")
        acts[key] = (at, xf, xq)
    if wl.get("dequant"):
        ys = [torch.empty((n_out * n_in,), dtype=torch.float32, device="cuda")
              for _, _, n_out, n_in, _ in wl["gemvs"]]
    elif quant_row:
        ys = [torch.empty((qk.qk_row_bytes(wt, n_in) * n_out,), dtype=torch.uint8, device="cuda")
              for _, wt, n_out, n_in, _ in wl["gemvs"]]
    else:
        ys = [torch.empty((ncols_of(wl, akey), n_out), dtype=torch.float32, device="cuda")
              for _, _, n_out, _, akey in wl["gemvs"]]
    torch.cuda.synchronize()
    log(f"[bench] {copies} weight copies x {step_w_bytes / 1e6:.2f} MB resident; "
        f"warmup {args.warmup}, steps {args.steps}")

    swiglu = bool(wl.get("swiglu_pair"))
    timed_names = ["gate_up", "down"] if swiglu else [gv[0] for gv in wl["gemvs"]]
    n_g = len(timed_names)
    quant_names = list(acts)  # one activation quantize per key (x, then h for the FFN step)
    n_q = len(quant_names)

    def quantize(i, at, xf, xq, qevs):
        if qevs is None:
            qk.qk_quantize_act(at, xf, xq)
        else:
            qk.qk_quantize_act_timed(at, xf, xq, qevs[i][0], qevs[i][1])

    def step(k, evs=None, qevs=None):
        mats = dev_w[k % copies]
        if swiglu:
            (_, gt, g_out, g_in, _), _, (_, dt, d_out, d_in, _) = wl["gemvs"]
            at, xf, xq = acts["x"]
            _, h, hq = acts["h"]
            quantize(0, at, xf, xq, qevs)
            if evs is None:
                qk.qk_gemv_pair(gt, mats[0], mats[1], g_out, g_in, xq, 1, qk.QK_EPI_SWIGLU, h)
            else:
                qk.qk_gemv_pair_timed(gt, mats[0], mats[1], g_out, g_in, xq, 1, qk.QK_EPI_SWIGLU, h,
                                      evs[0][0], evs[0][1])
            quantize(1, acts["h"][0], h, hq, qevs)
            if evs is None:
                qk.qk_gemv(dt, mats[2], d_out, d_in, hq, 1, ys[2])
            else:
                qk.qk_gemv_timed(dt, mats[2], d_out, d_in, hq, 1, ys[2], evs[1][0], evs[1][1])
            return
        for i, (at, xf, xq) in enumerate(acts.values()):
            quantize(i, at, xf, xq, qevs)
        for g, (wname, wt, n_out, n_in, akey) in enumerate(wl["gemvs"]):
            if wl.get("dequant") or quant_row:
                if evs is not None:
                    evs[g][0].record(stream)
                if quant_row:
                    qk.qk_quantize_row(wt, mats[g], ys[g])
                else:
                    qk.qk_dequantize_row(wt, mats[g], n_out * n_in, ys[g])
                if evs is not None:
                    evs[g][1].record(stream)
                continue
            xq = acts[akey][2]
            ncols = acts[akey][1].shape[0]
            if evs is None:
                qk.qk_gemv(wt, mats[g], n_out, n_in, xq, ncols, ys[g])
            else:
                e0, e1 = evs[g]
                qk.qk_gemv_timed(wt, mats[g], n_out, n_in, xq, ncols, ys[g], e0, e1)

    tw = time.perf_counter()
    for k in range(args.warmup):
        step(k)
    enqueue_ms_per_step = (time.perf_counter() - tw) * 1e3 / max(args.warmup, 1)
    torch.cuda.synchronize()

    # Region A - whole job.  The K steps are captured once into a HIP graph and
    # replayed, so the timed region holds no host-side enqueue work; events on the
    # launch stream bracket the replay.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(args.steps):
            step(args.warmup + k)
    graph.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    wall0 = time.perf_counter()
    t_start.record(stream)
    graph.replay()
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = t_start.elapsed_time(t_stop)
    # weight bytes per step; a dequantize workload counts the blocks read plus the f32
    # written, a weight-quantize workload the f32 read plus the blocks written
    value_bytes = algorithmic_bytes(wl, qk) if (wl.get("dequant") or quant_row) else step_w_bytes
    value = value_bytes * args.steps / (elapsed_ms / 1e3) / 1e9

    # Region B - the same K steps launched one by one; every kernel launch of the
    # step (the activation quantize as well as the GEMV) records a start / stop
    # event pair with its own kernel timestamps (HIP extended launch), giving
    # kernel durations free of enqueue gaps.  Timing every kernel the same way
    # matters: a launch-recorded start event on a kernel whose predecessor was
    # launched without events also takes in part of the boundary between the two
    # (about 1.7 us here), which rocprofv3's dispatch timestamps do not show.
    # torch creates the underlying events on their first record.
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_g)] for _ in range(args.steps)]
    qev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_q)] for _ in range(args.steps)]
    for per in ev + qev:
        for e0, e1 in per:
            e0.record(stream)
            e1.record(stream)
    torch.cuda.synchronize()
    # A bounded spin kernel holds the stream while the host enqueues all K steps,
    # so the GPU then runs them back to back as in the graph replay (an idle GPU
    # between host launches would add a start-up cost to every kernel).
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    torch.cuda._sleep(1_000_000)
    s1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(s0.elapsed_time(s1), 1e-3)
    hold_ms = 10.0 * enqueue_ms_per_step * args.steps + 20.0  # profilers slow the enqueue
    e_start = torch.cuda.Event(enable_timing=True)
    e_stop = torch.cuda.Event(enable_timing=True)
    hold_done = torch.cuda.Event()
    torch.cuda._sleep(int(cycles_per_ms * hold_ms))
    hold_done.record(stream)
    e_start.record(stream)
    for k in range(args.steps):
        step(args.warmup + k, ev[k], qev[k])
    e_stop.record(stream)
    backlog = not hold_done.query()  # still spinning: every step was queued in time
    torch.cuda.synchronize()
    eager_ms = e_start.elapsed_time(e_stop)
    if not backlog:
        log("[bench] warning: the stream hold ended before all steps were enqueued")

    kern_ms = np.array([[e0.elapsed_time(e1) for e0, e1 in per] for per in ev])  # [steps, n_g]
    gemv_ms_mean = kern_ms.sum(axis=1).mean()
    quant_ms = (np.array([[e0.elapsed_time(e1) for e0, e1 in per] for per in qev])
                if n_q else np.zeros((args.steps, 0)))  # [steps, n_q]

    # Region C - the read-stream ceiling: the library's read-only probe kernel over
    # the same weight tensors (same rotation, one launch per tensor, launch-recorded
    # events, back to back behind a stream hold), i.e. what HBM gives a launch that
    # reads the same bytes and does nothing else.  Two load patterns are timed: the
    # default (one wavefront per 2 KB group) and the fastest of the committed sweep
    # at 17-33 MB (2 KB groups, a persistent grid of 1024 four-wavefront
    # workgroups); the faster one is the ceiling.
    ceiling = None
    if not (wl.get("dequant") or quant_row):
        nbytes = [m.numel() // 16 * 16 for m in dev_w[0]]
        pouts = [torch.empty(((nb_ + 2047) // 2048,), dtype=torch.int32, device="cuda")
                 for nb_ in nbytes]
        patterns = {"2 KB per wavefront, one wavefront per group": 0,
                    "2 KB groups, persistent grid of 1024 workgroups": 1024}
        probe_us = {}
        backlog2 = True
        for pname, grid_blocks in patterns.items():
            pev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in nbytes] for _ in range(args.steps)]
            for per in pev:
                for e0, e1 in per:
                    e0.record(stream)
                    e1.record(stream)
            for k in range(args.warmup):
                for g, nb_ in enumerate(nbytes):
                    qk.qk_read_probe_ex(dev_w[k % copies][g], nb_, 2, grid_blocks, 0, out=pouts[g])
            torch.cuda.synchronize()
            hold2 = torch.cuda.Event()
            torch.cuda._sleep(int(cycles_per_ms * hold_ms))
            hold2.record(stream)
            for k in range(args.steps):
                for g, nb_ in enumerate(nbytes):
                    e0, e1 = pev[k][g]
                    qk.qk_read_probe_ex(dev_w[(args.warmup + k) % copies][g], nb_, 2, grid_blocks, 0,
                                        out=pouts[g], ev_start=e0, ev_stop=e1)
            backlog2 = backlog2 and not hold2.query()
            torch.cuda.synchronize()
            probe_us[pname] = float(np.array([[e0.elapsed_time(e1) for e0, e1 in per]
                                              for per in pev]).sum(axis=1).mean() * 1e3)
        best = min(probe_us, key=probe_us.get)
        probe_ms = probe_us[best] / 1e3
        ceiling = {"kernel": "qk_read_probe_ex (loads of the same weight bytes only; one launch per "
                             "weight tensor, launch-recorded events, back to back)" +
                             ("" if backlog2 else " (hold ended early)"),
                   "pattern": best,
                   "us_per_step_by_pattern": {k: round(v, 3) for k, v in probe_us.items()},
                   "us_per_step": round(float(probe_ms * 1e3), 3),
                   "weight_GBps": round(sum(nbytes) / (probe_ms / 1e3) / 1e9, 1),
                   "frac_of_hbm_peak": round(sum(nbytes) / (probe_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "gemv_frac_of_ceiling": round(float(probe_ms / gemv_ms_mean), 4)}
        log(f"[bench] read-stream ceiling {ceiling['us_per_step']} us/step "
            f"({ceiling['weight_GBps']} GB/s, {best}); GEMV at {ceiling['gemv_frac_of_ceiling']:.3f} of it")

    alg_bytes = algorithmic_bytes(wl, qk)
    achieved = alg_bytes / (gemv_ms_mean / 1e3) / 1e9
    def stats_us(col):
        return {"mean": round(float(col.mean() * 1e3), 3),
                "p10": round(float(np.percentile(col, 10) * 1e3), 3),
                "p50": round(float(np.percentile(col, 50) * 1e3), 3),
                "p90": round(float(np.percentile(col, 90) * 1e3), 3)}

    per_kernel_us = {timed_names[g]: stats_us(kern_ms[:, g]) for g in range(n_g)}
    quant_kernel_us = {quant_names[i]: stats_us(quant_ms[:, i]) for i in range(n_q)}
    log(f"[bench] graph replay {elapsed_ms:.3f} ms over {args.steps} steps "
        f"({elapsed_ms / args.steps * 1e3:.2f} us/step, host wall {wall * 1e3:.1f} ms); "
        f"eager {eager_ms / args.steps * 1e3:.2f} us/step; GEMV kernel time per step "
        f"{gemv_ms_mean * 1e3:.2f} us; per kernel {per_kernel_us}")

    if args.calibrate_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(args.workload, wl, inputs, args.cpu_seconds)

    first = wl["gemvs"][0]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed_ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "gemvs": [f"{qk.TYPE_NAMES[t]} {n_out}x{n_in}" for _, t, n_out, n_in, _ in wl["gemvs"]],
            "batch": acts[first[4]][1].shape[0] if first[4] is not None else None,
            "weight_bytes_per_step": step_w_bytes,
            "value_bytes_per_step": value_bytes,
            "weight_copies_rotated": copies,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(args.workload),
        },
        "cpu_baseline": cpu,
        "detail": {"gemv_kernel_us_per_step": round(float(gemv_ms_mean * 1e3), 3),
                   "kernel_timing": ("events recorded on the launch stream around each kernel"
                                     if (wl.get("dequant") or quant_row) else
                                     "HIP events recorded by every kernel launch of the step "
                                     "(activation quantize and GEMV)") +
                                    ", steps run back to back behind a stream hold" +
                                    ("" if backlog else " (hold ended early)"),
                   "traffic_unit": "bytes per step (FETCH_SIZE + WRITE_SIZE, copy-kernel scaled)",
                   "eager_us_per_step": round(eager_ms / args.steps * 1e3, 3),
                   "gemv_kernel_us": per_kernel_us,
                   "quantize_kernel_us": quant_kernel_us or None,
                   "algorithmic_bytes_per_step_gemv": alg_bytes,
                   "read_stream_ceiling": ceiling,
                   "pages_context": {k: v for k, v in PAGES_CONTEXT.items()
                                     if any(qk.TYPE_NAMES[t] == k for _, t, _, _, _ in wl["gemvs"])} or None},
    }
    if kernel_family(args.workload) == "gemm":
        # the batched path is also a contraction: 2 int8 ops per weight and column
        # (multiply, add), against the dense int8 matrix-core peak
        ops = sum(2 * n_out * n_in * ncols_of(wl, akey) for _, _, n_out, n_in, akey in wl["gemvs"])
        tops = ops / (gemv_ms_mean / 1e3) / 1e12
        out["detail"]["int8_tops"] = round(tops, 2)
        out["detail"]["int8_frac_of_dense_peak"] = round(tops / INT8_PEAK_TOPS, 4)
    print(json.dumps(out), flush=True)


def ncols_of(wl, akey):
    return wl["acts"][akey][2]


if __name__ == "__main__":
    main()
