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
             launch stream) against the 8 TB/s HBM peak
  cpu_baseline  the scalar C oracle on the host, single thread, on a bounded
             sample of the same workload
Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 * 1024 * 1024
METRIC = "quantized GEMV weight GB/s and % of HBM peak (Q4_K/Q6_K/Q8_0, batch 1)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Workloads: a list of GEMVs sharing activations.  Each GEMV: (name, w_type,
# n_out, n_in, activation key).  Activations: key -> (act_type, n, ncols).
# ---------------------------------------------------------------------------

def workloads(qk):
    T4K, T6K, T40, T80 = qk.QK_TYPE_Q4_K, qk.QK_TYPE_Q6_K, qk.QK_TYPE_Q4_0, qk.QK_TYPE_Q8_0
    T8K = qk.QK_TYPE_Q8_K
    return {
        "q4_K_decode_4096x11008": {
            "gemvs": [("W", T4K, 4096, 11008, "x")], "acts": {"x": (T8K, 11008, 1)}},
        "q4_K_4096x4096": {
            "gemvs": [("W_q4_K", T4K, 4096, 4096, "x")], "acts": {"x": (T8K, 4096, 1)}},
        "q4_0_4096x4096": {
            "gemvs": [("W_q4_0", T40, 4096, 4096, "x")], "acts": {"x": (T80, 4096, 1)}},
        "ffn_7b_q4_K_q6_K": {
            "gemvs": [("gate", T4K, 11008, 4096, "x"), ("up", T4K, 11008, 4096, "x"),
                      ("down", T6K, 4096, 11008, "x2")],
            "acts": {"x": (T8K, 4096, 1), "x2": (T8K, 11008, 1)}},
        "q6_K_head_32000x4096": {
            "gemvs": [("W", T6K, 32000, 4096, "x")], "acts": {"x": (T8K, 4096, 1)}},
        "q8_0_256x1024": {
            "gemvs": [("W", T80, 256, 1024, "x")], "acts": {"x": (T80, 1024, 1)}},
        "q4_K_batched_14336x4096_n16": {
            "gemvs": [("W", T4K, 14336, 4096, "X")], "acts": {"X": (T8K, 4096, 16)}},
        "q4_K_batched_14336x4096_n64": {
            "gemvs": [("W", T4K, 14336, 4096, "X")], "acts": {"X": (T8K, 4096, 64)}},
    }


def host_inputs(name, qk):
    """Seeded synthetic inputs (numpy) of a workload: weights and f32 activations."""
    from quantized_gemv_quantize_amd import synth
    if name == "q4_K_decode_4096x11008":
        return synth.q4_K_decode_4096x11008()
    if name in ("q4_K_4096x4096", "q4_0_4096x4096"):
        return synth.q4_gemv_4096x4096()
    if name == "ffn_7b_q4_K_q6_K":
        return synth.ffn_7b()
    if name == "q6_K_head_32000x4096":
        return synth.q6_K_head_32000x4096()
    if name.startswith("q4_K_batched"):
        d = synth.q4_K_batched_14336x4096()
        return {"W": d["W"], "X": d["X"]}
    if name == "q8_0_256x1024":
        return synth.q8_0_gemv_256x1024()
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

    if w_type == synth.Q4_K:
        w[:, :, 0:2] = f16(1e-4, 1e-3)
        w[:, :, 2:4] = f16(1e-4, 1e-3)
    elif w_type == synth.Q6_K:
        sc = torch.randint(-64, 64, (n_out, nb, 16), dtype=torch.int8, device="cuda", generator=gen)
        w[:, :, 192:208] = sc.view(torch.uint8)
        w[:, :, 208:210] = f16(1e-4, 1e-3)
    elif w_type == synth.Q4_0:
        w[:, :, 0:2] = f16(1e-3, 4e-3)
    else:
        raise ValueError("GPU copies are drawn for block-byte weight formats only")
    return w.reshape(n_out, nb * bb)


def cpu_baseline(name, wl, inputs, seconds):
    """The scalar C oracle (single thread) on a bounded sample of the workload:
    the first rows of each GEMV, repeated until `seconds` have passed."""
    from oracle import oracle as orc
    t_end = time.perf_counter() + seconds
    done_bytes = 0
    reps = 0
    sample_rows = {}
    t0 = time.perf_counter()
    while True:
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
                done_bytes += rows * W.shape[1]
        reps += 1
        if time.perf_counter() >= t_end:
            break
    dt = time.perf_counter() - t0
    desc = ", ".join(f"{k}: first {r} rows" for k, r in sample_rows.items())
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{desc}; quantize + GEMV repeated {reps}x in {dt:.1f} s, single thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="q4_K_decode_4096x11008")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
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
    copies = max(1, -(-ROTATE_BYTES // step_w_bytes))
    dev_w = []  # per copy: list of weight tensors, one per GEMV
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    for c in range(copies):
        mats = []
        for wname, wt, n_out, n_in, _ in wl["gemvs"]:
            if c == 0 or wt == qk.QK_TYPE_Q8_0:
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
    ys = [torch.empty((ncols_of(wl, akey), n_out), dtype=torch.float32, device="cuda")
          for _, _, n_out, _, akey in wl["gemvs"]]
    torch.cuda.synchronize()
    log(f"[bench] {copies} weight copies x {step_w_bytes / 1e6:.2f} MB resident; "
        f"warmup {args.warmup}, steps {args.steps}")

    n_g = len(wl["gemvs"])

    def step(k, evs=None):
        mats = dev_w[k % copies]
        for key, (at, xf, xq) in acts.items():
            qk.qk_quantize_act(at, xf, xq)
        for g, (wname, wt, n_out, n_in, akey) in enumerate(wl["gemvs"]):
            xq = acts[akey][2]
            ncols = acts[akey][1].shape[0]
            if evs is None:
                qk.qk_gemv(wt, mats[g], n_out, n_in, xq, ncols, ys[g])
            else:
                e0, e1 = evs[g]
                qk.qk_gemv_timed(wt, mats[g], n_out, n_in, xq, ncols, ys[g], e0, e1)

    for k in range(args.warmup):
        step(k)
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
    value = step_w_bytes * args.steps / (elapsed_ms / 1e3) / 1e9

    # Region B - the same K steps launched one by one; each GEMV launch records
    # a start / stop event pair with its own kernel timestamps (HIP extended
    # launch), giving kernel durations free of enqueue gaps.  torch creates the
    # underlying events on their first record.
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_g)] for _ in range(args.steps)]
    for per in ev:
        for e0, e1 in per:
            e0.record(stream)
            e1.record(stream)
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_stop = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for k in range(args.steps):
        step(args.warmup + k, ev[k])
    e_stop.record(stream)
    torch.cuda.synchronize()
    eager_ms = e_start.elapsed_time(e_stop)

    kern_ms = np.array([[e0.elapsed_time(e1) for e0, e1 in per] for per in ev])  # [steps, n_g]
    gemv_ms_mean = kern_ms.sum(axis=1).mean()

    # algorithmic bytes per GEMV launch: weights + activation blocks + f32 outputs
    alg_bytes = 0
    for _, wt, n_out, n_in, akey in wl["gemvs"]:
        at, xf, xq = acts[akey]
        ncols = xf.shape[0]
        alg_bytes += qk.qk_row_bytes(wt, n_in) * n_out + xq.numel() + 4 * n_out * ncols
    achieved = alg_bytes / (gemv_ms_mean / 1e3) / 1e9
    per_kernel_us = {wl["gemvs"][g][0]: {"mean": round(float(kern_ms[:, g].mean() * 1e3), 3),
                                          "p10": round(float(np.percentile(kern_ms[:, g], 10) * 1e3), 3),
                                          "p50": round(float(np.percentile(kern_ms[:, g], 50) * 1e3), 3),
                                          "p90": round(float(np.percentile(kern_ms[:, g], 90) * 1e3), 3)}
                     for g in range(n_g)}
    log(f"[bench] graph replay {elapsed_ms:.3f} ms over {args.steps} steps "
        f"({elapsed_ms / args.steps * 1e3:.2f} us/step, host wall {wall * 1e3:.1f} ms); "
        f"eager {eager_ms / args.steps * 1e3:.2f} us/step; GEMV kernel time per step "
        f"{gemv_ms_mean * 1e3:.2f} us; per kernel {per_kernel_us}")

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
            "batch": acts[first[4]][1].shape[0],
            "weight_bytes_per_step": step_w_bytes,
            "weight_copies_rotated": copies,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
        "cpu_baseline": cpu,
        "detail": {"gemv_kernel_us_per_step": round(float(gemv_ms_mean * 1e3), 3),
                   "eager_us_per_step": round(eager_ms / args.steps * 1e3, 3),
                   "gemv_kernel_us": per_kernel_us,
                   "algorithmic_bytes_per_step_gemv": alg_bytes},
    }
    print(json.dumps(out), flush=True)


def ncols_of(wl, akey):
    return wl["acts"][akey][2]


if __name__ == "__main__":
    main()
