"""Benchmark of one Muon optimizer step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: the Llama-3-8B-shaped weight set (32 layers x {q, k, v, o,
gate, up, down} in bf16 with fp32 momentum, Newton-Schulz standard method,
five quintic steps, plus AdamW on the 128256 x 4096 embedding and lm_head and
65 RMSNorm vectors).  Inputs are synthetic and already resident in HBM when
the timed region starts: rank-64 geometric-spectrum gradients plus noise,
generated on the GPU from seeded torch generators.

Prints one JSON line: value = nominal Newton-Schulz TFLOP/s of the whole step
(5 x sum over units of 4 m^2 n + 2 m^3, m <= n, divided by the step time),
ms_per_step, the roofline of the dominant kernel (the P X update GEMM,
timed live with HIP events around each of its launches) and the fp64 oracle
timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="llama3_8b_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ns-method", choices=["standard", "gram", "auto", "gram_restart"], default=None,
                   help="override the workload's Newton-Schulz method")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the measured MFMA and copy ceilings")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run the library's two streaming copies of 1 GiB (non-temporal, and through the "
                        "GEMMs' global -> LDS loads) three times each and exit: the reference dispatches "
                        "that scale the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "owner-computes step is a design, not built", file=sys.stderr)
        sys.exit(2)
    import torch

    import matrix_orthogonalizing_optimizer_amd as mo
    from workloads import configs, gen

    mo.lib()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for _ in range(3):
            mo.muon_probe_copy(src, dst, nbytes)
        for _ in range(3):
            mo.muon_probe_copy_lds(src, dst, nbytes)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_per_dispatch": nbytes, "dispatches": 3,
                                               "kernels": ["probe_copy_kernel", "probe_copy_lds_kernel"]}}))
        return
    wl = configs.ALL[args.workload]()
    if args.ns_method:
        wl.method = args.ns_method
    method = {"standard": 0, "gram": 1, "auto": 2, "gram_restart": 3}[wl.method]
    table = wl.table

    # ---- inputs (untimed), resident in HBM
    t0 = time.time()
    params, grads, moms, eas, ess = [], [], [], [], []
    for p, (kind, dt, rows, cols, _s, _sd) in enumerate(table):
        tdt = gen.torch_dtype(dt)
        params.append(gen.normal(rows, cols, gen.W_STD, gen.stream_seed(0, 4, p, 1 << 20), dev, tdt))
        if kind == 0:
            grads.append(gen.lowrank_gradient(rows, cols, wl.rank, gen.stream_seed(0, 4, p, 0), dev, tdt))
            moms.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
            eas.append(None)
            ess.append(None)
        else:
            grads.append(gen.normal(rows, cols, gen.ADAM_G_STD, gen.stream_seed(0, 4, p, 0), dev, tdt))
            moms.append(None)
            eas.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
            ess.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
    plan = mo.muon_plan_create(table, method)
    ws = torch.empty(mo.muon_plan_workspace_bytes(plan), dtype=torch.uint8, device=dev)
    hp = mo.make_hparams(**{k: v for k, v in wl.hp.items()})
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f} s; workspace {ws.numel() / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        mo.muon_step(plan, params, grads, moms, eas, ess, hp, ws, stream=stream)
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # ---- timed region: K whole steps, kernel launches bracketed by HIP events
    mo.muon_timing_enable(True)
    mo.muon_timing_collect()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    host_s = 0.0
    for _ in range(args.steps):
        h0 = time.perf_counter()
        mo.muon_step(plan, params, grads, moms, eas, ess, hp, ws, stream=stream)
        host_s += time.perf_counter() - h0
    t_enqueued = time.perf_counter()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    mo.muon_timing_enable(False)
    kt = mo.muon_timing_collect()
    ms_per_step = 1e3 * elapsed / args.steps
    print(f"# timed {args.steps} steps: {ms_per_step:.2f} ms/step", file=sys.stderr, flush=True)

    ns_flops = wl.hp["ns_steps"] * configs.ns_flops(table)
    tflops = ns_flops / (ms_per_step * 1e-3) / 1e12
    exe = executed_flops(mo.muon_plan_buckets(plan), wl.hp["ns_steps"])
    exe_total = sum(exe.values())
    probes = None if args.no_probes else measure_probes(mo, torch, stream)

    kernels = {}
    for name, r in kt.items():
        avg = r["total_ms"] / max(r["launches"], 1)
        e = {"launches": r["launches"] // args.steps, "ms_per_step": r["total_ms"] / args.steps,
             "avg_launch_ms": avg}
        if r["flops"] > 0:
            # the symmetric products compute only upper-triangle tiles: their
            # dense-equivalent rate is nominal, executed_tflops is what ran
            key = "nominal_tflops" if name in SYMMETRIC_FAMILIES else "tflops"
            e[key] = r["flops"] / (r["total_ms"] * 1e-3) / 1e12
        if name in exe:
            e["executed_tflops"] = exe[name] * args.steps / (r["total_ms"] * 1e-3) / 1e12
        if r["bytes"] > 0:
            e["gbs"] = r["bytes"] / (r["total_ms"] * 1e-3) / 1e9
        kernels[name] = e
    dom = "ns_update_PX" if "ns_update_PX" in kt else max(kt, key=lambda k: kt[k]["total_ms"])
    d = kt[dom]
    achieved = d["flops"] / d["launches"] / (d["total_ms"] / d["launches"] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_PEAK_TFLOPS,
                "flops_per_launch": d["flops"] / d["launches"],
                "avg_launch_ms": d["total_ms"] / d["launches"], "traffic": None}
    if probes:
        roofline["frac_of_probed_peak"] = achieved / probes["mfma_bf16_tflops"]
    if dom == "ns_update_PX" and wl.method == "standard":
        # algorithmic HBM bytes of the update GEMM Y' = Y P^T: read Y (n x m)
        # and P (m x m), write Y'
        es = 2 if table[0][1] == 1 else 4
        per_step = sum(es * (2.0 * m * n + 1.0 * m * m) for m, n in unit_shapes(table))
        roofline["algorithmic_bytes_per_launch"] = (wl.hp["ns_steps"] - 1) * per_step * args.steps / d["launches"]
        roofline["traffic"] = measured_traffic(wl.name)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, table, {1: "gram", 3: "gram_restart"}.get(method, "standard"))

    # muon_step only enqueues: its host time per call against the GPU's time
    # per step (the host had queued all K steps after this long)
    host = {"host_ms_per_call": 1e3 * host_s / args.steps,
            "all_steps_enqueued_after_ms": 1e3 * (t_enqueued - t_start),
            "gpu_ms_for_all_steps": 1e3 * elapsed}
    n_units = len(mo.muon_plan_units(plan))
    adam_elems = sum(r[2] * r[3] for r in table if r[0] == 1)
    muon_elems = sum(r[2] * r[3] for r in table if r[0] == 0)
    out = {
        "metric": "Muon step ms + NS TFLOP/s (% bf16 MFMA peak), 8B-shaped weight set, 1 GPU",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if table[0][1] == 1 else "f32",
        "data": "synthetic",
        "pct_bf16_peak": 100.0 * tflops / BF16_PEAK_TFLOPS,
        "executed_tflops": exe_total / (ms_per_step * 1e-3) / 1e12,
        "executed_pct_bf16_peak": 100.0 * exe_total / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "probed_peaks": probes,
        "config": {"workload": wl.name, "units": n_units, "buckets": len(mo.muon_plan_buckets(plan)),
                   "ns_steps": wl.hp["ns_steps"], "ns_method": wl.method,
                   "muon_elements": muon_elems, "adamw_elements": adam_elems,
                   "ns_nominal_tflop_per_step": ns_flops / 1e12,
                   "ns_executed_tflop_per_step": exe_total / 1e12},
        "roofline": roofline,
        "kernels": kernels,
        "enqueue": host,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


SYMMETRIC_FAMILIES = ("ns_gram_A", "ns_poly_P", "gram_r0", "gram_p", "gram_q", "gram_t", "gram_r")


def executed_flops(buckets, steps):
    """FLOPs the GEMM kernels execute in one step, per timing family: output
    tiles computed x 2 T^2 K, T the tile side (256, or 128 when m <= 192).
    Padded tiles count; symmetric products compute upper-triangle tiles only.
    Bucket tuples: (m, n, tall, param dtype, compute dtype, method, first, count)."""
    out = {}

    def add(name, v):
        out[name] = out.get(name, 0.0) + v

    for m, n, _tall, _pdt, _cdt, method, _first, count in buckets:
        T = 256 if m > 192 else 128
        t, tn = -(-m // T), -(-n // T)
        tri, rect = t * (t + 1) // 2, tn * t
        f = 2.0 * T * T * count
        if method == 0:  # standard
            add("ns_gram_A", steps * tri * f * n)
            add("ns_poly_P", steps * tri * f * m)
            if steps > 1:
                add("ns_update_PX", (steps - 1) * rect * f * m)
            add("ns_final_update", rect * f * m)
        else:  # Gram (1), or restarted Gram (3): after ceil(steps / 2) steps one
            # n x m product forms X_r and one Gram product recomputes R; that
            # step has no Z P, P R, R P products
            rs = 1 if method == 3 and steps >= 2 else 0
            add("gram_r0", (1 + rs) * tri * f * n)
            add("gram_p", steps * tri * f * m)
            if steps - 1 - rs > 0:
                add("gram_q", (steps - 1 - rs) * tri * f * m)
                add("gram_t", (steps - 1 - rs) * tri * f * m)
                add("gram_r", (steps - 1 - rs) * tri * f * m)
            if rs:
                add("ns_update_PX", rect * f * m)
            add("ns_final_update", rect * f * m)
    return out


def measure_probes(mo, torch, stream):
    """Ceilings measured in this process on this device, each timed with
    events on the launch stream, best of three: the library's register-only
    bf16 MFMA loop (two workgroups of 4 waves per compute unit) and its
    streaming copy of 2 GiB (2 x 2 GiB through HBM)."""
    sink = torch.empty(512, dtype=torch.float32, device="cuda:0")
    src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty(1 << 31, dtype=torch.uint8, device="cuda:0")

    def best_of(fn, amount):
        fn()  # warm
        best = 0.0
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            best = max(best, amount / (e0.elapsed_time(e1) * 1e-3))
        return best

    flops = 512 * 4 * 1024 * 8 * 32768.0
    mfma = best_of(lambda: mo.muon_probe_mfma(512, 1024, sink, stream=stream), flops) / 1e12
    copy = best_of(lambda: mo.muon_probe_copy(src, dst, 1 << 31, stream=stream), 2.0 * (1 << 31)) / 1e9
    del src, dst
    return {"mfma_bf16_tflops": mfma, "mfma_frac_of_nominal": mfma / BF16_PEAK_TFLOPS,
            "copy_gbs": copy, "copy_frac_of_nominal": copy / HBM_PEAK_GBS}


def unit_shapes(table):
    """(m, n) of every Muon unit, m <= n."""
    out = []
    for kind, _dt, rows, cols, split, _sd in table:
        if kind != 0 or rows == 0 or cols == 0:
            continue
        h = split if split > 0 else rows
        out += [(min(h, cols), max(h, cols))] * (rows // h)
    return out


# the update GEMM's traffic depends on the kernel and on the launch arguments
GEMM_SOURCES = ("matrix_orthogonalizing_optimizer_amd/csrc/gemm.hpp",
                "matrix_orthogonalizing_optimizer_amd/csrc/gemm_bf16.hip",
                "matrix_orthogonalizing_optimizer_amd/csrc/api.cpp")


def gemm_source_digest() -> str:
    """SHA-256 of the GEMM sources with // comments and whitespace removed, so
    that only a change of code (not of its comments) invalidates counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        code = re.sub(r"//[^\n]*", "", text)
        h.update("".join(code.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the update GEMM from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's
    readings), or None when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_update_gemm_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- `"):
                k, v = line[3:].split("`", 1)
                vals[k] = v.split(":", 1)[1].strip()
    if vals.get("kernel_source_sha256") != gemm_source_digest():
        return None
    return float(vals["traffic_bytes_per_launch"])


SMALL_WORKLOADS = ("single_256x512_fp32", "gpt2_small_bf16")
CPU_SAMPLE_MAX_M = 1024   # largest m of a scaled-down per-bucket sample unit
ADAMW_CHUNK = 1 << 24     # AdamW elements per reference call


def cpu_baseline(wl, table, method: str):
    """The plain C++ fp64 reference (oracle/muon_ref.cpp, std::thread over
    every host core it sees; not tuned for this) timed on this host.

    The 256x512 and GPT-2-small-shaped workloads are timed in full: one whole
    step over the table (momentum, Newton-Schulz, scaled update for every
    unit; AdamW for every other element).  For the large workloads one unit
    per shape bucket is timed, at its real shape when m <= 1024 and otherwise
    at the same aspect ratio scaled down by the smallest power of two that
    brings m to 1024 or less; its time is scaled up by the ratio of nominal
    Newton-Schulz FLOPs (full unit / sample) and by the bucket's unit count.
    AdamW is timed on every element (in chunks of 2^24 elements).  Reported
    in the metric's unit (nominal NS TFLOP/s) and as ms per step."""
    import numpy as np
    import torch

    from oracle import cref
    from workloads import configs, gen

    hp = wl.hp
    ohp = _cref_hparams(hp)
    threads = cref.threads()
    step_flops = hp["ns_steps"] * configs.ns_flops(table)
    if wl.name in SMALL_WORKLOADS:
        P, M, EA, ES = gen.make_state(wl, "cpu")
        G = gen.make_grads(wl, 0, "cpu")
        f = lambda xs: [None if x is None else x.double().numpy() for x in xs]
        P, M, EA, ES, G = f(P), f(M), f(EA), f(ES), f(G)
        t = time.perf_counter()
        cref.muon_step(table, P, G, M, EA, ES, ohp, method=method)
        secs = time.perf_counter() - t
        return {"value": step_flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"whole step over the full {wl.name} table in the plain C++ fp64 reference "
                          f"({secs:.1f} s)",
                "ms_per_step": 1e3 * secs, "extrapolated": False}
    # large workloads: one (scaled) unit per bucket, AdamW in full
    buckets = {}
    for kind, _dt, rows, cols, split, _sd in table:
        if kind != 0 or rows == 0 or cols == 0:
            continue
        h = split if split > 0 else rows
        key = (h, cols)
        buckets[key] = buckets.get(key, 0) + rows // h
    total = 0.0
    parts = []
    for i, ((r, c), count) in enumerate(buckets.items()):
        sc = 1
        while min(r, c) // sc > CPU_SAMPLE_MAX_M:
            sc *= 2
        rs, cs = r // sc, c // sc
        G = gen.lowrank_gradient(rs, cs, wl.rank, 99 + i, "cpu", torch.float64).to(torch.bfloat16).double().numpy()
        t = time.perf_counter()
        cref.muon_step([(0, 1, rs, cs, 0, 0)], [np.zeros((rs, cs))], [G], [np.zeros((rs, cs))], [None], [None],
                       ohp, method=method)
        secs = time.perf_counter() - t
        ns = lambda a, b: 4.0 * min(a, b) ** 2 * max(a, b) + 2.0 * min(a, b) ** 3
        est = secs * ns(r, c) / ns(rs, cs) * count
        total += est
        parts.append(f"{count} x {r}x{c} from {rs}x{cs} ({secs:.1f} s)")
    adam = sum(r[2] * r[3] for r in table if r[0] == 1)
    adam_secs = 0.0
    if adam:
        n = min(adam, ADAMW_CHUNK)
        rng = np.random.default_rng(0)
        w = rng.standard_normal(n) * 0.02
        g = rng.standard_normal(n) * 1e-3
        z = np.zeros(n)
        t = time.perf_counter()
        done = 0
        while done < adam:
            k = min(n, adam - done)
            cref.adamw(w[:k], g[:k], z[:k], z[:k], 1, hp["adam_lr"], hp["adam_beta1"], hp["adam_beta2"],
                       hp["adam_eps"], hp["adam_weight_decay"])
            done += k
        adam_secs = time.perf_counter() - t
        parts.append(f"AdamW on all {adam} elements ({adam_secs:.1f} s, timed in full)")
    secs = total + adam_secs
    return {"value": step_flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "plain C++ fp64 reference; one unit per shape bucket, scaled to m <= 1024 at the "
                      "same aspect ratio and extrapolated by nominal NS FLOPs and unit count: "
                      + "; ".join(parts),
            "ms_per_step": 1e3 * secs, "extrapolated": True}


def _cref_hparams(hp):
    import oracle
    return oracle.OracleHparams(**{k: v for k, v in hp.items() if k in oracle.OracleHparams.__annotations__})


if __name__ == "__main__":
    main()
