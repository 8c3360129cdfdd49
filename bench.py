"""Benchmark of the MI355X ONNX MatMul library.

One step = one pass of the headline workload (FP32 square [1024,1024]^2 plus
the batch-broadcast [8,1,512,512] x [1,6,512,512]) through mm_execute, with
inputs resident in HBM and rotated over enough copies that no step finds
them in the 256 MB Infinity Cache.  The JSON line also carries:

* ``roofline``: the dominant kernel's algorithmic FLOPs per launch divided by
  its average launch time, measured with HIP events on the launch stream over
  the timed region, against the FP32 MFMA peak;
* ``cases``: every other workload product timed the same way (TFLOP/s,
  HBM GB/s and the fraction of its own roofline);
* ``cpu_baseline``: the fp64 CPU oracle timed over whole steps of the
  headline workload on the host cores (about ``--cpu-seconds`` of work).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cases]
       [--no-cpu] [--cpu-seconds S] [--only NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from onnx_broadcast_matmul_amd import binding as mm  # noqa: E402
from onnx_broadcast_matmul_amd import synth  # noqa: E402

HEADLINE = "fp32_square_and_batched_broadcast"
# MI355X published peaks: HBM3E 8 TB/s; dense MFMA FP32 157.3 TFLOP/s,
# FP16/BF16 2.5 PFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP/clk = 2516.6), FP64
# 78.6 TFLOP/s, INT8 5.0 POP/s (8192 OP/clk per CU = 5033.2 TOP/s).
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {mm.FLOAT: 157.3, mm.FLOAT16: 2516.6, mm.BFLOAT16: 2516.6, mm.DOUBLE: 78.6, mm.INT8: 5033.2}
ROTATE_BYTES = 1 << 30  # rotate input/output copies until a step touches >= 1 GiB
MAX_COPIES = 16


# Sources whose text fixes the tiled GEMM kernel's memory traffic; a traffic
# record taken from hardware counters holds only while their hash matches.
GEMM_SOURCES = ["k_gemm_impl.h", "k_gemm.hip", "tiles.h", "device.h", "internal.h"]


def gemm_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "onnx_broadcast_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(product: str, tile: int):
    """HBM bytes per launch that rocprofv3 FETCH_SIZE + WRITE_SIZE passes
    measured for this product and tile, scaled by the plain-copy calibration,
    from a ``TRAFFIC`` line of a summary under profiles/; None when there is
    no record or the kernel sources changed after the counters were taken."""
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return None
    sha = gemm_sources_sha256()
    for f in sorted(os.listdir(d)):
        if not f.endswith((".md", ".txt")):
            continue
        with open(os.path.join(d, f)) as fh:
            for line in fh:
                if not line.startswith("TRAFFIC "):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("product") == product and int(kv.get("tile", -1)) == tile and kv.get("sources_sha256") == sha:
                    return int(kv["bytes_per_launch"])
    return None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Case:
    """One workload product on the device, with rotated buffer copies."""

    def __init__(self, product: synth.Product, dev):
        import torch

        self.p = product
        self.dt = product.dtype
        self.plan = mm.Plan(product.a_shape, product.b_shape, self.dt)
        self.info = self.plan.info()
        a, b = product.make()
        A = synth.as_torch(a, self.dt).to(dev)
        B = synth.as_torch(b, self.dt).to(dev)
        del a, b
        tdt = mm.torch_dtype(self.dt)
        self.bytes = self.info["min_bytes"]
        self.flops = self.info["flops"]
        self.copies = int(min(MAX_COPIES, max(1, math.ceil(ROTATE_BYTES / max(self.bytes, 1)))))
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        self.Y = [torch.empty(self.plan.output_shape, dtype=tdt, device=dev) for _ in range(self.copies)]
        self.ptrs = [(self.A[i].data_ptr(), self.B[i].data_ptr(), self.Y[i].data_ptr()) for i in range(self.copies)]
        self.bound = "hbm" if self.flops / self.bytes < MFMA_PEAK_TFLOPS[self.dt] * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"

    def run(self, i: int, stream: int) -> None:
        a, b, y = self.ptrs[i % self.copies]
        self.plan.execute_ptr(a, b, y, stream)


class GemmCase:
    """One Gemm product on the device, with rotated buffer copies."""

    def __init__(self, product: synth.GemmProduct, dev):
        import torch

        self.p = product
        self.dt = product.dtype
        self.plan = mm.GemmPlan(product.a_shape, product.b_shape, self.dt, product.trans_a, product.trans_b,
                                product.c_shape, product.alpha, product.beta)
        self.info = self.plan.info()
        a, b, c = product.make()
        A = synth.as_torch(a, self.dt).to(dev)
        B = synth.as_torch(b, self.dt).to(dev)
        C = synth.as_torch(c, self.dt).to(dev)
        es = synth.ELEM_SIZE[self.dt]
        self.bytes = float(es * (a.size + b.size + c.size + product.M * product.N))
        self.flops = 2.0 * product.M * product.N * product.K
        del a, b, c
        self.copies = int(min(MAX_COPIES, max(1, math.ceil(ROTATE_BYTES / self.bytes))))
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        self.C = [C] + [C.clone() for _ in range(self.copies - 1)]
        self.Y = [torch.empty((product.M, product.N), dtype=mm.torch_dtype(self.dt), device=dev)
                  for _ in range(self.copies)]
        self.bound = "hbm" if self.flops / self.bytes < MFMA_PEAK_TFLOPS[self.dt] * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"

    def run(self, i: int, stream: int) -> None:
        k = i % self.copies
        self.plan.execute_ptr(self.A[k].data_ptr(), self.B[k].data_ptr(), self.Y[k].data_ptr(), stream,
                              self.C[k].data_ptr())


class IntCase:
    """One MatMulInteger product on the device, with rotated buffer copies;
    a launch is the whole mm_int_execute (sum passes and the tiled kernel)."""

    def __init__(self, product: synth.IntProduct, dev):
        import torch

        self.p = product
        self.dt = mm.INT8
        code = {True: mm.INT8, False: mm.UINT8}
        self.plan = mm.IntPlan(product.a_shape, product.b_shape, code[product.a_signed], code[product.b_signed],
                               product.a_zp, product.b_zp)
        self.info = self.plan.info()
        a, b, za, zb = product.make()
        A = torch.from_numpy(a).to(dev)
        B = torch.from_numpy(b).to(dev)
        self.za = None if za is None else torch.from_numpy(np.atleast_1d(za)).to(dev)
        self.zb = None if zb is None else torch.from_numpy(np.atleast_1d(zb)).to(dev)
        del a, b
        self.bytes = self.info["min_bytes"]
        self.flops = self.info["flops"]
        self.copies = int(min(MAX_COPIES, max(1, math.ceil(ROTATE_BYTES / self.bytes))))
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        self.Y = [torch.empty(self.plan.output_shape, dtype=torch.int32, device=dev) for _ in range(self.copies)]
        self.bound = "hbm" if self.flops / self.bytes < MFMA_PEAK_TFLOPS[self.dt] * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"

    def run(self, i: int, stream: int) -> None:
        k = i % self.copies
        self.plan.execute_ptr(self.A[k].data_ptr(), self.B[k].data_ptr(), self.Y[k].data_ptr(), stream,
                              self.za.data_ptr() if self.za is not None else 0,
                              self.zb.data_ptr() if self.zb is not None else 0)


def int_case_report(c: IntCase, durs_ms):
    r = case_report(c, durs_ms)
    r["tops"] = r.pop("tflops")
    if r["roofline_unit"] == "TFLOP/s":
        r["roofline_unit"] = "TOP/s"
    r["dtype"] = ("s8" if c.p.a_signed else "u8") + ("s8" if c.p.b_signed else "u8") + "->i32"
    r["op"] = f"MatMulInteger zero points A={['none', 'scalar', 'per row'][c.p.a_zp]} B={['none', 'scalar', 'per column'][c.p.b_zp]}"
    return r


def _capture(cases, count: int, offset: int):
    """A HIP graph holding `count` steps (each step: every case once)."""
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for k in range(count):
            for c in cases:
                c.run(offset + k, sp)
    return g


def time_cases(cases, steps: int, warmup: int, per_case_reps: int = 5):
    """Time `steps` steps (each step: every case once) as one replay of a
    captured HIP graph, bracketed by device synchronisation; launches then
    follow each other on the GPU without host round trips.  Per-case launch
    durations come from replays of a per-case graph of `steps` launches,
    timed with events on the launch stream.  Returns (ms per step, per-case
    lists of average launch durations in ms)."""
    import torch

    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for w in range(warmup):
        for c in cases:
            c.run(w, sp)
    torch.cuda.synchronize()
    step_graph = _capture(cases, steps, warmup)
    case_graphs = [_capture([c], steps, warmup) for c in cases]
    step_graph.replay()  # untimed
    for g in case_graphs:
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    step_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per = []
    for g in case_graphs:
        d = []
        for _ in range(per_case_reps):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            d.append(e0.elapsed_time(e1) / steps)
        per.append(d)
    return ms, per


def check_graph_against_eager(c) -> bool:
    """The graph-replayed output of the last buffer copy equals an eager
    execution into a fresh buffer, bit for bit."""
    import torch

    i = c.copies - 1
    ref = torch.empty_like(c.Y[i])
    c.plan.execute_ptr(c.A[i].data_ptr(), c.B[i].data_ptr(), ref.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return bool(torch.equal(ref.view(torch.uint8), c.Y[i].view(torch.uint8)))


def case_report(c: Case, durs_ms):
    d = np.array(durs_ms)
    med = float(np.median(d))
    tflops = c.flops / (med * 1e-3) / 1e12
    gbs = c.bytes / (med * 1e-3) / 1e9
    if c.bound == "hbm":
        achieved, peak, unit = gbs, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = tflops, MFMA_PEAK_TFLOPS[c.dt], "TFLOP/s"
    return {
        "algo": mm.ALGO_NAMES[c.plan.algo], "tile": c.info["tile"], "split_k": c.info["split_k"],
        "dtype": synth.DTYPE_NAMES.get(c.dt, str(c.dt)), "a_shape": list(c.p.a_shape), "b_shape": list(c.p.b_shape),
        "us_median": round(med * 1e3, 3), "us_p10": round(float(np.percentile(d, 10)) * 1e3, 3),
        "us_p90": round(float(np.percentile(d, 90)) * 1e3, 3),
        "tflops": round(tflops, 3), "hbm_gbs": round(gbs, 1), "bound": c.bound,
        "roofline_frac": round(achieved / peak, 4), "roofline_unit": unit, "copies": c.copies,
    }


def cpu_baseline(products, seconds: float):
    """The fp64 oracle run over whole steps of the workload.

    Every product of the step is computed in full by ``oracle.matmul``; steps
    repeat until ``seconds`` have passed, so the sample is a whole number of
    complete steps and the rate is directly comparable with ``value``.
    """
    import oracle

    oracle.lib()
    data = [(p, *p.make()) for p in products]
    step_flops = sum(synth_flops(p) for p in products)
    steps = 0
    t0 = time.perf_counter()
    while True:
        for p, a, b in data:
            oracle.matmul(a, b, p.dtype)
        steps += 1
        t = time.perf_counter() - t0
        if t >= seconds:
            break
    f = steps * step_flops
    return {
        "value": round(f / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
        "sample": (f"{steps} whole steps of the workload ({' + '.join(p.name for p in products)}); "
                   f"{f:.3e} FLOP in {t:.1f} s, fp64 accumulation, OpenMP over output rows"),
    }


def synth_flops(p: synth.Product) -> float:
    shape = np.broadcast_shapes(p.a_shape[:-2] if len(p.a_shape) > 2 else (), p.b_shape[:-2] if len(p.b_shape) > 2 else ())
    M = p.a_shape[-2] if len(p.a_shape) > 1 else 1
    N = p.b_shape[-1] if len(p.b_shape) > 1 else 1
    return 2.0 * float(np.prod(shape)) * M * N * p.K


def env_info():
    import torch

    props = torch.cuda.get_device_properties(0)
    return {
        "gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
        "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
        "host_cpus": os.cpu_count(), "omp_threads": os.environ.get("OMP_NUM_THREADS"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cases", action="store_true", help="skip the per-product table of the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", default=None, help="time only these products (comma-separated names; profiling runs)")
    ap.add_argument("--eager-only", action="store_true",
                    help="run --warmup eager steps of the headline workload and exit (hardware-counter passes)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run three plain device copies of this many MiB and exit (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mm.lib()

    headline = synth.WORKLOADS[HEADLINE].products
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.eager_only:
        cases = [Case(p, dev) for p in headline]
        sp = torch.cuda.current_stream().cuda_stream
        for w in range(args.warmup):
            for c in cases:
                c.run(w, sp)
        torch.cuda.synchronize()
        print(json.dumps({"eager_steps": args.warmup, "launches": {c.p.name: c.info for c in cases}}), flush=True)
        return
    if args.only:
        names = args.only.split(",")
        prods = [p for p in synth.all_products() + synth.GEMM_PRODUCTS + synth.INT_PRODUCTS if p.name in names]
        if len(prods) != len(names):
            sys.exit(f"unknown product in {args.only}")
        for p in prods:
            if isinstance(p, synth.IntProduct):
                c = IntCase(p, dev)
            else:
                c = GemmCase(p, dev) if isinstance(p, synth.GemmProduct) else Case(p, dev)
            _, per = time_cases([c], args.steps, args.warmup)
            rep = int_case_report(c, per[0]) if isinstance(c, IntCase) else case_report(c, per[0])
            print(json.dumps({"only": p.name, "case": rep}), flush=True)
            del c
            torch.cuda.empty_cache()
        return

    log(f"[bench] preparing {HEADLINE}")
    hcases = [Case(p, dev) for p in headline]
    ms, per = time_cases(hcases, args.steps, args.warmup)
    graph_ok = all(check_graph_against_eager(c) for c in hcases)
    flops = sum(c.flops for c in hcases)
    value = flops / (ms * 1e-3) / 1e12
    log(f"[bench] {HEADLINE}: {ms:.4f} ms/step, {value:.2f} TFLOP/s")

    # dominant kernel: the product with the largest average launch time
    avgs = [float(np.mean(d)) for d in per]
    dom = int(np.argmax(avgs))
    dc = hcases[dom]
    achieved = dc.flops / (avgs[dom] * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_PEAK_TFLOPS[dc.dt], "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_PEAK_TFLOPS[dc.dt], 4), "traffic": recorded_traffic(dc.p.name, dc.info["tile"]),
        "kernel": f"general {dc.info['tile']} on {dc.p.name}", "avg_launch_us": round(avgs[dom] * 1e3, 3),
        "flops_per_launch": dc.flops, "algorithmic_bytes_per_launch": dc.bytes,
    }

    out = {
        "metric": "TFLOP/s (and HBM GB/s for skinny) per dtype/shape; % of MFMA/HBM roofline",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded normal(0,1)/sqrt(K) inputs)",
        "config": {"workload": HEADLINE, "products": [[list(c.p.a_shape), list(c.p.b_shape)] for c in hcases],
                   "flops_per_step": flops, "parallelism": "single GPU"},
        "roofline": roofline,
        "timing": "HIP graph replay of the timed steps; events on the launch stream",
        "graph_matches_eager": graph_ok,
        "headline_cases": {c.p.name: case_report(c, d) for c, d in zip(hcases, per)},
    }
    del hcases
    torch.cuda.empty_cache()

    if not args.no_cases:
        table = {}
        for p in synth.all_products():
            if p in headline:
                continue
            log(f"[bench] case {p.name}")
            c = Case(p, dev)
            steps = max(10, args.steps // 2)
            _, per_c = time_cases([c], steps, max(3, args.warmup // 2))
            table[p.name] = case_report(c, per_c[0])
            log(f"[bench]   {table[p.name]}")
            del c
            torch.cuda.empty_cache()
        for gp in synth.GEMM_PRODUCTS:
            log(f"[bench] gemm case {gp.name}")
            c = GemmCase(gp, dev)
            steps = max(10, args.steps // 2)
            _, per_c = time_cases([c], steps, max(3, args.warmup // 2))
            table[gp.name] = case_report(c, per_c[0])
            table[gp.name]["op"] = f"Gemm transA={int(gp.trans_a)} transB={int(gp.trans_b)} C={list(gp.c_shape)}"
            log(f"[bench]   {table[gp.name]}")
            del c
            torch.cuda.empty_cache()
        for ip in synth.INT_PRODUCTS:
            log(f"[bench] integer case {ip.name}")
            c = IntCase(ip, dev)
            steps = max(10, args.steps // 2)
            _, per_c = time_cases([c], steps, max(3, args.warmup // 2))
            table[ip.name] = int_case_report(c, per_c[0])
            log(f"[bench]   {table[ip.name]}")
            del c
            torch.cuda.empty_cache()
        out["cases"] = table

    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(headline, args.cpu_seconds)
        log(f"[bench]   {out['cpu_baseline']}")
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
