"""Benchmark of the MI355X ONNX MatMul library.

One step = one pass of the headline workload through mm_execute: the BF16
transformer projection A [16,512,4096] x B [4096,11008] (B shared by every
batch; the plan folds the batch into 8192 rows), FP32 accumulation, BF16
output.  Inputs are resident in HBM and rotated over enough copies (>= 1
GiB per rotation) that no step finds them in the 256 MB Infinity Cache.

Timing.  Every launch (one mm_execute) is bracketed by its own pair of HIP
events recorded on the launch stream, so each launch is an individual
sample.  Ahead of each batch of launches a bounded spin kernel occupies the
GPU while the host enqueues, so the timed launches then run back to back and
the host's enqueue cost is never inside an event pair.  (The event between
two launches keeps them from overlapping, so short kernels read a little
slower than when they run back to back: each case also reports the mean of
a batch of launches between a single event pair.)  The headline runs W
untimed steps, then exactly K timed steps between device synchronisations;
``ms_per_step`` is the GPU time from the first step's start event to the
last step's end event divided by K.

The JSON line also carries:

* ``roofline``: the projection's algorithmic FLOPs (2 M N K) divided by the
  mean event-timed duration of its K launches, against the dense BF16 MFMA
  peak; ``traffic`` is the HBM bytes per launch that rocprofv3 FETCH_SIZE /
  WRITE_SIZE passes recorded under profiles/ (scaled by the plain-copy
  calibration), or null when the kernel sources changed since;
* ``cases``: every workload product (and the Gemm and MatMulInteger
  products) with >= 50 individually timed launches taken in passes whose
  case order alternates, the raw samples, median / p10 / p90, TFLOP/s, HBM
  GB/s and the fraction of its own roofline, plus the CPU oracle's rate on a
  bounded sample of that product;
* ``cpu_baseline``: the fp64 CPU oracle timed on blocks of rows of the
  projection on the host cores (about ``--cpu-seconds`` of work).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cases]
       [--no-cpu] [--cpu-seconds S] [--only NAMES] [--eager N] [--copy-mib M]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from onnx_broadcast_matmul_amd import binding as mm  # noqa: E402
from onnx_broadcast_matmul_amd import synth  # noqa: E402

HEADLINE = "bf16_transformer_projection"
METRIC = "TFLOP/s (and HBM GB/s for skinny) per dtype/shape; % of MFMA/HBM roofline"
# MI355X published peaks: HBM3E 8 TB/s; dense MFMA FP32 157.3 TFLOP/s,
# FP16/BF16 2.5 PFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP/clk = 2516.6), FP64
# 78.6 TFLOP/s, INT8 5.0 POP/s (8192 OP/clk per CU = 5033.2 TOP/s).
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {mm.FLOAT: 157.3, mm.FLOAT16: 2516.6, mm.BFLOAT16: 2516.6, mm.DOUBLE: 78.6, mm.INT8: 5033.2}
ROTATE_BYTES = 1 << 30  # rotate input/output copies until a rotation touches >= 1 GiB
MAX_COPIES = 128
CASE_PASSES = 5         # passes over the case list (order reversed on odd passes)
CASE_LAUNCHES = 10      # individually timed launches per case and pass
PAD_MS = 0.3            # spin ahead of each batch of timed launches (covers the batch's enqueue)
WARM_MS = 3.0           # untimed launches of the same case between the spin and a timed batch: the
                        # clock climbs over the first milliseconds of sustained matrix-core load
HEAD_PAD_MS = 0.3       # spin ahead of the headline's timed steps (covers the first enqueue only,
                        # so the GPU does not idle long enough to leave its sustained clock)

# Sources whose text fixes the tiled GEMM kernel's memory traffic; a traffic
# record taken from hardware counters holds only while their hash matches.
GEMM_SOURCES = ["k_gemm_impl.h", "k_gemm.hip", "tiles.h", "device.h", "internal.h", "plan.cpp"]


def gemm_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "onnx_broadcast_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(product: str):
    """HBM bytes per launch that rocprofv3 FETCH_SIZE + WRITE_SIZE passes
    measured for this product, scaled by the plain-copy calibration, from a
    ``TRAFFIC`` line of a summary under profiles/; None when there is no
    record or the kernel sources changed after the counters were taken."""
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
                if kv.get("product") == product and kv.get("sources_sha256") == sha:
                    return int(kv["bytes_per_launch"])
    return None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _copies(nbytes: float) -> int:
    return int(min(MAX_COPIES, max(1, math.ceil(ROTATE_BYTES / max(nbytes, 1.0)))))


class Case:
    """One MatMul product on the device, with rotated buffer copies."""

    def __init__(self, product: synth.Product, dev):
        import torch

        self.p = product
        self.name = product.name
        self.dt = product.dtype
        self.plan = mm.Plan(product.a_shape, product.b_shape, self.dt)
        self.info = self.plan.info()
        a, b = product.make()
        self.host = (a, b)
        A = synth.as_torch(a, self.dt).to(dev)
        B = synth.as_torch(b, self.dt).to(dev)
        self.bytes = self.info["min_bytes"]
        self.flops = self.info["flops"]
        self.copies = _copies(self.bytes)
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        tdt = mm.torch_dtype(self.dt)
        self.Y = [torch.empty(self.plan.output_shape, dtype=tdt, device=dev) for _ in range(self.copies)]
        self.ptrs = [(self.A[i].data_ptr(), self.B[i].data_ptr(), self.Y[i].data_ptr()) for i in range(self.copies)]
        self.bound = _bound(self.flops, self.bytes, self.dt)

    def run(self, i: int, stream: int) -> None:
        a, b, y = self.ptrs[i % self.copies]
        self.plan.execute_ptr(a, b, y, stream)

    def oracle_sample(self, seconds: float):
        """(FLOPs, seconds) of the CPU oracle on leading blocks of rows."""
        a, b = self.host
        return _oracle_rows(a, b, self.dt, seconds)

    def describe(self):
        return {"a_shape": list(self.p.a_shape), "b_shape": list(self.p.b_shape)}


class GemmCase(Case):
    """One Gemm product on the device, with rotated buffer copies."""

    def __init__(self, product: synth.GemmProduct, dev):
        import torch

        self.p = product
        self.name = product.name
        self.dt = product.dtype
        self.plan = mm.GemmPlan(product.a_shape, product.b_shape, self.dt, product.trans_a, product.trans_b,
                                product.c_shape, product.alpha, product.beta)
        self.info = self.plan.info()
        a, b, c = product.make()
        self.host = (a, b, c)
        A = synth.as_torch(a, self.dt).to(dev)
        B = synth.as_torch(b, self.dt).to(dev)
        C = synth.as_torch(c, self.dt).to(dev)
        es = synth.ELEM_SIZE[self.dt]
        self.bytes = float(es * (a.size + b.size + c.size + product.M * product.N))
        self.flops = 2.0 * product.M * product.N * product.K
        self.copies = _copies(self.bytes)
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        self.C = [C] + [C.clone() for _ in range(self.copies - 1)]
        self.Y = [torch.empty((product.M, product.N), dtype=mm.torch_dtype(self.dt), device=dev)
                  for _ in range(self.copies)]
        self.bound = _bound(self.flops, self.bytes, self.dt)

    def run(self, i: int, stream: int) -> None:
        k = i % self.copies
        self.plan.execute_ptr(self.A[k].data_ptr(), self.B[k].data_ptr(), self.Y[k].data_ptr(), stream,
                              self.C[k].data_ptr())

    def oracle_sample(self, seconds: float):
        import oracle

        a, b, c = self.host
        p = self.p
        rows, t, f = 16, 0.0, 0.0
        while True:  # leading rows of the output, through the per-element Gemm oracle
            idx = np.arange(min(rows, p.M) * p.N, dtype=np.int64)
            t0 = time.perf_counter()
            oracle.gemm_at(a, b, self.dt, idx, p.trans_a, p.trans_b, c, p.alpha, p.beta)
            t += time.perf_counter() - t0
            f += 2.0 * idx.size * p.K
            if t >= seconds or rows >= p.M:
                return f, t
            rows *= 2

    def describe(self):
        p = self.p
        return {"a_shape": list(p.a_shape), "b_shape": list(p.b_shape),
                "op": f"Gemm transA={int(p.trans_a)} transB={int(p.trans_b)} C={list(p.c_shape)}"}


class IntCase(Case):
    """One MatMulInteger product on the device, with rotated buffer copies."""

    def __init__(self, product: synth.IntProduct, dev):
        import torch

        self.p = product
        self.name = product.name
        self.dt = mm.INT8
        code = {True: mm.INT8, False: mm.UINT8}
        self.plan = mm.IntPlan(product.a_shape, product.b_shape, code[product.a_signed], code[product.b_signed],
                               product.a_zp, product.b_zp)
        self.info = self.plan.info()
        a, b, za, zb = product.make()
        self.host = (a, b, za, zb)
        A = torch.from_numpy(a).to(dev)
        B = torch.from_numpy(b).to(dev)
        self.za = None if za is None else torch.from_numpy(np.atleast_1d(za)).to(dev)
        self.zb = None if zb is None else torch.from_numpy(np.atleast_1d(zb)).to(dev)
        self.bytes = self.info["min_bytes"]
        self.flops = self.info["flops"]
        self.copies = _copies(self.bytes)
        self.A = [A] + [A.clone() for _ in range(self.copies - 1)]
        self.B = [B] + [B.clone() for _ in range(self.copies - 1)]
        self.Y = [torch.empty(self.plan.output_shape, dtype=torch.int32, device=dev) for _ in range(self.copies)]
        self.bound = _bound(self.flops, self.bytes, self.dt)

    def run(self, i: int, stream: int) -> None:
        k = i % self.copies
        self.plan.execute_ptr(self.A[k].data_ptr(), self.B[k].data_ptr(), self.Y[k].data_ptr(), stream,
                              self.za.data_ptr() if self.za is not None else 0,
                              self.zb.data_ptr() if self.zb is not None else 0)

    def oracle_sample(self, seconds: float):
        import oracle

        a, b, za, zb = self.host
        n_out = int(np.prod(self.plan.output_shape))
        K = self.p.a_shape[-1]
        N = self.p.b_shape[-1]
        rows, t, f = 16, 0.0, 0.0
        while True:
            idx = np.arange(min(rows * N, n_out), dtype=np.int64)
            t0 = time.perf_counter()
            oracle.matmul_integer_at(a, b, idx, za, zb)
            t += time.perf_counter() - t0
            f += 2.0 * idx.size * K
            if t >= seconds or idx.size >= n_out:
                return f, t
            rows *= 2

    def describe(self):
        p = self.p
        return {"a_shape": list(p.a_shape), "b_shape": list(p.b_shape),
                "op": f"MatMulInteger zero points A={['none', 'scalar', 'per row'][p.a_zp]} "
                      f"B={['none', 'scalar', 'per column'][p.b_zp]}",
                "dtype": ("s8" if p.a_signed else "u8") + ("s8" if p.b_signed else "u8") + "->i32"}


def _bound(flops: float, nbytes: float, dt: int) -> str:
    ridge = MFMA_PEAK_TFLOPS[dt] * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "hbm" if flops / nbytes < ridge else "mfma"


def _oracle_rows(a, b, dt, seconds: float):
    """Run the oracle on growing leading blocks of rows of the first output
    batch until `seconds` have passed; returns (FLOPs, seconds)."""
    import oracle

    aa = a.reshape((-1,) + a.shape[-2:])[0] if a.ndim > 2 else a
    bb = b.reshape((-1,) + b.shape[-2:])[0] if b.ndim > 2 else b
    if aa.ndim == 1:  # a rank-one A: one row
        t0 = time.perf_counter()
        oracle.matmul(aa, bb, dt)
        n = bb.shape[-1] if bb.ndim > 1 else 1
        return 2.0 * aa.shape[0] * n, time.perf_counter() - t0
    M, K = aa.shape
    N = bb.shape[-1] if bb.ndim > 1 else 1
    rows, r0, t, f = 16, 0, 0.0, 0.0
    while True:
        blk = np.ascontiguousarray(aa[r0:r0 + rows])
        t0 = time.perf_counter()
        oracle.matmul(blk, bb, dt)
        t += time.perf_counter() - t0
        f += 2.0 * blk.shape[0] * N * K
        r0 = (r0 + rows) % M
        if t >= seconds:
            return f, t
        rows = min(rows * 2, M)


# ---------------------------------------------------------------- timing

def _cycles_per_ms() -> float:
    """Clock cycles of torch's spin kernel per millisecond (measured)."""
    import torch

    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record(s)
    torch.cuda._sleep(2_000_000)
    e1.record(s)
    torch.cuda.synchronize()
    return 2_000_000 / max(e0.elapsed_time(e1), 1e-3)


class Timer:
    """Individually event-timed launches on the current stream."""

    def __init__(self):
        import torch

        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream
        self.cpm = _cycles_per_ms()

    def pad(self, ms: float) -> None:
        # A bounded spin kernel (it ends after a fixed number of cycles).
        self.torch.cuda._sleep(int(self.cpm * ms))

    def launches(self, case, n: int, offset: int, pad_ms: float = PAD_MS, warm: int = 0):
        """Enqueue `warm` untimed launches of `case`, then n launches each
        between its own start and end events; returns the event pairs (read
        them after synchronising)."""
        E = self.torch.cuda.Event
        pairs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(n)]
        if pad_ms > 0:
            self.pad(pad_ms)
        for i in range(warm):
            case.run(offset + n + i, self.sp)
        for i, (s, e) in enumerate(pairs):
            s.record(self.stream)
            case.run(offset + i, self.sp)
            e.record(self.stream)
        return pairs


def _ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


def warm_count(case) -> int:
    """Untimed launches of a case that make about WARM_MS of GPU work."""
    return int(min(64, max(2, math.ceil(WARM_MS / max(getattr(case, "est_ms", WARM_MS), 1e-3)))))


def calibrate(cases, timer) -> None:
    """Rough per-launch time of every case (sets case.est_ms)."""
    for c in cases:
        pairs = timer.launches(c, 3, 0, warm=2)
        timer.torch.cuda.synchronize()
        c.est_ms = float(np.median(_ms(pairs)))


def back_to_back(case, timer, n: int, offset: int) -> float:
    """Mean time of n launches run back to back between one event pair (no
    events between them, behind a spin kernel and warm-up launches), in ms."""
    E = timer.torch.cuda.Event
    s, e = E(enable_timing=True), E(enable_timing=True)
    timer.pad(PAD_MS)
    for i in range(warm_count(case)):
        case.run(offset + n + i, timer.sp)
    s.record(timer.stream)
    for i in range(n):
        case.run(offset + i, timer.sp)
    e.record(timer.stream)
    timer.torch.cuda.synchronize()
    return s.elapsed_time(e) / n


def case_report(c, samples_ms, oracle=None, b2b_ms=None):
    d = np.array(samples_ms)
    med = float(np.median(d))
    tflops = c.flops / (med * 1e-3) / 1e12
    gbs = c.bytes / (med * 1e-3) / 1e9
    if c.bound == "hbm":
        achieved, peak, unit = gbs, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = tflops, MFMA_PEAK_TFLOPS[c.dt], ("TOP/s" if c.dt == mm.INT8 else "TFLOP/s")
    r = {
        "algo": mm.ALGO_NAMES[c.plan.algo], "tile": c.info["tile"], "split_k": c.info["split_k"],
        "tail_tile": c.info["tail_tile"], "tail_col": c.info["tail_col"],
        "dtype": synth.DTYPE_NAMES.get(c.dt, str(c.dt)), **c.describe(),
        "launches": int(d.size), "us_median": round(med * 1e3, 3), "us_mean": round(float(d.mean()) * 1e3, 3),
        "us_p10": round(float(np.percentile(d, 10)) * 1e3, 3), "us_p90": round(float(np.percentile(d, 90)) * 1e3, 3),
        "tflops": round(tflops, 3), "hbm_gbs": round(gbs, 1), "bound": c.bound,
        "roofline_frac": round(achieved / peak, 4), "roofline_unit": unit, "copies": c.copies,
        "flops": c.flops, "algorithmic_bytes": c.bytes,
        "us_samples": [round(x * 1e3, 3) for x in d.tolist()],
    }
    if b2b_ms is not None:
        r["us_back_to_back_mean"] = round(b2b_ms * 1e3, 3)
    if oracle is not None:
        f, t = oracle
        rate = f / t
        r["oracle"] = {"gflops": round(rate / 1e9, 3), "sample_flops": f, "sample_s": round(t, 3),
                       "full_product_s_est": round(c.flops / rate, 1)}
    return r


def time_case_table(cases, timer, passes: int, per_pass: int):
    """passes x per_pass individually timed launches of every case, each
    batch behind about WARM_MS of untimed launches of the same case; the
    case order is reversed on every other pass."""
    samples = {c.name: [] for c in cases}
    offset = 0
    for p in range(passes):
        order = cases if p % 2 == 0 else list(reversed(cases))
        for c in order:
            pairs = timer.launches(c, per_pass, offset, warm=warm_count(c))
            timer.torch.cuda.synchronize()
            samples[c.name] += _ms(pairs)
            offset += per_pass
        log(f"[bench] case pass {p + 1}/{passes} done")
    return samples


def check_against_eager(c) -> bool:
    """The last timed output of copy 0 equals a fresh launch into a new
    buffer, bit for bit (every launch of a plan gives the same bits)."""
    import torch

    ref = torch.empty_like(c.Y[0])
    c.plan.execute_ptr(c.A[0].data_ptr(), c.B[0].data_ptr(), ref.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return bool(torch.equal(ref.view(torch.uint8), c.Y[0].view(torch.uint8)))


# ---------------------------------------------------------------- host facts

def host_cpu():
    model, physical = None, None
    try:
        with open("/proc/cpuinfo") as f:
            cores = set()
            phys = core = None
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None:
                    cores.add((phys, core))
                    phys = core = None
            if phys is not None:
                cores.add((phys, core))
            physical = len(cores) or None
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "physical_cores": physical,
            "cpus_available": affinity}


def gpu_clocks():
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                           text=True, timeout=20)
        d = json.loads(r.stdout)
        card = d.get("card0", {})
        return {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()}
    except Exception:  # noqa: BLE001 -- informational only
        return None


def env_info():
    import torch

    props = torch.cuda.get_device_properties(0)
    return {
        "gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
        "torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "clocks": gpu_clocks(),
        **host_cpu(), "omp_threads": os.environ.get("OMP_NUM_THREADS"),
    }


def cpu_baseline(c: Case, seconds: float):
    """The fp64 oracle on consecutive blocks of rows of the projection."""
    import oracle

    oracle.lib()
    f, t = c.oracle_sample(seconds)
    hc = host_cpu()
    return {
        "value": round(f / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
        "sample": (f"leading row blocks of {c.name} (A {list(c.p.a_shape)} x B {list(c.p.b_shape)}, all 11008 "
                   f"columns, full K): {f:.3e} FLOP in {t:.1f} s; fp64 accumulation, OpenMP over row groups"),
        "cpu_model": hc["cpu_model"], "physical_cores": hc["physical_cores"], "logical_cpus": hc["logical_cpus"],
    }


def all_cases():
    prods = synth.all_products()
    return prods, synth.GEMM_PRODUCTS, synth.INT_PRODUCTS


_SHAPE_DTYPES = {"bf16": mm.BFLOAT16, "fp16": mm.FLOAT16, "fp32": mm.FLOAT, "fp64": mm.DOUBLE}
_SHAPE_INT = {"u8s8": (False, True), "s8s8": (True, True), "u8u8": (False, False), "s8u8": (True, False)}


def parse_shapes(spec: str):
    """Products named on the command line, for timing and profiling shapes
    outside the workload list: comma-separated items, each either
    ``<type>:<A dims>/<B dims>`` (MatMul, dims joined by ``x``) or
    ``<type>:linear:<M>x<K>x<N>`` (Gemm X W^T + b, W stored [N, K]), with
    <type> one of bf16, fp16, fp32, fp64 (inputs normal(0, 0.02), seed 7),
    or u8s8, s8s8, u8u8, s8u8 for MatMulInteger without zero points (A's and
    B's types; inputs uniform over the type)."""
    out = []
    for item in spec.split(","):
        parts = item.split(":")
        if len(parts) == 2 and parts[0] in _SHAPE_INT:
            sa, sb = parts[1].split("/")
            a = tuple(int(v) for v in sa.split("x"))
            b = tuple(int(v) for v in sb.split("x"))
            sgn = _SHAPE_INT[parts[0]]
            out.append(synth.IntProduct(f"{parts[0]}_{sa}_by_{sb}", a, b, sgn[0], sgn[1], 0, 0, 7))
            continue
        if len(parts) < 2 or parts[0] not in _SHAPE_DTYPES:
            raise ValueError(f"bad product spec {item!r}")
        dt = _SHAPE_DTYPES[parts[0]]
        if parts[1] == "linear":
            M, K, N = (int(v) for v in parts[2].split("x"))
            out.append(synth.GemmProduct(f"{parts[0]}_linear_{M}x{K}_by_{N}x{K}T_bias", M, N, K, False, True, (N,),
                                         1.0, 1.0, dt, ("normal", 0.02), 7))
        else:
            sa, sb = parts[1].split("/")
            a = tuple(int(v) for v in sa.split("x"))
            b = tuple(int(v) for v in sb.split("x"))
            out.append(synth.Product(f"{parts[0]}_{sa}_by_{sb}", a, b, dt, ("normal", 0.02), 7))
    return out


def make_case(p, dev):
    if isinstance(p, synth.IntProduct):
        return IntCase(p, dev)
    if isinstance(p, synth.GemmProduct):
        return GemmCase(p, dev)
    return Case(p, dev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cases", action="store_true", help="skip the per-product table")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and per-case oracle rates")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--oracle-seconds", type=float, default=0.5, help="oracle sample per case")
    ap.add_argument("--only", default=None, help="time only these products (comma-separated names)")
    ap.add_argument("--shapes", default=None,
                    help="time only these products given by shape (see parse_shapes); like --only")
    ap.add_argument("--eager", type=int, default=0,
                    help="with --only or --shapes: run this many plain launches of each product and exit "
                         "(counter passes)")
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

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return

    prods, gprods, iprods = all_cases()
    everything = prods + gprods + iprods
    if args.only or args.shapes:
        sel = []
        if args.only:
            names = args.only.split(",")
            sel = [p for p in everything if p.name in names]
            if len(sel) != len(names):
                sys.exit(f"unknown product in {args.only}")
        if args.shapes:
            sel += parse_shapes(args.shapes)
        cases = [make_case(p, dev) for p in sel]
        timer = Timer()
        sp = timer.sp
        if args.eager > 0:
            for c in cases:
                for i in range(args.eager):
                    c.run(i, sp)
                torch.cuda.synchronize()
                print(json.dumps({"eager": c.name, "launches": args.eager, "plan": c.info}), flush=True)
            return
        for c in cases:
            for i in range(args.warmup):
                c.run(i, sp)
        torch.cuda.synchronize()
        calibrate(cases, timer)
        samples = time_case_table(cases, timer, CASE_PASSES, max(1, args.steps // CASE_PASSES))
        for c in cases:
            b2b = back_to_back(c, timer, max(1, args.steps // CASE_PASSES), 3)
            print(json.dumps({"only": c.name, "case": case_report(c, samples[c.name], None, b2b)}), flush=True)
        return

    headline = synth.WORKLOADS[HEADLINE].products[0]
    log(f"[bench] preparing {len(everything)} products")
    cases = [make_case(p, dev) for p in everything] if not args.no_cases else [make_case(headline, dev)]
    hc = [c for c in cases if c.name == headline.name][0]
    timer = Timer()
    sp = timer.sp
    torch.cuda.synchronize()
    log(f"[bench] spin kernel: {timer.cpm:.0f} cycles/ms")

    # Per-product table first (it also warms the GPU up).
    table = None
    if not args.no_cases:
        for c in cases:
            for i in range(3):
                c.run(i, sp)
        torch.cuda.synchronize()
        calibrate(cases, timer)
        samples = time_case_table(cases, timer, CASE_PASSES, CASE_LAUNCHES)
        b2b = {c.name: back_to_back(c, timer, CASE_LAUNCHES, 7) for c in cases}

    # Headline: W untimed steps, then exactly K timed steps, right after the
    # case table so that the GPU has not idled (an idle gap changes the clock
    # for the next few hundred microseconds of MFMA work).
    for w in range(args.warmup):
        hc.run(w, sp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pairs = timer.launches(hc, args.steps, args.warmup, pad_ms=HEAD_PAD_MS)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = _ms(pairs)
    span_ms = pairs[0][0].elapsed_time(pairs[-1][1])
    ms = span_ms / args.steps
    value = hc.flops / (ms * 1e-3) / 1e12
    same = check_against_eager(hc)
    log(f"[bench] {HEADLINE}: {ms:.4f} ms/step, {value:.2f} TFLOP/s")

    # CPU work (the oracle) only after all GPU timing.
    if not args.no_cases:
        table = {}
        for c in cases:
            orc = None
            if not args.no_cpu:
                orc = c.oracle_sample(args.oracle_seconds)
            table[c.name] = case_report(c, samples[c.name], orc, b2b[c.name])
            r = table[c.name]
            log(f"[bench]   {c.name}: {r['us_median']} us ({r['tflops']} TFLOP/s, {r['hbm_gbs']} GB/s, "
                f"{r['roofline_frac']} of {r['roofline_unit']} peak)")

    mean_launch = float(np.mean(per))
    achieved = hc.flops / (mean_launch * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[hc.dt]
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4), "traffic": recorded_traffic(hc.name),
        "kernel": (f"tiled MFMA GEMM (k_gemm_lds_dma), tile entry {hc.info['tile']}"
                   + (f" for columns [0, {hc.info['tail_col']}) and entry {hc.info['tail_tile']} for the rest"
                      if hc.info["tail_col"] else "")
                   + f": every launch of one mm_execute of {hc.name}"),
        "avg_launch_us": round(mean_launch * 1e3, 3), "flops_per_launch": hc.flops,
        "algorithmic_bytes_per_launch": hc.bytes,
    }
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal(0, 0.02) inputs rounded to bf16)",
        "config": {"workload": HEADLINE, "a_shape": list(headline.a_shape), "b_shape": list(headline.b_shape),
                   "flops_per_step": hc.flops, "accumulation": "fp32", "output": "bf16",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "timing": ("each launch between its own HIP events on the launch stream, behind a bounded spin kernel; "
                   "ms_per_step = first start to last end event / steps"),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "us_samples": [round(x * 1e3, 3) for x in per],
        "repeat_matches_bitwise": same,
    }
    if table is not None:
        out["cases_timing"] = (f"{CASE_PASSES} passes over the products (order reversed on odd passes); per pass "
                               f"and product a {PAD_MS} ms spin, about {WARM_MS} ms of untimed launches of that "
                               f"product, then {CASE_LAUNCHES} launches each between its own HIP events; "
                               "us_back_to_back_mean: the same launches between one event pair")
        out["cases"] = table
    if not args.no_cpu:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(hc, args.cpu_seconds)
        log(f"[bench]   {out['cpu_baseline']}")
    out["env"] = env_info()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
