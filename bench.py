#!/usr/bin/env python
"""Benchmark of the MXFP4 hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  dynamic BF16 -> MXFP4 quantization of the activation A (the weight B is
  quantized once beforehand with the same kernel, as a weight packer would),
  then the block-scaled FP4 NT GEMM to BF16.
Primary workload: M = N = K = 4096 (TFLOP/s, 2*M*N*K per step).
Secondary workload: decode M=128, N=14336, K=4096 (achieved HBM GB/s).

Inputs are resident in HBM before timing.  Steps rotate over enough copies of
the inputs (>= 512 MiB in total) that the 256 MiB Infinity Cache cannot serve
them.  Each timed region is a HIP graph of whole steps replayed on the stream
the kernels run on, bracketed by events and device synchronisations.

Prints one JSON line on stdout.  The roofline object is for the GEMM kernel:
algorithmic flops (or bytes) per launch divided by the kernel's mean duration,
measured with events over a region of back-to-back GEMM launches.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROTATION_BYTES = 512 << 20


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_algorithmic_bytes(m, n, k, out_bytes=2):
    """Each packed code and scale byte of A and B once, plus C once."""
    return m * k // 2 + m * k // 32 + n * k // 2 + n * k // 32 + m * n * out_bytes


def quant_algorithmic_bytes(rows, k):
    return rows * k * 2 + rows * k // 2 + rows * k // 32


class DenseBench:
    def __init__(self, w: workloads.DenseWorkload, dev):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.w = w
        self.dev = dev
        a, b = w.make()
        self.a_cpu, self.b_cpu = a, b
        a_d, b_d = a.to(dev), b.to(dev)
        bq, bs = B.mxfp4_quantize(b_d)            # weight quantized once (not timed)
        m, n, k = w.m, w.n, w.k
        per_set = m * k * 2 + m * k // 2 + m * k // 32 + n * k // 2 + n * k // 32 + m * n * 2
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.per_set_bytes = per_set
        self.sets = []
        for _ in range(self.sets_n):
            self.sets.append(dict(
                a=a_d.clone(), aq=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
                as_=torch.empty((m, k // 32), dtype=torch.uint8, device=dev),
                bq=bq.clone(), bs=bs.clone(), c=torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
        need = B.load_library().mxfp4_gemm_nt_workspace_size(m, n, k)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        del a_d, b_d
        torch.cuda.synchronize()

    def quantize(self, s):
        self.B.mxfp4_quantize(s["a"], s["aq"], s["as_"])

    def gemm(self, s):
        self.B.mxfp4_gemm_nt(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"], ws=self.ws)

    def step(self, s):
        self.quantize(s)
        self.gemm(s)

    def _graph(self, fn, count, start=0):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(self.sets[(start + i) % self.sets_n])
        return g

    def timed(self, fn, steps, warmup):
        """Mean ms per call of fn over `steps` calls rotating through the input sets."""
        for i in range(2):                    # eager warm-up before capture
            fn(self.sets[i % self.sets_n])
        torch.cuda.synchronize()
        cycle = self._graph(fn, self.sets_n)
        rem = steps % self.sets_n
        tail = self._graph(fn, rem) if rem else None
        for _ in range(max(1, math.ceil(warmup / self.sets_n))):
            cycle.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps // self.sets_n):
            cycle.replay()
        if tail is not None:
            tail.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps


def cpu_baseline(bench: DenseBench, target_seconds: float):
    """The CPU oracle (as it stands) on a bounded sample of the same step: quantize
    `rows` rows of A and multiply them by the full pre-quantized B."""
    import oracle
    from threadpoolctl import threadpool_info
    w = bench.w
    bq, bs = oracle.quantize(workloads.bf16_bits(bench.b_cpu))   # weight packing, untimed
    a_bits = workloads.bf16_bits(bench.a_cpu)

    def run(rows):
        t = time.perf_counter()
        aq, as_ = oracle.quantize(a_bits[:rows])
        oracle.gemm_nt(aq, as_, bq, bs)
        return time.perf_counter() - t

    pilot_rows = min(w.m, 32)
    t_pilot = run(pilot_rows)
    rows = int(min(w.m, max(pilot_rows, pilot_rows * target_seconds / max(t_pilot, 1e-3))))
    t = run(rows)
    flops = 2 * rows * w.n * w.k
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {w.m} rows of A: oracle quantize + float64 GEMM against the full "
                      f"pre-quantized {w.n}x{w.k} B ({t:.1f} s); numpy/BLAS threads as listed in cores"}


def traffic_from_profiles(kernel_key: str):
    """HBM bytes per launch recorded under profiles/ for this kernel, if the kernel
    sources have not changed since the counters were taken (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()[:16]
    for line in open(path):
        parts = dict(p.split("=", 1) for p in line.split() if "=" in p)
        if parts.get("workload") == kernel_key and parts.get("sources") == sha and "bytes_per_launch" in parts:
            return float(parts["bytes_per_launch"])
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.SQUARE4096.name, choices=sorted(workloads.DENSE))
    ap.add_argument("--secondary", default=workloads.DECODE.name,
                    help="second dense workload reported in the same line ('none' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        eprint("bench.py runs on one GPU only: this build has no multi-GPU path "
               "(sharding across GPUs is described in the design notes, not implemented).")
        sys.exit(2)
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda", 0)
    from block_scaled_fp4_mxfp4_amd import load_library
    load_library()

    w = workloads.DENSE[args.workload]
    eprint(f"[bench] building inputs for {w.name}")
    bench = DenseBench(w, dev)
    eprint(f"[bench] {bench.sets_n} rotating input sets of {bench.per_set_bytes / 2**20:.1f} MiB")
    step_ms = bench.timed(bench.step, args.steps, args.warmup)
    gemm_ms = bench.timed(bench.gemm, args.steps, args.warmup)
    quant_ms = bench.timed(bench.quantize, args.steps, args.warmup)
    eprint(f"[bench] step {step_ms*1e3:.2f} us, gemm {gemm_ms*1e3:.2f} us, quantize {quant_ms*1e3:.2f} us")

    flops = w.flops
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    step_tflops = flops / (step_ms * 1e-3) / 1e12
    qbytes = quant_algorithmic_bytes(w.m, w.k)
    result = {
        "metric": "MXFP4 GEMM TFLOP/s at 4096^3; achieved HBM GB/s at decode M=128",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1, e8m0 block scales, fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded Gaussian BF16; weights pre-quantized once)",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k,
                   "step": "quantize A (bf16->mxfp4) + mxfp4 NT GEMM -> bf16",
                   "rotating_input_sets": bench.sets_n, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": traffic_from_profiles(w.name)},
        "kernels": {
            "gemm_us": round(gemm_ms * 1e3, 3), "gemm_tflops": round(gemm_tflops, 2),
            "quantize_us": round(quant_ms * 1e3, 3),
            "quantize_gbs": round(qbytes / (quant_ms * 1e-3) / 1e9, 1),
            "quantize_hbm_frac": round(qbytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        },
    }

    if args.secondary != "none":
        w2 = workloads.DENSE[args.secondary]
        eprint(f"[bench] building inputs for {w2.name}")
        b2 = DenseBench(w2, dev)
        s2 = b2.timed(b2.step, args.steps, args.warmup)
        g2 = b2.timed(b2.gemm, args.steps, args.warmup)
        q2 = b2.timed(b2.quantize, args.steps, args.warmup)
        gbytes = gemm_algorithmic_bytes(w2.m, w2.n, w2.k)
        qb2 = quant_algorithmic_bytes(w2.m, w2.k)
        gemm_gbs = gbytes / (g2 * 1e-3) / 1e9
        result["secondary"] = {
            "metric": "achieved HBM GB/s at decode M=128", "workload": w2.name,
            "value": round((gbytes + qb2) / (s2 * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(s2, 6), "rotating_input_sets": b2.sets_n,
            "step": "quantize A + split-K mxfp4 GEMM (B pre-quantized)",
            "roofline": {"bound": "hbm", "achieved": round(gemm_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gemm_gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_from_profiles(w2.name)},
            "kernels": {"gemm_us": round(g2 * 1e3, 3), "quantize_us": round(q2 * 1e3, 3),
                        "gemm_tflops": round(w2.flops / (g2 * 1e-3) / 1e12, 2)},
        }
        eprint(f"[bench] {w2.name}: step {s2*1e3:.2f} us, gemm {g2*1e3:.2f} us ({gemm_gbs:.0f} GB/s)")
        del b2

    if not args.no_cpu_baseline:
        eprint("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(bench, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
