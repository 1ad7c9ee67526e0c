#!/usr/bin/env python
"""Benchmark of the MXFP4 hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  dynamic BF16 -> MXFP4 quantization of the activation A, then the
  block-scaled FP4 NT GEMM to BF16.  The weight B is quantized once beforehand
  with the same kernel (a weight packer's job, outside the step); its
  quantization time is reported separately.  The prefill GEMMs and the MoE
  layer keep their scale bytes in the interleaved layout the tile kernels copy
  from (include/mxfp4.h): the activation quantizers write it directly, the
  weights' scales are interleaved once with the weights; the same GEMMs on
  row-major scales are reported beside them (`row_major_scales`).
Primary workload: M = N = K = 4096 (TFLOP/s, 2*M*N*K per step).
Secondary workload: decode M=128, N=14336, K=4096 (achieved HBM GB/s).
Also reported: the grouped MoE layer (8192 tokens, top-4 of 64 experts,
N=2816, K=4096) in TFLOP/s and GB/s, and the same layer run wholly on the
device (`moe_layer`: top-k routing of the router logits, the expert-sorted
permutation, MXFP4 quantization scattered into the routed rows, the grouped
GEMM and the weighted combine), each step's time against its algorithmic
bytes.  Also the fused producers (`producers`): residual add + RMSNorm and
SwiGLU kernels that write their output straight as MXFP4, against HBM; and
NVFP4 (`nvfp4`: two-level quantization of A and the dequantizing GEMM, which
runs on the BF16 MFMA) on the primary workload, against the BF16 peak.

Inputs are resident in HBM before timing.  Steps rotate over enough copies of
the inputs (>= 512 MiB in total) that the 256 MiB Infinity Cache cannot serve
them.  Each timed region is a HIP graph of whole steps replayed on the stream
the kernels run on, bracketed by events and device synchronisations; one event
pair per graph replay also gives min / median / max per-step times.

Also reported (`--no-w4a8` skips it): the same workloads with MXFP8 activations
(W4A8: MXFP8 quantization of A + the MXFP8 x MXFP4 GEMM), against the FP8 MFMA
peak (a mixed FP8 x FP4 MFMA runs at the FP8 rate) or HBM.

Measured ceilings (probe kernels in the same library) are reported beside the
published peaks: the FP4 MFMA rate of a kernel that only runs MFMAs, and the
streaming read rate (`--no-ceilings` skips them).

Prints one JSON line on stdout.  The roofline object is for the GEMM kernel:
algorithmic flops (or bytes) per launch divided by the kernel's mean duration,
measured with events over a region of back-to-back GEMM launches.

`--only {step,gemm,quantize,quantize_b,copy}` instead runs that work eagerly
`--steps` times and prints nothing on stdout: the mode used under rocprofv3
(kernel traces and counter passes; `copy` is the plain device copy that
calibrates the byte counters; `--w4a8-only` selects the W4A8 kernels,
`--row-major-scales` the MXFP4 path on row-major scales).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_FP4_TFLOPS = 10100.0     # MI355X dense FP4 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (an FP8 x FP4 MFMA runs at the FP8 rate)
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16 MFMA (the NVFP4 GEMM's dequantized operands)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROTATION_BYTES = 512 << 20
COPY_BYTES = 512 << 20        # size of the counter-calibration copy


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_algorithmic_bytes(m, n, k, out_bytes=2):
    """Each packed code and scale byte of A and B once, plus C once."""
    return m * k // 2 + m * k // 32 + n * k // 2 + n * k // 32 + m * n * out_bytes


def quant_algorithmic_bytes(rows, k, code_bytes_per_elem=0.5):
    """BF16 in, codes (half a byte per element for MXFP4, one for MXFP8) and scale bytes out."""
    return rows * k * 2 + int(rows * k * code_bytes_per_elem) + rows * k // 32


def w4a8_algorithmic_bytes(m, n, k, out_bytes=2):
    """MXFP8 A (one byte per element + scales), MXFP4 B, C once."""
    return m * k + m * k // 32 + n * k // 2 + n * k // 32 + m * n * out_bytes


DETAIL_STEPS = 200    # calls timed for every line but the headline step (at least)
DETAIL_WARMUP = 20


def calls_per_replay(steps: int) -> int:
    """Calls per graph replay for `steps` timed calls: the largest divisor of
    `steps` that leaves at least four replays (samples), at most 64 calls; one
    call per replay below four steps."""
    if steps < 4:
        return 1
    return max(d for d in range(1, min(64, steps // 4) + 1) if steps % d == 0)


def summarize(samples, calls_per_sample=1):
    """mean / min / median / max (ms per call) over one list of per-call samples."""
    return {"mean": statistics.fmean(samples), "min": min(samples), "median": statistics.median(samples),
            "max": max(samples), "samples": len(samples), "calls_per_sample": calls_per_sample}


def us(t):
    """A timing summary in microseconds (sample counts kept as they are)."""
    return {k: (v if k in ("samples", "calls_per_sample") else round(v * 1e3, 3)) for k, v in t.items()}


def roofline(bound, achieved, peak, unit, traffic=None, kernel=None):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
    return r


def dense_inputs_record(w) -> dict:
    """Seeds and SHA-256 of the BF16 operands a dense workload draws."""
    a, b = w.make()
    return {"seeds": {"a": w.seed + workloads.ROLE_A, "a_outlier_channels": w.seed + workloads.ROLE_OUTLIER,
                      "b": w.seed + workloads.ROLE_B},
            "a_outliers": w.a_outliers, "b_sigma": w.b_sigma,
            "sha256": {"a_bf16": workloads.sha256_of(a), "b_bf16": workloads.sha256_of(b)}}


def moe_inputs_record(w) -> dict:
    """Seeds and SHA-256 of the MoE workload's inputs: token activations, router
    logits, expert weights and the offsets of the host routing."""
    x = w.tokens_bf16()
    wts = workloads.gaussian_bf16((w.experts, w.n, w.k), w.w_sigma, w.seed + workloads.ROLE_B)
    _, offsets = w.routing()
    return {"seeds": {"x": w.seed + workloads.ROLE_A, "w": w.seed + workloads.ROLE_B,
                      "route_bias": w.seed + workloads.ROLE_ROUTE_BIAS, "route_noise": w.seed + workloads.ROLE_ROUTE_NOISE},
            "bias_sigma": w.bias_sigma, "w_sigma": w.w_sigma,
            "sha256": {"x_bf16": workloads.sha256_of(x), "logits_f32": workloads.sha256_of(w.logits()),
                       "w_bf16": workloads.sha256_of(wts), "offsets_i32": workloads.sha256_of(offsets)}}


class DenseBench:
    """act = "mxfp4": the MXFP4 path; act = "mxfp8": W4A8 (MXFP8 activations,
    MXFP4 weights); act = "mxfp8x8": both operands MXFP8."""

    def __init__(self, w: workloads.DenseWorkload, dev, act: str = "mxfp4", quantize_b_in_step: bool = False,
                 interleaved: bool | None = None):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.w = w
        self.dev = dev
        self.act = act
        self.with_b = quantize_b_in_step
        # interleaved scales (the tile kernels' copy layout) wherever the tile
        # kernels run: prefill shapes with k % 512 == 0
        il_ok = w.m > 128 and w.k % 512 == 0
        self.il = il_ok if interleaved is None else (interleaved and il_ok)
        a8 = act in ("mxfp8", "mxfp8x8")
        k_a = w.k if a8 else w.k // 2                    # A code bytes per row
        k_b = w.k if act == "mxfp8x8" else w.k // 2      # B code bytes per row
        a, b = w.make()
        self.a_cpu, self.b_cpu = a, b
        a_d, b_d = a.to(dev), b.to(dev)
        # weight quantized once (not in the step)
        bq, bs = B.mxfp8_quantize(b_d) if act == "mxfp8x8" else B.mxfp4_quantize(b_d)
        if self.il:
            bs = B.mxfp4_scales_interleave(bs)
        m, n, k = w.m, w.n, w.k
        per_set = m * k * 2 + m * k_a + m * k // 32 + n * k_b + n * k // 32 + m * n * 2
        if self.with_b:
            per_set += n * k * 2       # each set also holds the weight in BF16, quantized in the step
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.per_set_bytes = per_set
        self.sets = []
        # the small-M workloads also keep each weight copy prepacked for mxfp4_gemm_nt_prepacked
        # (and, with MXFP8 activations, for mxfp8_gemm_w4a8_nt_prepacked)
        self.prepacked = act == "mxfp4" and m <= 128 and k % 512 == 0
        self.prepacked_b = act in ("mxfp4", "mxfp8") and m <= 128 and k % 512 == 0
        for _ in range(self.sets_n):
            a_s_shape = (k // 512, m, 16) if self.il else (m, k // 32)
            st = dict(a=a_d.clone(), aq=torch.empty((m, k_a), dtype=torch.uint8, device=dev),
                      as_=torch.empty(a_s_shape, dtype=torch.uint8, device=dev),
                      bq=bq.clone(), bs=bs.clone(), c=torch.empty((m, n), dtype=torch.bfloat16, device=dev))
            if self.with_b:
                st["b"] = b_d.clone()
            if self.prepacked_b:
                st["bp_q"], st["bp_s"] = B.mxfp4_prepack_weight(st["bq"], st["bs"])
            if self.prepacked or (self.prepacked_b and act == "mxfp8"):
                cb, sb = B.mxfp4_prepacked_weight_size(m, k)
                # the activation in the MXFP4 prepacked layout, or in the FP8 one (twice the code bytes)
                st["ap_q"] = torch.empty(cb if act == "mxfp4" else 2 * cb, dtype=torch.uint8, device=dev)
                st["ap_s"] = torch.empty(sb, dtype=torch.uint8, device=dev)
            self.sets.append(st)
        need = B.load_library().mxfp4_gemm_nt_workspace_size(m, n, k)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        del a_d, b_d
        torch.cuda.synchronize()

    def quantize(self, i):
        s = self.sets[i % self.sets_n]
        if self.act in ("mxfp8", "mxfp8x8"):
            (self.B.mxfp8_quantize_interleaved if self.il else self.B.mxfp8_quantize)(s["a"], s["aq"], s["as_"])
        elif self.il:
            self.B.mxfp4_quantize_interleaved(s["a"], s["aq"], s["as_"])
        else:
            self.B.mxfp4_quantize(s["a"], s["aq"], s["as_"])

    def quantize_b(self, i):
        """Quantizes the set's BF16 weight into the set's B operand (the bytes it
        already holds: the same quantization of the same weight)."""
        s = self.sets[i % self.sets_n]
        if self.il:
            self.B.mxfp4_quantize_interleaved(s["b"], s["bq"], s["bs"])
        else:
            self.B.mxfp4_quantize(s["b"], s["bq"], s["bs"])

    def step_quantize_both(self, i):
        self.quantize(i)
        self.quantize_b(i)
        self.gemm(i)

    def gemm(self, i):
        s = self.sets[i % self.sets_n]
        if self.act == "mxfp8":
            if self.il:
                self.B.mxfp8_gemm_w4a8_nt_interleaved(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"])
            else:
                self.B.mxfp8_gemm_w4a8_nt(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"])
        elif self.act == "mxfp8x8":
            if self.il:
                self.B.mxfp8_gemm_nt_interleaved(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"])
            else:
                self.B.mxfp8_gemm_nt(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"])
        elif self.il:
            self.B.mxfp4_gemm_nt_interleaved(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"])
        else:
            self.B.mxfp4_gemm_nt(s["aq"], s["as_"], s["bq"], s["bs"], c=s["c"], ws=self.ws)

    def gemm_prepacked(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_gemm_nt_prepacked(s["aq"], s["as_"], s["bp_q"], s["bp_s"], self.w.n, c=s["c"])

    def gemm_w4a8_prepacked(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp8_gemm_w4a8_nt_prepacked(s["aq"], s["as_"], s["bp_q"], s["bp_s"], self.w.n, c=s["c"])

    def step_w4a8_prepacked(self, i):
        self.quantize(i)
        self.gemm_w4a8_prepacked(i)

    def quantize_w4a8_both_prepacked(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp8_quantize_prepacked(s["a"], s["ap_q"], s["ap_s"])

    def gemm_w4a8_both_prepacked(self, i):
        s = self.sets[i % self.sets_n]
        w = self.w
        self.B.mxfp8_gemm_w4a8_nt_prepacked_ab(s["ap_q"], s["ap_s"], s["bp_q"], s["bp_s"], w.m, w.n, w.k, c=s["c"])

    def step_w4a8_both_prepacked(self, i):
        self.quantize_w4a8_both_prepacked(i)
        self.gemm_w4a8_both_prepacked(i)

    def step(self, i):
        self.quantize(i)
        self.gemm(i)

    def step_prepacked(self, i):
        self.quantize(i)
        self.gemm_prepacked(i)

    def quantize_prepacked(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_quantize_prepacked(s["a"], s["ap_q"], s["ap_s"])

    def gemm_prepacked_ab(self, i):
        s = self.sets[i % self.sets_n]
        w = self.w
        self.B.mxfp4_gemm_nt_prepacked_ab(s["ap_q"], s["ap_s"], s["bp_q"], s["bp_s"], w.m, w.n, w.k, c=s["c"])

    def step_prepacked_ab(self, i):
        self.quantize_prepacked(i)
        self.gemm_prepacked_ab(i)

    @staticmethod
    def _graph(fn, first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + count):
                fn(i)
        return g

    def timed(self, fn, steps, warmup, period=None):
        """Times exactly `steps` calls fn(0), fn(1), ..., fn(steps - 1).

        The calls run as `samples` graph replays of p calls each (p from
        calls_per_replay: p divides `steps`).  The input rotation continues across
        replays: replay r runs calls r*p ... r*p + p - 1, so with `period` (default:
        the number of input sets) rotating sets, ceil-free graph reuse needs
        lcm(p, period) / p distinct graphs.  Every statistic is over the same
        per-call samples (one replay's event time / p); the mean over the samples
        is the events' total over exactly `steps` calls divided by `steps`."""
        period = period or self.sets_n
        p = calls_per_replay(steps)
        graphs_n = math.lcm(p, period) // p
        for i in range(2):                    # eager warm-up before capture
            fn(i)
        torch.cuda.synchronize()
        graphs = [self._graph(fn, j * p, p) for j in range(graphs_n)]
        for r in range(max(1, math.ceil(warmup / p))):
            graphs[r % graphs_n].replay()
        torch.cuda.synchronize()
        samples_n = steps // p
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples_n + 1)]
        ev[0].record()
        for r in range(samples_n):
            graphs[r % graphs_n].replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        return summarize([ev[r].elapsed_time(ev[r + 1]) / p for r in range(samples_n)], p)


class MoEBench:
    """The grouped per-expert workload: routed rows sorted by expert, one
    weight matrix per expert (quantized once), device offsets."""

    def __init__(self, w: workloads.MoEWorkload, dev, act: str = "mxfp4", interleaved: bool = True):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.w = w
        self.act = act
        self.il = interleaved and w.k % 512 == 0   # interleaved scales (see DenseBench)
        a, wts, offsets = w.make()
        self.counts = (offsets[1:] - offsets[:-1]).tolist()
        rows, n, k, e = w.total_rows, w.n, w.k, w.experts
        a_d = a.to(dev)
        wq, ws = B.mxfp4_quantize(wts.view(e * n, k).to(dev))
        del wts
        wq, ws = wq.view(e, n, k // 2), ws.view(e, n, k // 32)
        if self.il:
            ws = B.mxfp4_scales_interleave(ws)
        off_d = offsets.to(dev)
        k_a = k if act == "mxfp8" else k // 2
        per_set = rows * k * 2 + rows * k_a + rows * k // 32 + e * n * k // 2 + e * n * k // 32 + rows * n * 2
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.sets = []
        for _ in range(self.sets_n):
            self.sets.append(dict(
                a=a_d.clone(), aq=torch.empty((rows, k_a), dtype=torch.uint8, device=dev),
                as_=torch.empty((k // 512, rows, 16) if self.il else (rows, k // 32), dtype=torch.uint8, device=dev),
                wq=wq.clone(), ws=ws.clone(), off=off_d.clone(),
                c=torch.empty((rows, n), dtype=torch.bfloat16, device=dev)))
        del a_d, wq, ws
        torch.cuda.synchronize()

    def quantize(self, i):
        s = self.sets[i % self.sets_n]
        if self.act == "mxfp8":
            (self.B.mxfp8_quantize_interleaved if self.il else self.B.mxfp8_quantize)(s["a"], s["aq"], s["as_"])
        elif self.il:
            self.B.mxfp4_quantize_interleaved(s["a"], s["aq"], s["as_"])
        else:
            self.B.mxfp4_quantize(s["a"], s["aq"], s["as_"])

    def gemm(self, i):
        s = self.sets[i % self.sets_n]
        if self.act == "mxfp8":
            fn = self.B.mxfp8_grouped_gemm_w4a8_nt_interleaved if self.il else self.B.mxfp8_grouped_gemm_w4a8_nt
            fn(s["aq"], s["as_"], s["wq"], s["ws"], s["off"], c=s["c"])
        elif self.il:
            self.B.mxfp4_grouped_gemm_nt_interleaved(s["aq"], s["as_"], s["wq"], s["ws"], s["off"], c=s["c"])
        else:
            self.B.mxfp4_grouped_gemm_nt(s["aq"], s["as_"], s["wq"], s["ws"], s["off"], c=s["c"])

    def step(self, i):
        self.quantize(i)
        self.gemm(i)

    def algorithmic_bytes(self):
        """Codes and scales of A and of every expert that has rows, plus C."""
        w = self.w
        used = sum(1 for c in self.counts if c > 0)
        rows = w.total_rows
        a_code = w.k if self.act == "mxfp8" else w.k // 2
        return (used * (w.n * w.k // 2 + w.n * w.k // 32) + rows * a_code + rows * w.k // 32
                + rows * w.n * 2)

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed


class MoELayerBench:
    """The whole MoE layer on the device: top-k routing of the router logits,
    the expert-sorted permutation, MXFP4 quantization scattered into the routed
    rows (scales interleaved), the grouped GEMM over the expert weights
    (quantized once, scales interleaved once), and the weighted combine back to
    tokens."""

    def __init__(self, w: workloads.MoEWorkload, dev):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.w = w
        t, e, kk, n, k = w.tokens, w.experts, w.top_k, w.n, w.k
        rows = t * kk
        x_d = w.tokens_bf16().to(dev)
        lg_d = w.logits().to(dev)
        wts = workloads.gaussian_bf16((e * n, k), w.w_sigma, w.seed + workloads.ROLE_B)
        wq, ws = B.mxfp4_quantize(wts.to(dev))
        del wts
        wq, ws = wq.view(e, n, k // 2), B.mxfp4_scales_interleave(ws.view(e, n, k // 32))
        per_set = (t * k * 2 + t * e * 4 + rows * (k // 2 + k // 32) + e * n * (k // 2 + k // 32)
                   + rows * n * 2 + t * n * 2)
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.sets = []
        for _ in range(self.sets_n):
            self.sets.append(dict(
                x=x_d.clone(), lg=lg_d.clone(), wq=wq.clone(), ws=ws.clone(),
                ids=torch.empty((t, kk), dtype=torch.int32, device=dev),
                gate=torch.empty((t, kk), dtype=torch.float32, device=dev),
                off=torch.empty((e + 1,), dtype=torch.int32, device=dev),
                rt=torch.empty((rows,), dtype=torch.int32, device=dev),
                tr=torch.empty((t, kk), dtype=torch.int32, device=dev),
                aq=torch.empty((rows, k // 2), dtype=torch.uint8, device=dev),
                as_=torch.empty((k // 512, rows, 16), dtype=torch.uint8, device=dev),
                y=torch.empty((rows, n), dtype=torch.bfloat16, device=dev),
                out=torch.empty((t, n), dtype=torch.bfloat16, device=dev)))
        del x_d, lg_d, wq, ws
        for i in range(self.sets_n):   # every set holds a complete layer's intermediates before timing
            self.step(i)
        torch.cuda.synchronize()
        self.counts = torch.diff(self.sets[0]["off"]).cpu().tolist()

    def route(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_moe_route(s["lg"], self.w.top_k, s["ids"], s["gate"])

    def permute(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_moe_permute(s["ids"], self.w.experts, s["off"], s["rt"], s["tr"])

    def scatter(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_moe_quantize_scatter_interleaved(s["x"], s["tr"], self.w.total_rows, s["aq"], s["as_"])

    def gemm(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_grouped_gemm_nt_interleaved(s["aq"], s["as_"], s["wq"], s["ws"], s["off"], c=s["y"])

    def combine(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_moe_combine(s["y"], s["tr"], s["gate"], out=s["out"])

    def step(self, i):
        self.route(i)
        self.permute(i)
        self.scatter(i)
        self.gemm(i)
        self.combine(i)

    def algorithmic_bytes(self):
        """What each step must move once: inputs read, outputs written."""
        w = self.w
        t, e, kk, n, k, rows = w.tokens, w.experts, w.top_k, w.n, w.k, w.total_rows
        used = sum(1 for c in self.counts if c > 0)
        return {
            "route": t * e * 4 + rows * 8,
            "permute": rows * 4 + (e + 1) * 4 + rows * 8,
            "scatter": t * k * 2 + rows * (k // 2 + k // 32) + rows * 4,
            "gemm": used * n * (k // 2 + k // 32) + rows * (k // 2 + k // 32) + rows * n * 2,
            "combine": rows * n * 2 + rows * 8 + t * n * 2,
        }

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed


def measure_moe_layer(args, dev, us):
    wm = workloads.ALL[args.moe]
    eprint(f"[bench] building inputs for the on-device MoE layer of {wm.name}")
    lb = MoELayerBench(wm, dev)
    # at least 16 launches per graph replay (64 steps = 4 samples of 16): replays of only a few
    # short routing and permutation launches would add the replay gap to each of them
    msteps = max(64, args.detail_steps // 2)
    nbytes = lb.algorithmic_bytes()
    out = {"workload": wm.name, "steps": msteps, "rotating_input_sets": lb.sets_n,
           "step": "route + permute + scatter-quantize + grouped mxfp4 GEMM + combine (interleaved scales)",
           "rows_per_expert": {"min": min(lb.counts), "max": max(lb.counts),
                               "empty": sum(c == 0 for c in lb.counts)}}
    st = lb.timed(lb.step, msteps, 2)
    out["step_us"] = us(st)
    out["step_tflops"] = round(wm.flops / (st["mean"] * 1e-3) / 1e12, 2)
    kern = {}
    for name in ("route", "permute", "scatter", "gemm", "combine"):
        tk = lb.timed(getattr(lb, name), msteps, 2)
        gbs = nbytes[name] / (tk["mean"] * 1e-3) / 1e9
        kern[name] = {"us": us(tk), "algorithmic_bytes": nbytes[name], "gbs": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        kname = {"scatter": "quantize_scatter_kernel", "combine": "combine_kernel"}.get(name)
        if kname:
            kern[name]["traffic"] = traffic_from_profiles(wm.name, kname)
    kern["gemm"]["tflops"] = round(wm.flops / (kern["gemm"]["us"]["mean"] * 1e-6) / 1e12, 2)
    out["kernels"] = kern
    eprint(f"[bench] MoE layer {wm.name}: step {st['mean']*1e3:.1f} us; " +
           ", ".join(f"{k} {v['us']['mean']:.1f} us" for k, v in kern.items()))
    del lb
    return out


class ProducerBench:
    """Fused producers on the prefill shapes: residual add + RMSNorm + MXFP4 of
    a [4096, 4096] activation (writing the updated residual stream), and
    SwiGLU + MXFP4 of the [4096, 14336] FFN activation read from the two
    halves of a [4096, 28672] gate|up buffer."""

    def __init__(self, dev, rows=4096, hidden=4096, inter=14336):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.rows, self.hidden, self.inter = rows, hidden, inter
        x = workloads.activation_bf16(rows, hidden, 300, outliers=True).to(dev)
        res = workloads.activation_bf16(rows, hidden, 301, outliers=False).to(dev)
        gamma = workloads.gaussian_bf16((hidden,), 0.1, 302).to(dev)
        gu = workloads.gaussian_bf16((rows, 2 * inter), 1.0, 401).to(dev)
        per_set = rows * hidden * 2 * 3 + rows * hidden * 17 // 32 + rows * inter * 4 + rows * inter * 17 // 32
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.sets = []
        for _ in range(self.sets_n):
            self.sets.append(dict(
                x=x.clone(), res=res.clone(), gamma=gamma.clone(), h=torch.empty_like(x), gu=gu.clone(),
                q=torch.empty((rows, hidden // 2), dtype=torch.uint8, device=dev),
                s=torch.empty((rows, hidden // 32), dtype=torch.uint8, device=dev),
                qi=torch.empty((rows, inter // 2), dtype=torch.uint8, device=dev),
                si=torch.empty((rows, inter // 32), dtype=torch.uint8, device=dev)))
        del x, res, gamma, gu
        torch.cuda.synchronize()

    def rmsnorm(self, i):
        s = self.sets[i % self.sets_n]
        self.B.mxfp4_rmsnorm_quantize(s["x"], s["gamma"], 1e-5, residual=s["res"], residual_out=s["h"],
                                      q=s["q"], scales=s["s"])

    def swiglu(self, i):
        s = self.sets[i % self.sets_n]
        k = self.inter
        self.B.mxfp4_swiglu_quantize(s["gu"][:, :k], s["gu"][:, k:], q=s["qi"], scales=s["si"])

    def algorithmic_bytes(self):
        r, h, f = self.rows, self.hidden, self.inter
        return {
            # x, residual and gamma in; the updated residual, codes and scales out
            "rmsnorm": r * h * 2 * 2 + h * 2 + r * h * 2 + r * h // 2 + r * h // 32,
            # gate and up in; codes and scales out
            "swiglu": r * f * 2 * 2 + r * f // 2 + r * f // 32,
        }

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed


def measure_producers(args, dev, us):
    eprint("[bench] fused producers (RMSNorm and SwiGLU emitting MXFP4)")
    pb = ProducerBench(dev)
    nbytes = pb.algorithmic_bytes()
    out = {}
    for name, shape in (("rmsnorm", f"{pb.rows}x{pb.hidden}, residual add"),
                        ("swiglu", f"{pb.rows}x{pb.inter} from a {pb.rows}x{2 * pb.inter} gate|up buffer")):
        t = pb.timed(getattr(pb, name), max(64, args.detail_steps // 2), 4)
        gbs = nbytes[name] / (t["mean"] * 1e-3) / 1e9
        kname = f"{name}_quantize_kernel"
        out[name] = {"shape": shape, "us": us(t), "algorithmic_bytes": nbytes[name], "gbs": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4),
                                  "traffic": traffic_from_profiles(f"producer_{name}", kname)}}
        eprint(f"[bench] {name}_quantize {shape}: {t['mean']*1e3:.2f} us ({gbs:.0f} GB/s)")
    del pb
    return out


class NvBench:
    """NVFP4 on the prefill workload: two-level quantization of A (the step's
    activation), and the dequantizing NT GEMM against a weight quantized once."""

    def __init__(self, w: workloads.DenseWorkload, dev):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.w = w
        a, b = w.make()
        a_d = a.to(dev)
        bq, bs, bg = B.nvfp4_quantize(b.to(dev))
        m, n, k = w.m, w.n, w.k
        per_set = m * k * 2 + m * (k // 2 + k // 16 + 4) + n * (k // 2 + k // 16 + 4) + m * n * 2
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.sets = []
        for _ in range(self.sets_n):
            self.sets.append(dict(
                a=a_d.clone(), aq=torch.empty((m, k // 2), dtype=torch.uint8, device=dev),
                as_=torch.empty((m, k // 16), dtype=torch.uint8, device=dev),
                ag=torch.empty((m,), dtype=torch.float32, device=dev),
                bq=bq.clone(), bs=bs.clone(), bg=bg.clone(),
                c=torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
        for i in range(self.sets_n):
            self.quantize(i)
        del a_d
        torch.cuda.synchronize()

    def quantize(self, i):
        s = self.sets[i % self.sets_n]
        self.B.nvfp4_quantize(s["a"], s["aq"], s["as_"], s["ag"])

    def gemm(self, i):
        s = self.sets[i % self.sets_n]
        self.B.nvfp4_gemm_nt(s["aq"], s["as_"], s["ag"], s["bq"], s["bs"], s["bg"], c=s["c"])

    def step(self, i):
        self.quantize(i)
        self.gemm(i)

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed


def measure_nvfp4(args, dev, w, us):
    eprint(f"[bench] NVFP4 on {w.name}")
    nb = NvBench(w, dev)
    s = nb.timed(nb.step, args.detail_steps, args.detail_warmup)
    g = nb.timed(nb.gemm, args.detail_steps, args.detail_warmup)
    q = nb.timed(nb.quantize, args.detail_steps, args.detail_warmup)
    tf = w.flops / (g["mean"] * 1e-3) / 1e12
    qbytes = w.m * w.k * 2 + w.m * (w.k // 2 + w.k // 16 + 4)
    out = {"workload": w.name,
           "dtype": "nvfp4 (e2m1, ue4m3 per 16, fp32 per row), exact bf16 dequantization, bf16 MFMA, fp32 accumulate",
           "step_us": us(s), "gemm_us": us(g), "quantize_a_us": us(q),
           "quantize_a_gbs": round(qbytes / (q["mean"] * 1e-3) / 1e9, 1),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_from_profiles(w.name, "nvfp4_gemm_kernel")}}
    eprint(f"[bench] NVFP4 {w.name}: step {s['mean']*1e3:.2f} us, gemm {g['mean']*1e3:.2f} us ({tf:.0f} TFLOP/s), "
           f"quantize {q['mean']*1e3:.2f} us")
    del nb
    return out


class Ceilings:
    """Measured ceilings on this GPU (include/mxfp4_probe.h), reported next to the
    published peaks: the FP4 scaled-MFMA rate of a kernel that only runs MFMAs
    (8 waves per CU like the tile GEMM; one launch about as long as the 4096^3
    GEMM, and one ~8x longer), and the streaming read rate over buffers of the
    decode weight's size (rotated past the Infinity Cache) and over 1 GiB."""

    READ_SMALL = 14336 * 4096 // 2        # the decode weight's packed codes

    def __init__(self, dev):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        props = torch.cuda.get_device_properties(dev)
        self.cus = props.multi_processor_count
        g = torch.Generator(device="cpu").manual_seed(7)
        self.seed = torch.randint(0, 256, (B.PROBE_SEED_BYTES,), dtype=torch.uint8, generator=g).to(dev)
        self.mfma_out = torch.empty(self.cus * 512, dtype=torch.float32, device=dev)
        self.read_blocks = self.cus          # one 256-thread workgroup per CU reads fastest
        self.read_out = torch.empty(self.read_blocks * 256, dtype=torch.int32, device=dev)
        self.small = [torch.full((self.READ_SMALL,), i + 1, dtype=torch.uint8, device=dev)
                      for i in range(max(2, math.ceil(ROTATION_BYTES / self.READ_SMALL)))]
        self.big = torch.full((1 << 30,), 3, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed

    def measure(self, steps):
        # Several launches per captured graph, as for the GEMMs: a graph of one
        # launch adds a replay gap of several microseconds to every launch.
        out = {}
        for fmt, a_fp8 in (("fp4", False), ("w4a8", True)):
            for label, iters in (("short", 128), ("long", 1024)):
                if a_fp8:
                    iters //= 2           # FP8-rate MFMAs take twice as long each
                self.sets_n = 1
                flops = self.B.load_library().mxfp4_probe_mfma_flops(self.cus, iters)
                t = self.timed(lambda i: self.B.mxfp4_probe_mfma(self.seed, self.mfma_out, self.cus, iters,
                                                                 a_fp8=a_fp8),
                               steps, max(4, steps // 10))
                out[f"mfma_{fmt}_tflops_{label}"] = round(flops / (t["mean"] * 1e-3) / 1e12, 1)
                out[f"mfma_{fmt}_probe_{label}_us"] = round(t["mean"] * 1e3, 2)
        self.sets_n = len(self.small)
        t = self.timed(lambda i: self.B.mxfp4_probe_read(self.small[i % self.sets_n], self.read_out,
                                                          self.read_blocks), steps, max(4, steps // 10))
        out["read_gbs_29MB"] = round(self.READ_SMALL / (t["mean"] * 1e-3) / 1e9, 1)
        out["read_29MB_us"] = round(t["mean"] * 1e3, 2)
        self.sets_n = 4
        t = self.timed(lambda i: self.B.mxfp4_probe_read(self.big, self.read_out, self.read_blocks),
                       max(8, steps // 10), 4)
        out["read_gbs_1GiB"] = round((1 << 30) / (t["mean"] * 1e-3) / 1e9, 1)
        return out


def cpu_baseline(bench: DenseBench, target_seconds: float):
    """The CPU oracle, as it stands, on a bounded sample of the same step: oracle
    quantization of A, then its float64 GEMM against the pre-quantized B (the
    weight packing is outside the step, as on the GPU).  The whole step is
    repeated to fill about `target_seconds`; if one step would take longer than
    that, only the first rows of A are used."""
    import oracle
    from threadpoolctl import threadpool_info
    w = bench.w
    bq, bs = oracle.quantize(workloads.bf16_bits(bench.b_cpu))
    a_bits = workloads.bf16_bits(bench.a_cpu)

    def run(rows):
        t = time.perf_counter()
        aq, as_ = oracle.quantize(a_bits[:rows])
        oracle.gemm_nt(aq, as_, bq, bs)
        return time.perf_counter() - t

    pilot_rows = min(w.m, 64)
    t_pilot = run(pilot_rows)
    est_full = t_pilot * w.m / pilot_rows
    if est_full <= target_seconds:
        rows = w.m
        reps = max(1, round(target_seconds / max(run(rows), 1e-3)))
    else:
        rows = max(pilot_rows, int(w.m * target_seconds / est_full))
        reps = 1
    t0 = time.perf_counter()
    for _ in range(reps):
        run(rows)
    t = time.perf_counter() - t0
    flops = 2 * rows * w.n * w.k * reps
    blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    avail = len(os.sched_getaffinity(0))
    # the oracle quantizer alone (NumPy, one thread) on A's rows, about a fifth of the budget
    q_rows, q_reps, tq = w.m, 0, 0.0
    while tq < target_seconds / 5:
        t1 = time.perf_counter()
        oracle.quantize(a_bits[:q_rows])
        tq += time.perf_counter() - t1
        q_reps += 1
    q_bytes = quant_algorithmic_bytes(q_rows, w.k) * q_reps
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": int(blas), "kind": "oracle",
            "sample": f"{rows} of {w.m} rows of A, {reps} repetition(s), {t:.1f} s: oracle quantize of A "
                      f"(NumPy, one thread) + float64 BLAS GEMM against the pre-quantized {w.n}x{w.k} B "
                      f"({blas} BLAS threads of {avail} available cores)",
            "quantize": {"value": round(q_bytes / tq / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": f"oracle quantize of the {q_rows}x{w.k} BF16 A, {q_reps} repetition(s), "
                                   f"{tq:.1f} s (NumPy, one thread; bytes = 2 in + 0.5 + 1/32 out per element)"}}


# The sources each measured kernel is built from: recorded counter data stays
# valid while these files are unchanged.
KERNEL_SOURCES = {
    "gemm_tile_kernel": ("gemm_tile.hip", "common.hpp"),
    "gemm_stream_kernel": ("gemm_stream.hip", "common.hpp"),
    "gemm_stream_pre_kernel": ("gemm_stream.hip", "common.hpp"),
    "gemm_pp_kernel": ("gemm_stream.hip", "common.hpp"),
    "quantize_kernel": ("quantize.hip", "common.hpp"),
    "quantize_prepacked_kernel": ("quantize.hip", "common.hpp"),
    "quantize_scatter_kernel": ("moe.hip", "common.hpp"),
    "combine_kernel": ("moe.hip", "common.hpp"),
    "rmsnorm_quantize_kernel": ("producers.hip", "common.hpp"),
    "swiglu_quantize_kernel": ("producers.hip", "common.hpp"),
    "nvfp4_quantize_kernel": ("nvfp4.hip", "common.hpp"),
    "nvfp4_gemm_kernel": ("nvfp4.hip", "common.hpp"),
    "gemm_tile_kernel_f8f8": ("gemm_tile.hip", "common.hpp"),
    "grouped_persistent_kernel": ("gemm_tile.hip", "common.hpp"),
}


def sources_sha(kernel: str) -> str:
    """Hash of the HIP sources of one kernel (first 16 hex digits of a SHA-256)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` recorded in profiles/traffic.md,
    if the kernel's sources have not changed since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    sha = sources_sha(kernel)
    for line in open(path):
        parts = dict(p.split("=", 1) for p in line.split() if "=" in p)
        if (parts.get("workload") == workload and parts.get("kernel") == kernel and parts.get("sources") == sha
                and "bytes_per_launch" in parts):
            return float(parts["bytes_per_launch"])
    return None


def measure_w4a8(args, dev, w, us):
    """W4A8 (MXFP8 activations x MXFP4 weights) on the primary, decode and MoE
    workloads: step = MXFP8 quantization of A + the W4A8 GEMM."""
    out = {"dtype": "mxfp8 e4m3 x mxfp4 e2m1, e8m0 block scales, fp32 accumulate, bf16 out",
           "scales": "interleaved for the prefill and MoE GEMMs (written by the quantizers); decode: both operands "
                     "prepacked (A in the FP8 prepacked layout)"}
    eprint(f"[bench] W4A8 on {w.name}")
    b = DenseBench(w, dev, "mxfp8")
    s = b.timed(b.step, args.detail_steps, args.detail_warmup)
    g = b.timed(b.gemm, args.detail_steps, args.detail_warmup)
    q = b.timed(b.quantize, args.detail_steps, args.detail_warmup)
    tf = w.flops / (g["mean"] * 1e-3) / 1e12
    qbytes = quant_algorithmic_bytes(w.m, w.k, 1.0)
    out["prefill"] = {
        "workload": w.name, "step_us": us(s), "step_tflops": round(w.flops / (s["mean"] * 1e-3) / 1e12, 2),
        "gemm_us": us(g), "quantize_a_us": us(q),
        "quantize_a_gbs": round(qbytes / (q["mean"] * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
    }
    eprint(f"[bench] W4A8 {w.name}: step {s['mean']*1e3:.2f} us, gemm {g['mean']*1e3:.2f} us ({tf:.0f} TFLOP/s)")
    del b
    if args.secondary != "none":
        w2 = workloads.DENSE[args.secondary]
        b2 = DenseBench(w2, dev, "mxfp8")
        pre = b2.prepacked_b
        # with the weight held prepacked: the prepacked-weight kernel; the streaming
        # kernel on the row-major weight timed beside it
        s2 = b2.timed(b2.step_w4a8_prepacked if pre else b2.step, args.detail_steps, args.detail_warmup)
        g2 = b2.timed(b2.gemm_w4a8_prepacked if pre else b2.gemm, args.detail_steps, args.detail_warmup)
        gu = b2.timed(b2.gemm, args.detail_steps, args.detail_warmup) if pre else g2
        gpp = b2.timed(b2.gemm_w4a8_both_prepacked, args.detail_steps, args.detail_warmup) if pre else None
        spp = b2.timed(b2.step_w4a8_both_prepacked, args.detail_steps, args.detail_warmup) if pre else None
        gbytes = w4a8_algorithmic_bytes(w2.m, w2.n, w2.k)
        gbs = gbytes / (g2["mean"] * 1e-3) / 1e9
        if pre:
            # both operands prepacked leads, as on the MXFP4 decode line: A quantized
            # straight into the FP8 prepacked layout, no LDS in the GEMM; the
            # prepacked-weight kernel (row-major A) and the streaming kernel beside it
            gbs_pp = gbytes / (gpp["mean"] * 1e-3) / 1e9
            out["decode"] = {
                "workload": w2.name, "step_us": us(spp), "gemm_us": us(gpp),
                "step": "quantize A into the FP8 prepacked layout + W4A8 GEMM on both prepacked operands",
                "roofline": {"bound": "hbm", "achieved": round(gbs_pp, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs_pp / PEAK_HBM_GBS, 4), "kernel": "gemm_pp_kernel (fp8 A)"},
                "prepacked_weight": {
                    "step": "quantize A to MXFP8 (row-major) + W4A8 GEMM on the prepacked weight",
                    "step_us": us(s2), "gemm_us": us(g2), "gemm_gbs": round(gbs, 1),
                    "gemm_hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "gemm_stream_pre_kernel (fp8 A)"},
                "gemm_unpacked_weight_us": us(gu),
            }
            eprint(f"[bench] W4A8 {w2.name}: gemm {gpp['mean']*1e3:.2f} us ({gbs_pp:.0f} GB/s, both operands "
                   f"prepacked; prepacked weight {g2['mean']*1e3:.2f} us, row-major weight {gu['mean']*1e3:.2f} us)")
        else:
            out["decode"] = {
                "workload": w2.name, "step_us": us(s2), "gemm_us": us(g2),
                "step": "quantize A to MXFP8 + streaming W4A8 GEMM",
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "gemm_stream_kernel (fp8 A)"},
            }
            eprint(f"[bench] W4A8 {w2.name}: gemm {g2['mean']*1e3:.2f} us ({gbs:.0f} GB/s)")
        del b2
    if args.moe != "none":
        wm = workloads.ALL[args.moe]
        mb = MoEBench(wm, dev, "mxfp8")
        msteps = max(16, args.detail_steps // 2)
        sm = mb.timed(mb.step, msteps, 2)
        gm = mb.timed(mb.gemm, msteps, 2)
        tfm = wm.flops / (gm["mean"] * 1e-3) / 1e12
        out["moe"] = {
            "workload": wm.name, "step_us": us(sm), "gemm_us": us(gm),
            "step_tflops": round(wm.flops / (sm["mean"] * 1e-3) / 1e12, 2),
            "roofline": {"bound": "mfma", "achieved": round(tfm, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfm / PEAK_FP8_TFLOPS, 4)},
        }
        eprint(f"[bench] W4A8 {wm.name}: grouped gemm {gm['mean']*1e3:.1f} us ({tfm:.0f} TFLOP/s)")
        del mb
    return out


def measure_large(args, dev):
    """The two larger prefill GEMMs: ffn-down 4096x4096x14336 and square 8192^3
    (step: quantize A + GEMM against the pre-quantized weight), each with its
    roofline against the FP4 MFMA peak."""
    out = {}
    for wl in (workloads.FFN_DOWN, workloads.SQUARE8192):
        eprint(f"[bench] building inputs for {wl.name}")
        b = DenseBench(wl, dev)
        rows_sets = b.sets_n
        s = b.timed(b.step, args.detail_steps, args.detail_warmup)
        g = b.timed(b.gemm, args.detail_steps, args.detail_warmup)
        q = b.timed(b.quantize, args.detail_steps, args.detail_warmup)
        tf = wl.flops / (g["mean"] * 1e-3) / 1e12
        qbytes = quant_algorithmic_bytes(wl.m, wl.k)
        del b
        g_rm = None
        if not args.no_row_major:
            rm = DenseBench(wl, dev, interleaved=False)
            g_rm = rm.timed(rm.gemm, args.detail_steps, args.detail_warmup)
            del rm
        out[wl.name] = {
            "m": wl.m, "n": wl.n, "k": wl.k, "rotating_input_sets": rows_sets,
            "step": "quantize A + mxfp4 NT GEMM -> bf16 (B pre-quantized; interleaved scales)",
            "step_us": us(s), "step_tflops": round(wl.flops / (s["mean"] * 1e-3) / 1e12, 2),
            "gemm_us": us(g), "gemm_tflops": round(tf, 2),
            "quantize_a_us": us(q), "quantize_a_gbs": round(qbytes / (q["mean"] * 1e-3) / 1e9, 1),
            "roofline": roofline("mfma", tf, PEAK_FP4_TFLOPS, "TFLOP/s",
                                 traffic_from_profiles(wl.name, "gemm_tile_kernel"), kernel="gemm_tile_kernel"),
            "inputs": dense_inputs_record(wl),
        }
        if g_rm:
            out[wl.name]["row_major_scales"] = {"gemm_us": us(g_rm),
                                                "gemm_tflops": round(wl.flops / (g_rm["mean"] * 1e-3) / 1e12, 2)}
        eprint(f"[bench] {wl.name}: step {s['mean']*1e3:.1f} us, gemm {g['mean']*1e3:.1f} us ({tf:.0f} TFLOP/s)"
               + (f"; row-major scales {g_rm['mean']*1e3:.1f} us" if g_rm else ""))
    return out


def measure_decode(args, dev, w2, primary: bool):
    """A decode-shaped workload.  With the weight held prepacked, the step quantizes
    A straight into the prepacked layout and runs the GEMM that loads both operands
    into registers; the same GEMM with only B prepacked and on the row-major weight
    is timed beside it."""
    eprint(f"[bench] building inputs for {w2.name}")
    b2 = DenseBench(w2, dev)
    pre = b2.prepacked
    s2 = b2.timed(b2.step_prepacked_ab if pre else b2.step, args.detail_steps, args.detail_warmup)
    g2 = b2.timed(b2.gemm_prepacked_ab if pre else b2.gemm, args.detail_steps, args.detail_warmup)
    gb = b2.timed(b2.gemm_prepacked, args.detail_steps, args.detail_warmup) if pre else g2
    gu = b2.timed(b2.gemm, args.detail_steps, args.detail_warmup) if pre else g2
    q2 = b2.timed(b2.quantize_prepacked if pre else b2.quantize, args.detail_steps, args.detail_warmup)
    gbytes = gemm_algorithmic_bytes(w2.m, w2.n, w2.k)
    qb2 = quant_algorithmic_bytes(w2.m, w2.k)
    gemm_gbs = gbytes / (g2["mean"] * 1e-3) / 1e9
    kname = "gemm_pp_kernel" if pre else "gemm_stream_kernel"
    out = {
        "workload": w2.name, "m": w2.m, "n": w2.n, "k": w2.k,
        "value": round((gbytes + qb2) / (s2["mean"] * 1e-3) / 1e9, 1), "unit": "GB/s",
        "ms_per_step": round(s2["mean"], 6), "step_us": us(s2), "rotating_input_sets": b2.sets_n,
        "step": ("quantize A into the prepacked layout + mxfp4 GEMM on prepacked A and B "
                 "(B quantized and prepacked once)" if pre
                 else "quantize A + streaming mxfp4 GEMM (B pre-quantized)"),
        "roofline": roofline("hbm", gemm_gbs, PEAK_HBM_GBS, "GB/s", traffic_from_profiles(w2.name, kname),
                             kernel=kname),
        "kernels": {"gemm_us": us(g2), "quantize_a_us": us(q2),
                    "gemm_tflops": round(w2.flops / (g2["mean"] * 1e-3) / 1e12, 2),
                    "gemm_prepacked_b_only_us": us(gb),
                    "gemm_prepacked_b_only_gbs": round(gbytes / (gb["mean"] * 1e-3) / 1e9, 1),
                    "gemm_unpacked_weight_us": us(gu),
                    "gemm_unpacked_weight_gbs": round(gbytes / (gu["mean"] * 1e-3) / 1e9, 1)},
        "inputs": dense_inputs_record(w2),
    }
    if primary:
        out["metric"] = "achieved HBM GB/s at decode M=128"
    eprint(f"[bench] {w2.name}: step {s2['mean']*1e3:.2f} us, gemm {g2['mean']*1e3:.2f} us "
           f"({gemm_gbs:.0f} GB/s; B-only prepacked {gb['mean']*1e3:.2f} us, unpacked {gu['mean']*1e3:.2f} us)")
    del b2
    return out


def measure_mxfp8(args, dev, w):
    """Both operands MXFP8 on the primary workload: step = MXFP8 quantization of
    A + the MXFP8 x MXFP8 GEMM against a weight quantized to MXFP8 once, against
    the FP8 MFMA peak."""
    eprint(f"[bench] MXFP8 x MXFP8 on {w.name}")
    b = DenseBench(w, dev, "mxfp8x8")
    s = b.timed(b.step, args.detail_steps, args.detail_warmup)
    g = b.timed(b.gemm, args.detail_steps, args.detail_warmup)
    tf = w.flops / (g["mean"] * 1e-3) / 1e12
    out = {"workload": w.name, "dtype": "mxfp8 e4m3 x mxfp8 e4m3, e8m0 block scales, fp32 accumulate, bf16 out",
           "step": "quantize A (bf16->mxfp8) + mxfp8 x mxfp8 NT GEMM -> bf16 (B quantized to mxfp8 once; "
                   "interleaved scales)",
           "step_us": us(s), "step_tflops": round(w.flops / (s["mean"] * 1e-3) / 1e12, 2), "gemm_us": us(g),
           "roofline": roofline("mfma", tf, PEAK_FP8_TFLOPS, "TFLOP/s",
                                traffic_from_profiles(w.name, "gemm_tile_kernel_f8f8"),
                                kernel="gemm_tile_kernel (mxfp8 x mxfp8, 256x256)")}
    eprint(f"[bench] MXFP8 x MXFP8 {w.name}: step {s['mean']*1e3:.2f} us, gemm {g['mean']*1e3:.2f} us ({tf:.0f} TFLOP/s)")
    del b
    return out


class FusedDecodeBench:
    """Decode from the activation's producer (the quantization fused into the
    producer): RMSNorm of a [128, 4096] hidden state before the 14336 x 4096
    up projection, and SwiGLU of a [128, 2 x 14336] gate|up buffer before the
    4096 x 14336 down projection, each followed by the GEMM on prepacked
    operands against its weight (quantized and prepacked once).  Two forms of
    each step:
      fused:      producer writing the prepacked layout, GEMM (2 launches);
      two_launch: producer writing BF16 (and row-major MXFP4), the prepacked
                  quantizer on the BF16 output, GEMM (3 launches)."""

    def __init__(self, dev):
        from block_scaled_fp4_mxfp4_amd import binding as B
        self.B = B
        self.m, self.hidden, self.inter = 128, 4096, 14336
        m, h, f = self.m, self.hidden, self.inter
        x = workloads.activation_bf16(m, h, 800, outliers=True).to(dev)
        gamma = workloads.gaussian_bf16((h,), 0.1, 801).to(dev)
        gu = workloads.gaussian_bf16((m, 2 * f), 1.0, 802).to(dev)
        w_up = workloads.gaussian_bf16((f, h), 0.02, 803).to(dev)
        w_dn = workloads.gaussian_bf16((h, f), 0.02, 804).to(dev)
        up_p = B.mxfp4_prepack_weight(*B.mxfp4_quantize(w_up))
        dn_p = B.mxfp4_prepack_weight(*B.mxfp4_quantize(w_dn))
        del w_up, w_dn
        per_set = sum(t.numel() for t in (*up_p, *dn_p)) + m * (h + 2 * f) * 2
        self.sets_n = max(2, math.ceil(ROTATION_BYTES / per_set))
        self.sets = []
        for _ in range(self.sets_n):
            st = dict(x=x.clone(), gamma=gamma.clone(), gu=gu.clone(), up=[t.clone() for t in up_p],
                      dn=[t.clone() for t in dn_p], y=torch.empty((m, h), dtype=torch.bfloat16, device=dev),
                      yd=torch.empty((m, f), dtype=torch.bfloat16, device=dev),
                      q=torch.empty((m, h // 2), dtype=torch.uint8, device=dev),
                      s=torch.empty((m, h // 32), dtype=torch.uint8, device=dev),
                      qd=torch.empty((m, f // 2), dtype=torch.uint8, device=dev),
                      sd=torch.empty((m, f // 32), dtype=torch.uint8, device=dev),
                      c_up=torch.empty((m, f), dtype=torch.bfloat16, device=dev),
                      c_dn=torch.empty((m, h), dtype=torch.bfloat16, device=dev))
            st["ap"] = [torch.empty(n_, dtype=torch.uint8, device=dev) for n_ in B.mxfp4_prepacked_weight_size(m, h)]
            st["apd"] = [torch.empty(n_, dtype=torch.uint8, device=dev) for n_ in B.mxfp4_prepacked_weight_size(m, f)]
            self.sets.append(st)
        del x, gamma, gu, up_p, dn_p
        torch.cuda.synchronize()

    def up_fused(self, i):
        s, B = self.sets[i % self.sets_n], self.B
        B.mxfp4_rmsnorm_quantize(s["x"], s["gamma"], 1e-5, q=s["ap"][0], scales=s["ap"][1], prepacked=True)
        B.mxfp4_gemm_nt_prepacked_ab(*s["ap"], *s["up"], self.m, self.inter, self.hidden, c=s["c_up"])

    def up_two_launch(self, i):
        s, B = self.sets[i % self.sets_n], self.B
        B.mxfp4_rmsnorm_quantize(s["x"], s["gamma"], 1e-5, y=s["y"], q=s["q"], scales=s["s"])
        B.mxfp4_quantize_prepacked(s["y"], *s["ap"])
        B.mxfp4_gemm_nt_prepacked_ab(*s["ap"], *s["up"], self.m, self.inter, self.hidden, c=s["c_up"])

    def down_fused(self, i):
        s, B, f = self.sets[i % self.sets_n], self.B, self.inter
        B.mxfp4_swiglu_quantize(s["gu"][:, :f], s["gu"][:, f:], q=s["apd"][0], scales=s["apd"][1], prepacked=True)
        B.mxfp4_gemm_nt_prepacked_ab(*s["apd"], *s["dn"], self.m, self.hidden, f, c=s["c_dn"])

    def down_two_launch(self, i):
        s, B, f = self.sets[i % self.sets_n], self.B, self.inter
        B.mxfp4_swiglu_quantize(s["gu"][:, :f], s["gu"][:, f:], y=s["yd"], q=s["qd"], scales=s["sd"])
        B.mxfp4_quantize_prepacked(s["yd"], *s["apd"])
        B.mxfp4_gemm_nt_prepacked_ab(*s["apd"], *s["dn"], self.m, self.hidden, f, c=s["c_dn"])

    _graph = staticmethod(DenseBench._graph)
    timed = DenseBench.timed


def measure_fused_decode(args, dev):
    eprint("[bench] decode steps from the producer: quantization fused into RMSNorm / SwiGLU vs a separate launch")
    fb = FusedDecodeBench(dev)
    steps = max(64, args.detail_steps)
    out = {"rotating_input_sets": fb.sets_n, "steps": steps}
    for name, shape in (("up", "RMSNorm 128x4096 -> GEMM 128x14336x4096"),
                        ("down", "SwiGLU 128x14336 (gate|up 128x28672) -> GEMM 128x4096x14336")):
        fused = fb.timed(getattr(fb, f"{name}_fused"), steps, 8)
        two = fb.timed(getattr(fb, f"{name}_two_launch"), steps, 8)
        out[name] = {"shape": shape, "fused_us": us(fused), "two_launch_us": us(two),
                     "saving_frac": round(1.0 - fused["mean"] / two["mean"], 4)}
        eprint(f"[bench] {name}: fused {fused['mean']*1e3:.2f} us, two-launch {two['mean']*1e3:.2f} us")
    del fb
    return out


def run_only(args, dev):
    """Eager launches for profiling runs."""
    if args.only == "copy":
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"[bench] {args.steps} copies of {COPY_BYTES} bytes")
        return
    if args.only in ("probe_mfma", "probe_mfma_w4a8"):
        # the MFMA-only probe at the tile kernel's occupancy, one 4096^3-length launch each
        cl = Ceilings(dev)
        a_fp8 = args.only == "probe_mfma_w4a8"
        iters = 64 if a_fp8 else 128
        for i in range(args.warmup + args.steps):
            if i == args.warmup:
                torch.cuda.synchronize()
            cl.B.mxfp4_probe_mfma(cl.seed, cl.mfma_out, cl.cus, iters, a_fp8=a_fp8)
        torch.cuda.synchronize()
        eprint(f"[bench] {args.steps} eager '{args.only}' launches ({cl.cus} workgroups, {iters} iterations)")
        return
    w = workloads.ALL[args.workload]
    act = "mxfp8x8" if args.mxfp8_only else ("mxfp8" if args.w4a8_only else "mxfp4")
    if args.nvfp4_only and isinstance(w, workloads.DenseWorkload) and args.only in ("gemm", "quantize", "step"):
        bench = NvBench(w, dev)
    elif args.only in ("rmsnorm", "swiglu"):
        bench = ProducerBench(dev)
    elif args.only in ("route", "permute", "scatter", "combine", "layer"):
        if not isinstance(w, workloads.MoEWorkload):
            eprint(f"--only {args.only} needs the MoE workload")
            sys.exit(2)
        bench = MoELayerBench(w, dev)
        if args.only == "layer":
            args.only = "step"
    elif isinstance(w, workloads.MoEWorkload):
        bench = MoEBench(w, dev, act, interleaved=not args.row_major_scales)
    else:
        bench = DenseBench(w, dev, act, quantize_b_in_step=args.only in ("quantize_b", "step_quantize_both"),
                           interleaved=False if args.row_major_scales else None)
    if not hasattr(bench, args.only):
        eprint(f"'{args.only}' is not a mode of {w.name}")
        sys.exit(2)
    fn = getattr(bench, args.only)
    for i in range(args.warmup):
        fn(i)
    torch.cuda.synchronize()
    for i in range(args.steps):
        fn(i)
    torch.cuda.synchronize()
    eprint(f"[bench] {args.steps} eager '{args.only}' launches on {w.name}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.SQUARE4096.name, choices=sorted(workloads.ALL),
                    help="primary dense workload; with --only, any workload (MoE: gemm, quantize, step)")
    ap.add_argument("--secondary", default=workloads.DECODE.name,
                    help="second dense workload reported in the same line ('none' to skip)")
    ap.add_argument("--moe", default=workloads.MOE.name,
                    help="grouped MoE workload reported in the same line ('none' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the MFMA and read-rate probes")
    ap.add_argument("--only", choices=["step", "gemm", "gemm_prepacked", "step_prepacked", "gemm_prepacked_ab",
                                       "gemm_w4a8_prepacked", "gemm_w4a8_both_prepacked",
                                       "step_prepacked_ab", "quantize_prepacked", "quantize", "quantize_b", "copy",
                                       "route", "permute", "scatter", "combine", "layer", "rmsnorm", "swiglu",
                                       "probe_mfma", "probe_mfma_w4a8", "step_quantize_both"],
                    help="eager launches for profiling; route/permute/scatter/combine/layer run the "
                         "on-device MoE layer's steps (layer = all five) on the MoE workload")
    ap.add_argument("--no-moe-layer", action="store_true", help="skip the on-device MoE layer measurement")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the ffn-down 4096x4096x14336 and square 8192^3 prefill GEMMs")
    ap.add_argument("--no-decode-down", action="store_true",
                    help="skip the ffn-down decode shape 128x4096x14336")
    ap.add_argument("--no-nvfp4", action="store_true", help="skip the NVFP4 measurement")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the fused producer (RMSNorm / SwiGLU emitting MXFP4) measurement")
    ap.add_argument("--nvfp4-only", action="store_true",
                    help="with --only gemm/quantize/step: the NVFP4 kernels on the dense workload")
    ap.add_argument("--w4a8-only", action="store_true",
                    help="with --only: MXFP8 activations (W4A8 quantizer / GEMM) instead of MXFP4")
    ap.add_argument("--no-w4a8", action="store_true", help="skip the W4A8 (MXFP8 activation) measurements")
    ap.add_argument("--no-mxfp8", action="store_true", help="skip the MXFP8 x MXFP8 measurement")
    ap.add_argument("--no-row-major", action="store_true",
                    help="skip the row-major-scale comparisons (the same kernels on the other scale layout)")
    ap.add_argument("--row-major-scales", action="store_true",
                    help="with --only: the MXFP4 dense and grouped kernels on row-major scales")
    ap.add_argument("--mxfp8-only", action="store_true",
                    help="with --only gemm/quantize/step: both operands MXFP8 (the MXFP8 x MXFP8 GEMM)")
    args = ap.parse_args()
    # The headline step is timed over exactly --steps calls; every other line
    # (the step's kernels, decode, MoE, widenings, ceilings) over at least 200
    # calls after at least 20 warm-ups, so that microsecond kernels are not
    # timed in replays of a handful of calls whatever --steps is.
    args.detail_steps = max(args.steps, DETAIL_STEPS)
    args.detail_warmup = max(args.warmup, DETAIL_WARMUP)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        eprint("bench.py runs on one GPU only: the library has no multi-GPU path "
               "(how the GEMMs would shard across GPUs is described in the design notes, not implemented).")
        sys.exit(2)
    if not torch.cuda.is_available():
        eprint("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda", 0)
    from block_scaled_fp4_mxfp4_amd import load_library
    load_library()
    if args.only:
        run_only(args, dev)
        return

    if args.workload not in workloads.DENSE:
        eprint(f"the primary workload must be dense ({', '.join(sorted(workloads.DENSE))}); "
               f"use --moe for the grouped one")
        sys.exit(2)
    w = workloads.DENSE[args.workload]
    eprint(f"[bench] building inputs for {w.name}")
    bench = DenseBench(w, dev, quantize_b_in_step=True)
    eprint(f"[bench] {bench.sets_n} rotating input sets of {bench.per_set_bytes / 2**20:.1f} MiB")
    step = bench.timed(bench.step, args.steps, args.warmup)
    gemm = bench.timed(bench.gemm, args.detail_steps, args.detail_warmup)
    quant = bench.timed(bench.quantize, args.detail_steps, args.detail_warmup)
    quant_b = bench.timed(bench.quantize_b, args.detail_steps, args.detail_warmup)
    step_ab = bench.timed(bench.step_quantize_both, args.detail_steps, args.detail_warmup)
    eprint(f"[bench] step {step['mean']*1e3:.2f} us, gemm {gemm['mean']*1e3:.2f} us, "
           f"quantize {quant['mean']*1e3:.2f} us, weight quantize {quant_b['mean']*1e3:.2f} us, "
           f"step quantizing both operands {step_ab['mean']*1e3:.2f} us")
    # the same step and GEMM on row-major scales (the quantizer's default layout)
    if not args.no_row_major:
        rm = DenseBench(w, dev, interleaved=False)
        step_rm = rm.timed(rm.step, args.detail_steps, args.detail_warmup)
        gemm_rm = rm.timed(rm.gemm, args.detail_steps, args.detail_warmup)
        quant_rm = rm.timed(rm.quantize, args.detail_steps, args.detail_warmup)
        del rm
        eprint(f"[bench] row-major scales: step {step_rm['mean']*1e3:.2f} us, gemm {gemm_rm['mean']*1e3:.2f} us, "
               f"quantize {quant_rm['mean']*1e3:.2f} us")

    flops = w.flops
    gemm_tflops = flops / (gemm["mean"] * 1e-3) / 1e12
    step_tflops = flops / (step["mean"] * 1e-3) / 1e12
    qbytes = quant_algorithmic_bytes(w.m, w.k)
    qbbytes = quant_algorithmic_bytes(w.n, w.k)

    result = {
        "metric": "MXFP4 GEMM TFLOP/s at 4096^3; achieved HBM GB/s at decode M=128",
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "detail_steps": args.detail_steps,
        "ms_per_step": round(step["mean"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1, e8m0 block scales, fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded Gaussian BF16; weights pre-quantized once)",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k,
                   "step": "quantize A (bf16->mxfp4) + mxfp4 NT GEMM -> bf16",
                   "scales": "interleaved [k/512, rows, 16] (written by the quantizer; the weight's once)",
                   "rotating_input_sets": bench.sets_n, "parallelism": "single GPU"},
        "roofline": roofline("mfma", gemm_tflops, PEAK_FP4_TFLOPS, "TFLOP/s",
                             traffic_from_profiles(w.name, "gemm_tile_kernel"), kernel="gemm_tile_kernel"),
        "inputs": dense_inputs_record(w),
        "step_us": us(step),
        "kernels": {
            "gemm_us": us(gemm), "gemm_tflops": round(gemm_tflops, 2),
            "quantize_a_us": us(quant),
            "quantize_a_gbs": round(qbytes / (quant["mean"] * 1e-3) / 1e9, 1),
            "quantize_a_hbm_frac": round(qbytes / (quant["mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "quantize_b_us": us(quant_b),
            "quantize_b_gbs": round(qbbytes / (quant_b["mean"] * 1e-3) / 1e9, 1),
        },
        # the step as the workload states it: both operands quantized on the fly
        "step_quantize_both": {"step": "quantize A + quantize B + mxfp4 NT GEMM -> bf16",
                               "step_us": us(step_ab),
                               "step_tflops": round(flops / (step_ab["mean"] * 1e-3) / 1e12, 2)},
    }
    if not args.no_row_major:
        result["row_major_scales"] = {"step": "the same step and GEMM with row-major scales [rows, k/32]",
                                      "step_us": us(step_rm),
                                      "step_tflops": round(flops / (step_rm["mean"] * 1e-3) / 1e12, 2),
                                      "gemm_us": us(gemm_rm),
                                      "gemm_tflops": round(flops / (gemm_rm["mean"] * 1e-3) / 1e12, 2),
                                      "quantize_a_us": us(quant_rm)}

    if not args.no_large:
        result["prefill_large"] = measure_large(args, dev)

    if args.secondary != "none":
        result["secondary"] = measure_decode(args, dev, workloads.DENSE[args.secondary], primary=True)
        if not args.no_decode_down:
            result["decode_down"] = measure_decode(args, dev, workloads.DECODE_DOWN, primary=False)

    if args.moe != "none":
        wm = workloads.ALL[args.moe]
        eprint(f"[bench] building inputs for {wm.name}")
        mb = MoEBench(wm, dev)
        msteps = max(16, args.detail_steps // 2)
        sm = mb.timed(mb.step, msteps, 2)
        gm = mb.timed(mb.gemm, msteps, 2)
        qm = mb.timed(mb.quantize, msteps, 2)
        mbytes = mb.algorithmic_bytes()
        tf = wm.flops / (gm["mean"] * 1e-3) / 1e12
        gbs = mbytes / (gm["mean"] * 1e-3) / 1e9
        counts = mb.counts
        result["moe"] = {
            "workload": wm.name, "tokens": wm.tokens, "experts": wm.experts, "top_k": wm.top_k,
            "n": wm.n, "k": wm.k, "steps": msteps, "rotating_input_sets": mb.sets_n,
            "rows_per_expert": {"min": min(counts), "max": max(counts), "empty": sum(c == 0 for c in counts)},
            "step": "quantize routed A + grouped mxfp4 GEMM (expert weights pre-quantized; interleaved scales)",
            "step_us": us(sm), "step_tflops": round(wm.flops / (sm["mean"] * 1e-3) / 1e12, 2),
            "gemm_us": us(gm), "quantize_a_us": us(qm),
            "gemm_tflops": round(tf, 2), "gemm_mfma_frac": round(tf / PEAK_FP4_TFLOPS, 4),
            "gemm_gbs": round(gbs, 1), "gemm_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": mbytes,
            # the workload sits near the ridge: report both roofs and the fraction of the
            # binding one (roof time = max(flops / MFMA peak, bytes / HBM peak))
            "roofline": roofline("mfma", tf, PEAK_FP4_TFLOPS, "TFLOP/s",
                                 traffic_from_profiles(wm.name, "grouped_persistent_kernel"),
                                 kernel="grouped_persistent_kernel"),
            "roofline_hbm": roofline("hbm", gbs, PEAK_HBM_GBS, "GB/s",
                                     traffic_from_profiles(wm.name, "grouped_persistent_kernel"),
                                     kernel="grouped_persistent_kernel"),
            "min_roof_frac": round(max(wm.flops / (PEAK_FP4_TFLOPS * 1e12), mbytes / (PEAK_HBM_GBS * 1e9))
                                   / (gm["mean"] * 1e-3), 4),
            "inputs": moe_inputs_record(wm),
        }
        eprint(f"[bench] {wm.name}: step {sm['mean']*1e3:.1f} us, grouped gemm {gm['mean']*1e3:.1f} us "
               f"({tf:.0f} TFLOP/s, {gbs:.0f} GB/s)")
        del mb
        if not args.no_row_major:
            mr = MoEBench(wm, dev, interleaved=False)
            gm_rm = mr.timed(mr.gemm, msteps, 2)
            del mr
            result["moe"]["row_major_scales"] = {
                "gemm_us": us(gm_rm), "gemm_tflops": round(wm.flops / (gm_rm["mean"] * 1e-3) / 1e12, 2)}
            eprint(f"[bench] {wm.name}: grouped gemm on row-major scales {gm_rm['mean']*1e3:.1f} us")

    if args.moe != "none" and not args.no_moe_layer:
        result["moe_layer"] = measure_moe_layer(args, dev, us)

    if not args.no_producers:
        result["producers"] = measure_producers(args, dev, us)
        result["fused_decode"] = measure_fused_decode(args, dev)

    if not args.no_w4a8:
        result["w4a8"] = measure_w4a8(args, dev, w, us)

    if not args.no_mxfp8:
        result["mxfp8"] = measure_mxfp8(args, dev, w)

    if not args.no_nvfp4:
        result["nvfp4"] = measure_nvfp4(args, dev, w, us)

    if not args.no_ceilings:
        eprint("[bench] measuring MFMA and streaming-read ceilings with the probe kernels")
        cl = Ceilings(dev)
        ceil = cl.measure(args.detail_steps)
        del cl
        ceil["gemm_frac_of_mfma_ceiling"] = round(gemm_tflops / ceil["mfma_fp4_tflops_short"], 4)
        if "w4a8" in result:
            ceil["w4a8_gemm_frac_of_mfma_ceiling"] = round(
                result["w4a8"]["prefill"]["roofline"]["achieved"] / ceil["mfma_w4a8_tflops_short"], 4)
        if "secondary" in result:
            ceil["decode_gemm_frac_of_read_ceiling"] = round(
                result["secondary"]["roofline"]["achieved"] / ceil["read_gbs_29MB"], 4)
        ceil["note"] = ("measured on this GPU by probe kernels (include/mxfp4_probe.h); "
                        "roofline.peak stays the published figure")
        result["ceilings"] = ceil
        eprint(f"[bench] ceilings: {ceil}")

    if not args.no_cpu_baseline:
        eprint("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(bench, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
