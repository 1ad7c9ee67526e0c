"""Every output element of the full-size workloads against the float64 oracle.

The sampled full-size tests elsewhere check a few rows and columns; these
compare the whole output of the benchmarked paths:
  * decode 128 x 14336 x 4096: A quantized into the prepacked layout, the
    weight prepacked, the both-prepacked decode GEMM (BF16 and fp32 output);
  * the decode down projection 128 x 4096 x 14336 through the same path,
    where the automatic choice splits K over four workgroups per panel;
  * prefill 4096 x 4096 x 4096: GPU quantize of both operands and the
    automatic GEMM (256x256 tiles), BF16 and fp32 output;
  * the 64-expert MoE layer: every element of the smallest non-empty and of
    the largest expert through the grouped GEMM.
The oracle quantizes the same BF16 inputs on the CPU.  Bars as elsewhere:
fp32 output within floored max-rel 1e-5 of the float64 result, BF16 output
the nearest-even rounding of it except at rounding midpoints.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_gemm_nt, mxfp4_gemm_nt_prepacked_ab, mxfp4_grouped_gemm_nt,
                                        mxfp4_prepack_weight, mxfp4_quantize, mxfp4_quantize_prepacked)
from tests.gpu_common import assert_bf16_matches_rounded, device, log, to_np

pytestmark = pytest.mark.gpu


def _bf16_bits(c: torch.Tensor) -> np.ndarray:
    return to_np(c.view(torch.int16)).view(np.uint16)


def _check(got16: np.ndarray, got32: np.ndarray, c64: np.ndarray) -> None:
    assert oracle.floored_max_rel(got32, c64) <= 1e-5
    assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got16), c64) <= 1e-2
    assert_bf16_matches_rounded(got16, c64)


def test_decode_full_output():
    dev = device()
    w = workloads.DECODE
    a, b = w.make()
    log(f"{w.name}: every output element, prepacked A and B")
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    ap_q, ap_s = mxfp4_quantize_prepacked(a.to(dev))
    c16 = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, out_dtype=torch.bfloat16)
    c32 = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oaq, oas = oracle.quantize(workloads.bf16_bits(a))
    obq, obs = oracle.quantize(workloads.bf16_bits(b))
    _check(_bf16_bits(c16), to_np(c32), oracle.gemm_nt(oaq, oas, obq, obs))


def test_decode_down_split_k_full_output():
    """The down projection at decode, 128 x 4096 x 14336: 64 column panels, so
    the automatic choice splits K over four workgroups per panel."""
    dev = device()
    w = workloads.DECODE_DOWN
    a, b = w.make()
    log(f"{w.name}: every output element, prepacked A and B, automatic split-K")
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    ap_q, ap_s = mxfp4_quantize_prepacked(a.to(dev))
    c16 = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, out_dtype=torch.bfloat16)
    c32 = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oaq, oas = oracle.quantize(workloads.bf16_bits(a))
    obq, obs = oracle.quantize(workloads.bf16_bits(b))
    _check(_bf16_bits(c16), to_np(c32), oracle.gemm_nt(oaq, oas, obq, obs))


def test_prefill_4096_full_output():
    dev = device()
    w = workloads.DENSE["prefill_4096x4096x4096"]
    a, b = w.make()
    log(f"{w.name}: every output element, automatic kernel")
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    c16 = mxfp4_gemm_nt(aq, as_, bq, bs)
    c32 = mxfp4_gemm_nt(aq, as_, bq, bs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oaq, oas = oracle.quantize(workloads.bf16_bits(a))
    obq, obs = oracle.quantize(workloads.bf16_bits(b))
    _check(_bf16_bits(c16), to_np(c32), oracle.gemm_nt(oaq, oas, obq, obs))


def test_moe_smallest_and_largest_expert_full_output():
    dev = device()
    w = workloads.MOE
    a, wts, offsets = w.make()
    counts = np.diff(offsets.numpy())
    nonempty = np.flatnonzero(counts)
    picks = [int(nonempty[np.argmin(counts[nonempty])]), int(np.argmax(counts))]
    log(f"moe: experts {picks} with {[int(counts[g]) for g in picks]} rows, every output element")
    aq, as_ = mxfp4_quantize(a.to(dev))
    wq, wsc = mxfp4_quantize(wts.view(-1, w.k).to(dev))
    wq = wq.view(w.experts, w.n, w.k // 2)
    wsc = wsc.view(w.experts, w.n, w.k // 32)
    d_off = offsets.to(dev)
    c16 = mxfp4_grouped_gemm_nt(aq, as_, wq, wsc, d_off)
    c32 = mxfp4_grouped_gemm_nt(aq, as_, wq, wsc, d_off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for g in picks:
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        oaq, oas = oracle.quantize(workloads.bf16_bits(a[lo:hi]))
        obq, obs = oracle.quantize(workloads.bf16_bits(wts[g]))
        c64 = oracle.gemm_nt(oaq, oas, obq, obs)
        _check(_bf16_bits(c16[lo:hi]), to_np(c32[lo:hi]), c64)
