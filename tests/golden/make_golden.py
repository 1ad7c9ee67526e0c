"""Writes tests/golden/oracle_digests.txt from the CPU oracle alone.

The pages print no worked numerical example of the format or the GEMM, so the
stored values here are the oracle's own results on the seeded workloads:
SHA-256 digests of its quantized code and scale bytes and of the BF16
(nearest-even) GEMM output, plus a few output values; likewise for the MoE
steps (routing, permutation, scatter-quantize), the fused producers and NVFP4.  They freeze the oracle:
a later change to its arithmetic shows up as a mismatch and has to be justified
against the pages.  Run from the repository root:

    python tests/golden/make_golden.py
"""
from __future__ import annotations

import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.txt")


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def entries():
    tiny = workloads.TINY
    a, b = tiny.make()
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    c = oracle.gemm_nt(aq, as_, bq, bs)
    c16 = oracle.f64_to_bf16_bits(c)
    yield f"{tiny.name}.a_q", digest(aq)
    yield f"{tiny.name}.a_s", digest(as_)
    yield f"{tiny.name}.b_q", digest(bq)
    yield f"{tiny.name}.b_s", digest(bs)
    yield f"{tiny.name}.c_bf16", digest(c16)
    for (i, j) in [(0, 0), (17, 100), (63, 255)]:
        yield f"{tiny.name}.c[{i},{j}]", float(c[i, j]).hex()
    dec = workloads.DECODE
    a, _ = dec.make()
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    yield f"{dec.name}.a_q", digest(aq)
    yield f"{dec.name}.a_s", digest(as_)
    # MoE steps on the first 1024 tokens of the MoE workload's router logits and activations
    moe = workloads.MOE
    lg = moe.logits()[:1024].numpy()
    ids, gate = oracle.route_topk(lg, moe.top_k)
    off, row_token, token_rows = oracle.permute(ids, moe.experts)
    yield "moe1024.ids", digest(ids)
    yield "moe1024.gate_f32", digest(gate.astype(np.float32))
    yield "moe1024.offsets", digest(off)
    yield "moe1024.row_token", digest(row_token)
    x = moe.tokens_bf16()[:1024, :512]
    q, s, _ = oracle.quantize_scatter(workloads.bf16_bits(x), token_rows, ids.size)
    yield "moe1024.scatter_q", digest(q)
    yield "moe1024.scatter_s", digest(s)
    # fused producers and NVFP4 on the tiny workload's A
    gamma = workloads.gaussian_bf16((tiny.k,), 1.0, 13)
    a_bits = workloads.bf16_bits(tiny.make()[0])
    yield f"{tiny.name}.rmsnorm_bf16", digest(oracle.rmsnorm_bf16(a_bits, workloads.bf16_bits(gamma), 1e-5))
    yield f"{tiny.name}.swiglu_bf16", digest(oracle.swiglu_bf16(a_bits[:, :512], a_bits[:, 512:]))
    nq, ns, ng = oracle.quantize_nvfp4(a_bits)
    yield f"{tiny.name}.nvfp4_q", digest(nq)
    yield f"{tiny.name}.nvfp4_s", digest(ns)
    yield f"{tiny.name}.nvfp4_gs", digest(ng)
    nc = oracle.gemm_nvfp4_nt(nq, ns, ng, nq[:32], ns[:32], ng[:32])
    yield f"{tiny.name}.nvfp4_c[5,7]", float(nc[5, 7]).hex()


def main():
    lines = [f"{k} {v}" for k, v in entries()]
    with open(OUT, "w") as f:
        f.write("# written by tests/golden/make_golden.py from the CPU oracle; do not edit by hand\n")
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
