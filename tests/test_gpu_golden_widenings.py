"""The GPU paths beyond the MXFP4 GEMM reproduce the stored oracle digests
(tests/golden/oracle_digests.txt, written from the oracle alone by
tests/golden/make_golden.py): MoE routing and permutation on 1024 tokens of the
MoE workload, scatter-quantize of their activations, and NVFP4 quantization of
the tiny workload's A."""
import hashlib

import numpy as np
import pytest
import torch

import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_moe_permute, mxfp4_moe_quantize_scatter, mxfp4_moe_route,
                                        nvfp4_quantize)
from tests.gpu_common import device, log, to_np
from tests.test_golden import load_golden

pytestmark = pytest.mark.gpu


def _digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_moe_steps_match_stored_digests():
    dev = device()
    gold = load_golden()
    moe = workloads.MOE
    log("golden: moe route / permute / scatter on 1024 tokens")
    ids, gate = mxfp4_moe_route(moe.logits()[:1024].to(dev), moe.top_k)
    off, rt, tr = mxfp4_moe_permute(ids, moe.experts)
    x = moe.tokens_bf16()[:1024, :512].contiguous()
    q, s = mxfp4_moe_quantize_scatter(x.to(dev), tr, ids.numel())
    torch.cuda.synchronize()
    assert _digest(to_np(ids)) == gold["moe1024.ids"]
    assert _digest(to_np(off)) == gold["moe1024.offsets"]
    assert _digest(to_np(rt)) == gold["moe1024.row_token"]
    assert _digest(to_np(q)) == gold["moe1024.scatter_q"]
    assert _digest(to_np(s)) == gold["moe1024.scatter_s"]


def test_nvfp4_quantize_matches_stored_digests():
    dev = device()
    gold = load_golden()
    tiny = workloads.TINY
    q, s, gs = nvfp4_quantize(tiny.make()[0].to(dev))
    torch.cuda.synchronize()
    assert _digest(to_np(q)) == gold[f"{tiny.name}.nvfp4_q"]
    assert _digest(to_np(s)) == gold[f"{tiny.name}.nvfp4_s"]
    assert _digest(to_np(gs)) == gold[f"{tiny.name}.nvfp4_gs"]
