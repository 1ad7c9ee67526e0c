"""W4A8 with both operands prepacked: the MXFP8 quantizer writing the FP8
prepacked layout, byte for byte against that layout's host definition
(tests/prepack_layout.py, from include/mxfp8.h) applied to the oracle's MXFP8
bytes; the GEMM on the FP8 prepacked A and the prepacked weight bit for bit
equal to the W4A8 GEMM on the row-major A and the prepacked weight (fp32 and
BF16), within the MFMA group-rule bound of the oracle, nothing written past C.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_prepack_weight, mxfp4_prepacked_weight_size, mxfp8_gemm_w4a8_nt_prepacked,
                                        mxfp8_gemm_w4a8_nt_prepacked_ab, mxfp8_quantize, mxfp8_quantize_prepacked)
from tests.gpu_common import device, log, poisoned, random_bf16, to_np, upload
from tests.prepack_layout import prepack_fp8_numpy
from tests.test_gpu_w4a8 import PREPACKED_SHAPES, _check_general, _quantized_operands, w4a8_tolerance

pytestmark = pytest.mark.gpu


QUANT_CASES = [(1, 512), (64, 1024), (100, 4096), (130, 2048), (128, 14336)]


@pytest.mark.parametrize("rows,k", QUANT_CASES)
def test_mxfp8_quantize_prepacked_is_the_layout_of_the_oracle_bytes(rows, k):
    dev = device()
    log(f"mxfp8 prepacked quantize rows={rows} k={k}")
    x = random_bf16((rows, k), rows + 7 * k, spread=6, outlier_frac=0.01)
    bits = workloads.bf16_bits(x)
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    qf = poisoned((2 * cb + 256,), torch.uint8, dev, 0x77)
    sf = poisoned((sb + 256,), torch.uint8, dev, 0x77)
    mxfp8_quantize_prepacked(x.to(dev), qf[:2 * cb], sf[:sb])
    torch.cuda.synchronize()
    wq, ws = prepack_fp8_numpy(*oracle.quantize_mxfp8(bits))
    assert np.array_equal(to_np(qf)[:2 * cb], wq), "code bytes"
    assert np.array_equal(to_np(sf)[:sb], ws), "scale bytes"
    assert np.all(to_np(qf)[2 * cb:] == 0x77) and np.all(to_np(sf)[sb:] == 0x77), "write past the end"


@pytest.mark.parametrize("shape", PREPACKED_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in PREPACKED_SHAPES])
def test_w4a8_both_prepacked_matches_prepacked_weight_kernel(shape):
    dev = device()
    m, n, k = shape
    log(f"w4a8 both prepacked {shape}")
    aq, as_, bq, bs = _quantized_operands(m, n, k, 5 * m + n)
    d_aq, d_as, d_bq, d_bs = (upload(t, dev) for t in (aq, as_, bq, bs))
    bp_q, bp_s = mxfp4_prepack_weight(d_bq, d_bs)
    apq, aps = (upload(t, dev) for t in prepack_fp8_numpy(aq, as_))
    for out_dtype, bits in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        c_all = poisoned((m + 1, n), out_dtype, dev, 0x7F)
        mxfp8_gemm_w4a8_nt_prepacked_ab(apq, aps, bp_q, bp_s, m, n, k, c=c_all[:m])
        ref = mxfp8_gemm_w4a8_nt_prepacked(d_aq, d_as, bp_q, bp_s, n, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.all(c_all[m:].view(torch.uint8) == 0x7F), "write past C"
        assert torch.equal(c_all[:m].view(bits), ref.view(bits)), f"{out_dtype} differs from the prepacked-weight kernel"
        if out_dtype == torch.float32:
            _check_general(to_np(c_all[:m]), None, oracle.gemm_w4a8_nt(aq, as_, bq, bs),
                           w4a8_tolerance(aq, as_, bq, bs))


def test_w4a8_decode_step_quantize_prepacked_then_gemm():
    """The decode step on the device: BF16 activation -> FP8 prepacked -> GEMM,
    equal to MXFP8 quantization + the prepacked-weight kernel."""
    dev = device()
    m, n, k = 128, 2048, 4096
    x = random_bf16((m, k), 3, spread=4).to(dev)
    b = random_bf16((n, k), 4, spread=3)
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    bp_q, bp_s = mxfp4_prepack_weight(upload(bq, dev), upload(bs, dev))
    apq, aps = mxfp8_quantize_prepacked(x)
    c = mxfp8_gemm_w4a8_nt_prepacked_ab(apq, aps, bp_q, bp_s, m, n, k, out_dtype=torch.float32)
    aq, as_ = mxfp8_quantize(x)
    ref = mxfp8_gemm_w4a8_nt_prepacked(aq, as_, bp_q, bp_s, n, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))
