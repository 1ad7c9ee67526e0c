"""Seeded random shapes through every MXFP4 GEMM entry point and its automatic
kernel choice, against the float64 oracle.

The other GEMM tests pick shapes at each kernel's boundaries by hand; this one
draws them (ragged M, N and K, K a multiple of 32, 512 or 1024 as the entry
point needs), so the automatic dispatch between the tile, streaming, split-K
and persistent kernels meets shapes nobody chose.  Bars as elsewhere: fp32
output within floored max-rel 1e-5 of the float64 oracle, BF16 output the
nearest-even rounding of the same kernel's fp32 result and within floored
max-rel 1e-2 of the oracle, nothing written past C.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp4_mxfp4_amd import (mxfp4_gemm_nt, mxfp4_gemm_nt_prepacked, mxfp4_gemm_nt_prepacked_ab,
                                        mxfp4_grouped_gemm_nt, mxfp4_prepack_weight)
from tests.gpu_common import device, log, poisoned, random_codes, to_np, upload

pytestmark = pytest.mark.gpu


def _shapes(seed, count, k_unit, k_max):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(np.exp(rng.uniform(0, np.log(700))))
        n = int(rng.integers(1, 700))
        k = int(rng.integers(1, k_max // k_unit + 1)) * k_unit
        out.append((m, n, k))
    return out


def _check(c32_all, c16_all, m, c64):
    assert np.all(to_np(c32_all[m:].view(torch.uint8)) == 0xFF), "write past the end of C (fp32)"
    assert np.all(to_np(c16_all[m:].view(torch.uint8)) == 0xFF), "write past the end of C (bf16)"
    got32 = to_np(c32_all[:m])
    got16 = to_np(c16_all[:m].view(torch.int16)).view(np.uint16)
    assert oracle.floored_max_rel(got32, c64) <= 1e-5
    # the BF16 output is the nearest-even rounding of the same call's fp32 result,
    # bit for bit (random codes with scales 2^-7..2^7 cancel heavily, so the fp32
    # error can reach a BF16 midpoint of the exact result)
    assert np.array_equal(got16, oracle.round_output_bf16(got32.astype(np.float64)))
    assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got16), c64) <= 1e-2


def _operands(m, n, k, seed):
    aq, as_ = random_codes(m, k, seed)
    bq, bs = random_codes(n, k, seed + 1)
    return aq, as_, bq, bs


@pytest.mark.parametrize("m,n,k", _shapes(11, 24, 32, 2048))
def test_random_shape_auto_kernel(m, n, k):
    dev = device()
    log(f"random shape auto m={m} n={n} k={k}")
    aq, as_, bq, bs = _operands(m, n, k, m * 7 + n * 3 + k)
    ops = [upload(x, dev) for x in (aq, as_, bq, bs)]
    c32 = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    c16 = poisoned((m + 1, n), torch.bfloat16, dev, 0xFF)
    mxfp4_gemm_nt(*ops, c=c32[:m])
    mxfp4_gemm_nt(*ops, c=c16[:m])
    torch.cuda.synchronize()
    _check(c32, c16, m, oracle.gemm_nt(aq, as_, bq, bs))


@pytest.mark.parametrize("m,n,k", _shapes(12, 12, 1024, 4096))
def test_random_shape_persistent_and_streaming(m, n, k):
    """k % 1024 == 0: the persistent loop and the streaming kernel forced, each
    against the oracle."""
    dev = device()
    log(f"random shape persistent/stream m={m} n={n} k={k}")
    aq, as_, bq, bs = _operands(m, n, k, m * 5 + n + k)
    ops = [upload(x, dev) for x in (aq, as_, bq, bs)]
    c64 = oracle.gemm_nt(aq, as_, bq, bs)
    for kernel in ("persistent", "stream"):
        c32 = poisoned((m + 1, n), torch.float32, dev, 0xFF)
        c16 = poisoned((m + 1, n), torch.bfloat16, dev, 0xFF)
        mxfp4_gemm_nt(*ops, c=c32[:m], kernel=kernel)
        mxfp4_gemm_nt(*ops, c=c16[:m], kernel=kernel)
        torch.cuda.synchronize()
        _check(c32, c16, m, c64)


@pytest.mark.parametrize("m,n,k", _shapes(13, 12, 512, 8192))
def test_random_shape_prepacked(m, n, k):
    """The prepacked weight (streaming kernel) and both operands prepacked with
    the automatic K split, against the oracle."""
    dev = device()
    log(f"random shape prepacked m={m} n={n} k={k}")
    aq, as_, bq, bs = _operands(m, n, k, m * 3 + n * 5 + k)
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    bp_q, bp_s = mxfp4_prepack_weight(upload(bq, dev), upload(bs, dev))
    ap_q, ap_s = mxfp4_prepack_weight(d_aq, d_as)
    c64 = oracle.gemm_nt(aq, as_, bq, bs)
    c32 = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    c16 = poisoned((m + 1, n), torch.bfloat16, dev, 0xFF)
    mxfp4_gemm_nt_prepacked(d_aq, d_as, bp_q, bp_s, n, c=c32[:m])
    mxfp4_gemm_nt_prepacked(d_aq, d_as, bp_q, bp_s, n, c=c16[:m])
    torch.cuda.synchronize()
    _check(c32, c16, m, c64)
    c32 = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    c16 = poisoned((m + 1, n), torch.bfloat16, dev, 0xFF)
    mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, c=c32[:m])
    mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, c=c16[:m])
    torch.cuda.synchronize()
    _check(c32, c16, m, c64)


def _group_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        groups = int(rng.integers(1, 40))
        counts = rng.integers(0, 600, size=groups) * (rng.random(groups) < 0.85)
        n = int(rng.integers(1, 600))
        k = int(rng.choice([256, 512, 1024, 2048]))
        out.append((tuple(int(x) for x in counts), n, k))
    return out


@pytest.mark.parametrize("counts,n,k", _group_cases(14, 10))
def test_random_grouped(counts, n, k):
    """Random expert sizes (some empty): every group's rows against the oracle
    (k % 1024 == 0 with groups averaging 192 rows or more takes the persistent
    loop, other cases the one-tile-per-workgroup kernel)."""
    dev = device()
    total = int(sum(counts))
    log(f"random grouped: {len(counts)} groups, {total} rows, n={n} k={k}")
    if total == 0:
        pytest.skip("no rows drawn")
    aq, as_ = random_codes(total, k, total + n)
    wq, ws = random_codes(len(counts) * n, k, total + 2 * n)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    d_wq = upload(wq, dev).view(len(counts), n, k // 2)
    d_ws = upload(ws, dev).view(len(counts), n, k // 32)
    c32 = poisoned((total + 1, n), torch.float32, dev, 0xFF)
    mxfp4_grouped_gemm_nt(upload(aq, dev), upload(as_, dev), d_wq, d_ws, upload(offsets, dev), c=c32[:total])
    torch.cuda.synchronize()
    assert np.all(to_np(c32[total:].view(torch.uint8)) == 0xFF), "write past the end of C"
    got = to_np(c32[:total])
    for g in range(len(counts)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        ref = oracle.gemm_nt(aq[lo:hi], as_[lo:hi], wq[g * n:(g + 1) * n], ws[g * n:(g + 1) * n])
        assert oracle.floored_max_rel(got[lo:hi], ref) <= 1e-5, f"group {g}"
