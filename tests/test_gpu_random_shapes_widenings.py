"""Seeded random shapes through the widening GEMMs (W4A8 dense and grouped,
MXFP8 x MXFP8, NVFP4) and their automatic kernel choices, against the CPU
oracle, with each suite's own bars: the W4A8 and MXFP8 results within the
bound derived from the FP8 MFMA rounding rule (checked on up to 16 rows per
case, the bound's cost growing with rows x n x k / 8), the NVFP4 result within
floored max-rel 1e-5 of the float64 oracle; BF16 outputs the nearest-even
rounding of the same kernel's fp32 result; nothing written past C.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import mxfp8_gemm_nt, mxfp8_gemm_w4a8_nt, mxfp8_grouped_gemm_w4a8_nt, nvfp4_gemm_nt
from tests.gpu_common import device, log, poisoned, random_bf16, to_np, upload
from tests.test_gpu_mxfp8_gemm import mxfp8_tolerance
from tests.test_gpu_nvfp4 import _random_nvfp4
from tests.test_gpu_w4a8 import w4a8_tolerance

pytestmark = pytest.mark.gpu


def _shapes(seed, count, k_unit, k_max, mn_max=600):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m = int(np.exp(rng.uniform(0, np.log(mn_max))))
        n = int(rng.integers(1, mn_max))
        k = int(rng.integers(1, k_max // k_unit + 1)) * k_unit
        out.append((m, n, k))
    return out


def _run(fn, ops, m, n, dev):
    c32 = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    c16 = poisoned((m + 1, n), torch.bfloat16, dev, 0xFF)
    fn(*ops, c=c32[:m])
    fn(*ops, c=c16[:m])
    torch.cuda.synchronize()
    assert np.all(to_np(c32[m:].view(torch.uint8)) == 0xFF), "write past the end of C (fp32)"
    assert np.all(to_np(c16[m:].view(torch.uint8)) == 0xFF), "write past the end of C (bf16)"
    got32 = to_np(c32[:m]).astype(np.float64)
    got16 = to_np(c16[:m].view(torch.int16)).view(np.uint16)
    assert np.array_equal(got16, oracle.f64_to_bf16_bits(got32))
    return got32


def _rows(m, seed):
    return np.unique(np.random.default_rng(seed).choice(m, size=min(16, m), replace=False))


def _bound_check(got32, c64, tol):
    assert not (np.abs(got32 - c64) > tol).any(), "outputs outside the MFMA group-rule bound"
    assert oracle.floored_max_rel(got32, c64) <= 1e-2


@pytest.mark.parametrize("m,n,k", _shapes(21, 14, 32, 2048))
def test_random_shape_w4a8(m, n, k):
    dev = device()
    log(f"random w4a8 m={m} n={n} k={k}")
    a = random_bf16((m, k), m + k, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), n + 2 * k, spread=3)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    got32 = _run(mxfp8_gemm_w4a8_nt, [upload(x, dev) for x in (aq, as_, bq, bs)], m, n, dev)
    r = _rows(m, m + n + k)
    _bound_check(got32[r], oracle.gemm_w4a8_nt(aq[r], as_[r], bq, bs), w4a8_tolerance(aq[r], as_[r], bq, bs))


@pytest.mark.parametrize("m,n,k", _shapes(22, 14, 32, 2048))
def test_random_shape_mxfp8(m, n, k):
    dev = device()
    log(f"random mxfp8 m={m} n={n} k={k}")
    a = random_bf16((m, k), 3 * m + k, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), 3 * n + k, spread=3)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    bq, bs = oracle.quantize_mxfp8(workloads.bf16_bits(b))
    got32 = _run(mxfp8_gemm_nt, [upload(x, dev) for x in (aq, as_, bq, bs)], m, n, dev)
    r = _rows(m, 2 * m + n + k)
    _bound_check(got32[r], oracle.gemm_mxfp8_nt(aq[r], as_[r], bq, bs), mxfp8_tolerance(aq[r], as_[r], bq, bs))


@pytest.mark.parametrize("m,n,k", _shapes(23, 14, 64, 2048))
def test_random_shape_nvfp4(m, n, k):
    dev = device()
    log(f"random nvfp4 m={m} n={n} k={k}")
    aq, as_, ag = _random_nvfp4(m, k, 5 * m + k)
    bq, bs, bg = _random_nvfp4(n, k, 5 * n + 3 * k)
    got32 = _run(nvfp4_gemm_nt, [upload(t, dev) for t in (aq, as_, ag, bq, bs, bg)], m, n, dev)
    assert oracle.floored_max_rel(got32, oracle.gemm_nvfp4_nt(aq, as_, ag, bq, bs, bg)) <= 1e-5


def _group_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        groups = int(rng.integers(1, 24))
        counts = rng.integers(0, 500, size=groups) * (rng.random(groups) < 0.85)
        n = int(rng.integers(1, 500))
        k = int(rng.choice([256, 512, 1024, 2048]))
        out.append((tuple(int(x) for x in counts), n, k))
    return out


@pytest.mark.parametrize("counts,n,k", _group_cases(24, 8))
def test_random_grouped_w4a8(counts, n, k):
    """Random expert sizes (some empty; k % 1024 == 0 takes the persistent tile
    loop): each group against the oracle bound on up to 16 sampled rows."""
    dev = device()
    total = int(sum(counts))
    log(f"random grouped w4a8: {len(counts)} groups, {total} rows, n={n} k={k}")
    if total == 0:
        pytest.skip("no rows drawn")
    a = random_bf16((total, k), total + k, spread=3)
    w = random_bf16((len(counts) * n, k), n + k, spread=3)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    wq, ws = oracle.quantize(workloads.bf16_bits(w))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    d_wq = upload(wq, dev).view(len(counts), n, k // 2)
    d_ws = upload(ws, dev).view(len(counts), n, k // 32)
    c32 = poisoned((total + 1, n), torch.float32, dev, 0xFF)
    mxfp8_grouped_gemm_w4a8_nt(upload(aq, dev), upload(as_, dev), d_wq, d_ws, upload(offsets, dev), c=c32[:total])
    torch.cuda.synchronize()
    assert np.all(to_np(c32[total:].view(torch.uint8)) == 0xFF), "write past the end of C"
    got = to_np(c32[:total]).astype(np.float64)
    for g in range(len(counts)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        r = lo + _rows(hi - lo, g + total)
        wg, sg = wq[g * n:(g + 1) * n], ws[g * n:(g + 1) * n]
        _bound_check(got[r], oracle.gemm_w4a8_nt(aq[r], as_[r], wg, sg), w4a8_tolerance(aq[r], as_[r], wg, sg))
