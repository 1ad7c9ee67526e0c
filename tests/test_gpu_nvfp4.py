"""GPU NVFP4 (two-level: UE4M3 per 16 elements, fp32 per row) against the CPU oracle.

* quantization: code bytes, UE4M3 scale bytes and global scales bit-exact (every
  step of the rule is an IEEE fp32 operation on both sides), over spread-out
  blocks, outlier channels, zero rows, tiny (BF16-subnormal) rows and every
  register-slot configuration of the kernel;
* GEMM: fp32 output within floored max-rel 1e-5 of the float64 oracle (the
  products of exactly dequantized values are exact; fp32 accumulation and the
  two global-scale multiplies round), BF16 output equal to the nearest-even
  rounding of the kernel's own fp32 result, over ragged M and N, random code
  and scale bytes, and a sampled 4096^3 problem.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import nvfp4_gemm_nt, nvfp4_quantize
from tests.gpu_common import device, log, poisoned, random_bf16, sampled_indices, to_np, upload

pytestmark = pytest.mark.gpu


QUANT_CASES = [(1, 32), (7, 96), (64, 4096), (33, 4160), (5, 8192), (3, 32768)]


@pytest.mark.parametrize("rows,k", QUANT_CASES)
def test_nvfp4_quantize_bitexact(rows, k):
    dev = device()
    log(f"nvfp4 quantize rows={rows} k={k}")
    x = random_bf16((rows, k), 11 + k, spread=10, outlier_frac=0.01)
    if rows > 2:
        x[1] = 0                                               # zero row: gs = 1, all scales 0
        x[2] = x[2] * 2.0 ** -120                              # tiny row: subnormal BF16 and fp32 values
    q = poisoned((rows, k // 2), torch.uint8, dev, 0xA5)
    s = poisoned((rows, k // 16), torch.uint8, dev, 0xA5)
    gs = poisoned((rows,), torch.float32, dev, 0xA5)
    nvfp4_quantize(x.to(dev), q, s, gs)
    torch.cuda.synchronize()
    rq, rs, rg = oracle.quantize_nvfp4(workloads.bf16_bits(x))
    assert np.array_equal(to_np(gs).view(np.uint32), rg.view(np.uint32)), "global scales"
    assert np.array_equal(to_np(s), rs), "scale bytes"
    assert np.array_equal(to_np(q), rq), "code bytes"


def test_nvfp4_quantize_prefill_activation_full_size():
    dev = device()
    w = workloads.SQUARE4096
    a = workloads.activation_bf16(w.m, w.k, w.seed, outliers=True)
    q, s, gs = nvfp4_quantize(a.to(dev))
    torch.cuda.synchronize()
    idx = sampled_indices(w.m, 64, 3)
    rq, rs, rg = oracle.quantize_nvfp4(workloads.bf16_bits(a[idx]))
    assert np.array_equal(to_np(q)[idx], rq) and np.array_equal(to_np(s)[idx], rs)
    assert np.array_equal(to_np(gs)[idx].view(np.uint32), rg.view(np.uint32))


def _random_nvfp4(rows, k, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    s = rng.integers(0x20, 0x60, size=(rows, k // 16), dtype=np.uint8)   # UE4M3 2^-3 .. 2^4-ish
    gs = (rng.random(rows) * 4 + 0.25).astype(np.float32)
    return q, s, gs


GEMM_CASES = [(1, 1, 64), (64, 256, 1024), (130, 200, 192), (257, 129, 512), (512, 512, 4096), (3, 1000, 128)]


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_nvfp4_gemm_random_operands(m, n, k):
    dev = device()
    log(f"nvfp4 gemm random m={m} n={n} k={k}")
    aq, as_, ag = _random_nvfp4(m, k, m + k)
    bq, bs, bg = _random_nvfp4(n, k, n + 7 * k)
    ops = [upload(t, dev) for t in (aq, as_, ag, bq, bs, bg)]
    c_all = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    c32 = c_all[:m]
    nvfp4_gemm_nt(*ops, c=c32)
    c16 = nvfp4_gemm_nt(*ops, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(c_all[m:].view(torch.uint8) == 0xFF), "write past C"
    ref = oracle.gemm_nvfp4_nt(aq, as_, ag, bq, bs, bg)
    got = to_np(c32).astype(np.float64)
    assert oracle.floored_max_rel(got, ref) <= 1e-5
    assert np.array_equal(to_np(c16.view(torch.int16)).view(np.uint16), oracle.f64_to_bf16_bits(got))


def test_nvfp4_quantize_then_gemm_vs_oracle():
    dev = device()
    m, n, k = 192, 320, 2048
    a = random_bf16((m, k), 21, spread=4, outlier_frac=0.01)
    b = random_bf16((n, k), 22, spread=2)
    ga = nvfp4_quantize(a.to(dev))
    gb = nvfp4_quantize(b.to(dev))
    c = nvfp4_gemm_nt(*ga, *gb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ra = oracle.quantize_nvfp4(workloads.bf16_bits(a))
    rb = oracle.quantize_nvfp4(workloads.bf16_bits(b))
    ref = oracle.gemm_nvfp4_nt(*ra, *rb)
    assert oracle.floored_max_rel(to_np(c).astype(np.float64), ref) <= 1e-5


def test_nvfp4_gemm_prefill_full_size_sampled():
    dev = device()
    w = workloads.SQUARE4096
    log(f"nvfp4 gemm {w.name}")
    a, b = w.make()
    ga = nvfp4_quantize(a.to(dev))
    gb = nvfp4_quantize(b.to(dev))
    c = nvfp4_gemm_nt(*ga, *gb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sampled_indices(w.m, 16, 4)
    cols = sampled_indices(w.n, 64, 5)
    ra = oracle.quantize_nvfp4(workloads.bf16_bits(a[rows]))
    rb = oracle.quantize_nvfp4(workloads.bf16_bits(b[cols]))
    ref = oracle.gemm_nvfp4_nt(*ra, *rb)
    got = to_np(c)[np.ix_(rows, cols)].astype(np.float64)
    assert oracle.floored_max_rel(got, ref) <= 1e-5


def test_nvfp4_gemm_large_tiles_ragged_sampled():
    """4100 x 4000 needs 17 x 16 >= 256 tiles of 256 x 256: the large-tile configuration, ragged on both edges."""
    dev = device()
    m, n, k = 4100, 4000, 128
    log(f"nvfp4 gemm large tiles m={m} n={n} k={k}")
    aq, as_, ag = _random_nvfp4(m, k, 31)
    bq, bs, bg = _random_nvfp4(n, k, 32)
    c_all = poisoned((m + 1, n), torch.float32, dev, 0xFF)
    nvfp4_gemm_nt(*[upload(t, dev) for t in (aq, as_, ag, bq, bs, bg)], c=c_all[:m])
    torch.cuda.synchronize()
    assert torch.all(c_all[m:].view(torch.uint8) == 0xFF), "write past C"
    rows = np.unique(np.concatenate([sampled_indices(m, 24, 6), np.arange(m - 8, m)]))
    cols = np.unique(np.concatenate([sampled_indices(n, 48, 7), np.arange(n - 8, n)]))
    ref = oracle.gemm_nvfp4_nt(aq[rows], as_[rows], ag[rows], bq[cols], bs[cols], bg[cols])
    got = to_np(c_all[:m])[np.ix_(rows, cols)].astype(np.float64)
    assert oracle.floored_max_rel(got, ref) <= 1e-5
