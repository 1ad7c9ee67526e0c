"""GPU fused producers (residual add + RMSNorm, SwiGLU) emitting MXFP4, against the CPU oracle.

* residual add: the updated residual stream bit-exact;
* RMSNorm: the kernel's BF16 output equals the nearest BF16 of the oracle's
  float64 value, except where that value lies within 2^-40 (relative) of a
  rounding midpoint (fp64 arithmetic in the kernel differs from the oracle's
  correctly rounded sum of squares by a few fp64 ulps at most);
* SwiGLU: the kernel's BF16 output is within one BF16 step of the oracle's
  float64 value and equals its nearest BF16 except within (|g| + 8) * 2^-24
  (relative) of a rounding midpoint (fp32 arithmetic with the hardware exp2 and
  reciprocal: g*u exact, -g*log2(e) rounding by |g| * 2^-24 in the exponent,
  about an ulp each for exp2 and rcp, half an ulp each for the add and the
  final product);
* MXFP4: codes and scale bytes bit-exact against the oracle's quantization of
  the kernel's own BF16 output (and so of the oracle's wherever the two agree);
  a call without the BF16 output writes the same bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_gemm_nt_prepacked_ab, mxfp4_prepack_weight, mxfp4_prepacked_weight_size,
                                        mxfp4_quantize, mxfp4_quantize_prepacked, mxfp4_rmsnorm_quantize,
                                        mxfp4_swiglu_quantize)
from tests.gpu_common import device, log, poisoned, random_bf16, sampled_indices, to_np

pytestmark = pytest.mark.gpu


def _bits(t):
    return workloads.bf16_bits(t.cpu())


def _assert_nearest_or_midpoint(got_bits, y64, rel_window):
    want = oracle.f64_to_bf16_bits(y64)
    bad = got_bits != want
    if not bad.any():
        return
    lo = oracle.bf16_bits_to_f64(want[bad])
    hi = oracle.bf16_bits_to_f64(got_bits[bad])
    mid = (lo + hi) / 2
    window = rel_window[bad] if np.ndim(rel_window) else rel_window
    near = np.abs(y64[bad] - mid) <= window * np.abs(y64[bad])
    one_step = np.abs(got_bits[bad].astype(np.int32) - want[bad].astype(np.int32)) == 1
    assert np.all(near & one_step), f"{int((~(near & one_step)).sum())} outputs are not the nearest BF16"


RMS_CASES = [
    (1, 32, True, 1e-5), (5, 96, False, 1e-6), (64, 4096, True, 1e-5), (130, 8192, True, 0.0),
    (33, 4160, False, 1e-5), (9, 32768, True, 1e-5), (3, 2048, True, 1.0),
]


@pytest.mark.parametrize("rows,k,with_res,eps", RMS_CASES)
def test_rmsnorm_quantize_matches_oracle(rows, k, with_res, eps):
    dev = device()
    log(f"rmsnorm rows={rows} k={k} residual={with_res} eps={eps}")
    x = random_bf16((rows, k), 100 + k, spread=6, outlier_frac=0.01)
    res = random_bf16((rows, k), 200 + k, spread=6)
    g = torch.Generator().manual_seed(k)
    gamma = (1.0 + 0.2 * torch.randn(k, generator=g)).to(torch.bfloat16)
    xd, gd = x.to(dev), gamma.to(dev)
    resd = res.to(dev) if with_res else None
    h_out = poisoned((rows, k), torch.bfloat16, dev, 0x7F) if with_res else None
    y = poisoned((rows, k), torch.bfloat16, dev, 0x7F)
    q, s = mxfp4_rmsnorm_quantize(xd, gd, eps, residual=resd, residual_out=h_out, y=y)
    q2, s2 = mxfp4_rmsnorm_quantize(xd, gd, eps, residual=resd)          # no BF16 outputs
    torch.cuda.synchronize()
    hb = oracle.add_residual(_bits(x), _bits(res)) if with_res else _bits(x)
    if with_res:
        assert np.array_equal(_bits(h_out), hb)
    y64 = oracle.rmsnorm_f64(hb, _bits(gamma), eps)
    yb = _bits(y)
    _assert_nearest_or_midpoint(yb, y64, 2.0 ** -40)
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q), rq) and np.array_equal(to_np(s), rs)
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_rmsnorm_exact_midpoints_round_to_even():
    """Rows whose RMSNorm output is exact in float64 and lands on BF16 rounding
    midpoints (and on quarter points and zeros): each row repeats
    [1.5, 1.5, 1.5, 0.5, 0.5, 0.5, 0.5, 0.5] times 2^r, so mean(h^2) = 4^r and
    with eps = 0 the scale is exactly 2^-r; gamma runs over 1 + j/128 (with
    signs and zeros), so y = h * gamma has up to 10 significant bits.  The BF16
    output must be the nearest-even rounding exactly, ties included."""
    dev = device()
    rows, k = 6, 1024
    base = np.array([1.5, 1.5, 1.5, 0.5, 0.5, 0.5, 0.5, 0.5])
    h = np.stack([np.tile(base, k // 8) * 2.0 ** (r - 2) * (-1) ** r for r in range(rows)])
    j = np.arange(k) % 128
    gamma = (1.0 + j / 128.0) * np.where(np.arange(k) % 3 == 0, -1.0, 1.0) * 2.0 ** ((np.arange(k) // 128) % 4 - 1)
    gamma[::97] = 0.0
    hb = oracle.f64_to_bf16_bits(h)
    gb = oracle.f64_to_bf16_bits(gamma)
    assert np.array_equal(oracle.bf16_bits_to_f64(hb), h) and np.array_equal(oracle.bf16_bits_to_f64(gb), gamma)
    want = oracle.rmsnorm_bf16(hb, gb, 0.0)
    ties = oracle.rmsnorm_f64(hb, gb, 0.0)
    lo = oracle.bf16_bits_to_f64(want)
    log(f"rmsnorm exact midpoints: {int(np.sum(np.abs(ties) != np.abs(lo)))} of {ties.size} outputs rounded")
    x = torch.from_numpy(hb.astype(np.int16)).view(torch.bfloat16).to(dev)
    g = torch.from_numpy(gb.astype(np.int16)).view(torch.bfloat16).to(dev)
    y = poisoned((rows, k), torch.bfloat16, dev, 0x7F)
    q, s = mxfp4_rmsnorm_quantize(x, g, 0.0, y=y)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), want)
    rq, rs = oracle.quantize(want)
    assert np.array_equal(to_np(q), rq) and np.array_equal(to_np(s), rs)


def test_rmsnorm_in_place_residual_and_zero_rows():
    dev = device()
    rows, k, eps = 16, 1024, 1e-5
    x = random_bf16((rows, k), 5, spread=3)
    x[3] = 0                                    # a zero row with eps > 0 normalizes to zeros
    res = random_bf16((rows, k), 6, spread=3)
    res[3] = 0
    gamma = torch.ones(k, dtype=torch.bfloat16)
    resd = res.to(dev)
    q, s = mxfp4_rmsnorm_quantize(x.to(dev), gamma.to(dev), eps, residual=resd, residual_out=resd)
    torch.cuda.synchronize()
    hb = oracle.add_residual(_bits(x), _bits(res))
    assert np.array_equal(_bits(resd), hb)
    rq, rs = oracle.quantize(oracle.rmsnorm_bf16(hb, _bits(gamma), eps))
    assert np.array_equal(to_np(q), rq) and np.array_equal(to_np(s), rs)
    assert np.all(to_np(q)[3] == 0) and np.all(to_np(s)[3] == 0)


def test_rmsnorm_prefill_activation_full_size_sampled():
    dev = device()
    rows, k, eps = 4096, 4096, 1e-5
    log(f"rmsnorm full size {rows}x{k}")
    x = workloads.activation_bf16(rows, k, 300, outliers=True)
    res = workloads.activation_bf16(rows, k, 301, outliers=False)
    gamma = workloads.gaussian_bf16((k,), 0.1, 302)
    y = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    h_out = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    q, s = mxfp4_rmsnorm_quantize(x.to(dev), gamma.to(dev), eps, residual=res.to(dev), residual_out=h_out, y=y)
    torch.cuda.synchronize()
    idx = sampled_indices(rows, 48, 9)
    hb = oracle.add_residual(_bits(x[idx]), _bits(res[idx]))
    assert np.array_equal(_bits(h_out)[idx], hb)
    yb = _bits(y)[idx]
    _assert_nearest_or_midpoint(yb, oracle.rmsnorm_f64(hb, _bits(gamma), eps), 2.0 ** -40)
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q)[idx], rq) and np.array_equal(to_np(s)[idx], rs)


SWIGLU_CASES = [(1, 32, 32), (17, 96, 192), (64, 2816, 5632), (40, 14336, 14336), (7, 160, 168)]


def _silu_window(gate_bf16):
    """Relative distance from a BF16 midpoint within which the fp32 kernel may round either way."""
    return (np.abs(oracle.bf16_bits_to_f64(_bits(gate_bf16))) + 8.0) * 2.0 ** -24


def _gate_up(rows, k, ld, seed, dev):
    g = torch.Generator().manual_seed(seed)
    base = (torch.randn(rows, ld + k, generator=g) * 3).to(torch.bfloat16)
    base[:, :8] = torch.tensor([-1000.0, -100.0, -20.0, -0.0, 0.0, 20.0, 100.0, 1000.0]).to(torch.bfloat16)
    buf = base.to(dev)
    # gate = columns [0, k) and up = columns [ld, ld + k) of the same rows: one row stride, ld + k
    return buf[:, :k], buf[:, ld:ld + k], base[:, :k].contiguous(), base[:, ld:ld + k].contiguous()


@pytest.mark.parametrize("rows,k,ld", SWIGLU_CASES)
def test_swiglu_quantize_matches_oracle(rows, k, ld):
    dev = device()
    log(f"swiglu rows={rows} k={k} ld={ld}")
    gate, up, gate_c, up_c = _gate_up(rows, k, ld, rows + k, dev)
    y = poisoned((rows, k), torch.bfloat16, dev, 0x7F)
    q, s = mxfp4_swiglu_quantize(gate, up, y=y)
    q2, s2 = mxfp4_swiglu_quantize(gate, up)
    torch.cuda.synchronize()
    y64 = oracle.swiglu_f64(_bits(gate_c), _bits(up_c))
    yb = _bits(y)
    _assert_nearest_or_midpoint(yb, y64, _silu_window(gate_c))
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q), rq) and np.array_equal(to_np(s), rs)
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_swiglu_ffn_full_size_sampled():
    dev = device()
    rows, k = 4096, 14336
    log(f"swiglu full size {rows}x{k} (gate|up halves of one [rows, 2k] buffer)")
    gu = workloads.gaussian_bf16((rows, 2 * k), 1.0, 401)
    gud = gu.to(dev)
    y = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    q, s = mxfp4_swiglu_quantize(gud[:, :k], gud[:, k:], y=y)
    torch.cuda.synchronize()
    idx = sampled_indices(rows, 24, 10)
    y64 = oracle.swiglu_f64(_bits(gu[idx, :k]), _bits(gu[idx, k:]))
    yb = _bits(y)[idx]
    _assert_nearest_or_midpoint(yb, y64, _silu_window(gu[idx, :k]))
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q)[idx], rq) and np.array_equal(to_np(s)[idx], rs)


# ---------------------------------------------------------------------------
# producers writing the prepacked operand layout of the decode GEMM

PREPACKED_CASES = [(1, 512), (64, 1024), (100, 4096), (128, 4096), (130, 2048)]


@pytest.mark.parametrize("rows,k", PREPACKED_CASES)
def test_rmsnorm_quantize_prepacked_is_the_layout_of_the_row_major_bytes(rows, k):
    """The prepacked producer's buffers equal the prepacked layout (built on the
    host from its definition) of the row-major producer's codes and scales, bit
    for bit, padding rows as zero blocks; the BF16 outputs are the same."""
    from tests.prepack_layout import prepack_numpy
    dev = device()
    log(f"rmsnorm prepacked rows={rows} k={k}")
    x = random_bf16((rows, k), 40 + k, spread=5, outlier_frac=0.01)
    res = random_bf16((rows, k), 41 + k, spread=5)
    gamma = (1.0 + 0.2 * torch.randn(k, generator=torch.Generator().manual_seed(k))).to(torch.bfloat16)
    xd, rd, gd = x.to(dev), res.to(dev), gamma.to(dev)
    h1, y1 = (torch.empty((rows, k), dtype=torch.bfloat16, device=dev) for _ in range(2))
    h2, y2 = (torch.empty((rows, k), dtype=torch.bfloat16, device=dev) for _ in range(2))
    q, s = mxfp4_rmsnorm_quantize(xd, gd, 1e-5, residual=rd, residual_out=h1, y=y1)
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    pq, ps = poisoned((cb,), torch.uint8, dev, 0x77), poisoned((sb,), torch.uint8, dev, 0x77)
    mxfp4_rmsnorm_quantize(xd, gd, 1e-5, residual=rd, residual_out=h2, y=y2, q=pq, scales=ps, prepacked=True)
    torch.cuda.synchronize()
    wq, ws = prepack_numpy(to_np(q), to_np(s))
    assert np.array_equal(to_np(pq), wq) and np.array_equal(to_np(ps), ws)
    assert torch.equal(h1, h2) and torch.equal(y1, y2)


@pytest.mark.parametrize("rows,k", PREPACKED_CASES)
def test_swiglu_quantize_prepacked_is_the_layout_of_the_row_major_bytes(rows, k):
    from tests.prepack_layout import prepack_numpy
    dev = device()
    log(f"swiglu prepacked rows={rows} k={k}")
    gate, up, _, _ = _gate_up(rows, k, 2 * k, rows * 3 + k, dev)
    y1 = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    q, s = mxfp4_swiglu_quantize(gate, up, y=y1)
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    pq, ps = poisoned((cb,), torch.uint8, dev, 0x77), poisoned((sb,), torch.uint8, dev, 0x77)
    mxfp4_swiglu_quantize(gate, up, y=y2, q=pq, scales=ps, prepacked=True)
    torch.cuda.synchronize()
    wq, ws = prepack_numpy(to_np(q), to_np(s))
    assert np.array_equal(to_np(pq), wq) and np.array_equal(to_np(ps), ws)
    assert torch.equal(y1, y2)


def test_fused_decode_step_matches_two_launch_step_and_oracle():
    """Decode from the producer: RMSNorm writing the prepacked layout, then the
    GEMM on prepacked operands, equals the two-launch step (producer BF16 output,
    prepacked quantizer, the same GEMM) bit for bit, and the oracle within the
    fp32 bar on sampled columns."""
    dev = device()
    w = workloads.DECODE
    m, n, k = w.m, w.n, w.k
    log(f"fused decode step {w.name}")
    x = workloads.activation_bf16(m, k, 700, outliers=True)
    gamma = workloads.gaussian_bf16((k,), 0.1, 701)
    b = workloads.gaussian_bf16((n, k), w.b_sigma, 702)
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    xd, gd = x.to(dev), gamma.to(dev)
    y = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    mxfp4_rmsnorm_quantize(xd, gd, 1e-5, y=y)
    ap_q, ap_s = mxfp4_quantize_prepacked(y)
    c_two = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, out_dtype=torch.float32)
    fq, fs = mxfp4_rmsnorm_quantize(xd, gd, 1e-5, prepacked=True)
    c_fused = mxfp4_gemm_nt_prepacked_ab(fq, fs, bp_q, bp_s, m, n, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(fq, ap_q) and torch.equal(fs, ap_s)
    assert torch.equal(c_fused, c_two)
    cols = sampled_indices(n, 96, seed=3)
    aq, as_ = oracle.quantize(_bits(y))
    obq, obs = oracle.quantize(workloads.bf16_bits(b[torch.from_numpy(cols)]))
    ref = oracle.gemm_nt(aq, as_, obq, obs)
    assert oracle.floored_max_rel(to_np(c_fused)[:, cols].astype(np.float64), ref) <= 1e-5
