"""GPU W4A8 GEMMs (MXFP8 A x MXFP4 B, dense and grouped) vs the CPU oracle.

Numerics of the hardware.  gfx950's scaled MFMA with an FP8 operand does not
form an exact dot product: along K it sums products in aligned groups of 8
(K [8g, 8g + 8)), first aligning them to the group's largest exponent sum
(E4M3 exponent + E2M1 exponent, from the exponent fields) and truncating each
toward zero to a multiple of 2**(E - 13); within one 64-deep MFMA the group
sums are aligned to the largest exponent sum E' of its products and rounded
down to a multiple of 2**(E' - 24) (measured with both operands FP8,
tests/test_gpu_mxfp8_gemm.py); the MFMA's sum then meets the fp32
accumulator.  (Measured through this library with one big and one small
element per row; test_w4a8_mfma_group_rule pins the group rule.)  FP4 x FP4
never loses a bit under that rule, FP8 x FP4 can, so the FP4 GEMM's 1e-5 fp32
bar becomes a bound derived from the rule:
    |C - C_exact| <= sum_g n_g * 2**(E_g - 13) * scale_a * scale_b
                     + sum_t 8 * 2**(E'_t + S_t - 24)
                     + (k / 16) * 2**-24 * sum_k |a_k * b_k|
with n_g the group's nonzero products and E_g taken over every element of
the group (an upper bound whether or not the hardware skips zeros), E'_t over
every element of 64-deep step t and S_t the step's largest sum of block
scale exponents.

Bars:
  * exact regime (no product can leave its group's grid and every partial sum
    is exact in fp32): fp32 output bit-identical to the float64 oracle, with
    varied block scales;
  * general data: the bound above element by element, and floored max-rel
    <= 1e-2 against the float64 oracle;
  * bf16 output: the nearest-even rounding of the kernel's own fp32 result;
  * outputs poisoned with NaN bytes beforehand, a canary row after C untouched;
  * grouped: bit-identical to the dense tile kernel on each expert's row slice.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_prepack_weight, mxfp4_quantize, mxfp8_gemm_w4a8_nt,
                                        mxfp8_gemm_w4a8_nt_prepacked, mxfp8_grouped_gemm_w4a8_nt, mxfp8_quantize)
from tests.gpu_common import device, log, poisoned, random_bf16, random_codes, sampled_indices, to_np, upload

pytestmark = pytest.mark.gpu

# (m, n, k): one tile, several 128 x 256 tiles with ragged M / N tails, k % 512 != 0
# (register path), tiles whose second wave row holds 0, 1 or 2 stored row blocks
SHAPES = [(128, 256, 512), (300, 520, 1024), (513, 263, 2048), (130, 900, 1056), (64, 64, 32),
          (257, 129, 4096), (1, 300, 96), (200, 300, 512), (40, 256, 512), (80, 256, 512),
          (100, 256, 512), (129, 1000, 1536)]
# streaming kernel (k % 512 == 0): 32- and 64-row M tiles, several M tiles sharing a
# 64-column slice, ragged M / N, a column count that is not a multiple of 8 slices
STREAM_SHAPES = [(1, 64, 512), (17, 200, 1024), (32, 1000, 4096), (33, 70, 512), (64, 129, 8192),
                 (100, 512, 2048), (128, 320, 4096), (129, 66, 1536), (300, 190, 1024), (128, 14336, 512)]
CASES = [("tile128", s) for s in SHAPES] + [("stream", s) for s in STREAM_SHAPES]
CASE_IDS = [f"{kern}-{m}x{n}x{k}" for kern, (m, n, k) in CASES]


def _fp8_exponents(q8):
    """Exponent of each E4M3 code from its field (field 0, subnormal or zero, counts as 1)."""
    return np.maximum((q8.astype(np.int64) >> 3) & 15, 1) - 7


def _fp4_exponents(q4):
    """Exponent of each E2M1 element [rows, k] from its field (field 0 counts as 1)."""
    lo, hi = q4 & 0xF, q4 >> 4
    codes = np.empty((q4.shape[0], q4.shape[1] * 2), np.int64)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    return np.maximum((codes >> 1) & 3, 1) - 1, codes


def w4a8_tolerance(aq, as_, bq, bs):
    """Per-element bound on |C_gpu - C_exact| from the MFMA's group rule (module docstring)."""
    m, k = aq.shape
    n = bq.shape[0]
    ea = _fp8_exponents(aq)
    eb, bcodes = _fp4_exponents(bq)
    a_nz = (aq & 0x7F) != 0
    b_nz = (bcodes & 7) != 0
    groups = k // 8
    E = np.full((m, n, groups), -10 ** 6, np.int64)
    cnt = np.zeros((m, n, groups), np.int64)
    for u in range(8):
        E = np.maximum(E, ea[:, None, u::8] + eb[None, :, u::8])
        cnt += a_nz[:, None, u::8] & b_nz[None, :, u::8]
    sa = np.repeat(as_.astype(np.int64) - 127, 4, axis=1)        # scale exponent per group
    sb = np.repeat(bs.astype(np.int64) - 127, 4, axis=1)
    trunc = (cnt * np.ldexp(1.0, E - 13 + sa[:, None, :] + sb[None, :, :])).sum(-1)
    cross = np.zeros((m, n))
    for t in range((groups + 7) // 8):
        g0, g1 = 8 * t, min(8 * t + 8, groups)
        cross += 8 * np.ldexp(1.0, E[:, :, g0:g1].max(-1) + (sa[:, None, g0:g1] + sb[None, :, g0:g1]).max(-1) - 24)
    trunc = trunc + cross
    a_abs = np.abs(oracle.dequantize_mxfp8(aq, as_))
    b_abs = np.abs(oracle.dequantize(bq, bs))
    acc = (k / 16) * 2.0 ** -24 * (a_abs @ b_abs.T)
    return trunc + acc


def _check_general(got32, got16, c64, tol):
    bad = np.abs(got32.astype(np.float64) - c64) > tol
    assert not bad.any(), f"{int(bad.sum())} outputs outside the MFMA group-rule bound"
    assert oracle.floored_max_rel(got32, c64) <= 1e-2
    if got16 is not None:
        assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got16), c64) <= 1e-2
        assert np.array_equal(got16, oracle.f64_to_bf16_bits(got32.astype(np.float64)))


def _gemm(aq, as_, bq, bs, dev, out_dtype, m, n, kernel="auto"):
    c_all = poisoned((m + 1, n), out_dtype, dev, 0xFF)        # NaN poison, one canary row after
    c = c_all[:m]
    mxfp8_gemm_w4a8_nt(upload(aq, dev), upload(as_, dev), upload(bq, dev), upload(bs, dev), c=c, kernel=kernel)
    torch.cuda.synchronize()
    assert np.all(to_np(c_all[m:].view(torch.uint8)) == 0xFF), "write past the end of C"
    return to_np(c.float()) if out_dtype == torch.float32 else to_np(c.view(torch.int16)).view(np.uint16)


def _exact_fp8_codes(rows, k, seed, top_field):
    """E4M3 codes of value 0 or +-(1 + j/8) * 2**p, p in 0 .. top_field - 7 (multiples of 1/8)."""
    rng = np.random.default_rng(seed)
    mag = rng.integers(7 << 3, (top_field + 1) << 3, size=(rows, k), dtype=np.uint8)
    mag[rng.random((rows, k)) < 0.1] = 0
    sign = (rng.random((rows, k)) < 0.5).astype(np.uint8) << 7
    return mag | sign


@pytest.mark.parametrize("kernel,shape", CASES, ids=CASE_IDS)
def test_w4a8_exact_regime_bitexact(kernel, shape):
    """A values are multiples of 1/8 with exponents 0 .. 3 and B values multiples
    of 1/2 up to 6 (exponents 0 .. 2): every exponent sum is at most 5, so the
    group grid is at most 2**-8 and every product (a multiple of 1/16 before
    scaling) lies on it.  For k <= 2048 A stays below 4 (exponents 0 .. 1) and
    the block scales vary over 2**-1 .. 2**1 (products multiples of 2**-6 below
    90, sums below 2**18), otherwise scales are 1 and A below 16 (products
    multiples of 1/16 below 96, sums below 2**19): every partial sum is exact in
    fp32, so the result is bit-exact."""
    dev = device()
    m, n, k = shape
    log(f"w4a8 exact regime {kernel} {shape}")
    bq, _ = random_codes(n, k, 2)
    if k <= 2048:
        aq = _exact_fp8_codes(m, k, 1, 8)
        rng = np.random.default_rng(3)
        as_ = rng.integers(126, 129, size=(m, k // 32), dtype=np.uint8)
        bs = rng.integers(126, 129, size=(n, k // 32), dtype=np.uint8)
    else:
        aq = _exact_fp8_codes(m, k, 1, 10)
        as_ = np.full((m, k // 32), 127, np.uint8)
        bs = np.full((n, k // 32), 127, np.uint8)
    ref = oracle.gemm_w4a8_nt(aq, as_, bq, bs)
    got = _gemm(aq, as_, bq, bs, dev, torch.float32, m, n, kernel)
    assert np.array_equal(got, ref.astype(np.float32))


def test_w4a8_mfma_group_rule():
    """Pins the hardware rule the tolerance is derived from: a big product (448,
    times 1 or 6) and a small one in the same aligned group of 8 lose the small
    one's bits below 2**(E - 13), truncated toward zero; in different groups
    both survive exactly."""
    dev = device()
    k = 512
    cases = []
    for bval, bbyte, eb in ((1.0, 0x22, 0), (6.0, 0x77, 2)):
        for big in (0x7E, 0xFE):
            for small in (0x01, 0x08, 0x0C, 0x14, 0x8C, 0x94):
                for pb, ps in ((0, 1), (0, 7), (13, 8), (13, 15), (0, 8), (7, 8), (40, 47), (40, 39), (63, 56)):
                    cases.append((bval, bbyte, eb, big, small, pb, ps))
    for bval, bbyte, eb in ((1.0, 0x22, 0), (6.0, 0x77, 2)):
        rows = [c for c in cases if c[1] == bbyte]
        a = np.zeros((len(rows), k), np.uint8)
        for i, (_, _, _, big, small, pb, ps) in enumerate(rows):
            a[i, pb], a[i, ps] = big, small
        b = np.full((64, k // 2), bbyte, np.uint8)
        got = _gemm(a, np.full((len(rows), k // 32), 127, np.uint8), b, np.full((64, k // 32), 127, np.uint8), dev,
                    torch.float32, len(rows), 64)[:, 0]
        for g, (_, _, _, big, small, pb, ps) in zip(got, rows):
            pbig = oracle.E4M3_TABLE[big] * bval
            psmall = oracle.E4M3_TABLE[small] * bval
            if pb // 8 == ps // 8:
                grid = 2.0 ** (8 + eb - 13)          # 448 has exponent 8
                psmall = np.trunc(psmall / grid) * grid
            assert g == pbig + psmall, (hex(big), hex(small), pb, ps, bval, g, pbig + psmall)


def _quantized_operands(m, n, k, seed):
    a = random_bf16((m, k), 10 + seed, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), 20 + seed, spread=3)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    return aq, as_, bq, bs


@pytest.mark.parametrize("kernel,shape", CASES, ids=CASE_IDS)
def test_w4a8_quantized_gaussian(kernel, shape):
    dev = device()
    m, n, k = shape
    log(f"w4a8 gaussian {kernel} {shape}")
    aq, as_, bq, bs = _quantized_operands(m, n, k, m + n)
    c64 = oracle.gemm_w4a8_nt(aq, as_, bq, bs)
    got32 = _gemm(aq, as_, bq, bs, dev, torch.float32, m, n, kernel)
    got16 = _gemm(aq, as_, bq, bs, dev, torch.bfloat16, m, n, kernel)
    _check_general(got32, got16, c64, w4a8_tolerance(aq, as_, bq, bs))


def test_w4a8_unaligned_scales_take_the_register_path():
    """k % 512 == 0 but scale arrays only 4-byte aligned: the register path runs
    and gives the copy path's result bit for bit."""
    dev = device()
    m, n, k = 200, 300, 1024
    aq, as_, bq, bs = _quantized_operands(m, n, k, 5)
    d_aq, d_bq = upload(aq, dev), upload(bq, dev)
    ref = to_np(mxfp8_gemm_w4a8_nt(d_aq, upload(as_, dev), d_bq, upload(bs, dev), out_dtype=torch.float32))
    a_buf = torch.zeros(as_.size + 4, dtype=torch.uint8, device=dev)
    b_buf = torch.zeros(bs.size + 4, dtype=torch.uint8, device=dev)
    a_s = a_buf[4:].view(m, k // 32)
    b_s = b_buf[4:].view(n, k // 32)
    a_s.copy_(upload(as_, dev))
    b_s.copy_(upload(bs, dev))
    got = to_np(mxfp8_gemm_w4a8_nt(d_aq, a_s, d_bq, b_s, out_dtype=torch.float32))
    torch.cuda.synchronize()
    assert np.array_equal(got, ref)
    _check_general(got, None, oracle.gemm_w4a8_nt(aq, as_, bq, bs), w4a8_tolerance(aq, as_, bq, bs))


def test_w4a8_long_k():
    """k = 2^19 over 130 rows (two m-tiles): A row offsets inside a tile reach
    127 * k bytes.  Values 0, +-1/2, +-1 with unit scales keep every partial sum
    a multiple of 1/4 below 2^19, exact in fp32, so the result is bit-exact."""
    dev = device()
    m, n, k = 130, 16, 1 << 19
    log(f"w4a8 long k {m}x{n}x{k}")
    g = np.random.default_rng(7)
    small8 = np.array([0x00, 0x30, 0x38, 0xB0, 0xB8], np.uint8)     # 0, 1/2, 1, -1/2, -1
    small4 = np.array([0, 1, 2, 8, 9, 10], np.uint8)                # 0, 1/2, 1, -0, -1/2, -1
    aq = small8[g.integers(0, 5, (m, k))]
    bq = (small4[g.integers(0, 6, (n, k // 2))] | (small4[g.integers(0, 6, (n, k // 2))] << 4)).astype(np.uint8)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    ref = oracle.gemm_w4a8_nt(aq, as_, bq, bs)
    got = _gemm(aq, as_, bq, bs, dev, torch.float32, m, n)
    assert np.array_equal(got, ref.astype(np.float32))


def test_w4a8_kernels_agree_and_stream_rejects_unsupported_k():
    """The tile and streaming kernels give results within each other's bound on
    one decode-like shape, and the streaming kernel refuses k % 512 != 0."""
    dev = device()
    m, n, k = 128, 640, 4096
    aq, as_, bq, bs = _quantized_operands(m, n, k, 77)
    tile = _gemm(aq, as_, bq, bs, dev, torch.float32, m, n, "tile128")
    strm = _gemm(aq, as_, bq, bs, dev, torch.float32, m, n, "stream")
    tol = w4a8_tolerance(aq, as_, bq, bs)
    assert np.all(np.abs(tile.astype(np.float64) - strm) <= 2 * tol)
    from block_scaled_fp4_mxfp4_amd import MXFP4Error
    aq2, as2, bq2, bs2 = (upload(t, dev) for t in _quantized_operands(8, 64, 1056, 3))
    with pytest.raises(MXFP4Error):
        mxfp8_gemm_w4a8_nt(aq2, as2, bq2, bs2, kernel="stream")


# the W4A8 GEMM on a prepacked weight: 32-, 64- and 128-row A tiles (two pairs of
# FP8 A in LDS at 128 rows), K in chunks of 8, 4 and 1 pairs, ragged M and N
PREPACKED_SHAPES = [(1, 64, 512), (17, 200, 1024), (32, 1000, 4096), (33, 70, 512), (64, 129, 8192),
                    (100, 512, 2048), (128, 320, 4096), (128, 192, 4608), (129, 66, 1536), (200, 190, 14336),
                    (128, 14336, 512)]


@pytest.mark.parametrize("shape", PREPACKED_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in PREPACKED_SHAPES])
def test_w4a8_prepacked_weight_matches_stream_kernel(shape):
    """Bit-identical to the streaming kernel (same per-wave K split, MFMA order
    and reduction) in fp32 and BF16, within the derived bound of the oracle,
    nothing written past C."""
    dev = device()
    m, n, k = shape
    log(f"w4a8 prepacked weight {shape}")
    aq, as_, bq, bs = _quantized_operands(m, n, k, 3 * m + n)
    d_aq, d_as, d_bq, d_bs = (upload(t, dev) for t in (aq, as_, bq, bs))
    bp_q, bp_s = mxfp4_prepack_weight(d_bq, d_bs)
    for out_dtype, bits in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        c_all = poisoned((m + 1, n), out_dtype, dev, 0x7F)
        mxfp8_gemm_w4a8_nt_prepacked(d_aq, d_as, bp_q, bp_s, n, c=c_all[:m])
        ref = mxfp8_gemm_w4a8_nt(d_aq, d_as, d_bq, d_bs, out_dtype=out_dtype, kernel="stream")
        torch.cuda.synchronize()
        assert torch.all(c_all[m:].view(torch.uint8) == 0x7F), "write past C"
        assert torch.equal(c_all[:m].view(bits), ref.view(bits)), f"{out_dtype} differs from the streaming kernel"
        if out_dtype == torch.float32:
            _check_general(to_np(c_all[:m]), None, oracle.gemm_w4a8_nt(aq, as_, bq, bs),
                           w4a8_tolerance(aq, as_, bq, bs))


def test_w4a8_prepacked_rejects_bad_k():
    from block_scaled_fp4_mxfp4_amd import MXFP4Error
    dev = device()
    aq, as_, bq, bs = (upload(t, dev) for t in _quantized_operands(8, 64, 1024, 3))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    with pytest.raises(MXFP4Error):   # the weight is prepacked for k = 1024; A claims 992
        mxfp8_gemm_w4a8_nt_prepacked(aq[:, :992].contiguous(), as_[:, :31].contiguous(), bp_q, bp_s, 64)


def test_w4a8_empty_problems():
    dev = device()
    aq, as_, bq, bs = (upload(t, dev) for t in _quantized_operands(96, 80, 256, 1))
    assert mxfp8_gemm_w4a8_nt(aq[:0], as_[:0], bq, bs).shape == (0, 80)
    assert mxfp8_gemm_w4a8_nt(aq, as_, bq[:0], bs[:0]).shape == (96, 0)


@pytest.mark.parametrize("name", ["tiny_64x256x1024", "decode_128x14336x4096", "prefill_4096x4096x4096",
                                  "ffn_down_4096x4096x14336", "square_8192x8192x8192"])
def test_w4a8_workload_full_size_sampled(name):
    """Full-size dense workloads with MXFP8 activations (GPU quantizers + W4A8
    GEMM), checked on sampled output rows and columns against the oracle."""
    dev = device()
    w = workloads.DENSE[name]
    a, b = w.make()
    log(f"{name}: full-size W4A8 GEMM")
    aq, as_ = mxfp8_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    c = mxfp8_gemm_w4a8_nt(aq, as_, bq, bs)
    c32 = mxfp8_gemm_w4a8_nt(aq, as_, bq, bs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sampled_indices(w.m, 64, seed=1)
    cols = sampled_indices(w.n, 64, seed=2)
    oaq, oas = oracle.quantize_mxfp8(workloads.bf16_bits(a[torch.from_numpy(rows)]))
    obq, obs = oracle.quantize(workloads.bf16_bits(b[torch.from_numpy(cols)]))
    ref = oracle.gemm_w4a8_nt(oaq, oas, obq, obs)
    got16 = to_np(c.view(torch.int16)).view(np.uint16)[np.ix_(rows, cols)]
    got32 = to_np(c32)[np.ix_(rows, cols)]
    _check_general(got32, got16, ref, w4a8_tolerance(oaq, oas, obq, obs))


# ---------------------------------------------------------------------------
# grouped

def _grouped_case(counts, n, k, seed, dev, out_dtype=torch.float32):
    counts = np.asarray(counts)
    groups = len(counts)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    total = int(offsets[-1])
    a = random_bf16((max(total, 1), k), seed)[:total]
    w = random_bf16((groups * n, k), seed + 1)
    if total:
        aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    else:
        aq, as_ = np.zeros((0, k), np.uint8), np.zeros((0, k // 32), np.uint8)
    wq, ws = oracle.quantize(workloads.bf16_bits(w))
    wq = wq.reshape(groups, n, k // 2)
    ws = ws.reshape(groups, n, k // 32)
    c_all = poisoned((total + 1, n), out_dtype, dev, 0xFF)
    c = c_all[:total]
    d_ops = upload(aq, dev), upload(as_, dev), upload(wq, dev), upload(ws, dev)
    mxfp8_grouped_gemm_w4a8_nt(*d_ops, upload(offsets, dev), c=c)
    torch.cuda.synchronize()
    assert torch.all(c_all[total:].view(torch.uint8) == 0xFF), "write past the end of C"
    return aq, as_, wq, ws, offsets, c, d_ops


GROUP_PATTERNS = {
    "single_group": ([300], 192, 256),
    "all_rows_one_expert": ([0, 0, 517, 0], 130, 512),
    "empty_first_middle_last": ([0, 40, 0, 129, 0], 96, 1024),
    "tile_boundaries_128": ([1, 127, 128, 129, 255, 256, 257], 64, 256),
    "ragged_k": ([33, 70, 5], 72, 160),
    "many_groups": (list(np.random.default_rng(0).integers(0, 40, size=70)), 64, 256),
    # k % 1024 == 0: the persistent tile loop (128 x 256 tiles), with ragged
    # groups and n, and more tiles than compute units
    "persistent_ragged": ([0, 127, 128, 129, 255, 1, 700, 0], 200, 1024),
    "persistent_ragged_n": ([300, 0, 600, 45, 256, 1000], 600, 1024),
    "persistent_many_tiles": (list(np.random.default_rng(1).integers(0, 600, size=32)), 1536, 2048),
}


@pytest.mark.parametrize("pattern", list(GROUP_PATTERNS))
def test_grouped_w4a8_bitexact_vs_dense_per_group(pattern):
    dev = device()
    counts, n, k = GROUP_PATTERNS[pattern]
    log(f"grouped w4a8 {pattern}: counts={counts[:10]} n={n} k={k}")
    aq, as_, wq, ws, offsets, c, (d_aq, d_as, d_wq, d_ws) = _grouped_case(counts, n, k, 7, dev)
    got = to_np(c)
    for g in range(len(counts)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        a_s_g = d_as[lo:hi] if k % 128 == 0 else d_as[lo:hi].clone()
        dense = mxfp8_gemm_w4a8_nt(d_aq[lo:hi], a_s_g, d_wq[g], d_ws[g], out_dtype=torch.float32, kernel="tile128")
        torch.cuda.synchronize()
        assert np.array_equal(got[lo:hi], to_np(dense)), f"group {g}"
        # the oracle bound on up to 16 rows of the group (its cost grows with rows x n x k / 8)
        rows = np.unique(np.linspace(lo, hi - 1, min(16, hi - lo)).astype(np.int64))
        ref = oracle.gemm_w4a8_nt(aq[rows], as_[rows], wq[g], ws[g])
        _check_general(got[rows], None, ref, w4a8_tolerance(aq[rows], as_[rows], wq[g], ws[g]))


def test_grouped_w4a8_bf16_output():
    dev = device()
    counts = [17, 0, 300, 64]
    aq, as_, wq, ws, offsets, c, d_ops = _grouped_case(counts, 200, 1024, 9, dev, out_dtype=torch.bfloat16)
    c32 = torch.empty(c.shape, dtype=torch.float32, device=dev)
    mxfp8_grouped_gemm_w4a8_nt(*d_ops, upload(offsets, dev), c=c32)
    torch.cuda.synchronize()
    got = to_np(c.view(torch.int16)).view(np.uint16)
    got32 = to_np(c32)
    for g in range(len(counts)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        ref = oracle.gemm_w4a8_nt(aq[lo:hi], as_[lo:hi], wq[g], ws[g])
        _check_general(got32[lo:hi], got[lo:hi], ref, w4a8_tolerance(aq[lo:hi], as_[lo:hi], wq[g], ws[g]))


def test_grouped_w4a8_moe_workload_full_size_sampled():
    """The 64-expert top-4 MoE layer at full size with MXFP8 activations (GPU
    quantizers + grouped W4A8 GEMM), checked on sampled rows of every expert."""
    dev = device()
    w = workloads.MOE
    a, wts, offsets = w.make()
    aq, as_ = mxfp8_quantize(a.to(dev))
    wq, wsc = mxfp4_quantize(wts.view(-1, w.k).to(dev))
    wq = wq.view(w.experts, w.n, w.k // 2)
    wsc = wsc.view(w.experts, w.n, w.k // 32)
    d_off = offsets.to(dev)
    c = mxfp8_grouped_gemm_w4a8_nt(aq, as_, wq, wsc, d_off)
    c32 = mxfp8_grouped_gemm_w4a8_nt(aq, as_, wq, wsc, d_off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got_all = to_np(c.view(torch.int16)).view(np.uint16)
    got32_all = to_np(c32)
    cols = sampled_indices(w.n, 48, seed=3)
    for g in range(w.experts):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        rows = lo + sampled_indices(hi - lo, 4, seed=g)
        oaq, oas = oracle.quantize_mxfp8(workloads.bf16_bits(a[torch.from_numpy(rows)]))
        obq, obs = oracle.quantize(workloads.bf16_bits(wts[g][torch.from_numpy(cols)]))
        ref = oracle.gemm_w4a8_nt(oaq, oas, obq, obs)
        _check_general(got32_all[np.ix_(rows, cols)], got_all[np.ix_(rows, cols)], ref,
                       w4a8_tolerance(oaq, oas, obq, obs))


@pytest.mark.parametrize("k", [512, 1024])
def test_grouped_w4a8_malformed_offsets_stay_in_bounds(k):
    """Negative, decreasing and past-the-end offsets neither write outside C nor
    disturb rows that exactly one clamped group covers (k = 1024: the
    persistent tile loop)."""
    dev = device()
    total, n, groups = 300, 96, 4
    offsets = np.array([-5, 120, 80, 500, 300], np.int32)   # g0 = [0, 120), g2 = [80, 300)
    a = random_bf16((total, k), 31)
    w = random_bf16((groups * n, k), 32)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    wq, ws = oracle.quantize(workloads.bf16_bits(w))
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    d_wq, d_ws = upload(wq.reshape(groups, n, k // 2), dev), upload(ws.reshape(groups, n, k // 32), dev)
    c_all = poisoned((total + 3, n), torch.float32, dev, 0xFF)
    c = c_all[:total]
    mxfp8_grouped_gemm_w4a8_nt(d_aq, d_as, d_wq, d_ws, upload(offsets, dev), c=c)
    torch.cuda.synchronize()
    assert torch.all(c_all[total:].view(torch.uint8) == 0xFF), "write past the end of C"
    got = to_np(c)
    g0 = to_np(mxfp8_gemm_w4a8_nt(d_aq[0:120], d_as[0:120], d_wq[0], d_ws[0], out_dtype=torch.float32,
                                  kernel="tile128"))
    g2 = to_np(mxfp8_gemm_w4a8_nt(d_aq[80:300], d_as[80:300], d_wq[2], d_ws[2], out_dtype=torch.float32,
                                  kernel="tile128"))
    torch.cuda.synchronize()
    assert np.array_equal(got[0:80], g0[0:80])
    assert np.array_equal(got[120:300], g2[40:220])
    overlap = got[80:120]
    assert np.all((overlap == g0[80:120]) | (overlap == g2[0:40]))
