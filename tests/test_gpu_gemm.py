"""GPU block-scaled FP4 NT GEMM vs the CPU oracle.

Each kernel the library can select (256x256 tiles, 128x128 tiles, the small-M
split-K path at several split counts, the small-M streaming path) runs on
shapes with several tiles and ragged M, N and K tails.  Bars:
  * exact regime (every partial sum representable in fp32): fp32 output
    bit-identical to the float64 oracle;
  * fp32 output: floored max-rel <= 1e-5 against the fp32 CPU reference and
    against the float64 oracle;
  * bf16 output: floored max-rel <= 1e-2 against the float64 oracle, and equal
    to the nearest-even rounding of the exact result except at rounding
    midpoints;
  * outputs poisoned with NaN bytes beforehand, neighbouring memory untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import MXFP4Error, mxfp4_gemm_nt, mxfp4_quantize, workspace
from tests.gpu_common import (assert_bf16_matches_rounded, device, log, poisoned, random_bf16,
                              random_codes, sampled_indices, to_np, upload)

pytestmark = pytest.mark.gpu

TILE_SHAPES = [  # (m, n, k): several tiles, ragged tails, k % 128 != 0 cases
    (256, 256, 128), (300, 520, 1024), (513, 263, 2048), (130, 900, 1056), (64, 64, 32),
    (257, 129, 4096), (1, 300, 96),
    # last 256-row tile with 96 and with 200 stored rows: a wave row with 3 of its
    # 4 row blocks stored (first / second wave row)
    (352, 520, 1024), (200, 300, 512),
]
SPLITK_SHAPES = [(1, 64, 128), (17, 200, 1024), (32, 1000, 4096), (33, 70, 160), (100, 512, 2048),
                 (128, 320, 4096), (64, 129, 8192),
                 # K in 128-chunks not divisible by 4 (15, 17, 30): waves of unequal K
                 # ranges over several column tiles
                 (2, 281, 1920), (64, 300, 2176), (128, 200, 3840)]
# the persistent loop needs k % 1024 == 0; k = 1024 is the two-stage tile (no loop body)
PERSISTENT_SHAPES = [(300, 520, 1024), (513, 263, 2048), (257, 129, 4096), (352, 520, 1024), (1, 300, 1024),
                     (200, 300, 3072)]
STREAM_SHAPES = [(1, 64, 512), (17, 200, 1024), (32, 1000, 4096), (33, 70, 512), (64, 129, 8192),
                 (100, 512, 2048), (128, 320, 4096), (129, 66, 1536), (300, 190, 1024)]


def _gemm(aq, as_, bq, bs, dev, kernel, splits, out_dtype, m, n):
    c_all = poisoned((m + 1, n), out_dtype, dev, 0xFF)        # NaN poison, one canary row after
    c = c_all[:m]
    mxfp4_gemm_nt(upload(aq, dev), upload(as_, dev), upload(bq, dev), upload(bs, dev), c=c,
                  kernel=kernel, splits=splits)
    torch.cuda.synchronize()
    canary = to_np(c_all[m:].view(torch.uint8))
    assert np.all(canary == 0xFF), "write past the end of C"
    out = to_np(c.float()) if out_dtype == torch.float32 else to_np(c.view(torch.int16)).view(np.uint16)
    return out


def _cases():
    for kern in ("tile256", "tile128"):
        for shape in TILE_SHAPES:
            yield kern, 0, shape
    for splits in (1, 2, 3, 0):
        for shape in SPLITK_SHAPES:
            yield "splitk", splits, shape
    for shape in STREAM_SHAPES:
        yield "stream", 0, shape
    for shape in PERSISTENT_SHAPES:
        yield "persistent", 0, shape


CASES = list(_cases())


@pytest.mark.parametrize("kernel,splits,shape", CASES, ids=[f"{k}-s{s}-{m}x{n}x{kk}" for k, s, (m, n, kk) in CASES])
def test_gemm_exact_regime_bitexact(kernel, splits, shape):
    dev = device()
    m, n, k = shape
    log(f"exact regime {kernel} splits={splits} {shape}")
    aq, _ = random_codes(m, k, 1)
    bq, _ = random_codes(n, k, 2)
    if k <= 256:   # varied block scales keep every sum exact while K is small
        _, as_ = random_codes(m, k, 3, 125, 129)
        _, bs = random_codes(n, k, 4, 125, 129)
    else:
        as_ = np.full((m, k // 32), 127, np.uint8)
        bs = np.full((n, k // 32), 127, np.uint8)
    ref = oracle.gemm_nt(aq, as_, bq, bs)
    got = _gemm(aq, as_, bq, bs, dev, kernel, splits, torch.float32, m, n)
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("kernel,splits,shape", CASES, ids=[f"{k}-s{s}-{m}x{n}x{kk}" for k, s, (m, n, kk) in CASES])
def test_gemm_quantized_gaussian(kernel, splits, shape):
    dev = device()
    m, n, k = shape
    log(f"gaussian {kernel} splits={splits} {shape}")
    a = random_bf16((m, k), 10 + m, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), 20 + n, spread=3)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    c64 = oracle.gemm_nt(aq, as_, bq, bs)
    c32 = oracle.gemm_nt_f32(aq, as_, bq, bs)
    got32 = _gemm(aq, as_, bq, bs, dev, kernel, splits, torch.float32, m, n)
    assert oracle.floored_max_rel(got32, c32) <= 1e-5
    assert oracle.floored_max_rel(got32, c64) <= 1e-5
    got16 = _gemm(aq, as_, bq, bs, dev, kernel, splits, torch.bfloat16, m, n)
    assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got16), c64) <= 1e-2
    assert_bf16_matches_rounded(got16, c64)
    # the bf16 output is the nearest-even rounding of this kernel's own fp32 result
    assert np.array_equal(got16, oracle.f64_to_bf16_bits(got32.astype(np.float64)))


def test_gemm_auto_dispatch_and_empty_problems():
    dev = device()
    a = random_bf16((96, 256), 1)
    b = random_bf16((80, 256), 2)
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    c = mxfp4_gemm_nt(aq, as_, bq, bs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oaq, oas = oracle.quantize(workloads.bf16_bits(a))
    obq, obs = oracle.quantize(workloads.bf16_bits(b))
    assert oracle.floored_max_rel(to_np(c), oracle.gemm_nt(oaq, oas, obq, obs)) <= 1e-5
    # m == 0 and n == 0 are no-ops
    e = mxfp4_gemm_nt(aq[:0], as_[:0], bq, bs)
    assert e.shape == (0, 80)
    e = mxfp4_gemm_nt(aq, as_, bq[:0], bs[:0])
    assert e.shape == (96, 0)


def test_stream_kernel_rejects_unsupported_k():
    """The streaming kernel copies 512-K units: any other k is refused, not miscomputed."""
    dev = device()
    aq, as_ = random_codes(8, 1056, 1)
    bq, bs = random_codes(64, 1056, 2)
    with pytest.raises(MXFP4Error):
        mxfp4_gemm_nt(upload(aq, dev), upload(as_, dev), upload(bq, dev), upload(bs, dev), kernel="stream")


def test_persistent_kernel_rejects_unsupported_k():
    """The persistent loop takes an even number of 512-K scale groups per tile:
    k = 1536 is refused, not miscomputed."""
    dev = device()
    aq, as_ = random_codes(300, 1536, 1)
    bq, bs = random_codes(64, 1536, 2)
    with pytest.raises(MXFP4Error):
        mxfp4_gemm_nt(upload(aq, dev), upload(as_, dev), upload(bq, dev), upload(bs, dev), kernel="persistent")


@pytest.mark.parametrize("shape", [(4400, 4200, 2048), (8192, 8192, 1024)])
def test_persistent_matches_tile256_many_tiles_per_workgroup(shape):
    """More output tiles than compute units: every workgroup of the persistent
    launch runs several tiles back to back (the next tile's first stage is
    loaded during the previous tile's epilogue).  The result is bit-identical
    to the one-tile-per-workgroup kernel, and sampled entries match the oracle."""
    dev = device()
    m, n, k = shape
    log(f"persistent vs tile256 {shape}")
    a = random_bf16((m, k), 30 + m, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), 40 + n, spread=3)
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    got = {}
    for dt, bits in ((torch.float32, torch.int32), (torch.bfloat16, torch.int16)):
        ref = mxfp4_gemm_nt(aq, as_, bq, bs, out_dtype=dt, kernel="tile256")
        got[dt] = mxfp4_gemm_nt(aq, as_, bq, bs, out_dtype=dt, kernel="persistent")
        torch.cuda.synchronize()
        assert torch.equal(got[dt].view(bits), ref.view(bits)), f"{dt} differs from the tile256 kernel"
    rows = sampled_indices(m, 48, seed=3)
    cols = sampled_indices(n, 48, seed=4)
    oaq, oas = oracle.quantize(workloads.bf16_bits(a[torch.from_numpy(rows)]))
    obq, obs = oracle.quantize(workloads.bf16_bits(b[torch.from_numpy(cols)]))
    c64 = oracle.gemm_nt(oaq, oas, obq, obs)
    assert oracle.floored_max_rel(to_np(got[torch.float32])[np.ix_(rows, cols)], c64) <= 1e-5
    got16 = to_np(got[torch.bfloat16].view(torch.int16)).view(np.uint16)[np.ix_(rows, cols)]
    assert_bf16_matches_rounded(got16, c64)


@pytest.mark.parametrize("kernel", ["tile256", "tile128", "stream", "splitk", "persistent"])
def test_gemm_long_k(kernel):
    """A long reduction (k = 2^19): row offsets inside a tile reach 255 * k/2
    bytes.  Codes of magnitude <= 1 with unit scales keep every partial sum a
    multiple of 1/4 below 2^19, exact in fp32, so the result is bit-exact
    whatever the summation order, and any misaddressed row or block shows."""
    dev = device()
    m, n, k = 3, 70, 1 << 19
    log(f"long k {kernel} {m}x{n}x{k}")
    g = np.random.default_rng(7)
    small = np.array([0, 1, 2, 8, 9, 10], np.uint8)          # 0, +-0.5, +-1
    aq = (small[g.integers(0, 6, (m, k // 2))] | (small[g.integers(0, 6, (m, k // 2))] << 4)).astype(np.uint8)
    bq = (small[g.integers(0, 6, (n, k // 2))] | (small[g.integers(0, 6, (n, k // 2))] << 4)).astype(np.uint8)
    as_ = np.full((m, k // 32), 127, np.uint8)
    bs = np.full((n, k // 32), 127, np.uint8)
    ref = oracle.gemm_nt(aq, as_, bq, bs)
    got = _gemm(aq, as_, bq, bs, dev, kernel, 0, torch.float32, m, n)
    assert np.array_equal(got, ref.astype(np.float32))


def test_splitk_workspace_reuse_across_calls():
    """The arrival counters return to zero, so one workspace serves consecutive
    calls of different shapes (the partial sums of a small-N call must not land
    where a larger-N call keeps its counters)."""
    dev = device()
    ws = torch.zeros(1 << 25, dtype=torch.uint8, device=dev)
    for seed, (m, n, k) in enumerate([(64, 512, 2048), (128, 640, 4096), (7, 64, 1024), (128, 9000, 1024)]):
        a = random_bf16((m, k), 100 + seed)
        b = random_bf16((n, k), 200 + seed)
        aq, as_ = oracle.quantize(workloads.bf16_bits(a))
        bq, bs = oracle.quantize(workloads.bf16_bits(b))
        c = mxfp4_gemm_nt(upload(aq, dev), upload(as_, dev), upload(bq, dev), upload(bs, dev),
                          out_dtype=torch.float32, kernel="splitk", splits=4, ws=ws)
        torch.cuda.synchronize()
        assert oracle.floored_max_rel(to_np(c), oracle.gemm_nt(aq, as_, bq, bs)) <= 1e-5
        assert torch.all(ws[:65536] == 0), "counters not returned to zero"


@pytest.mark.parametrize("name", ["tiny_64x256x1024", "decode_128x14336x4096", "prefill_4096x4096x4096",
                                  "ffn_down_4096x4096x14336", "square_8192x8192x8192"])
def test_gemm_workload_full_size_sampled(name):
    """Full-size workloads through the benchmark's path (GPU quantize + auto GEMM),
    checked on sampled output rows and columns against the oracle."""
    dev = device()
    w = workloads.DENSE[name]
    a, b = w.make()
    log(f"{name}: full-size GEMM")
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    c = mxfp4_gemm_nt(aq, as_, bq, bs)
    c32 = mxfp4_gemm_nt(aq, as_, bq, bs, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = sampled_indices(w.m, 64, seed=1)
    cols = sampled_indices(w.n, 64, seed=2)
    oaq, oas = oracle.quantize(workloads.bf16_bits(a[torch.from_numpy(rows)]))
    obq, obs = oracle.quantize(workloads.bf16_bits(b[torch.from_numpy(cols)]))
    ref = oracle.gemm_nt(oaq, oas, obq, obs)
    got16 = to_np(c.view(torch.int16)).view(np.uint16)[np.ix_(rows, cols)]
    got32 = to_np(c32)[np.ix_(rows, cols)]
    assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got16), ref) <= 1e-2
    assert oracle.floored_max_rel(got32, ref) <= 1e-5
    assert_bf16_matches_rounded(got16, ref)
