"""GPU MXFP8 quantizer vs the CPU oracle, byte for byte (E4M3 codes and scale bytes)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import mxfp8_quantize
from tests.gpu_common import bf16_from_np_bits, device, log, random_bf16, sampled_indices, to_np

pytestmark = pytest.mark.gpu


def _run(x_bits: np.ndarray, dev):
    rows, k = x_bits.shape
    x = bf16_from_np_bits(x_bits).to(dev)
    outs = []
    for poison in (0x00, 0xFF):   # an unwritten byte differs between the two runs
        q = torch.full((rows, k), poison, dtype=torch.uint8, device=dev)
        s = torch.full((rows, k // 32), poison, dtype=torch.uint8, device=dev)
        mxfp8_quantize(x, q, s)
        torch.cuda.synchronize()
        outs.append((to_np(q), to_np(s)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    return outs[0]


def _exhaustive_blocks() -> np.ndarray:
    """Every finite BF16 magnitude (both signs) inside a block of every reachable exponent.

    A block whose largest magnitude is A = (2 - 2**-7) * 2**(e+8) has shared
    exponent e = floor(log2 A) - 8; its other 31 elements run through every
    BF16 value of magnitude <= A, so |x| / 2**e covers [0, 512) at every e,
    including the saturating range (448, 510].  The anchor's position inside
    the block rotates.  Blocks whose maximum lies below 2**-119 (normal,
    subnormal, zero, negative zero) all take the clamped exponent -127.
    """
    mags = np.arange(0, 0x7F80, dtype=np.uint16)
    mag_vals = oracle.bf16_bits_to_f64(mags)
    blocks = []
    pos = 0
    for e in range(-127, 120):
        anchor = float(np.ldexp(255.0, e + 1))            # (2 - 2**-7) * 2**(e+8)
        anchor_bits = oracle.f64_to_bf16_bits(np.array([anchor]))[0]
        vals = mags[mag_vals <= anchor]
        vals = np.concatenate([vals, vals | np.uint16(0x8000)])
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blk = np.empty((vals.shape[0], 32), np.uint16)
        for r in range(vals.shape[0]):
            p = pos % 32
            pos += 1
            blk[r, :p] = vals[r, :p]
            blk[r, p] = anchor_bits if (r & 1) == 0 else (anchor_bits | 0x8000)
            blk[r, p + 1:] = vals[r, p:]
        blocks.append(blk)
    # maxima in the normal binades below 2**-119 (exponent fields 1..7): clamped scale
    rng = np.random.default_rng(5)
    for f in range(1, 8):
        blk = rng.integers(0, (f << 7) | 0x7F, size=(4, 32), dtype=np.uint16)
        blk[:, 3] = (f << 7) | 0x7F
        blk[1::2] |= 0x8000
        blocks.append(blk)
    # subnormal / zero / negative-zero maxima
    sub = np.arange(0, 0x80, dtype=np.uint16)
    tiny = np.concatenate([sub, sub | 0x8000, np.zeros(64 - (2 * 128) % 64, np.uint16)])
    blocks.append(tiny.reshape(-1, 32))
    blocks.append(np.zeros((2, 32), np.uint16))
    blocks.append(np.full((2, 32), 0x8000, np.uint16))
    allb = np.concatenate(blocks)
    pad = (-allb.shape[0]) % 32
    allb = np.concatenate([allb, np.zeros((pad, 32), np.uint16)])
    return allb.reshape(-1, 32 * 32)                        # rows of K = 1024


def test_mxfp8_quantize_exhaustive_bf16_values_every_exponent():
    dev = device()
    x = _exhaustive_blocks()
    log(f"exhaustive mxfp8 quantize: {x.shape[0]} rows x {x.shape[1]}")
    q, s = _run(x, dev)
    oq, os_ = oracle.quantize_mxfp8(x)
    assert np.array_equal(s, os_), "scale bytes"
    bad = np.flatnonzero(q != oq)
    assert bad.size == 0, (f"{bad.size} codes differ; first: x={x.reshape(-1)[bad[:4]]} "
                           f"got={q.reshape(-1)[bad[:4]]} want={oq.reshape(-1)[bad[:4]]}")


@pytest.mark.parametrize("rows,k,seed", [(1, 32, 0), (3, 96, 1), (7, 160, 2), (64, 1024, 3),
                                         (129, 4096, 4), (33, 14336, 5), (1000, 64, 6)])
def test_mxfp8_quantize_random_shapes(rows, k, seed):
    dev = device()
    xb = random_bf16((rows, k), seed, spread=20, outlier_frac=0.01)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    log(f"mxfp8 quantize random rows={rows} k={k}")
    q, s = _run(bits, dev)
    oq, os_ = oracle.quantize_mxfp8(bits)
    assert np.array_equal(s, os_) and np.array_equal(q, oq)


def test_mxfp8_quantize_leaves_neighbouring_memory_alone():
    dev = device()
    rows, k = 5, 96
    xb = random_bf16((rows, k), 11)
    q_all = torch.full((rows * k + 64,), 0xA5, dtype=torch.uint8, device=dev)
    s_all = torch.full((rows * k // 32 + 64,), 0x5A, dtype=torch.uint8, device=dev)
    q = q_all[: rows * k].view(rows, k)
    s = s_all[: rows * k // 32].view(rows, k // 32)
    mxfp8_quantize(xb.to(dev), q, s)
    torch.cuda.synchronize()
    assert torch.all(q_all[rows * k:] == 0xA5)
    assert torch.all(s_all[rows * k // 32:] == 0x5A)


@pytest.mark.parametrize("name", ["tiny_64x256x1024", "decode_128x14336x4096", "prefill_4096x4096x4096",
                                  "ffn_down_4096x4096x14336", "square_8192x8192x8192"])
def test_mxfp8_quantize_workload_activations(name):
    """Full-size activation operands of every dense workload, checked on sampled rows."""
    dev = device()
    w = workloads.DENSE[name]
    a, _ = w.make()
    log(f"{name}: mxfp8 quantize A {tuple(a.shape)}")
    q, s = mxfp8_quantize(a.to(dev))
    torch.cuda.synchronize()
    rows = sampled_indices(a.shape[0], 96, seed=a.shape[0])
    bits = workloads.bf16_bits(a[torch.from_numpy(rows)])
    oq, os_ = oracle.quantize_mxfp8(bits)
    assert np.array_equal(to_np(s)[rows], os_), "scales"
    assert np.array_equal(to_np(q)[rows], oq), "codes"
