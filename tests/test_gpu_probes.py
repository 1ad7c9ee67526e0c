"""GPU checks of the measurement probes (include/mxfp4_probe.h).

The read probe backs a bandwidth figure, so it must read every byte exactly
once: the XOR of its per-thread results equals the XOR of all 32-bit words of
the buffer (a byte read twice or skipped changes it, for the seeded random
contents).  The MFMA probe's result values mean nothing; it must run, be
deterministic and stay finite, and its flop count follows its definition."""
import numpy as np
import pytest
import torch

from block_scaled_fp4_mxfp4_amd import binding as B
from tests.gpu_common import device, log, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), (1 << 20, 7), (29360128, 2048),
                                           ((1 << 20) + 48, 64)])
def test_read_probe_reads_every_byte_once(nbytes, blocks):
    dev = device()
    log(f"read probe: {nbytes} bytes, {blocks} blocks")
    g = torch.Generator().manual_seed(nbytes % 1000003 + blocks)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    src = host.to(dev)
    out = torch.full((blocks * 256,), 0x5a5a5a5a, dtype=torch.int32, device=dev)
    assert B.mxfp4_probe_read(src, out, blocks) == nbytes
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(to_np(out).view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def test_mfma_probe_runs_deterministically():
    dev = device()
    blocks, iters = 8, 16
    log(f"mfma probe: {blocks} blocks x {iters} iterations")
    g = torch.Generator().manual_seed(7)
    seed = torch.randint(0, 256, (B.PROBE_SEED_BYTES,), dtype=torch.uint8, generator=g).to(dev)
    runs = []
    for _ in range(2):
        out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device=dev)
        flops = B.mxfp4_probe_mfma(seed, out, blocks, iters)
        torch.cuda.synchronize()
        runs.append(to_np(out))
    assert flops == blocks * 8 * iters * 8 * 2 * 32 * 32 * 64
    assert np.all(np.isfinite(runs[0]))
    assert np.array_equal(runs[0], runs[1])


def test_mfma_w4a8_probe_runs_deterministically():
    """FP8 operands are built with NaN codes masked off, so the sums stay finite."""
    dev = device()
    blocks, iters = 8, 16
    g = torch.Generator().manual_seed(8)
    seed = torch.randint(0, 256, (B.PROBE_SEED_BYTES,), dtype=torch.uint8, generator=g).to(dev)
    runs = []
    for _ in range(2):
        out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device=dev)
        B.mxfp4_probe_mfma(seed, out, blocks, iters, a_fp8=True)
        torch.cuda.synchronize()
        runs.append(to_np(out))
    assert np.all(np.isfinite(runs[0]))
    assert np.array_equal(runs[0], runs[1])
    # the FP8 probe computes something different from the FP4 one on the same seed
    out4 = torch.empty((blocks * 512,), dtype=torch.float32, device=dev)
    B.mxfp4_probe_mfma(seed, out4, blocks, iters)
    torch.cuda.synchronize()
    assert not np.array_equal(to_np(out4), runs[0])
