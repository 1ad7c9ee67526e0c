"""Helpers shared by the GPU parity tests (inputs, oracle comparisons, poisoning)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from block_scaled_fp4_mxfp4_amd import load_library
    load_library()            # raises if the HIP library is missing: no fallback exists
    return torch.device("cuda", 0)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_from_np_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def random_bf16(shape, seed, spread=4, outlier_frac=0.0):
    """Gaussian BF16 test data whose 32-blocks span 2**-spread .. 2**spread in magnitude."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if spread:
        rows, k = shape
        e = torch.randint(-spread, spread + 1, (rows, k // 32, 1), generator=g).float()
        x = (x.view(rows, k // 32, 32) * torch.exp2(e)).view(rows, k)
    if outlier_frac:
        k = shape[1]
        ch = torch.randperm(k, generator=g)[: max(1, int(k * outlier_frac))]
        x[:, ch] *= 20
    return x.to(torch.bfloat16)


def random_codes(rows, k, seed, lo=120, hi=134):
    """Random MXFP4 operand bytes (every code pattern, scale bytes in [lo, hi])."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    s = rng.integers(lo, hi + 1, size=(rows, k // 32), dtype=np.uint8)
    return q, s


def upload(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def poisoned(shape, dtype, dev, byte: int) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=dev)
    t.view(torch.uint8).fill_(byte)
    return t


def assert_bf16_matches_rounded(c_bf16: np.ndarray, c64: np.ndarray, tol_rel_rms: float = 1e-5):
    """BF16 output equals RNE_bf16 of the exact result, except where the exact
    result lies within tol * rms of a BF16 rounding midpoint (there any fp32
    summation order may round either way)."""
    want = oracle.round_output_bf16(c64)
    got = np.ascontiguousarray(c_bf16).view(np.uint16)
    bad = got != want
    if not bad.any():
        return
    rms = float(np.sqrt(np.mean(c64 * c64))) or 1.0
    # midpoint between the two candidates nearest to c64
    lo = oracle.bf16_bits_to_f64(want[bad])
    hi = oracle.bf16_bits_to_f64(got[bad])
    mid = (lo + hi) / 2
    near = np.abs(c64[bad] - mid) <= tol_rel_rms * rms
    one_ulp = np.abs(got[bad].astype(np.int32) - want[bad].astype(np.int32)) == 1
    assert np.all(near & one_ulp), (
        f"{int((~(near & one_ulp)).sum())} BF16 outputs differ from the rounded exact result "
        f"away from rounding midpoints")


def sampled_indices(n: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(n, size=min(count, n), replace=False)
    edges = np.array([0, n - 1])
    return np.unique(np.concatenate([pick, edges]))
