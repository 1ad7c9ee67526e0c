"""Seeded random shapes and values through the quantizers, the fused producers
and the MoE routing plumbing, against the CPU oracle.

The other tests pick shapes and values by hand; these draw them: ragged row
counts, K a multiple of 32 (512 for the prepacked layout), BF16 inputs mixing
Gaussian blocks at random exponents, raw random finite bit patterns, zero and
subnormal blocks; MoE token counts, expert counts and top-k drawn together
with dropped routing entries.  Bars as in the hand-picked suites: quantizer
codes, scale bytes and global scales bit-exact; RMSNorm and SwiGLU outputs the
nearest BF16 of the float64 value outside each kernel's stated midpoint window,
their MXFP4 bytes exact; routing ids, offsets and row maps exact, gate weights
and the combine within their stated bounds; nothing written outside the
outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_moe_permute, mxfp4_moe_quantize_scatter, mxfp4_prepacked_weight_size,
                                        mxfp4_quantize, mxfp4_quantize_prepacked, mxfp4_rmsnorm_quantize,
                                        mxfp4_swiglu_quantize, mxfp8_moe_quantize_scatter, mxfp8_quantize,
                                        nvfp4_quantize)
from tests.gpu_common import bf16_from_np_bits, device, log, poisoned, random_bf16, to_np, upload
from tests.test_gpu_moe import _check_combine, _check_route
from tests.test_gpu_producers import _assert_nearest_or_midpoint, _gate_up, _silu_window

pytestmark = pytest.mark.gpu


def _random_bits(rows, k, seed):
    """Finite BF16 bit patterns, one regime per 32-block: Gaussian at a random
    exponent in [-133, 120], raw random finite patterns, all zeros, one nonzero
    element among signed zeros."""
    rng = np.random.default_rng(seed)
    blocks = rows * (k // 32)
    g = rng.standard_normal((blocks, 32)) * np.exp2(rng.integers(-133, 121, size=(blocks, 1)))
    out = workloads.bf16_bits(torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16))
    raw = rng.integers(0, 1 << 16, size=(blocks, 32), dtype=np.uint32).astype(np.uint16)
    raw[(raw & 0x7F80) == 0x7F80] &= 0xBFFF                     # exponent field 255 (Inf/NaN) cleared to finite
    regime = rng.choice(4, size=blocks, p=[0.6, 0.25, 0.05, 0.1])
    out[regime == 1] = raw[regime == 1]
    out[regime == 2] = 0
    single = np.flatnonzero(regime == 3)
    out[single] = rng.choice(np.array([0x0000, 0x8000], np.uint16), size=(single.size, 32))
    out[single, rng.integers(0, 32, size=single.size)] = raw[single, 0]
    return np.ascontiguousarray(out.reshape(rows, k))


def _quant_shapes(seed, count, k_unit, k_max):
    rng = np.random.default_rng(seed)
    return [(int(np.exp(rng.uniform(0, np.log(600)))), int(rng.integers(1, k_max // k_unit + 1)) * k_unit)
            for _ in range(count)]


@pytest.mark.parametrize("rows,k", _quant_shapes(31, 12, 32, 8192))
def test_random_quantizers_bitexact(rows, k):
    """MXFP4, MXFP8 and NVFP4 quantizers on the same random input, each byte
    for byte against the oracle, with a poisoned row past each output."""
    dev = device()
    log(f"random quantizers rows={rows} k={k}")
    bits = _random_bits(rows, k, rows * 13 + k)
    x = bf16_from_np_bits(bits).to(dev)
    q4, s4 = poisoned((rows + 1, k // 2), torch.uint8, dev, 0xA5), poisoned((rows + 1, k // 32), torch.uint8, dev, 0x5A)
    q8, s8 = poisoned((rows + 1, k), torch.uint8, dev, 0xA5), poisoned((rows + 1, k // 32), torch.uint8, dev, 0x5A)
    mxfp4_quantize(x, q4[:rows], s4[:rows])
    mxfp8_quantize(x, q8[:rows], s8[:rows])
    qn = poisoned((rows + 1, k // 2), torch.uint8, dev, 0xA5)
    sn = poisoned((rows + 1, k // 16), torch.uint8, dev, 0x5A)
    gn = poisoned((rows + 1,), torch.float32, dev, 0xA5)
    nvfp4_quantize(x, qn[:rows], sn[:rows], gn[:rows])
    torch.cuda.synchronize()
    checks = [(q4, s4, oracle.quantize(bits)), (q8, s8, oracle.quantize_mxfp8(bits))]
    for q, s, (rq, rs) in checks:
        gq, gs = to_np(q), to_np(s)
        assert np.all(gq[rows] == 0xA5) and np.all(gs[rows] == 0x5A), "write past the end of the output"
        assert np.array_equal(gs[:rows], rs), "scale bytes"
        assert np.array_equal(gq[:rows], rq), "code bytes"
    rq, rs, rg = oracle.quantize_nvfp4(bits)
    gg = to_np(gn).view(np.uint32)
    assert gg[rows] == 0xA5A5A5A5 and np.all(to_np(sn)[rows] == 0x5A) and np.all(to_np(qn)[rows] == 0xA5)
    assert np.array_equal(gg[:rows], rg.view(np.uint32)), "NVFP4 global scales"
    assert np.array_equal(to_np(sn)[:rows], rs) and np.array_equal(to_np(qn)[:rows], rq), "NVFP4 bytes"


@pytest.mark.parametrize("rows,k", _quant_shapes(32, 8, 512, 8192))
def test_random_quantize_prepacked_is_the_layout_of_the_oracle_bytes(rows, k):
    """The prepacked quantizer equals the prepacked layout (built on the host
    from its definition) of the oracle's row-major bytes, padding included."""
    from tests.prepack_layout import prepack_numpy
    dev = device()
    log(f"random prepacked quantizer rows={rows} k={k}")
    bits = _random_bits(rows, k, rows * 17 + k)
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    pq, ps = poisoned((cb,), torch.uint8, dev, 0x77), poisoned((sb,), torch.uint8, dev, 0x77)
    mxfp4_quantize_prepacked(bf16_from_np_bits(bits).to(dev), pq, ps)
    torch.cuda.synchronize()
    wq, ws = prepack_numpy(*oracle.quantize(bits))
    assert np.array_equal(to_np(pq), wq) and np.array_equal(to_np(ps), ws)


def _producer_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        rows = int(np.exp(rng.uniform(0, np.log(300))))
        k = int(rng.integers(1, 8192 // 32 + 1)) * 32
        out.append((rows, k, bool(rng.random() < 0.6), float(rng.choice([0.0, 1e-6, 1e-5, 0.25])),
                    int(rng.integers(1, 9))))
    return out


@pytest.mark.parametrize("rows,k,with_res,eps,spread", _producer_cases(33, 12))
def test_random_rmsnorm_quantize(rows, k, with_res, eps, spread):
    dev = device()
    log(f"random rmsnorm rows={rows} k={k} residual={with_res} eps={eps} spread={spread}")
    x = random_bf16((rows, k), rows + 3 * k, spread=spread, outlier_frac=0.01)
    res = random_bf16((rows, k), rows + 5 * k, spread=spread)
    gamma = (torch.randn(k, generator=torch.Generator().manual_seed(rows + k)) * 0.5).to(torch.bfloat16)
    xd, gd = x.to(dev), gamma.to(dev)
    resd = res.to(dev) if with_res else None
    h_out = poisoned((rows + 1, k), torch.bfloat16, dev, 0x7F) if with_res else None
    y = poisoned((rows + 1, k), torch.bfloat16, dev, 0x7F)
    q = poisoned((rows + 1, k // 2), torch.uint8, dev, 0xA5)
    s = poisoned((rows + 1, k // 32), torch.uint8, dev, 0x5A)
    mxfp4_rmsnorm_quantize(xd, gd, eps, residual=resd, residual_out=h_out[:rows] if with_res else None,
                           y=y[:rows], q=q[:rows], scales=s[:rows])
    torch.cuda.synchronize()
    for t, byte in ((y, 0x7F), (q, 0xA5), (s, 0x5A)) + (((h_out, 0x7F),) if with_res else ()):
        assert np.all(to_np(t[rows:].view(torch.uint8)) == byte), "write past the end of an output"
    hb = oracle.add_residual(workloads.bf16_bits(x), workloads.bf16_bits(res)) if with_res else workloads.bf16_bits(x)
    if with_res:
        assert np.array_equal(workloads.bf16_bits(h_out[:rows].cpu()), hb)
    yb = workloads.bf16_bits(y[:rows].cpu())
    _assert_nearest_or_midpoint(yb, oracle.rmsnorm_f64(hb, workloads.bf16_bits(gamma), eps), 2.0 ** -40)
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q[:rows]), rq) and np.array_equal(to_np(s[:rows]), rs)


@pytest.mark.parametrize("rows,k,_res,_eps,pad", _producer_cases(34, 12))
def test_random_swiglu_quantize(rows, k, _res, _eps, pad):
    """Gate and up read from one buffer with a random row stride ld >= k
    (ld % 8 == 0)."""
    dev = device()
    ld = k + 8 * pad * (pad % 3)
    log(f"random swiglu rows={rows} k={k} ld={ld}")
    gate, up, gate_c, up_c = _gate_up(rows, k, ld, rows * 7 + k, dev)
    y = poisoned((rows + 1, k), torch.bfloat16, dev, 0x7F)
    q = poisoned((rows + 1, k // 2), torch.uint8, dev, 0xA5)
    s = poisoned((rows + 1, k // 32), torch.uint8, dev, 0x5A)
    mxfp4_swiglu_quantize(gate, up, y=y[:rows], q=q[:rows], scales=s[:rows])
    torch.cuda.synchronize()
    for t, byte in ((y, 0x7F), (q, 0xA5), (s, 0x5A)):
        assert np.all(to_np(t[rows:].view(torch.uint8)) == byte), "write past the end of an output"
    yb = workloads.bf16_bits(y[:rows].cpu())
    _assert_nearest_or_midpoint(yb, oracle.swiglu_f64(workloads.bf16_bits(gate_c), workloads.bf16_bits(up_c)),
                                _silu_window(gate_c))
    rq, rs = oracle.quantize(yb)
    assert np.array_equal(to_np(q[:rows]), rq) and np.array_equal(to_np(s[:rows]), rs)


def _moe_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        experts = int(rng.integers(1, 257))
        top_k = int(rng.integers(1, min(8, experts) + 1))
        tokens = int(np.exp(rng.uniform(0, np.log(1500))))
        k = int(rng.integers(1, 64 + 1)) * 32
        n = int(rng.integers(1, 700))
        out.append((tokens, experts, top_k, k, n))
    return out


@pytest.mark.parametrize("tokens,experts,top_k,k,n", _moe_cases(35, 12))
def test_random_moe_plumbing(tokens, experts, top_k, k, n):
    """Routing, permutation, the MXFP4 and MXFP8 scatter-quantizers and the
    weighted combine on one random draw: routing on random logits (ties
    included), the permutation on the routed ids with about a tenth of the
    entries dropped (ids below 0 or at or past the expert count)."""
    dev = device()
    log(f"random moe T={tokens} E={experts} k={top_k} K={k} N={n}")
    rng = np.random.default_rng(tokens * 3 + experts * 5 + top_k)
    lg = (rng.standard_normal((tokens, experts)) * 2).astype(np.float32)
    tie = rng.random(tokens) < 0.2
    lg[tie] = np.round(lg[tie, :1])                                   # whole rows of equal logits
    _check_route(lg, top_k, dev)

    ids, _ = oracle.route_topk(lg, top_k)
    ids = ids.astype(np.int32)
    drop = rng.random(ids.shape) < 0.1
    ids[drop] = rng.choice(np.array([-1, -5, experts, experts + 9], np.int32), size=int(drop.sum()))
    off, rt, tr = mxfp4_moe_permute(upload(ids, dev), experts)
    torch.cuda.synchronize()
    ro, rrt, rtr = oracle.permute(ids, experts)
    assert np.array_equal(to_np(off), ro) and np.array_equal(to_np(rt), rrt) and np.array_equal(to_np(tr), rtr)

    rows = tokens * top_k
    x = random_bf16((tokens, k), tokens + k, spread=8, outlier_frac=0.01)
    for fmt, fn, ref in (("mxfp4", mxfp4_moe_quantize_scatter, oracle.quantize_scatter),
                         ("mxfp8", mxfp8_moe_quantize_scatter, oracle.quantize_scatter_mxfp8)):
        cols = k // 2 if fmt == "mxfp4" else k
        q = poisoned((rows, cols), torch.uint8, dev, 0xA5)
        s = poisoned((rows, k // 32), torch.uint8, dev, 0x5A)
        fn(x.to(dev), tr, rows, q, s)
        torch.cuda.synchronize()
        rq, rs, written = ref(workloads.bf16_bits(x), rtr, rows)
        gq, gs = to_np(q), to_np(s)
        assert np.array_equal(gq[written], rq[written]) and np.array_equal(gs[written], rs[written]), fmt
        assert np.all(gq[~written] == 0xA5) and np.all(gs[~written] == 0x5A), fmt

    wide = (n + 31) // 32 * 32
    y = workloads.bf16_bits(random_bf16((rows, wide), rows + n, spread=5)[:, :n].contiguous())
    w = rng.random((tokens, top_k)).astype(np.float32)
    _check_combine(np.ascontiguousarray(y), rtr, w, dev)
