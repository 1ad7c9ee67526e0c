"""GPU MoE steps around the grouped GEMM against the CPU oracle.

* routing: expert ids bit-exact (both sides compare the same float32 logits);
  gate weights within a bound derived from fp32 arithmetic: the subtraction
  l_j - l_0 rounds by at most 2^-24 |l_j - l_0| relative, expf is within a
  few ulp, the sum of <= 8 terms and the division add <= 9 roundings, so
  |w - w_exact| <= 2^-20 (1 + |l_j - l_0|) w_exact;
* permutation: offsets, row_token and token_rows bit-exact (integer work);
* scatter-quantize: code and scale bytes bit-exact, untouched rows keep their
  poison;
* combine: fp32 output within the fused multiply-add bound
  top_k * 2^-24 * sum_j |w_j y_j| of the exact sum (the float32 weights and
  BF16 inputs taken exactly by the oracle); BF16 output equal to the
  nearest-even rounding of the kernel's own fp32 result;
* the whole layer at the MoE workload's size (route -> permute ->
  scatter-quantize -> grouped GEMM -> combine), the index work checked in
  full and the numbers on sampled tokens and columns; and a smaller layer with
  MXFP8 activations (W4A8 grouped GEMM), its scattered bytes exact and its
  outputs within 1e-2 floored max-rel of the float64 oracle (the GEMM's BF16
  output and the MFMA's FP8 group rule each add a few 2^-9 at most).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_grouped_gemm_nt, mxfp4_moe_combine, mxfp4_moe_permute,
                                        mxfp4_moe_quantize_scatter, mxfp4_moe_route, mxfp4_quantize,
                                        mxfp8_moe_quantize_scatter)
from tests.gpu_common import device, log, poisoned, random_bf16, sampled_indices, to_np, upload

pytestmark = pytest.mark.gpu


def _check_route(lg: np.ndarray, top_k: int, dev):
    ids, w = mxfp4_moe_route(upload(lg, dev), top_k)
    torch.cuda.synchronize()
    rid, rw = oracle.route_topk(lg, top_k)
    got_ids, got_w = to_np(ids), to_np(w).astype(np.float64)
    assert np.array_equal(got_ids, rid), "expert ids differ"
    sel = np.take_along_axis(lg.astype(np.float64), rid.astype(np.int64), axis=1)
    bound = 2.0 ** -20 * (1.0 + np.abs(sel - sel[:, :1])) * rw
    assert np.all(np.abs(got_w - rw) <= bound), float(np.max(np.abs(got_w - rw) / rw))


# experts % 32 == 0 takes the vector loads (64, 256, 32, 96); 16 and 48 the scalar ones
ROUTE_CASES = [(1, 1, 1), (257, 8, 2), (1000, 64, 4), (333, 200, 8), (100, 256, 8), (64, 3, 3), (50, 65, 1),
               (77, 16, 4), (129, 48, 6), (64, 32, 8), (40, 96, 5)]


@pytest.mark.parametrize("tokens,experts,top_k", ROUTE_CASES)
def test_route_matches_oracle(tokens, experts, top_k):
    dev = device()
    log(f"route T={tokens} E={experts} k={top_k}")
    rng = np.random.default_rng(tokens + experts)
    _check_route((rng.standard_normal((tokens, experts)) * 2).astype(np.float32), top_k, dev)


def test_route_ties_and_signed_zeros():
    dev = device()
    rng = np.random.default_rng(9)
    lg = rng.integers(-2, 3, size=(400, 64)).astype(np.float32)      # many equal logits
    lg[::7, :] = -0.0
    lg[::11, ::2] = 0.0
    for k in (1, 4, 8):
        log(f"route ties k={k}")
        _check_route(lg, k, dev)


def test_route_moe_workload_logits():
    dev = device()
    moe = workloads.MOE
    log(f"route {moe.name}")
    _check_route(moe.logits().numpy(), moe.top_k, dev)


PERMUTE_CASES = [(1, 1, 1, 0), (7, 3, 2, 1), (1000, 64, 4, 2), (333, 1000, 3, 3), (2049, 17, 5, 4), (4096, 64, 1, 5)]


@pytest.mark.parametrize("tokens,experts,top_k,seed", PERMUTE_CASES)
def test_permute_matches_oracle(tokens, experts, top_k, seed):
    dev = device()
    log(f"permute T={tokens} E={experts} k={top_k}")
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, experts, size=(tokens, top_k)).astype(np.int32)
    drop = rng.random((tokens, top_k)) < 0.1            # dropped entries: ids below 0 and at or past E
    ids[drop] = rng.choice(np.array([-1, -7, experts, experts + 3, 1 << 30], np.int32), size=int(drop.sum()))
    off, rt, tr = mxfp4_moe_permute(upload(ids, dev), experts)
    torch.cuda.synchronize()
    ro, rrt, rtr = oracle.permute(ids, experts)
    assert np.array_equal(to_np(off), ro)
    assert np.array_equal(to_np(rt), rrt)
    assert np.array_equal(to_np(tr), rtr)


def test_permute_no_tokens_writes_zero_offsets():
    dev = device()
    off = poisoned((9,), torch.int32, dev, 0x7F)
    mxfp4_moe_permute(torch.empty((0, 2), dtype=torch.int32, device=dev), 8, offsets=off)
    torch.cuda.synchronize()
    assert to_np(off).tolist() == [0] * 9


def test_permute_routing_of_moe_workload():
    dev = device()
    moe = workloads.MOE
    lg = moe.logits()
    ids, _ = mxfp4_moe_route(lg.to(dev), moe.top_k)
    off, rt, tr = mxfp4_moe_permute(ids, moe.experts)
    torch.cuda.synchronize()
    ro, rrt, rtr = oracle.permute(oracle.route_topk(lg.numpy(), moe.top_k)[0], moe.experts)
    assert np.array_equal(to_np(off), ro) and np.array_equal(to_np(rt), rrt) and np.array_equal(to_np(tr), rtr)
    counts = np.diff(ro)
    log(f"rows per expert min {counts.min()} max {counts.max()} empty {(counts == 0).sum()}")


# top_k > 4: the slots past the four whose rows load with the blocks
SCATTER_CASES = [(1, 32, 1, 1), (37, 96, 8, 3), (300, 1024, 64, 4), (129, 4160, 5, 2), (41, 256, 16, 6),
                 (23, 512, 12, 12)]


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("tokens,k,experts,top_k", SCATTER_CASES)
def test_quantize_scatter_bitexact(fmt, tokens, k, experts, top_k):
    dev = device()
    log(f"scatter {fmt} T={tokens} K={k} E={experts} k={top_k}")
    x = random_bf16((tokens, k), 17 + tokens, spread=8)
    rng = np.random.default_rng(tokens)
    ids = rng.integers(-1, experts, size=(tokens, top_k)).astype(np.int32)
    _, _, tr = oracle.permute(ids, experts)
    rows = tokens * top_k
    cols = k // 2 if fmt == "mxfp4" else k
    q = poisoned((rows, cols), torch.uint8, dev, 0xA5)
    s = poisoned((rows, k // 32), torch.uint8, dev, 0x5A)
    fn = mxfp4_moe_quantize_scatter if fmt == "mxfp4" else mxfp8_moe_quantize_scatter
    fn(x.to(dev), upload(tr, dev), rows, q, s)
    torch.cuda.synchronize()
    ref = oracle.quantize_scatter if fmt == "mxfp4" else oracle.quantize_scatter_mxfp8
    rq, rs, written = ref(workloads.bf16_bits(x), tr, rows)
    gq, gs = to_np(q), to_np(s)
    assert np.array_equal(gq[written], rq[written]) and np.array_equal(gs[written], rs[written])
    assert np.all(gq[~written] == 0xA5) and np.all(gs[~written] == 0x5A)


def test_quantize_scatter_equals_dense_quantizer_on_gathered_rows():
    dev = device()
    x = random_bf16((512, 2048), 3, spread=6).to(dev)
    ids = torch.from_numpy(np.random.default_rng(1).integers(0, 16, size=(512, 4)).astype(np.int32)).to(dev)
    off, rt, tr = mxfp4_moe_permute(ids, 16)
    q, s = mxfp4_moe_quantize_scatter(x, tr, 2048)
    gq, gs = mxfp4_quantize(x[rt.long()].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(q, gq) and torch.equal(s, gs)


def _check_combine(y_bits, tr, w, dev):
    total, n = y_bits.shape
    y = upload(y_bits.view(np.int16), dev).view(torch.bfloat16)
    out32 = mxfp4_moe_combine(y, upload(tr, dev), upload(w, dev), out_dtype=torch.float32)
    out16 = mxfp4_moe_combine(y, upload(tr, dev), upload(w, dev), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.combine(y_bits, tr, w)
    scale = oracle.combine_abs(y_bits, tr, w)
    got = to_np(out32).astype(np.float64)
    top_k = tr.shape[1]
    assert np.all(np.abs(got - ref) <= top_k * 2.0 ** -24 * scale + 2.0 ** -140)
    assert np.array_equal(to_np(out16.view(torch.int16)).view(np.uint16), oracle.f64_to_bf16_bits(got))


# top_k > 8: more than one group of slots loaded together, the last one partial
COMBINE_CASES = [(1, 8, 1, 1), (300, 64, 4, 64), (97, 100, 3, 7), (1000, 2816, 4, 64), (5, 1, 2, 3), (33, 200, 12, 16), (11, 100, 10, 12),
                 (9, 72, 20, 24)]


@pytest.mark.parametrize("tokens,n,top_k,experts", COMBINE_CASES)
def test_combine_within_fma_bound(tokens, n, top_k, experts):
    dev = device()
    log(f"combine T={tokens} N={n} k={top_k}")
    rng = np.random.default_rng(n + tokens)
    ids = rng.integers(-1, experts, size=(tokens, top_k)).astype(np.int32)
    _, _, tr = oracle.permute(ids, experts)
    rows = tokens * top_k
    wide = (n + 31) // 32 * 32
    y = workloads.bf16_bits(random_bf16((rows, wide), 5 + n, spread=5)[:, :n].contiguous())
    w = rng.random((tokens, top_k)).astype(np.float32)
    _check_combine(np.ascontiguousarray(y), tr, w, dev)


def test_moe_layer_full_size_sampled():
    """route -> permute -> scatter-quantize -> grouped GEMM -> combine at the MoE workload's size."""
    dev = device()
    moe = workloads.MOE
    log(f"moe layer {moe.name}")
    x = moe.tokens_bf16()
    lg = moe.logits()
    w_bf16 = workloads.gaussian_bf16((moe.experts * moe.n, moe.k), moe.w_sigma, moe.seed + workloads.ROLE_B)
    wq, ws = mxfp4_quantize(w_bf16.to(dev))
    wq = wq.view(moe.experts, moe.n, moe.k // 2)
    ws = ws.view(moe.experts, moe.n, moe.k // 32)
    rows = moe.tokens * moe.top_k
    ids, gate = mxfp4_moe_route(lg.to(dev), moe.top_k)
    off, rt, tr = mxfp4_moe_permute(ids, moe.experts)
    aq, as_ = mxfp4_moe_quantize_scatter(x.to(dev), tr, rows)
    y = mxfp4_grouped_gemm_nt(aq, as_, wq, ws, off)
    out = mxfp4_moe_combine(y, tr, gate)
    torch.cuda.synchronize()
    # index work in full
    rid, rgate = oracle.route_topk(lg.numpy(), moe.top_k)
    ro, rrt, rtr = oracle.permute(rid, moe.experts)
    assert np.array_equal(to_np(ids), rid) and np.array_equal(to_np(off), ro)
    assert np.array_equal(to_np(rt), rrt) and np.array_equal(to_np(tr), rtr)
    # numbers on sampled tokens and columns: exact fp64 expert outputs from the oracle's
    # own quantization of the sampled token rows and weight rows
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.choice(moe.tokens, 12, replace=False), [0, moe.tokens - 1]]))
    cols = np.unique(np.concatenate([rng.choice(moe.n, 48, replace=False), [0, moe.n - 1]]))
    xq, xs = oracle.quantize(workloads.bf16_bits(x[toks]))
    gq, gs = to_np(aq), to_np(as_)
    got = to_np(out.float()).astype(np.float64)
    wb = w_bf16.view(moe.experts, moe.n, moe.k)
    for i, t in enumerate(toks):
        ref = np.zeros(len(cols))
        for j in range(moe.top_k):
            e, r = int(rid[t, j]), int(rtr[t, j])
            assert np.array_equal(gq[r], xq[i]) and np.array_equal(gs[r], xs[i]), f"row {r} of token {t}"
            eq, es = oracle.quantize(workloads.bf16_bits(wb[e, torch.from_numpy(cols)]))
            ref += rgate[t, j] * oracle.gemm_nt(xq[i:i + 1], xs[i:i + 1], eq, es)[0]
        err = oracle.floored_max_rel(got[t, cols], ref)
        assert err <= 1e-2, f"token {t}: floored max-rel {err}"


def test_w4a8_moe_layer_sampled():
    """The same layer with MXFP8 activations: route -> permute -> MXFP8 scatter-quantize ->
    W4A8 grouped GEMM -> combine, on a 1024-token, 16-expert layer."""
    from block_scaled_fp4_mxfp4_amd import mxfp8_grouped_gemm_w4a8_nt
    dev = device()
    tokens, experts, top_k, n, k = 1024, 16, 2, 256, 1024
    log(f"w4a8 moe layer T={tokens} E={experts} k={top_k} N={n} K={k}")
    x = workloads.activation_bf16(tokens, k, 950, outliers=True)
    lg = workloads.gaussian_bf16((tokens, experts), 1.5, 951).float()
    w = workloads.gaussian_bf16((experts * n, k), 0.02, 952)
    wq, ws = mxfp4_quantize(w.to(dev))
    wq, ws = wq.view(experts, n, k // 2), ws.view(experts, n, k // 32)
    rows = tokens * top_k
    ids, gate = mxfp4_moe_route(lg.to(dev), top_k)
    off, rt, tr = mxfp4_moe_permute(ids, experts)
    aq, as_ = mxfp8_moe_quantize_scatter(x.to(dev), tr, rows)
    y = mxfp8_grouped_gemm_w4a8_nt(aq, as_, wq, ws, off)
    out = mxfp4_moe_combine(y, tr, gate, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rid, rgate = oracle.route_topk(lg.numpy(), top_k)
    ro, rrt, rtr = oracle.permute(rid, experts)
    assert np.array_equal(to_np(ids), rid) and np.array_equal(to_np(off), ro) and np.array_equal(to_np(tr), rtr)
    rq, rs, written = oracle.quantize_scatter_mxfp8(workloads.bf16_bits(x), rtr, rows)
    assert written.all() and np.array_equal(to_np(aq), rq) and np.array_equal(to_np(as_), rs)
    # float64 reference from the oracle's own operands: per token, the gate-weighted expert outputs
    wq_np, ws_np = to_np(wq), to_np(ws)
    toks = sampled_indices(tokens, 24, 12)
    got = to_np(out).astype(np.float64)
    for t in toks:
        ref = np.zeros(n)
        for j in range(top_k):
            e, r = int(rid[t, j]), int(rtr[t, j])
            ref += rgate[t, j] * oracle.gemm_w4a8_nt(rq[r:r + 1], rs[r:r + 1], wq_np[e], ws_np[e])[0]
        assert oracle.floored_max_rel(got[t], ref) <= 1e-2, f"token {t}"
