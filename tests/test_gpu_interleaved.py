"""GPU entry points on the interleaved scale layout ([k/512, rows, 16] per
operand): the interleaving kernel and the interleaved quantizers byte for byte
against the layout's host definition applied to the oracle's (or the row-major
kernel's) bytes; the dense and grouped GEMMs on interleaved scales bit for bit
against the same tile kernels on row-major scales (fp32 and BF16 outputs) and
within floored max-rel 1e-5 of the float64 oracle; the whole MoE layer through
the interleaved steps equal to the row-major layer."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (mxfp4_gemm_nt, mxfp4_gemm_nt_interleaved, mxfp4_grouped_gemm_nt,
                                        mxfp4_grouped_gemm_nt_interleaved, mxfp4_moe_combine, mxfp4_moe_permute,
                                        mxfp4_moe_quantize_scatter, mxfp4_moe_quantize_scatter_interleaved,
                                        mxfp4_moe_route, mxfp4_quantize, mxfp4_quantize_interleaved,
                                        mxfp4_scales_interleave)
from tests.gpu_common import (bf16_from_np_bits, device, log, poisoned, random_bf16, random_codes, sampled_indices,
                              to_np, upload)
from tests.scale_layout import interleave_numpy
from tests.test_gpu_random_shapes_producers import _random_bits

pytestmark = pytest.mark.gpu


def _with_canary(shape, dtype, dev, byte, extra=256):
    """A poisoned buffer of the given shape followed by `extra` poisoned bytes."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    flat = poisoned((n + extra,), torch.uint8, dev, byte)
    return flat, flat[:n].view(dtype).view(shape)


QUANT_CASES = [(1, 512), (3, 1024), (64, 4096), (100, 1536), (257, 8192), (1000, 512)]


@pytest.mark.parametrize("rows,k", QUANT_CASES)
def test_quantize_interleaved_is_the_layout_of_the_oracle_bytes(rows, k):
    dev = device()
    log(f"interleaved quantize rows={rows} k={k}")
    bits = _random_bits(rows, k, rows * 3 + k)
    qf, q = _with_canary((rows, k // 2), torch.uint8, dev, 0xA5)
    sf, s = _with_canary((k // 512, rows, 16), torch.uint8, dev, 0x5A)
    mxfp4_quantize_interleaved(bf16_from_np_bits(bits).to(dev), q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize(bits)
    assert np.array_equal(to_np(q), rq), "code bytes"
    assert np.array_equal(to_np(s), interleave_numpy(rs)), "interleaved scale bytes"
    assert np.all(to_np(qf)[q.numel():] == 0xA5) and np.all(to_np(sf)[s.numel():] == 0x5A), "write past the end"


@pytest.mark.parametrize("groups,rows,k", [(1, 1, 512), (1, 300, 2048), (5, 64, 1024), (64, 45, 4096), (3, 1000, 512)])
def test_scales_interleave_kernel(groups, rows, k):
    dev = device()
    log(f"scale interleave groups={groups} rows={rows} k={k}")
    s = np.random.default_rng(groups * rows + k).integers(0, 256, size=(groups, rows, k // 32), dtype=np.uint8)
    of, out = _with_canary((groups, k // 512, rows, 16), torch.uint8, dev, 0x77)
    mxfp4_scales_interleave(upload(s, dev), out=out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), interleave_numpy(s))
    assert np.all(to_np(of)[out.numel():] == 0x77)
    if groups == 1:   # the 2-D form
        out2 = mxfp4_scales_interleave(upload(s[0], dev))
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out2), interleave_numpy(s[0]))


def _tile_kernel_for(m, n, num_cus):
    # the interleaved dense entry point's tile choice
    return "tile256" if ((m + 255) // 256) * ((n + 255) // 256) >= num_cus else "tile128"


GEMM_CASES = [(1, 64, 512), (17, 300, 1536), (300, 257, 1024), (513, 700, 4096), (1000, 1000, 2048),
              (4096, 4096, 4096), (4100, 4000, 1024)]


@pytest.mark.parametrize("m,n,k", GEMM_CASES)
def test_gemm_interleaved_equals_row_major_tile_kernel(m, n, k):
    dev = device()
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    kernel = _tile_kernel_for(m, n, num_cus)
    log(f"interleaved gemm m={m} n={n} k={k} ({kernel})")
    aq, as_ = random_codes(m, k, m + 2 * k)
    bq, bs = random_codes(n, k, n + 3 * k)
    d_aq, d_as, d_bq, d_bs = (upload(t, dev) for t in (aq, as_, bq, bs))
    d_as_il, d_bs_il = mxfp4_scales_interleave(d_as), mxfp4_scales_interleave(d_bs)
    for dt in (torch.float32, torch.bfloat16):
        cf, c = _with_canary((m, n), dt, dev, 0xFF)
        mxfp4_gemm_nt_interleaved(d_aq, d_as_il, d_bq, d_bs_il, c=c)
        ref = mxfp4_gemm_nt(d_aq, d_as, d_bq, d_bs, out_dtype=dt, kernel=kernel)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.uint8), ref.view(torch.uint8)), f"{dt} differs from the row-major kernel"
        assert np.all(to_np(cf)[c.numel() * c.element_size():] == 0xFF), "write past the end of C"
        if dt == torch.float32:
            idx = sampled_indices(m, 24, m + n) if m * n * k > (1 << 31) else np.arange(m)
            assert oracle.floored_max_rel(to_np(c)[idx], oracle.gemm_nt(aq[idx], as_[idx], bq, bs)) <= 1e-5


GROUP_CASES = {
    "all_rows_one_expert": ([0, 0, 517, 0], 130, 512),
    "empty_first_middle_last": ([0, 40, 0, 129, 0], 96, 1024),
    "tile_boundaries_256": ([255, 256, 257, 511, 1], 256, 512),
    "ragged_k_1536": ([33, 70, 5, 300], 72, 1536),
    "persistent_ragged": ([0, 255, 256, 257, 511, 1, 700, 0], 200, 1024),
    "persistent_many_tiles": (list(np.random.default_rng(1).integers(0, 600, size=32)), 1536, 2048),
    "persistent_ragged_n": ([300, 0, 600, 45, 256, 1000], 600, 1024),
}


@pytest.mark.parametrize("name", list(GROUP_CASES))
def test_grouped_interleaved_equals_row_major(name):
    dev = device()
    counts, n, k = GROUP_CASES[name]
    counts = np.asarray(counts)
    groups, total = len(counts), int(np.sum(counts))
    log(f"interleaved grouped {name}: {groups} groups, {total} rows, n={n} k={k}")
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    aq, as_ = random_codes(total, k, total + k)
    wq, ws = random_codes(groups * n, k, groups + n + k)
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    d_wq = upload(wq, dev).view(groups, n, k // 2)
    d_ws = upload(ws, dev).view(groups, n, k // 32)
    d_off = upload(offsets, dev)
    d_as_il, d_ws_il = mxfp4_scales_interleave(d_as), mxfp4_scales_interleave(d_ws)
    for dt in (torch.float32, torch.bfloat16):
        cf, c = _with_canary((total, n), dt, dev, 0xFF)
        mxfp4_grouped_gemm_nt_interleaved(d_aq, d_as_il, d_wq, d_ws_il, d_off, c=c)
        ref = mxfp4_grouped_gemm_nt(d_aq, d_as, d_wq, d_ws, d_off, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.uint8), ref.view(torch.uint8)), f"{dt} differs from the row-major grouped GEMM"
        assert np.all(to_np(cf)[c.numel() * c.element_size():] == 0xFF), "write past the end of C"
    c32 = mxfp4_grouped_gemm_nt_interleaved(d_aq, d_as_il, d_wq, d_ws_il, d_off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = to_np(c32)
    for g in range(groups):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            r = lo + np.unique(np.random.default_rng(g).choice(hi - lo, size=min(8, hi - lo), replace=False))
            ref64 = oracle.gemm_nt(aq[r], as_[r], wq[g * n:(g + 1) * n], ws[g * n:(g + 1) * n])
            assert oracle.floored_max_rel(got[r], ref64) <= 1e-5, f"group {g}"


def test_grouped_interleaved_malformed_offsets_equal_row_major():
    """Offsets that decrease or leave [0, total_m] are sanitized the same way on
    both layouts: identical outputs, nothing written past C."""
    dev = device()
    total, groups, n, k = 700, 6, 256, 1024
    aq, as_ = random_codes(total, k, 5)
    wq, ws = random_codes(groups * n, k, 6)
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    d_wq = upload(wq, dev).view(groups, n, k // 2)
    d_ws = upload(ws, dev).view(groups, n, k // 32)
    d_as_il, d_ws_il = mxfp4_scales_interleave(d_as), mxfp4_scales_interleave(d_ws)
    for off in ([0, 300, 200, 650, 9000, -4, 700], [50, 50, 600, 600, 700, 700, 680]):
        log(f"interleaved grouped, offsets {off}")
        d_off = upload(np.asarray(off, np.int32), dev)
        cf, c = _with_canary((total, n), torch.float32, dev, 0x7F)
        rf, r = _with_canary((total, n), torch.float32, dev, 0x7F)
        mxfp4_grouped_gemm_nt_interleaved(d_aq, d_as_il, d_wq, d_ws_il, d_off, c=c)
        mxfp4_grouped_gemm_nt(d_aq, d_as, d_wq, d_ws, d_off, c=r)
        torch.cuda.synchronize()
        assert torch.equal(cf, rf)


@pytest.mark.parametrize("tokens,k,experts,top_k", [(1, 512, 1, 1), (37, 1024, 8, 3), (300, 4096, 64, 4),
                                                    (129, 1536, 5, 2)])
def test_scatter_interleaved_is_the_layout_of_the_row_major_scatter(tokens, k, experts, top_k):
    dev = device()
    log(f"interleaved scatter T={tokens} K={k} E={experts} k={top_k}")
    x = random_bf16((tokens, k), 17 + tokens, spread=8).to(dev)
    ids = np.random.default_rng(tokens).integers(-1, experts, size=(tokens, top_k)).astype(np.int32)
    _, _, tr = mxfp4_moe_permute(upload(ids, dev), experts)
    rows = tokens * top_k
    q1 = poisoned((rows, k // 2), torch.uint8, dev, 0xA5)
    s1 = poisoned((rows, k // 32), torch.uint8, dev, 0x5A)
    q2 = poisoned((rows, k // 2), torch.uint8, dev, 0xA5)
    sf, s2 = _with_canary((k // 512, rows, 16), torch.uint8, dev, 0x5A)
    mxfp4_moe_quantize_scatter(x, tr, rows, q1, s1)
    mxfp4_moe_quantize_scatter_interleaved(x, tr, rows, q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2)
    assert np.array_equal(to_np(s2), interleave_numpy(to_np(s1)))   # untouched rows keep the poison on both
    assert np.all(to_np(sf)[s2.numel():] == 0x5A)


def test_moe_layer_interleaved_equals_row_major():
    """The MoE workload's layer with the interleaved scatter-quantize and grouped
    GEMM (weights' scales interleaved once) gives the row-major layer's bits."""
    dev = device()
    moe = workloads.MOE
    log(f"moe layer {moe.name}, interleaved vs row-major")
    x = moe.tokens_bf16().to(dev)
    w_bf16 = workloads.gaussian_bf16((moe.experts * moe.n, moe.k), moe.w_sigma, moe.seed + workloads.ROLE_B)
    wq, ws = mxfp4_quantize(w_bf16.to(dev))
    del w_bf16
    wq = wq.view(moe.experts, moe.n, moe.k // 2)
    ws = ws.view(moe.experts, moe.n, moe.k // 32)
    ws_il = mxfp4_scales_interleave(ws)
    rows = moe.tokens * moe.top_k
    ids, gate = mxfp4_moe_route(moe.logits().to(dev), moe.top_k)
    off, _, tr = mxfp4_moe_permute(ids, moe.experts)
    aq, as_ = mxfp4_moe_quantize_scatter(x, tr, rows)
    out = mxfp4_moe_combine(mxfp4_grouped_gemm_nt(aq, as_, wq, ws, off), tr, gate)
    aq2, as_il = mxfp4_moe_quantize_scatter_interleaved(x, tr, rows)
    out2 = mxfp4_moe_combine(mxfp4_grouped_gemm_nt_interleaved(aq2, as_il, wq, ws_il, off), tr, gate)
    torch.cuda.synchronize()
    assert torch.equal(aq, aq2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


PRODUCER_CASES = [(1, 512, True), (37, 1536, False), (130, 4096, True), (64, 14336, False)]


@pytest.mark.parametrize("rows,k,with_res", PRODUCER_CASES)
def test_rmsnorm_interleaved_equals_row_major(rows, k, with_res):
    """Same BF16 outputs and codes as the row-major producer; scales = its scales interleaved."""
    from block_scaled_fp4_mxfp4_amd import mxfp4_rmsnorm_quantize
    dev = device()
    log(f"interleaved rmsnorm rows={rows} k={k} residual={with_res}")
    x = random_bf16((rows, k), 60 + k, spread=5, outlier_frac=0.01).to(dev)
    res = random_bf16((rows, k), 61 + k, spread=5).to(dev) if with_res else None
    gamma = (1.0 + 0.2 * torch.randn(k, generator=torch.Generator().manual_seed(k))).to(torch.bfloat16).to(dev)
    outs = []
    for il in (False, True):
        h = torch.empty((rows, k), dtype=torch.bfloat16, device=dev) if with_res else None
        y = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
        if il:
            sf, s = _with_canary((k // 512, rows, 16), torch.uint8, dev, 0x5A)
            q, s = mxfp4_rmsnorm_quantize(x, gamma, 1e-5, residual=res, residual_out=h, y=y, scales=s, interleaved=True)
        else:
            q, s = mxfp4_rmsnorm_quantize(x, gamma, 1e-5, residual=res, residual_out=h, y=y)
        outs.append((q, s, h, y))
    torch.cuda.synchronize()
    (q1, s1, h1, y1), (q2, s2, h2, y2) = outs
    assert torch.equal(q1, q2) and torch.equal(y1, y2) and (not with_res or torch.equal(h1, h2))
    assert np.array_equal(to_np(s2), interleave_numpy(to_np(s1)))
    assert np.all(to_np(sf)[s2.numel():] == 0x5A)


@pytest.mark.parametrize("rows,k,with_ld", [(1, 512, False), (37, 1536, True), (130, 4096, False), (64, 14336, True)])
def test_swiglu_interleaved_equals_row_major(rows, k, with_ld):
    from block_scaled_fp4_mxfp4_amd import mxfp4_swiglu_quantize
    dev = device()
    log(f"interleaved swiglu rows={rows} k={k}")
    ld = 2 * k + (64 if with_ld else 0)
    g = torch.Generator().manual_seed(rows + k)
    base = (torch.randn(rows, ld, generator=g) * 3).to(torch.bfloat16).to(dev)
    gate, up = base[:, :k], base[:, k:2 * k]
    y1 = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((rows, k), dtype=torch.bfloat16, device=dev)
    q1, s1 = mxfp4_swiglu_quantize(gate, up, y=y1)
    sf, s = _with_canary((k // 512, rows, 16), torch.uint8, dev, 0x5A)
    q2, s2 = mxfp4_swiglu_quantize(gate, up, y=y2, scales=s, interleaved=True)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(y1, y2)
    assert np.array_equal(to_np(s2), interleave_numpy(to_np(s1)))
    assert np.all(to_np(sf)[s2.numel():] == 0x5A)


def test_prefill_producer_to_interleaved_gemm():
    """RMSNorm producer -> GEMM on interleaved scales gives the bits of RMSNorm producer -> GEMM on
    row-major scales (the same tile kernel)."""
    from block_scaled_fp4_mxfp4_amd import mxfp4_rmsnorm_quantize
    dev = device()
    m, n, k = 1024, 2048, 4096
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    x = random_bf16((m, k), 9, spread=4).to(dev)
    gamma = torch.ones(k, dtype=torch.bfloat16, device=dev)
    bq, bs = random_codes(n, k, 10)
    d_bq, d_bs = upload(bq, dev), upload(bs, dev)
    q1, s1 = mxfp4_rmsnorm_quantize(x, gamma, 1e-5)
    q2, s2 = mxfp4_rmsnorm_quantize(x, gamma, 1e-5, interleaved=True)
    c1 = mxfp4_gemm_nt(q1, s1, d_bq, d_bs, out_dtype=torch.float32, kernel=_tile_kernel_for(m, n, num_cus))
    c2 = mxfp4_gemm_nt_interleaved(q2, s2, d_bq, mxfp4_scales_interleave(d_bs), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


# ---------------------------------------------------------------------------
# MXFP8 activations (W4A8) and MXFP8 x MXFP8 on interleaved scales


@pytest.mark.parametrize("rows,k", [(1, 512), (3, 1024), (257, 4096), (1000, 1536)])
def test_mxfp8_quantize_interleaved_is_the_layout_of_the_oracle_bytes(rows, k):
    from block_scaled_fp4_mxfp4_amd import mxfp8_quantize_interleaved
    dev = device()
    log(f"interleaved mxfp8 quantize rows={rows} k={k}")
    bits = _random_bits(rows, k, rows * 5 + k)
    sf, s = _with_canary((k // 512, rows, 16), torch.uint8, dev, 0x5A)
    q, s = mxfp8_quantize_interleaved(bf16_from_np_bits(bits).to(dev), scales_il=s)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_mxfp8(bits)
    assert np.array_equal(to_np(q), rq), "code bytes"
    assert np.array_equal(to_np(s), interleave_numpy(rs)), "interleaved scale bytes"
    assert np.all(to_np(sf)[s.numel():] == 0x5A)


def _w4a8_operands(m, n, k, seed, b_fp8=False):
    a = random_bf16((m, k), seed, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), seed + 1, spread=3)
    aq, as_ = oracle.quantize_mxfp8(workloads.bf16_bits(a))
    bq, bs = (oracle.quantize_mxfp8 if b_fp8 else oracle.quantize)(workloads.bf16_bits(b))
    return aq, as_, bq, bs


@pytest.mark.parametrize("m,n,k", [(1, 64, 512), (100, 300, 1536), (300, 257, 1024), (1024, 1000, 4096)])
def test_w4a8_and_mxfp8_interleaved_equal_row_major(m, n, k):
    from block_scaled_fp4_mxfp4_amd import (mxfp8_gemm_nt, mxfp8_gemm_nt_interleaved, mxfp8_gemm_w4a8_nt,
                                            mxfp8_gemm_w4a8_nt_interleaved)
    dev = device()
    log(f"interleaved w4a8 / mxfp8 m={m} n={n} k={k}")
    for b_fp8 in (False, True):
        aq, as_, bq, bs = (upload(t, dev) for t in _w4a8_operands(m, n, k, m + n + k, b_fp8))
        as_il, bs_il = mxfp4_scales_interleave(as_), mxfp4_scales_interleave(bs)
        for dt in (torch.float32, torch.bfloat16):
            cf, c = _with_canary((m, n), dt, dev, 0xFF)
            if b_fp8:
                mxfp8_gemm_nt_interleaved(aq, as_il, bq, bs_il, c=c)
                ref = mxfp8_gemm_nt(aq, as_, bq, bs, out_dtype=dt)
            else:
                mxfp8_gemm_w4a8_nt_interleaved(aq, as_il, bq, bs_il, c=c)
                ref = mxfp8_gemm_w4a8_nt(aq, as_, bq, bs, out_dtype=dt, kernel="tile128")
            torch.cuda.synchronize()
            assert torch.equal(c.view(torch.uint8), ref.view(torch.uint8)), f"b_fp8={b_fp8} {dt}"
            assert np.all(to_np(cf)[c.numel() * c.element_size():] == 0xFF), "write past the end of C"


@pytest.mark.parametrize("name", ["all_rows_one_expert", "empty_first_middle_last", "persistent_ragged",
                                  "persistent_many_tiles"])
def test_grouped_w4a8_interleaved_equals_row_major(name):
    from block_scaled_fp4_mxfp4_amd import mxfp8_grouped_gemm_w4a8_nt, mxfp8_grouped_gemm_w4a8_nt_interleaved
    dev = device()
    counts, n, k = GROUP_CASES[name]
    counts = np.asarray(counts)
    groups, total = len(counts), int(np.sum(counts))
    log(f"interleaved grouped w4a8 {name}: {groups} groups, {total} rows")
    offsets = upload(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), dev)
    aq, as_, _, _ = _w4a8_operands(total, 1, k, total + k)
    wq, ws = random_codes(groups * n, k, groups + n)
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    d_wq, d_ws = upload(wq, dev).view(groups, n, k // 2), upload(ws, dev).view(groups, n, k // 32)
    cf, c = _with_canary((total, n), torch.float32, dev, 0xFF)
    mxfp8_grouped_gemm_w4a8_nt_interleaved(d_aq, mxfp4_scales_interleave(d_as), d_wq, mxfp4_scales_interleave(d_ws),
                                           offsets, c=c)
    ref = mxfp8_grouped_gemm_w4a8_nt(d_aq, d_as, d_wq, d_ws, offsets, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))
    assert np.all(to_np(cf)[c.numel() * 4:] == 0xFF)


def test_w4a8_moe_layer_interleaved_equals_row_major():
    """Route -> permute -> MXFP8 scatter-quantize -> grouped W4A8 GEMM -> combine, 2048 tokens, 16 experts,
    on interleaved scales against row-major scales, bit for bit."""
    from block_scaled_fp4_mxfp4_amd import (mxfp8_grouped_gemm_w4a8_nt, mxfp8_grouped_gemm_w4a8_nt_interleaved,
                                            mxfp8_moe_quantize_scatter, mxfp8_moe_quantize_scatter_interleaved)
    dev = device()
    tokens, experts, top_k, n, k = 2048, 16, 4, 1024, 2048
    x = random_bf16((tokens, k), 77, spread=4).to(dev)
    lg = torch.from_numpy(np.random.default_rng(78).standard_normal((tokens, experts)).astype(np.float32)).to(dev)
    wq, ws = random_codes(experts * n, k, 79)
    d_wq, d_ws = upload(wq, dev).view(experts, n, k // 2), upload(ws, dev).view(experts, n, k // 32)
    ids, gate = mxfp4_moe_route(lg, top_k)
    off, _, tr = mxfp4_moe_permute(ids, experts)
    rows = tokens * top_k
    aq, as_ = mxfp8_moe_quantize_scatter(x, tr, rows)
    out = mxfp4_moe_combine(mxfp8_grouped_gemm_w4a8_nt(aq, as_, d_wq, d_ws, off), tr, gate)
    aq2, as_il = mxfp8_moe_quantize_scatter_interleaved(x, tr, rows)
    out2 = mxfp4_moe_combine(mxfp8_grouped_gemm_w4a8_nt_interleaved(aq2, as_il, d_wq, mxfp4_scales_interleave(d_ws),
                                                                    off), tr, gate)
    torch.cuda.synchronize()
    assert torch.equal(aq, aq2)
    assert np.array_equal(to_np(as_il), interleave_numpy(to_np(as_)))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
