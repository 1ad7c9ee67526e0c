"""GPU decode GEMM on prepacked weights against the CPU oracle and the streaming kernel.

* prepacking: the rearranged code and scale bytes equal a NumPy re-indexing of
  B written from the layout's definition (a pure byte permutation, zero rows
  past n), over ragged n and several k;
* GEMM: fp32 output within 1e-5 (floored max-rel) of the float64 oracle and
  bit-identical to the streaming kernel on the unpacked weight (same per-wave
  k-step split, same MFMA order, same fixed-order reduction), BF16 output
  bit-identical too; shapes cover both kernel forms (K = 4096 straight-line,
  other K looped, including more pairs than the register ring holds), the
  three row-tile sizes, ragged m and n, a single 512-K pair, and m > 128;
* the full decode workload (128 x 14336 x 4096) bit-identical to the streaming
  kernel over the whole output and within tolerance of the oracle on samples;
* the tiny workload's fp32 C at the points whose oracle values are stored in
  tests/golden; quantize + prepacked GEMM replayed from a HIP graph;
* both operands prepacked: the quantizer writing the prepacked layout equals
  the layout definition applied to the oracle's quantization (padded rows
  zero), and the GEMM on prepacked A and B is bit-identical to the other two
  kernels on every shape above and on the full decode workload.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import (MXFP4Error, mxfp4_gemm_nt, mxfp4_gemm_nt_prepacked, mxfp4_gemm_nt_prepacked_ab,
                                        mxfp4_prepack_weight, mxfp4_prepacked_weight_size, mxfp4_quantize,
                                        mxfp4_quantize_prepacked)
from block_scaled_fp4_mxfp4_amd import binding
from tests.gpu_common import (assert_bf16_matches_rounded, device, log, poisoned, random_bf16, random_codes,
                              sampled_indices, to_np, upload)
from tests.prepack_layout import prepack_numpy as _prepack_numpy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k", [(1, 512), (64, 512), (100, 1024), (130, 4096), (200, 1536)])
def test_prepack_layout_matches_definition(n, k):
    dev = device()
    log(f"prepack n={n} k={k}")
    bq, bs = random_codes(n, k, seed=n + k, lo=0, hi=254)
    cb, sb = mxfp4_prepacked_weight_size(n, k)
    assert cb == -(-n // 64) * 64 * k // 2 and sb == -(-n // 64) * 64 * k // 32
    bp_q = poisoned((cb,), torch.uint8, dev, 0xA5)
    bp_s = poisoned((sb,), torch.uint8, dev, 0xA5)
    mxfp4_prepack_weight(upload(bq, dev), upload(bs, dev), bp_q, bp_s)
    torch.cuda.synchronize()
    want_q, want_s = _prepack_numpy(bq, bs)
    assert np.array_equal(to_np(bp_q), want_q)
    assert np.array_equal(to_np(bp_s), want_s)


def _both(aq, as_, bq, bs, dev, out_dtype):
    """(prepacked-B result, streaming-kernel result); the result with A prepacked
    too is checked bit for bit against the first here."""
    a_q, a_s, b_q, b_s = (upload(t, dev) for t in (aq, as_, bq, bs))
    bp_q, bp_s = mxfp4_prepack_weight(b_q, b_s)
    ap_q, ap_s = mxfp4_prepack_weight(a_q, a_s)
    m, n = a_q.shape[0], b_q.shape[0]
    k = a_q.shape[1] * 2
    c_all = poisoned((m + 1, n), out_dtype, dev, 0x7F)
    mxfp4_gemm_nt_prepacked(a_q, a_s, bp_q, bp_s, n, c=c_all[:m])
    c2_all = poisoned((m + 1, n), out_dtype, dev, 0x7F)
    mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, c=c2_all[:m], splits=1)
    ref = mxfp4_gemm_nt(a_q, a_s, b_q, b_s, out_dtype=out_dtype, kernel="stream")
    torch.cuda.synchronize()
    assert torch.all(c_all[m:].view(torch.uint8) == 0x7F), "write past C"
    assert torch.all(c2_all[m:].view(torch.uint8) == 0x7F), "write past C (A prepacked)"
    assert torch.equal(c2_all[:m].view(torch.uint8), c_all[:m].view(torch.uint8)), "A-prepacked result differs"
    return c_all[:m], ref


# (m, n, k): K runs in straight-line chunks of 8, 4 and 1 pairs of 512 (K = 512:
# one pair, fewer than the 4-pair register ring; 2048: one chunk of 4; 4096: one
# chunk of 8; 4608: 8 + 1; 6144: 8 + 4; 8192: 8 + 8; 14336: 8 + 8 + 8 + 4, the
# ffn-down decode shape; 1536: three chunks of 1).
SHAPES = [(1, 64, 512), (5, 100, 1024), (33, 200, 512), (64, 256, 2048), (96, 130, 4096), (128, 192, 4096),
          (17, 640, 4096), (130, 64, 4096), (128, 320, 4608), (100, 64, 6144), (40, 96, 8192), (200, 72, 1536),
          (128, 192, 14336), (64, 130, 14336)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_prepacked_gemm_matches_oracle_and_stream_kernel(m, n, k):
    dev = device()
    log(f"prepacked gemm m={m} n={n} k={k}")
    a = random_bf16((m, k), 7 * m + k, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), 11 * n + k, spread=2)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    c32, s32 = _both(aq, as_, bq, bs, dev, torch.float32)
    c16, s16 = _both(aq, as_, bq, bs, dev, torch.bfloat16)
    got = to_np(c32).astype(np.float64)
    assert oracle.floored_max_rel(got, oracle.gemm_nt(aq, as_, bq, bs)) <= 1e-5
    assert torch.equal(c32.view(torch.int32), s32.view(torch.int32)), "fp32 differs from the streaming kernel"
    assert torch.equal(c16.view(torch.int16), s16.view(torch.int16)), "bf16 differs from the streaming kernel"


def test_prepacked_gemm_every_code_and_scale():
    """Random code bytes (every E2M1 pattern) and a wide scale range, m = 1 and 128."""
    dev = device()
    for m, n, k in [(1, 192, 4096), (128, 130, 2048)]:
        aq, as_ = random_codes(m, k, seed=m + 1, lo=110, hi=140)
        bq, bs = random_codes(n, k, seed=n + 2, lo=110, hi=140)
        c32, s32 = _both(aq, as_, bq, bs, dev, torch.float32)
        assert oracle.floored_max_rel(to_np(c32).astype(np.float64), oracle.gemm_nt(aq, as_, bq, bs)) <= 1e-5
        assert torch.equal(c32.view(torch.int32), s32.view(torch.int32))


def test_prepacked_rejects_bad_k_and_empty_problems_are_noops():
    dev = device()
    aq, as_ = random_codes(4, 1024, seed=3)
    bq, bs = random_codes(64, 1024, seed=4)
    bp_q, bp_s = mxfp4_prepack_weight(upload(bq, dev), upload(bs, dev))
    with pytest.raises(MXFP4Error):
        mxfp4_prepacked_weight_size(64, 992)
    with pytest.raises(MXFP4Error):
        mxfp4_prepack_weight(upload(bq[:, :496], dev), upload(bs[:, :31], dev))
    c = mxfp4_gemm_nt_prepacked(upload(aq[:0], dev), upload(as_[:0], dev), bp_q, bp_s, 64)
    assert c.shape == (0, 64)


@pytest.mark.parametrize("name", [workloads.DECODE.name, workloads.DECODE_DOWN.name])
def test_prepacked_decode_full_size(name):
    dev = device()
    w = workloads.DENSE[name]
    log(f"prepacked gemm {w.name}")
    a, b = w.make()
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    c = mxfp4_gemm_nt_prepacked(aq, as_, bp_q, bp_s, w.n)
    c32 = mxfp4_gemm_nt_prepacked(aq, as_, bp_q, bp_s, w.n, out_dtype=torch.float32)
    s = mxfp4_gemm_nt(aq, as_, bq, bs, kernel="stream")
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), s.view(torch.int16)), "bf16 differs from the streaming kernel"
    rows = sampled_indices(w.m, 32, seed=5)
    cols = sampled_indices(w.n, 96, seed=6)
    oaq, oas = oracle.quantize(workloads.bf16_bits(a[torch.from_numpy(rows)]))
    obq, obs = oracle.quantize(workloads.bf16_bits(b[torch.from_numpy(cols)]))
    ref = oracle.gemm_nt(oaq, oas, obq, obs)
    assert oracle.floored_max_rel(to_np(c32)[np.ix_(rows, cols)].astype(np.float64), ref) <= 1e-5


def test_prepacked_tiny_workload_matches_stored_oracle_values():
    """GPU quantize of the tiny workload, prepack, GEMM: fp32 C at the points whose
    float64 oracle values are stored in tests/golden/oracle_digests.txt."""
    from tests.test_golden import load_golden
    dev = device()
    gold = load_golden()
    w = workloads.TINY
    a, b = w.make()
    aq, as_ = mxfp4_quantize(a.to(dev))
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    c = to_np(mxfp4_gemm_nt_prepacked(aq, as_, bp_q, bp_s, w.n, out_dtype=torch.float32))
    for (i, j) in [(0, 0), (17, 100), (63, 255)]:
        want = float.fromhex(gold[f"{w.name}.c[{i},{j}]"])
        assert abs(float(c[i, j]) - want) <= 1e-5 * max(abs(want), 1.0), (i, j, float(c[i, j]), want)


def test_prepacked_graph_replays_match_eager():
    """Quantize + prepacked GEMM captured in a HIP graph: every replay, with eager
    work and synchronisation between replays, equals the eager result."""
    dev = device()
    m, n, k = 128, 448, 4096
    log(f"graph: quantize + prepacked gemm m={m} n={n} k={k}")
    a = workloads.activation_bf16(m, k, 970, outliers=True).to(dev)
    b = workloads.gaussian_bf16((n, k), 0.02, 971).to(dev)
    bq, bs = mxfp4_quantize(b)
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    aq = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    as_ = torch.empty((m, k // 32), dtype=torch.uint8, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def step():
        mxfp4_quantize(a, aq, as_)
        mxfp4_gemm_nt_prepacked(aq, as_, bp_q, bp_s, n, c=c)

    step()
    torch.cuda.synchronize()
    eager = c.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        c.view(torch.uint8).fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("rows,k", [(1, 512), (63, 1024), (64, 512), (130, 4096), (200, 1536)])
def test_quantize_prepacked_matches_oracle_layout(rows, k):
    dev = device()
    log(f"quantize prepacked rows={rows} k={k}")
    x = random_bf16((rows, k), 31 * rows + k, spread=8, outlier_frac=0.01)
    cb, sb = mxfp4_prepacked_weight_size(rows, k)
    ap_q = poisoned((cb,), torch.uint8, dev, 0xA5)
    ap_s = poisoned((sb,), torch.uint8, dev, 0xA5)
    mxfp4_quantize_prepacked(x.to(dev), ap_q, ap_s)
    torch.cuda.synchronize()
    rq, rs = oracle.quantize(workloads.bf16_bits(x))
    want_q, want_s = _prepack_numpy(rq, rs)
    assert np.array_equal(to_np(ap_q), want_q)
    assert np.array_equal(to_np(ap_s), want_s)


def test_prepacked_ab_decode_full_size_and_graph():
    """Decode 128 x 14336 x 4096 from BF16 A: quantize into the prepacked layout and
    multiply, bit-identical to quantize + streaming kernel; then the same two
    launches replayed from a HIP graph."""
    dev = device()
    w = workloads.DECODE
    log(f"prepacked A and B {w.name}")
    a, b = w.make()
    a_d = a.to(dev)
    aq, as_ = mxfp4_quantize(a_d)
    bq, bs = mxfp4_quantize(b.to(dev))
    bp_q, bp_s = mxfp4_prepack_weight(bq, bs)
    ap_q, ap_s = mxfp4_quantize_prepacked(a_d)
    c = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
    mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, c=c)
    s = mxfp4_gemm_nt(aq, as_, bq, bs, kernel="stream")
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), s.view(torch.int16))

    def step():
        mxfp4_quantize_prepacked(a_d, ap_q, ap_s)
        mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, w.m, w.n, w.k, c=c)

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        c.view(torch.uint8).fill_(0xCD)
        ap_q.fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), s.view(torch.int16)), f"replay {rep}"


# Split-K of the both-prepacked kernel: (m, n, k, splits).  K ranges of
# ceil(pairs / splits) pairs, rounded up to a multiple of 4 above 4: 14336 / 4
# -> 8 + 8 + 8 + 4; 14336 / 3 -> 12 + 12 + 4 (chunks 8 + 4); 2048 / 3 -> 2 + 2
# (two ranges: fewer than asked); 8192 / 16 -> one pair each; 1536 / 2 -> 2 + 1
# (a shorter last range); 5120 / 5 -> 2 each; 10240 / 3 -> 8 + 8 + 4; m = 200
# and 130: two row tiles; n = 130 and 200: a ragged last panel; 0 = the
# automatic choice.
SPLIT_SHAPES = [(128, 640, 14336, 4), (40, 256, 14336, 3), (64, 320, 2048, 3), (1, 200, 8192, 16),
                (33, 130, 1536, 2), (96, 64, 5120, 5), (200, 130, 2048, 4), (128, 130, 10240, 3),
                (130, 192, 4096, 0), (17, 64, 4096, 0)]


def _split_case(m, n, k, seed, dev):
    a = random_bf16((m, k), seed, spread=3, outlier_frac=0.01)
    b = random_bf16((n, k), seed + 1, spread=2)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    bq, bs = oracle.quantize(workloads.bf16_bits(b))
    bp_q, bp_s = mxfp4_prepack_weight(upload(bq, dev), upload(bs, dev))
    ap_q, ap_s = mxfp4_prepack_weight(upload(aq, dev), upload(as_, dev))
    return (aq, as_, bq, bs), (ap_q, ap_s, bp_q, bp_s)


@pytest.mark.parametrize("m,n,k,splits", SPLIT_SHAPES)
def test_prepacked_ab_split_k_matches_oracle(m, n, k, splits):
    """Every K split (including ranges fewer than asked and a shorter last range):
    fp32 within 1e-5 of the float64 oracle, BF16 the nearest-even rounding of the
    exact result, nothing written past C, the same bits on a second call, and the
    workspace's arrival counters back at zero."""
    dev = device()
    log(f"split-K prepacked m={m} n={n} k={k} splits={splits}")
    host, (ap_q, ap_s, bp_q, bp_s) = _split_case(m, n, k, 3 * m + n + k, dev)
    lib = binding.load_library()
    need = lib.mxfp4_gemm_nt_prepacked_ab_workspace_size(m, n, k, splits)
    ws = torch.zeros(max(need, 65536) + 4096, dtype=torch.uint8, device=dev)
    c64 = oracle.gemm_nt(*host)
    for out_dtype in (torch.float32, torch.bfloat16):
        c_all = poisoned((m + 1, n), out_dtype, dev, 0x7F)
        mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, c=c_all[:m], splits=splits, ws=ws)
        again = mxfp4_gemm_nt_prepacked_ab(ap_q, ap_s, bp_q, bp_s, m, n, k, out_dtype=out_dtype, splits=splits, ws=ws)
        torch.cuda.synchronize()
        assert torch.all(c_all[m:].view(torch.uint8) == 0x7F), "write past C"
        assert torch.all(ws[:65536] == 0), "arrival counters not returned to zero"
        c = c_all[:m]
        bits = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(c.view(bits), again.view(bits)), "split-K result not deterministic"
        if out_dtype == torch.float32:
            assert oracle.floored_max_rel(to_np(c).astype(np.float64), c64) <= 1e-5
        else:
            assert_bf16_matches_rounded(to_np(c.view(torch.int16)).view(np.uint16), c64)


def test_prepacked_ab_split_k_workspace_reuse_and_graph():
    """One zero-filled workspace serves consecutive calls of different shapes and
    split counts; the split-K launch replayed from a HIP graph gives the eager
    result on every replay (the counters reset in the kernel, no memset)."""
    dev = device()
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device=dev)
    for idx, (m, n, k, splits) in enumerate([(128, 256, 4096, 8), (64, 640, 2048, 2), (1, 64, 14336, 14)]):
        host, dev_ops = _split_case(m, n, k, 100 + idx, dev)
        c = mxfp4_gemm_nt_prepacked_ab(*dev_ops, m, n, k, out_dtype=torch.float32, splits=splits, ws=ws)
        torch.cuda.synchronize()
        assert oracle.floored_max_rel(to_np(c).astype(np.float64), oracle.gemm_nt(*host)) <= 1e-5
        assert torch.all(ws[:65536] == 0)
    m, n, k = 128, 512, 8192
    host, dev_ops = _split_case(m, n, k, 200, dev)
    eager = mxfp4_gemm_nt_prepacked_ab(*dev_ops, m, n, k, splits=4, ws=ws)
    c = torch.empty_like(eager)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        mxfp4_gemm_nt_prepacked_ab(*dev_ops, m, n, k, c=c, splits=4, ws=ws)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxfp4_gemm_nt_prepacked_ab(*dev_ops, m, n, k, c=c, splits=4, ws=ws)
    for rep in range(3):
        c.view(torch.uint8).fill_(0xCD)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.all(ws[:65536] == 0)


def test_prepacked_ab_split_k_refusals():
    dev = device()
    _, dev_ops = _split_case(128, 64, 2048, 5, dev)
    with pytest.raises(MXFP4Error):   # more than 16 ranges
        mxfp4_gemm_nt_prepacked_ab(*dev_ops, 128, 64, 2048, splits=17)
    small = torch.zeros(1024, dtype=torch.uint8, device=dev)
    with pytest.raises(MXFP4Error):   # workspace too small
        mxfp4_gemm_nt_prepacked_ab(*dev_ops, 128, 64, 2048, splits=4, ws=small)
