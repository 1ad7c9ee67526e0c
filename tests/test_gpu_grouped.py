"""GPU grouped per-expert GEMM: bit-exact against the dense kernel run on each
expert's slice with the same tile configuration, and within tolerance of the
CPU oracle, over routing patterns with empty, tiny and tile-boundary groups."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from block_scaled_fp4_mxfp4_amd import mxfp4_gemm_nt, mxfp4_grouped_gemm_nt, mxfp4_quantize
from tests.gpu_common import (assert_bf16_matches_rounded, device, log, poisoned, random_bf16,
                              sampled_indices, to_np, upload)

pytestmark = pytest.mark.gpu


def _tile_for(total_m, groups):
    # the grouped kernel's tile choice: 256x256 tiles when groups average >= 192 rows
    return "tile256" if total_m // groups >= 192 else "tile128"


def _grouped_case(counts, n, k, seed, dev, out_dtype=torch.float32):
    counts = np.asarray(counts)
    groups = len(counts)
    offsets = np.zeros(groups + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    total = int(offsets[-1])
    a = random_bf16((max(total, 1), k), seed)[:total]
    w = random_bf16((groups * n, k), seed + 1)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a)) if total else (np.zeros((0, k // 2), np.uint8), np.zeros((0, k // 32), np.uint8))
    wq, ws = oracle.quantize(workloads.bf16_bits(w))
    wq = wq.reshape(groups, n, k // 2)
    ws = ws.reshape(groups, n, k // 32)
    c_all = poisoned((total + 1, n), out_dtype, dev, 0xFF)
    c = c_all[:total]
    d_aq, d_as, d_wq, d_ws = upload(aq, dev), upload(as_, dev), upload(wq, dev), upload(ws, dev)
    mxfp4_grouped_gemm_nt(d_aq, d_as, d_wq, d_ws, upload(offsets, dev), c=c)
    torch.cuda.synchronize()
    assert torch.all(c_all[total:].view(torch.uint8) == 0xFF)
    return aq, as_, wq, ws, offsets, c, (d_aq, d_as, d_wq, d_ws)


PATTERNS = {
    "single_group": ([300], 192, 256),
    "all_rows_one_expert": ([0, 0, 517, 0], 130, 512),
    "empty_first_middle_last": ([0, 40, 0, 129, 0], 96, 1024),
    "tile_boundaries_128": ([1, 127, 128, 129, 255, 256, 257], 64, 256),
    "tile_boundaries_256": ([255, 256, 257, 511, 1], 256, 512),
    "ragged_k": ([33, 70, 5], 72, 160),
    "many_groups": (list(np.random.default_rng(0).integers(0, 40, size=70)), 64, 256),
    # 256 x 256 tiles with k % 1024 == 0 take the persistent loop: k = 1024 (two
    # stages, no loop body) with ragged groups, and more tiles than compute units
    # (every workgroup runs several tiles of different experts)
    "persistent_ragged": ([0, 255, 256, 257, 511, 1, 700, 0], 200, 1024),
    "persistent_many_tiles": (list(np.random.default_rng(1).integers(0, 600, size=32)), 1536, 2048),
    # several n-tiles with a ragged last one, and experts of 1 to 4 m-tiles: the
    # tiles of an expert run n-tile-major (its m-tiles of one n-tile adjacent)
    "persistent_ragged_n": ([300, 0, 600, 45, 256, 1000], 600, 1024),
}


@pytest.mark.parametrize("pattern", list(PATTERNS))
def test_grouped_bitexact_vs_dense_per_group(pattern):
    dev = device()
    counts, n, k = PATTERNS[pattern]
    log(f"grouped {pattern}: counts={counts[:10]} n={n} k={k}")
    aq, as_, wq, ws, offsets, c, dev_ops = _grouped_case(counts, n, k, 7, dev)
    total = int(offsets[-1])
    tile = _tile_for(total, len(counts))
    got = to_np(c)
    d_aq, d_as, d_wq, d_ws = dev_ops
    for g in range(len(counts)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        # row slices of the operands are valid arguments (scale rows need only 4-byte alignment
        # when k % 128 == 0); a copy keeps the k % 128 != 0 cases independent of that rule
        a_s_g = d_as[lo:hi] if k % 128 == 0 else d_as[lo:hi].clone()
        dense = mxfp4_gemm_nt(d_aq[lo:hi], a_s_g, d_wq[g], d_ws[g], out_dtype=torch.float32, kernel=tile)
        torch.cuda.synchronize()
        assert np.array_equal(got[lo:hi], to_np(dense)), f"group {g}"
    ref = oracle.grouped_gemm_nt(aq, as_, wq, ws, offsets)
    assert oracle.floored_max_rel(got, ref) <= 1e-5


def test_grouped_bf16_output():
    dev = device()
    counts = [17, 0, 300, 64]
    aq, as_, wq, ws, offsets, c, _ = _grouped_case(counts, 200, 1024, 9, dev, out_dtype=torch.bfloat16)
    ref = oracle.grouped_gemm_nt(aq, as_, wq, ws, offsets)
    got = to_np(c.view(torch.int16)).view(np.uint16)
    assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got), ref) <= 1e-2
    assert_bf16_matches_rounded(got, ref)


def test_grouped_moe_workload_full_size_sampled():
    """The 64-expert top-4 MoE layer at full size (GPU quantize + grouped GEMM),
    checked on sampled rows of every expert against the oracle."""
    dev = device()
    w = workloads.MOE
    a, wts, offsets = w.make()
    counts = np.diff(offsets.numpy())
    log(f"moe: rows per expert min={counts.min()} max={counts.max()} empty={(counts == 0).sum()}")
    aq, as_ = mxfp4_quantize(a.to(dev))
    wq, wsc = mxfp4_quantize(wts.view(-1, w.k).to(dev))
    wq = wq.view(w.experts, w.n, w.k // 2)
    wsc = wsc.view(w.experts, w.n, w.k // 32)
    c = mxfp4_grouped_gemm_nt(aq, as_, wq, wsc, offsets.to(dev))
    torch.cuda.synchronize()
    got_all = to_np(c.view(torch.int16)).view(np.uint16)
    cols = sampled_indices(w.n, 48, seed=3)
    for g in range(w.experts):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        rows = lo + sampled_indices(hi - lo, 4, seed=g)
        oaq, oas = oracle.quantize(workloads.bf16_bits(a[torch.from_numpy(rows)]))
        obq, obs = oracle.quantize(workloads.bf16_bits(wts[g][torch.from_numpy(cols)]))
        ref = oracle.gemm_nt(oaq, oas, obq, obs)
        got = got_all[np.ix_(rows, cols)]
        assert oracle.floored_max_rel(oracle.bf16_bits_to_f64(got), ref) <= 1e-2, f"expert {g}"
        assert_bf16_matches_rounded(got, ref)


def _sanitized_segments(offsets, total):
    """The segments the grouped kernel forms from any offsets: each offset clamped
    into [0, total], then the running maximum, so group g owns [lo_g, lo_{g+1})."""
    c = np.clip(np.asarray(offsets, np.int64), 0, total)
    run = np.maximum.accumulate(c)
    return [(int(run[g]), int(max(run[g], c[g + 1]))) for g in range(len(offsets) - 1)]


@pytest.mark.parametrize("case", ["few_groups", "across_chunks", "persistent"])
def test_grouped_malformed_offsets_give_disjoint_segments(case):
    """Offsets are only sanitized on the device (the host cannot read them without
    a sync): clamped into [0, total_m] and replaced by their running maximum.
    Negative, decreasing and past-the-end offsets must neither write outside C
    nor give overlapping groups: every row belongs to exactly one segment and
    holds that group's dense result, bit for bit."""
    dev = device()
    if case == "few_groups":
        total, n, k = 300, 96, 512
        # clamped: 0, 120, 80, 300, 300 -> segments [0,120), [120,120), [120,300), [300,300)
        offsets = np.array([-5, 120, 80, 500, 300], np.int32)
    elif case == "persistent":
        # 256 x 256 tiles with k % 1024 == 0: the persistent tile loop; clamped and
        # running max: 0, 500, 500, 1200, 1200 -> [0,500), [500,500), [500,1200), [1200,1200)
        total, n, k = 1200, 300, 1024
        offsets = np.array([-5, 500, 300, 1400, 1200], np.int32)
    else:
        # 70 groups (two 64-group chunks), a drop inside each chunk and one at the chunk edge
        total, n, k = 700, 64, 256
        rng = np.random.default_rng(5)
        offsets = np.sort(rng.integers(0, total, size=71)).astype(np.int32)
        offsets[0], offsets[-1] = 0, total
        offsets[10] = offsets[9] - 30
        offsets[64] = offsets[63] - 50
        offsets[66] = total + 40
    groups = len(offsets) - 1
    segs = _sanitized_segments(offsets, total)
    assert segs[0][0] == 0 and all(segs[g][1] == segs[g + 1][0] for g in range(groups - 1))
    a = random_bf16((total, k), 31)
    w = random_bf16((groups * n, k), 32)
    aq, as_ = oracle.quantize(workloads.bf16_bits(a))
    wq, ws = oracle.quantize(workloads.bf16_bits(w))
    d_aq, d_as = upload(aq, dev), upload(as_, dev)
    d_wq, d_ws = upload(wq.reshape(groups, n, k // 2), dev), upload(ws.reshape(groups, n, k // 32), dev)
    c_all = poisoned((total + 3, n), torch.float32, dev, 0xFF)
    c = c_all[:total]
    log(f"malformed offsets {case}: {groups} groups, total_m {total}")
    mxfp4_grouped_gemm_nt(d_aq, d_as, d_wq, d_ws, upload(offsets, dev), c=c)
    torch.cuda.synchronize()
    assert torch.all(c_all[total:].view(torch.uint8) == 0xFF), "write past the end of C"
    got = to_np(c)
    covered = np.zeros(total, bool)
    tile = _tile_for(total, groups)
    for g, (lo, hi) in enumerate(segs):
        if hi <= lo:
            continue
        ref = to_np(mxfp4_gemm_nt(d_aq[lo:hi], d_as[lo:hi], d_wq[g], d_ws[g], out_dtype=torch.float32, kernel=tile))
        assert np.array_equal(got[lo:hi], ref), f"group {g} rows [{lo}, {hi})"
        covered[lo:hi] = True
    rows_end = segs[-1][1]
    assert covered[:rows_end].all()
    # rows past the last segment end are no group's: they keep the poison
    assert torch.all(c[rows_end:].view(torch.uint8) == 0xFF)
