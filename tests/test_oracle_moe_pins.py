"""Pins for the MoE oracle (routing, permutation, scatter-quantize, combine).

Each check ties the oracle to something other than its own code:
* hand-worked routings and permutations whose expected values are written
  out below;
* order invariants of top-k checked with plain comparisons (every chosen
  logit at least every unchosen one, equal logits resolved by id);
* the softmax of all logits against scipy.special.softmax (k = E), the
  closed form w_i / w_j = exp(l_i - l_j), and k = 1 giving weight 1;
* the permutation against a brute-force scan in pure Python loops;
* scatter-quantize against quantizing the gathered rows (quantize then
  scatter vs gather then quantize: the row-independence of the format);
* combine against exact rational arithmetic on tiny cases.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle as O
import workloads


def test_route_hand_worked_ties():
    lg = np.array([[1.0, 3.0, 3.0, 2.0]], np.float32)
    ids, w = O.route_topk(lg, 2)
    assert ids.tolist() == [[1, 2]]
    assert w.tolist() == [[0.5, 0.5]]
    ids, w = O.route_topk(lg, 3)
    assert ids.tolist() == [[1, 2, 3]]
    d = 2.0 + math.exp(-1.0)
    assert np.allclose(w[0], [1 / d, 1 / d, math.exp(-1.0) / d], rtol=1e-15)


def test_route_signed_zero_is_a_tie():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    ids, _ = O.route_topk(lg, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]


def test_route_k1_weight_is_one():
    lg = np.random.default_rng(1).standard_normal((50, 8)).astype(np.float32)
    ids, w = O.route_topk(lg, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))   # argmax returns the first maximum


def test_route_k_equals_e_is_full_softmax():
    lg = (np.random.default_rng(2).standard_normal((40, 16)) * 3).astype(np.float32)
    ids, w = O.route_topk(lg, 16)
    ref = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, ids.astype(np.int64), axis=1), rtol=1e-12, atol=0)


def test_route_weight_ratios_closed_form():
    lg = (np.random.default_rng(3).standard_normal((30, 64))).astype(np.float32)
    ids, w = O.route_topk(lg, 4)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    for j in range(1, 4):
        assert np.allclose(w[:, j] / w[:, 0], np.exp(sel[:, j] - sel[:, 0]), rtol=1e-13)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_order_invariants_with_many_ties(seed):
    rng = np.random.default_rng(seed)
    lg = rng.integers(-3, 4, size=(60, 12)).astype(np.float32)    # small integers: ties everywhere
    k = 5
    ids, _ = O.route_topk(lg, k)
    for t in range(lg.shape[0]):
        chosen = [int(e) for e in ids[t]]
        assert len(set(chosen)) == k
        for a, b in zip(chosen, chosen[1:]):                       # descending, ties by id
            assert lg[t, a] > lg[t, b] or (lg[t, a] == lg[t, b] and a < b)
        for e in range(lg.shape[1]):
            if e in chosen:
                continue
            for c in chosen:                                       # no unchosen expert beats a chosen one
                assert lg[t, c] > lg[t, e] or (lg[t, c] == lg[t, e] and c < e)


def test_route_rejects_nan():
    with pytest.raises(ValueError):
        O.route_topk(np.array([[0.0, np.nan]], np.float32), 1)


def test_permute_hand_worked():
    ids = np.array([[1, 0], [1, 2], [0, 1]])
    offsets, row_token, token_rows = O.permute(ids, 3)
    assert offsets.tolist() == [0, 2, 5, 6]
    assert row_token.tolist() == [0, 2, 0, 1, 2, 1]
    assert token_rows.tolist() == [[2, 0], [3, 5], [1, 4]]


def test_permute_hand_worked_with_dropped_entries():
    ids = np.array([[2, -1], [5, 0], [0, 2]])   # -1 and 5 are outside [0, 3)
    offsets, row_token, token_rows = O.permute(ids, 3)
    assert offsets.tolist() == [0, 2, 2, 4]
    assert row_token.tolist() == [1, 2, 0, 2, -1, -1]
    assert token_rows.tolist() == [[2, -1], [-1, 0], [1, 3]]


def _permute_brute(ids, experts):
    tokens, k = len(ids), len(ids[0])
    rows = []
    for e in range(experts):                     # expert-major scan of every entry in (t, j) order
        for t in range(tokens):
            for j in range(k):
                if ids[t][j] == e:
                    rows.append((t, j))
    offsets = [0]
    for e in range(experts):
        offsets.append(offsets[-1] + sum(1 for t in range(tokens) for j in range(k) if ids[t][j] == e))
    row_token = [t for t, _ in rows] + [-1] * (tokens * k - len(rows))
    token_rows = [[-1] * k for _ in range(tokens)]
    for r, (t, j) in enumerate(rows):
        token_rows[t][j] = r
    return offsets, row_token, token_rows


@pytest.mark.parametrize("tokens,experts,k,seed", [(1, 1, 1, 0), (7, 3, 2, 1), (40, 9, 3, 2), (33, 5, 5, 3)])
def test_permute_brute_force(tokens, experts, k, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, experts + 2, size=(tokens, k))     # includes dropped ids and repeats
    offsets, row_token, token_rows = O.permute(ids, experts)
    bo, br, bt = _permute_brute(ids.tolist(), experts)
    assert offsets.tolist() == bo
    assert row_token.tolist() == br
    assert token_rows.tolist() == bt


def test_permute_of_workload_routing_invariants():
    moe = workloads.MOE
    lg = moe.logits()[:512].numpy()
    ids, _ = O.route_topk(lg, moe.top_k)
    offsets, row_token, token_rows = O.permute(ids, moe.experts)
    assert offsets[-1] == ids.size
    assert np.array_equal(np.diff(offsets), np.bincount(ids.reshape(-1), minlength=moe.experts))
    for e in range(moe.experts):
        seg = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)             # one row per token per expert, ascending tokens
    t_of = np.repeat(np.arange(ids.shape[0]), moe.top_k)
    assert np.array_equal(row_token[token_rows.reshape(-1)], t_of)
    assert sorted(token_rows.reshape(-1).tolist()) == list(range(ids.size))


def test_quantize_scatter_equals_quantize_of_gathered_rows():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((24, 128)) * np.exp2(rng.integers(-6, 7, size=(24, 1)))).astype(np.float32)
    xb = workloads.bf16_bits(__import__("torch").from_numpy(x).bfloat16())
    ids = rng.integers(-1, 6, size=(24, 3))
    offsets, row_token, token_rows = O.permute(ids, 6)
    total = int(offsets[-1])
    q, s, written = O.quantize_scatter(xb, token_rows, ids.size)
    assert written[:total].all() and not written[total:].any()
    gq, gs = O.quantize(xb[row_token[:total]])
    assert np.array_equal(q[:total], gq) and np.array_equal(s[:total], gs)
    q8, s8, _ = O.quantize_scatter_mxfp8(xb, token_rows, ids.size)
    g8, gs8 = O.quantize_mxfp8(xb[row_token[:total]])
    assert np.array_equal(q8[:total], g8) and np.array_equal(s8[:total], gs8)


def test_combine_hand_worked():
    y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    token_rows = np.array([[2, 0], [1, -1]])
    w = np.array([[0.25, 0.75], [0.5, 0.5]], np.float32)
    out = O.combine(y, token_rows, w)
    assert out.tolist() == [[0.25 * 5 + 0.75 * 1, 0.25 * 6 + 0.75 * 2], [1.5, 2.0]]


def test_combine_exact_rational():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((10, 5)).astype(np.float32).astype(np.float64)
    token_rows = rng.integers(-1, 10, size=(6, 3))
    w = rng.random((6, 3)).astype(np.float32)
    out = O.combine(y, token_rows, w)
    for t in range(6):
        for c in range(5):
            acc = Fraction(0)
            for j in range(3):
                r = int(token_rows[t, j])
                if r >= 0:
                    acc += Fraction(float(w[t, j])) * Fraction(float(y[r, c]))
            # float64 holds each product exactly (24 + 24 bits); only the sums round
            assert abs(Fraction(float(out[t, c])) - acc) <= abs(acc) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
