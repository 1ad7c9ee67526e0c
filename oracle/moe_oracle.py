"""CPU oracle for the MoE steps around the grouped MXFP4 GEMM.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it.  It shares
no code with the HIP library and imports nothing from the product package.

What it follows
---------------
* Grouped per-expert quantization.  The "fp4_quantization" Mojo module page
  lists grouped_quantize_dynamic_scaled_fp4_async: per-expert BF16 activation
  tiles quantized to MXFP4 (or NVFP4 / MXFP8) for the grouped matmul
  (grouped_matmul_block_scaled_mxfp4 on the same page).  Quantization is
  row-independent, so the row of expert-sorted position r is the quantized
  row of the token it came from.
* Routed rows in one launch.  The quadbit README ("Distributed sparse-FP4
  MoE") describes a segmented routed-row kernel in which every expert owns a
  contiguous segment of rows, and the DeepGEMM page (Summary, mega-MoE) fuses
  dispatch, the expert GEMMs and combine.  The pages print no router: the
  quadbit README keeps the router dense and outside the FP4 path.
* Readings taken where the pages are silent (each is the plainest one):
    - top-k: a token's experts are its k largest logits; equal logits go to
      the lower expert id;
    - gate weights: softmax over the k selected logits, so a token's weights
      sum to 1;
    - row order: rows sorted by (expert, token, slot j), i.e. the rows of one
      expert in ascending token order;
    - an expert id outside [0, E) marks an entry as dropped: it gets no row
      and contributes nothing to the combine;
    - combine: out[t] = sum over the token's kept slots j, in slot order, of
      weight[t, j] * y[row of (t, j)].
"""
from __future__ import annotations

import numpy as np

from .mxfp4_oracle import bf16_bits_to_f64, quantize
from .mxfp8_oracle import quantize_mxfp8


def route_topk(logits, top_k: int):
    """Top-k routing of float32 logits [T, E].

    Returns (ids int32 [T, k], weights float64 [T, k]).  ids[t] lists the k
    largest logits of token t in descending order, equal logits by ascending
    expert id.  weights[t, j] = exp(l_j) / sum over the k selected of exp(l_i),
    evaluated in float64 from the float32 logits.
    """
    lg = np.asarray(logits)
    if lg.dtype != np.float32 or lg.ndim != 2:
        raise ValueError("logits must be a float32 [T, E] array")
    tokens, experts = lg.shape
    if not 1 <= top_k <= experts:
        raise ValueError("top_k must be in [1, E]")
    if np.any(np.isnan(lg)):
        raise ValueError("NaN logits are outside the routing's definition")
    l64 = lg.astype(np.float64)
    ids = np.empty((tokens, top_k), dtype=np.int32)
    expert_ids = np.arange(experts)
    for t in range(tokens):
        # np.lexsort sorts by its last key first: descending logit, then ascending id
        order = np.lexsort((expert_ids, -l64[t]))
        ids[t] = order[:top_k]
    sel = np.take_along_axis(l64, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])          # the first selected logit is the largest
    weights = ex / ex.sum(axis=1, keepdims=True)
    return ids, weights


def permute(ids, experts: int):
    """Expert-sorted row layout of routed entries.

    ids int [T, k].  Entry (t, j) is kept when 0 <= ids[t, j] < experts.
    Kept entries are ordered by (expert, t, j); row r is the r-th of them.
    Returns
      offsets    int32 [E + 1]: rows of expert e are [offsets[e], offsets[e+1]);
      row_token  int32 [T * k]: token of each row, -1 past offsets[E];
      token_rows int32 [T, k]:  row of each entry, -1 for a dropped entry.
    """
    ids = np.asarray(ids, dtype=np.int64)
    if ids.ndim != 2:
        raise ValueError("ids must be [T, k]")
    tokens, top_k = ids.shape
    flat = ids.reshape(-1)
    kept = (flat >= 0) & (flat < experts)
    idx = np.nonzero(kept)[0]
    # key (expert, flat index); flat index = t * k + j orders (t, j)
    key = flat[idx] * (tokens * top_k) + idx
    order = idx[np.argsort(key, kind="stable")]
    counts = np.bincount(flat[kept], minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_token = np.full(tokens * top_k, -1, dtype=np.int32)
    row_token[: len(order)] = (order // top_k).astype(np.int32)
    token_rows = np.full(tokens * top_k, -1, dtype=np.int32)
    token_rows[order] = np.arange(len(order), dtype=np.int32)
    return offsets, row_token, token_rows.reshape(tokens, top_k)


def _scatter_rows(q_tok, s_tok, token_rows, total_rows):
    token_rows = np.asarray(token_rows, dtype=np.int64)
    q = np.zeros((total_rows, q_tok.shape[1]), dtype=np.uint8)
    s = np.zeros((total_rows, s_tok.shape[1]), dtype=np.uint8)
    written = np.zeros(total_rows, dtype=bool)
    for t in range(token_rows.shape[0]):
        for r in token_rows[t]:
            if 0 <= r < total_rows:
                q[r] = q_tok[t]
                s[r] = s_tok[t]
                written[r] = True
    return q, s, written


def quantize_scatter(x_bits, token_rows, total_rows: int):
    """MXFP4 operand of the grouped GEMM: row r holds the quantized row of its token.

    x_bits BF16 [T, K] as uint16; token_rows int [T, k].  Returns
    (q uint8 [R, K/2], s uint8 [R, K/32], written bool [R]); rows no entry
    points at stay zero and are flagged False in `written`.
    """
    q_tok, s_tok = quantize(x_bits)
    return _scatter_rows(q_tok, s_tok, token_rows, total_rows)


def quantize_scatter_mxfp8(x_bits, token_rows, total_rows: int):
    """The same with MXFP8 rows (E4M3 codes [R, K], E8M0 scales [R, K/32])."""
    q_tok, s_tok = quantize_mxfp8(x_bits)
    return _scatter_rows(q_tok, s_tok, token_rows, total_rows)


def combine(y, token_rows, weights):
    """out[t, :] = sum over kept slots j of weights[t, j] * y[token_rows[t, j], :], in float64.

    y: expert outputs [R, N], either float values or BF16 uint16 bit patterns;
    weights: [T, k] (their float32 values are taken exactly).  Dropped slots
    (row -1 or past R) contribute nothing.
    """
    y = np.asarray(y)
    y64 = bf16_bits_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    token_rows = np.asarray(token_rows, dtype=np.int64)
    w = np.asarray(weights).astype(np.float64)
    tokens, top_k = token_rows.shape
    out = np.zeros((tokens, y64.shape[1]), dtype=np.float64)
    for j in range(top_k):
        r = token_rows[:, j]
        ok = (r >= 0) & (r < y64.shape[0])
        out[ok] += w[ok, j][:, None] * y64[r[ok]]
    return out


def combine_abs(y, token_rows, weights):
    """sum over kept slots of |weights[t, j] * y[row, :]|: the scale of the combine's rounding error."""
    y = np.asarray(y)
    y64 = bf16_bits_to_f64(y) if y.dtype == np.uint16 else y.astype(np.float64)
    return combine(np.abs(y64), token_rows, np.abs(np.asarray(weights).astype(np.float64)))
