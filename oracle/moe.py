"""The FP8 mixture-of-experts layer built around the M-grouped product.

Test infrastructure (see the package docstring): not part of the product path.

The layer (deepgemm-rust README, "What's implemented" table, moe_fp8_layer
row) runs histogram, offsets, gather, a grouped product, SiLU-times-up, a
second grouped product and a weighted combine.  The steps, as this oracle
reads them (each reading is listed in the design notes):

route      Every (token t, slot j) pair whose expert e = topk_idx[t][j] lies in
           [0, G) is one row of the contiguous layout.  counts[e] is the number
           of such pairs (the histogram).  Expert e's rows start at
           starts[e] = sum_{e' < e} roundup(counts[e'], 128) (the offsets; the
           128-row alignment is the contiguous layout's, same table,
           m_grouped_fp8_gemm_nt_contiguous row) and hold its pairs in
           ascending (t, j) order.  m_indices[r] is the expert of row r or -1
           for a padding row; token_of_row[r] its token or -1; row_of[t][j]
           the row of pair (t, j) or -1 for a dropped slot.  Arrays are sized
           by an upper bound m_pad_max of the padded row count; rows past the
           real count are padding.
gather     Row r of the first operand is x[token_of_row[r]] (zeros for a
           padding row), quantized per 1x128 group like any activation.
gate_up    h = bf16(grouped product with w1), w1 [G][2I][H]: columns 0..I-1 of
           h are the gate, I..2I-1 the up projection.
act        a = bf16(silu(gate) * up), silu(g) = g / (1 + exp(-g)), each
           operation rounded to float32 (the precision the kernel takes the
           same decision in), then quantized per 1x128 group; padding rows
           are zero rows.
down       y = bf16(grouped product of the quantized act with w2 [G][H][I]).
combine    out[t] = bf16(sum_j topk_weights[t][j] * y[row_of[t][j]]), exact in
           FP64 before the one rounding.
"""

from __future__ import annotations

import numpy as np

from .gemm import grouped_gemm_nt, round_to_bf16
from .quantize import bf16_bits_to_f32, quantize_groups

ALIGN = 128


def max_padded_rows(tokens: int, topk: int, num_experts: int) -> int:
    """An upper bound of the padded row count: every pair one row, plus at
    most 127 padding rows per expert, rounded up to 128."""
    return (tokens * topk + num_experts * (ALIGN - 1) + ALIGN - 1) // ALIGN * ALIGN


def route_contiguous(topk_idx, num_experts: int, m_pad_max: int | None = None):
    """The routing layout of ``topk_idx`` int [T][topk] (see the module
    docstring).  Returns (counts int32 [G], m_indices int32 [m_pad_max],
    token_of_row int32 [m_pad_max], row_of int32 [T][topk])."""
    topk_idx = np.asarray(topk_idx, dtype=np.int64)
    tokens, topk = topk_idx.shape
    if m_pad_max is None:
        m_pad_max = max_padded_rows(tokens, topk, num_experts)
    flat = topk_idx.reshape(-1)  # pair p = t * topk + j, in (t, j) order
    valid = (flat >= 0) & (flat < num_experts)
    counts = np.bincount(flat[valid], minlength=num_experts).astype(np.int64)
    padded = (counts + ALIGN - 1) // ALIGN * ALIGN
    starts = np.concatenate(([0], np.cumsum(padded)[:-1]))
    if int(padded.sum()) > m_pad_max:
        raise ValueError("m_pad_max is smaller than the padded row count")
    # pairs sorted by expert, keeping (t, j) order within an expert
    key = np.where(valid, flat, num_experts)
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    expert_of_sorted = flat[order]
    rank = np.arange(order.size) - np.concatenate(([0], np.cumsum(counts)[:-1]))[expert_of_sorted]
    rows = starts[expert_of_sorted] + rank
    m_indices = np.full(m_pad_max, -1, dtype=np.int32)
    token_of_row = np.full(m_pad_max, -1, dtype=np.int32)
    row_of = np.full(tokens * topk, -1, dtype=np.int32)
    m_indices[rows] = expert_of_sorted
    token_of_row[rows] = order // topk
    row_of[order] = rows
    return counts.astype(np.int32), m_indices, token_of_row, row_of.reshape(tokens, topk)


def gather_rows(x_bf16, token_of_row) -> np.ndarray:
    """Row r = x[token_of_row[r]], a zero row where token_of_row[r] < 0."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    token_of_row = np.asarray(token_of_row, dtype=np.int64)
    out = np.zeros((token_of_row.size, x_bf16.shape[1]), dtype=np.uint16)
    live = token_of_row >= 0
    out[live] = x_bf16[token_of_row[live]]
    return out


def gather_quantize(x_bf16, token_of_row):
    """The gathered rows quantized per 1x128 group: (q uint8, sa float32)."""
    return quantize_groups(gather_rows(x_bf16, token_of_row))


def silu_mul(h_bf16) -> np.ndarray:
    """a = bf16(silu(gate) * up) for h bf16 bits [M][2I] (gate first), each
    step rounded to float32; returns bf16 bits [M][I]."""
    h = bf16_bits_to_f32(h_bf16)
    inter = h.shape[1] // 2
    g, u = h[:, :inter], h[:, inter:]
    with np.errstate(over="ignore"):
        e = np.exp(-g, dtype=np.float32)
    one = np.float32(1.0)
    act = (g / (one + e)).astype(np.float32) * u
    return round_to_bf16(act.astype(np.float32).astype(np.float64))


def silu_mul_quantize(h_bf16, m_indices):
    """silu_mul, zero rows where m_indices < 0, quantized per 1x128 group."""
    act = silu_mul(h_bf16)
    act[np.asarray(m_indices) < 0] = 0
    return quantize_groups(act)


def combine(y_bf16, row_of, topk_weights) -> np.ndarray:
    """FP64 out[t] = sum_j w[t][j] * y[row_of[t][j]] over slots with a row."""
    y = bf16_bits_to_f32(y_bf16).astype(np.float64)
    row_of = np.asarray(row_of, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    tokens, topk = row_of.shape
    out = np.zeros((tokens, y.shape[1]), dtype=np.float64)
    for j in range(topk):
        live = row_of[:, j] >= 0
        out[live] += w[live, j][:, None] * y[row_of[live, j]]
    return out


def moe_layer(x_bf16, topk_idx, topk_weights, w1, w2, num_experts: int):
    """The whole layer.  x bf16 bits [T][H]; w1 = (q [G][2I][H], sb
    [G][2I/128][H/128]); w2 = (q [G][H][I], sb [G][H/128][I/128]), both from
    the block quantizer.  Returns a dict of every intermediate (h64 and y64
    are the products in FP64 before their bf16 rounding, NaN on padding rows)
    and ``out`` (FP64 before its bf16 rounding) and ``out_bf16``."""
    (q1, s1), (q2, s2) = w1, w2
    counts, m_indices, token_of_row, row_of = route_contiguous(topk_idx, num_experts)
    qa1, sa1 = gather_quantize(x_bf16, token_of_row)
    h64 = grouped_gemm_nt(qa1, sa1, m_indices, q1, s1, num_experts)
    h = round_to_bf16(np.where(np.isnan(h64), 0.0, h64))  # padding rows carry no value; zero them
    qa2, sa2 = silu_mul_quantize(h, m_indices)
    y64 = grouped_gemm_nt(qa2, sa2, m_indices, q2, s2, num_experts)
    y = round_to_bf16(np.where(np.isnan(y64), 0.0, y64))
    out = combine(y, row_of, topk_weights)
    return {
        "counts": counts,
        "m_indices": m_indices,
        "token_of_row": token_of_row,
        "row_of": row_of,
        "qa1": qa1,
        "sa1": sa1,
        "h64": h64,
        "h": h,
        "qa2": qa2,
        "sa2": sa2,
        "y64": y64,
        "y": y,
        "out": out,
        "out_bf16": round_to_bf16(out),
    }
