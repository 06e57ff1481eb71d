"""Oracle runs spread over worker processes, for the full-size parity tests.

Test infrastructure.  The oracle's quantizers work one row (activation
groups) or one 128-row block row (weight blocks) at a time, and its product
one output row at a time, so a large operand can be cut at 128-row
boundaries, handed to worker processes, and the pieces put back together
without changing a single value: each piece is exactly what the oracle
computes for those rows.  This module holds only numpy code (the workers
never import torch or touch a GPU); the comparison statistics of the parity
criteria are defined here once and used by tests/parity.py as well.
"""

from __future__ import annotations

import atexit
import multiprocessing as mp
import os

import numpy as np

import oracle

# Row granularity of the pieces: a multiple of the 128-row weight block.
PIECE_ROWS = 1024

_POOL = None


def pool():
    """A process pool started with 'spawn' (fresh interpreters that import
    numpy and the oracle only), created on first use and kept for the
    session.  At most 8 workers, each limited to 2 BLAS threads."""
    global _POOL
    if _POOL is None:
        workers = max(1, min(8, (os.cpu_count() or 2) // 2))
        _POOL = mp.get_context("spawn").Pool(processes=workers, initializer=_init_worker)
        atexit.register(_close)
    return _POOL


def _close():
    global _POOL
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL = None


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(2)
    except Exception:
        pass


def _pieces(rows: int, piece: int = PIECE_ROWS):
    return [(r, min(rows, r + piece)) for r in range(0, rows, piece)]


# ------------------------------------------------------------- quantizers
def _quantize_blocks(w):
    return oracle.quantize_blocks(w)


def _quantize_groups(x):
    q, sa = oracle.quantize_groups(x, sa_ld=x.shape[0])
    return q, sa


def quantize_blocks(w: np.ndarray):
    """oracle.quantize_blocks(w), computed on 1024-row pieces in parallel."""
    parts = pool().map(_quantize_blocks, [w[a:b] for a, b in _pieces(w.shape[0])])
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def quantize_groups(x: np.ndarray):
    """oracle.quantize_groups(x), computed on 1024-row pieces in parallel;
    the scale array has sa_ld = roundup(M, 4) (rows past M are NaN)."""
    m, k = x.shape
    parts = pool().map(_quantize_groups, [x[a:b] for a, b in _pieces(m)])
    q = np.concatenate([p[0] for p in parts])
    sa = np.full((k // 128, -(-m // 4) * 4), np.nan, dtype=np.float32)
    sa[:, :m] = np.concatenate([p[1] for p in parts], axis=1)
    return q, sa


# ------------------------------------------------------ product criteria
def magnitude_sum(qa, sa, qb, sb) -> np.ndarray:
    """S[m, n] = sum_k |dequant(a)[m, k] * dequant(b)[n, k]| in FP64."""
    t = np.abs(oracle.e4m3_table())
    m, k = qa.shape
    n = qb.shape[0]
    fa = t[qa] * np.repeat(np.abs(sa[:, :m]).T.astype(np.float64), 128, axis=1)
    sbe = np.repeat(np.repeat(np.abs(sb).astype(np.float64), 128, axis=0)[:n], 128, axis=1)
    fb = t[qb] * sbe
    return fa @ fb.T


def error_stats(got: np.ndarray, ref: np.ndarray, s: np.ndarray, k: int) -> dict:
    """The two product criteria's ingredients for one block of outputs:
    squared error and reference norms (normwise), the largest excess over the
    elementwise FP32-order bound |D - D64| <= 2^-8 |D64| + 2 (K + K/128)
    2^-24 S, the count of elements that differ from bf16_RNE(D64), and
    whether every output is finite."""
    err = np.abs(got - ref)
    bound = 2.0**-8 * np.abs(ref) + 2.0 * (k + k // 128) * 2.0**-24 * s
    got_bits = (got.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return {
        "err2": float(np.sum((got - ref) ** 2)),
        "ref2": float(np.sum(ref**2)),
        "worst": float(np.max(err - bound)) if err.size else -np.inf,
        "ndiff": int(np.count_nonzero(got_bits != oracle.round_to_bf16(ref))),
        "count": int(got.size),
        "finite": bool(np.all(np.isfinite(got))),
    }


def _product_piece(args):
    qa, sa, qb, sb, got, k = args
    ref = oracle.gemm_nt(qa, sa, qb, sb)
    return error_stats(got, ref, magnitude_sum(qa, sa, qb, sb), k)


def product_stats(qa, sa, qb, sb, got, k: int, piece: int = 256) -> dict:
    """error_stats of `got` (FP64 [M][N]) against oracle.gemm_nt(qa, sa, qb,
    sb), computed on row pieces in parallel and summed."""
    m = qa.shape[0]
    jobs = [(qa[a:b], np.ascontiguousarray(sa[:, a:b]), qb, sb, got[a:b], k) for a, b in _pieces(m, piece)]
    return merge(pool().map(_product_piece, jobs))


def merge(parts) -> dict:
    out = {"err2": 0.0, "ref2": 0.0, "worst": -np.inf, "ndiff": 0, "count": 0, "finite": True}
    for p in parts:
        out["err2"] += p["err2"]
        out["ref2"] += p["ref2"]
        out["worst"] = max(out["worst"], p["worst"])
        out["ndiff"] += p["ndiff"]
        out["count"] += p["count"]
        out["finite"] = out["finite"] and p["finite"]
    return out
