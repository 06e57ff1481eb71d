"""Per-group and per-block FP8 quantization with FP32 scales.

Test infrastructure (see the package docstring): not part of the product path.

The recipe (the DeepSeek one the deepgemm-rust README names in its "What's
implemented" table, fp8_gemm_nt row: activation scales per 1x128 group,
weight scales per 128x128 block): every 128-element run of a row is rounded
to FP8 under its own scale
(Linnet "Backend plugins" page, module docstring of the DeepGEMM plugin
source), and the weight has one scale per 128x128 block.  Scales are FP32, not
powers of two: the Hopper kernels take f32 scales and the plugin asks for no
UE8M0 cast (Linnet page, DeepGemm.probe comment and the fp8_gemm_nt call with
disable_ue8m0_cast=True).

Readings where the pages are silent (each listed in the design notes):
* scale s = fl32(amax / 448) with amax the exact float32 maximum magnitude;
* an all-zero group gets s = 1;
* the element is y = fl32(x / s), a correctly rounded float32 division (not a
  multiplication by a reciprocal), then rounded to E4M3 (``e4m3_encode``);
* activation scales are stored one K group after another (MN-major), the rows padded to a
  multiple of four (Linnet page, module docstring and the `padded` row count
  in _BlockProduct.execute): SA is float32 [K/128][sa_ld], sa_ld = roundup(M, 4),
  entry [g][m] the scale of row m's group g; entries of rows >= M unspecified
  (this oracle fills them with NaN);
* weight scales are row-major float32 [ceil(N/128)][K/128] (deepgemm-rust
  README, "Quick start", the sfb shape); a partial last block of rows uses the
  rows present.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode

GROUP = 128


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _scale_of(amax: np.ndarray) -> np.ndarray:
    """FP32 scale for a set of float32 amax values: fl32(amax / 448), 1 if amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)  # IEEE float32 division
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_groups(x_bf16: np.ndarray, sa_ld: int | None = None):
    """Activation quantization, one scale per (row, 128-column group).

    x_bf16: uint16 [M][K] bfloat16 bit patterns, K a multiple of 128.
    Returns (q uint8 [M][K] E4M3 codes, sa float32 [K/128][sa_ld]).
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    m, k = x_bf16.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    if sa_ld is None:
        sa_ld = -(-m // 4) * 4
    if sa_ld < m:
        raise ValueError("sa_ld must be at least M")
    x = bf16_bits_to_f32(x_bf16).reshape(m, k // GROUP, GROUP)
    amax = np.max(np.abs(x), axis=2) if m else np.zeros((0, k // GROUP), np.float32)
    s = _scale_of(amax)  # [M][K/128]
    y = (x / s[:, :, None]).astype(np.float32)  # IEEE float32 division
    q = e4m3_encode(y).reshape(m, k)
    sa = np.full((k // GROUP, sa_ld), np.nan, dtype=np.float32)
    sa[:, :m] = s.T
    return q, sa


def quantize_blocks(w_bf16: np.ndarray):
    """Weight quantization, one scale per 128x128 block.

    w_bf16: uint16 [N][K] bfloat16 bit patterns, K a multiple of 128.
    Returns (q uint8 [N][K], sb float32 [ceil(N/128)][K/128]).
    """
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    n, k = w_bf16.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_bits_to_f32(w_bf16)
    nb, kb = -(-n // GROUP), k // GROUP
    q = np.empty((n, k), dtype=np.uint8)
    sb = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        rows = slice(i * GROUP, min(n, (i + 1) * GROUP))
        for j in range(kb):
            cols = slice(j * GROUP, (j + 1) * GROUP)
            block = w[rows, cols]
            s = _scale_of(np.max(np.abs(block)))
            sb[i, j] = s
            q[rows, cols] = e4m3_encode((block / s).astype(np.float32))
    return q, sb


def _scale_of_ue8m0(amax: np.ndarray) -> np.ndarray:
    """Power-of-two (UE8M0) scale: the FP32 scale fl32(amax/448) (1 for a zero
    group) rounded up to a power of two, 2^ceil(log2 s), kept within the E8M0
    range [2^-127, 2^127]."""
    s32 = _scale_of(amax).astype(np.float64)
    f, e = np.frexp(s32)  # s32 = f * 2^e, f in [0.5, 1)
    e = np.where(f == 0.5, e - 1, e)  # exact powers of two stay
    e = np.clip(e, -127, 127)
    return np.ldexp(1.0, e).astype(np.float32)


def quantize_groups_ue8m0(x_bf16: np.ndarray, sa_ld: int | None = None):
    """quantize_groups with power-of-two scales (the UE8M0 recipe of the
    Blackwell path: deepgemm-rust README, key techniques, scale factors as
    UE8M0 powers of two; and its note that FP32 scales are bridged to packed
    UE8M0).  The element is y = x / s (exact for a power of two unless it
    underflows float32), then E4M3; scales stay float32 values, powers of two."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    m, k = x_bf16.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    if sa_ld is None:
        sa_ld = -(-m // 4) * 4
    x = bf16_bits_to_f32(x_bf16).reshape(m, k // GROUP, GROUP)
    amax = np.max(np.abs(x), axis=2) if m else np.zeros((0, k // GROUP), np.float32)
    s = _scale_of_ue8m0(amax)
    y = (x / s[:, :, None]).astype(np.float32)
    q = e4m3_encode(y).reshape(m, k)
    sa = np.full((k // GROUP, sa_ld), np.nan, dtype=np.float32)
    sa[:, :m] = s.T
    return q, sa


def quantize_blocks_ue8m0(w_bf16: np.ndarray):
    """quantize_blocks with power-of-two (UE8M0) scales."""
    w_bf16 = np.asarray(w_bf16, dtype=np.uint16)
    n, k = w_bf16.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_bits_to_f32(w_bf16)
    nb, kb = -(-n // GROUP), k // GROUP
    q = np.empty((n, k), dtype=np.uint8)
    sb = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        rows = slice(i * GROUP, min(n, (i + 1) * GROUP))
        for j in range(kb):
            cols = slice(j * GROUP, (j + 1) * GROUP)
            block = w[rows, cols]
            s = _scale_of_ue8m0(np.max(np.abs(block)))
            sb[i, j] = s
            q[rows, cols] = e4m3_encode((block / s).astype(np.float32))
    return q, sb



MX_BLOCK = 32


def e8m0_code(s: np.ndarray) -> np.ndarray:
    """E8M0 code (exponent + 127) of power-of-two float32 scales in
    [2^-127, 2^127]."""
    f, e = np.frexp(np.asarray(s, dtype=np.float64))  # s = 0.5 * 2^e exactly
    if not np.all(f == 0.5):
        raise ValueError("scales must be powers of two")
    return (e - 1 + 127).astype(np.int64)


def quantize_mx(x_bf16: np.ndarray, s_ld: int | None = None):
    """MXFP8 recipe: one power-of-two scale per 1x32 block of each row (the
    gran-32 recipe of the deepgemm-rust README, "Full recipes"; the scale rule
    is _scale_of_ue8m0 over the block's amax, the same rule as the UE8M0
    recipe at gran-128), element code E4M3(x / s).  Scales are stored as E8M0
    codes, the four of a 128-column chunk packed in one int32 (byte j holds
    block 4c + j; the pages' packed UE8M0 scale factors), MN-major:
    s[c][row].  Entries of rows >= M are -1 (unspecified).

    x_bf16: uint16 [M][K], K a multiple of 128.  Returns (q uint8 [M][K],
    s int32 [K/128][s_ld]).  The same function quantizes a weight [N][K] (one
    scale per 1x32 block of each weight row)."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    m, k = x_bf16.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    if s_ld is None:
        s_ld = -(-m // 4) * 4
    x = bf16_bits_to_f32(x_bf16).reshape(m, k // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(x), axis=2) if m else np.zeros((0, k // MX_BLOCK), np.float32)
    s = _scale_of_ue8m0(amax)
    q = e4m3_encode((x / s[:, :, None]).astype(np.float32)).reshape(m, k)
    codes = e8m0_code(s).reshape(m, k // GROUP, 4) if m else np.zeros((0, k // GROUP, 4), np.int64)
    packed = codes[:, :, 0] | (codes[:, :, 1] << 8) | (codes[:, :, 2] << 16) | (codes[:, :, 3] << 24)
    out = np.full((k // GROUP, s_ld), -1, dtype=np.int32)
    out[:, :m] = packed.T.astype(np.uint32).view(np.int32)
    return q, out


def unpack_mx_scales(s_packed: np.ndarray, rows: int) -> np.ndarray:
    """E8M0 codes [rows][K/32] of a packed scale array [K/128][>= rows]."""
    p = np.asarray(s_packed, dtype=np.int32)[:, :rows].astype(np.uint32).T  # [rows][K/128]
    codes = np.stack([(p >> (8 * j)) & 0xFF for j in range(4)], axis=2)  # [rows][K/128][4]
    return codes.reshape(rows, -1).astype(np.int64)
