"""CPU oracle for the fine-grained block-scaled FP8 linear (test infrastructure).

THIS PACKAGE IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the
test suite, the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it.  It shares no code with the HIP library: no
kernels, headers, helpers, tables or constants, and it imports nothing from the
library package.

What it computes, and where the pages define it:

* ``e4m3``      FP8 E4M3 (OCP "FN" variant) decode table and a round-to-nearest-
                even, saturating encoder defined from that table.  The pages name
                the format "e4m3" / "f8e4m3" (Linnet "Backend plugins" page,
                DeepGemm.match; deepgemm-rust README, "What's implemented" table)
                and the Blackwell converter "cvt.rn.satfinite" (deepgemm-rust
                README, "Blackwell-native FP4/FP8" key techniques).
* ``quantize``  per-(1x128) activation group and per-(128x128) weight block
                quantization with FP32 scales = amax / 448 (deepgemm-rust README,
                "What's implemented" table, fp8_gemm_nt row; Linnet page, module
                docstring of the DeepGEMM plugin source).
                The UE8M0 variants round each scale up to a power of two
                (deepgemm-rust README, Blackwell key techniques: UE8M0 scale
                factors; FP32 scales bridged to packed UE8M0); the MX variant
                takes one such scale per 1x32 block (the README's gran-32
                recipe), packed as E8M0 codes.
* ``gemm``      the block-scaled product D = A.B^T with both scale sets applied
                once per 128-wide K chunk, in FP64, and its M-grouped contiguous
                variant (deepgemm-rust README, "What's implemented" table and
                "Quick start" grouped example), and its masked variant (same
                table, m_grouped_fp8_gemm_nt_masked row); and the MX product
                with per-1x32 power-of-two scales on both operands.
* ``moe``       the FP8 mixture-of-experts layer around the grouped product:
                routing layout, gather, SiLU-times-up, weighted combine and the
                whole layer (same table, moe_fp8_layer row).

Every function works in float64 (or exact integer / float32 steps where the
method fixes float32), favouring obviousness over speed.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
things other than itself (the torch CPU float8 cast, exact rational brute
force, closed forms and invariants).  No function is "parity unpinned".
"""

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_table
from .gemm import (
    gemm_nt,
    gemm_nt_mx,
    gemm_nt_dequantized,
    grouped_gemm_nt,
    masked_grouped_gemm_nt,
    round_to_bf16,
)
from . import moe
from .quantize import (
    GROUP,
    quantize_blocks,
    quantize_blocks_ue8m0,
    quantize_groups,
    quantize_groups_ue8m0,
    quantize_mx,
    unpack_mx_scales,
)

__all__ = [
    "E4M3_MAX",
    "GROUP",
    "e4m3_decode",
    "e4m3_encode",
    "e4m3_table",
    "gemm_nt",
    "gemm_nt_mx",
    "gemm_nt_dequantized",
    "grouped_gemm_nt",
    "masked_grouped_gemm_nt",
    "moe",
    "quantize_blocks",
    "quantize_groups",
    "quantize_groups_ue8m0",
    "quantize_blocks_ue8m0",
    "quantize_mx",
    "unpack_mx_scales",
    "round_to_bf16",
]
