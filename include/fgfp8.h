/*
 * fgfp8.h -- C ABI of libfgfp8, the fine-grained block-scaled FP8 linear for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (deepgemm-rust README, "What's implemented" table, rows
 * fp8_gemm_nt and m_grouped_fp8_gemm_nt_contiguous): D = A . B^T where A (the
 * activation, M x K) carries one FP32 scale per 1x128 group of each row and
 * B (the weight, N x K) one FP32 scale per 128x128 block; both operands are
 * FP8 E4M3 (OCP "FN": bias 7, largest finite 448, no infinities); the product
 * is accumulated in FP32, with both scales applied once per 128-wide K chunk,
 * and written as bfloat16.  Every 128-element run of an activation row is
 * rounded to FP8 under its own scale, and those scales are stored one K
 * group after another with the row count rounded up to four (Linnet
 * "Backend plugins" page, module docstring of the DeepGEMM plugin source and
 * _BlockProduct.execute).
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer (memory of the current HIP
 *    device), owned by the caller.  The library never allocates, frees or
 *    synchronizes, never reads device data on the host, and keeps no device
 *    state between calls (the one exception is the fixed routing workspace
 *    of moe_route_contiguous_noalloc, a device array inside the library);
 *    every call is legal under HIP graph capture.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    legacy default stream) and runs asynchronously: a return of FGFP8_OK
 *    means the work was enqueued, not that it finished.
 *  - Every array is dense row-major with the leading dimension stated.  Base
 *    pointers must be 16-byte aligned.
 *  - E4M3 arrays hold one byte per element; bf16 arrays two bytes.
 *  - Return value: FGFP8_OK (0) or an error code below; on error nothing was
 *    enqueued and fgfp8_last_error() describes the cause.  No C++ exception
 *    crosses this interface.
 *  - Empty problems (m == 0 or n == 0) enqueue nothing and return FGFP8_OK
 *    once the sizes are valid; their array pointers may then be null.
 *  - Size limits (the kernels address a tile with 32-bit buffer offsets):
 *    row counts below 2^31; k a positive multiple of 128 below 2^24; an
 *    activation scale array (k/128 * sa_ld floats) below 2 GiB.  Larger
 *    sizes are rejected with FGFP8_EINVAL.
 *  - Calls on one stream are ordered; calls on different streams that write
 *    the same output race.
 */
#ifndef FGFP8_H_
#define FGFP8_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FGFP8_OK = 0,
  FGFP8_EINVAL = 1,  /* bad shape, null pointer, misaligned base, bad leading dimension */
  FGFP8_ENODEV = 2,  /* no HIP device, or the current device is not gfx950 */
  FGFP8_ELAUNCH = 3, /* the HIP runtime refused a kernel launch */
};

/* Activation quantization, one scale per 1x128 group of each row.
 *
 * Defined by the per-(1x128) activation scales of the recipe (deepgemm-rust
 * README, "What's implemented", fp8_gemm_nt row) and the Linnet plugin's
 * input rounding, one FP8 scale per 128-element run of a row (Linnet
 * "Backend plugins" page, plugin module docstring).  For row m and
 * group g (columns 128g .. 128g+127):
 *     amax = max |x[m][k]|                       (exact, over the group)
 *     s    = fl32(amax / 448), or 1 when amax == 0
 *     q    = E4M3(fl32(x[m][k] / s))             (round to nearest even;
 *                                                 |.| >= 464 saturates to 448;
 *                                                 the sign of zero is kept)
 *
 * x_bf16  [m][k] bfloat16, input.
 * q_e4m3  [m][k] E4M3 bytes, output.
 * sa      [k/128][sa_ld] float32, output, MN-major: sa[g*sa_ld + m] is the
 *         scale of row m, group g.  Entries for m <= row < sa_ld are left
 *         untouched.
 * Requirements: k > 0 and k % 128 == 0; sa_ld % 4 == 0 and sa_ld >= m.
 * Non-finite inputs are outside the contract (results unspecified). */
int quantize_fp8_groups(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, float* sa, int64_t sa_ld,
                        void* stream);

/* Weight quantization, one scale per 128x128 block (the per-(128x128) weight
 * scales of the recipe; deepgemm-rust README, "What's implemented" and
 * "Quick start", where sfb has shape (n/128, k/128)).  Same rule as
 * quantize_fp8_groups over each block; the last block row of a matrix whose n
 * is not a multiple of 128 uses the rows present.  An offline step: weights
 * are quantized once and kept (Linnet plugin: weight and scale are persistent
 * parameters).
 *
 * w_bf16  [n][k] bfloat16, input.
 * q_e4m3  [n][k] E4M3 bytes, output.
 * sb      [ceil(n/128)][k/128] float32, output, row-major.
 * Requirements: k > 0 and k % 128 == 0. */
int quantize_fp8_blocks(const void* w_bf16, int64_t n, int64_t k, void* q_e4m3, float* sb, void* stream);

/* Block-scaled FP8 product, NT layout (both operands K-contiguous):
 *     D[m][n] = sum_kb  sa[kb][m] * sb[n/128][kb] * P(m, n, kb),
 *     P(m, n, kb) = sum over the 128 k of chunk kb of a[m][k] * b[n][k],
 * with P formed in FP32 by the matrix cores for each 128-wide chunk, then
 * scaled and accumulated in FP32 registers (the scales are applied to each
 * 128-wide block's partial in registers: deepgemm-rust README, kernel notes
 * under "What's implemented"), and rounded once to bfloat16 (round to nearest
 * even).  The summation order inside a chunk is the hardware's; results agree
 * with any other order to FP32 rounding (the Linnet "Backend plugins" page
 * notes that two such products differ only by summation order).
 *
 * a_e4m3  [m][k] E4M3, the quantized activation.
 * sa      [k/128][sa_ld] float32, MN-major activation scales (as written by
 *         quantize_fp8_groups).
 * b_e4m3  [n][k] E4M3, the quantized weight.
 * sb      [ceil(n/128)][k/128] float32, row-major weight scales.
 * d_bf16  [m][n] bfloat16, output (exactly m x n; no padded rows written).
 * Requirements: m >= 0, n >= 0, k > 0 and k % 128 == 0, sa_ld % 4 == 0,
 * sa_ld >= m. */
int fp8_gemm_nt(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream);

/* fp8_gemm_nt with a caller workspace.  On shapes whose 256x256 output
 * tiles would fill at most half of the compute units (few rows against a
 * modest N, e.g. M = 2048 with N = 4096), the 128-wide K chunks of every tile
 * are split over two workgroups: each accumulates its half exactly as
 * fp8_gemm_nt accumulates all of K (a fresh FP32 partial per chunk, promoted
 * with sa * sb), and the two FP32 sums meet through the workspace and are
 * added once before the bf16 rounding.  The result is deterministic; it
 * differs from fp8_gemm_nt's only in the FP32 summation order, which the
 * recipe leaves free.
 * Other shapes run exactly as fp8_gemm_nt.
 *
 * workspace        device memory, 256-byte aligned, of workspace_bytes >=
 *                  fp8_gemm_nt_workspace_bytes(m, n, k); it must be filled
 *                  with zeros before its first use, and every call leaves it
 *                  ready for the next one when it completes.  Calls that may
 *                  overlap in time (different streams) must not share it.
 *                  A smaller workspace (or NULL with 0 bytes) runs the
 *                  fp8_gemm_nt plan.
 * Other arguments and requirements: as fp8_gemm_nt. */
int fp8_gemm_nt_ws(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                   void* d_bf16, int64_t m, int64_t n, int64_t k, void* workspace, int64_t workspace_bytes,
                   void* stream);
/* Bytes of workspace fp8_gemm_nt_ws uses for (m, n, k): 0 when its plan for
 * the shape does not split K (or the shape is invalid).  Host-only. */
int64_t fp8_gemm_nt_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Block-scaled product with an FP8 output for the next layer: the bf16
 * result of fp8_gemm_nt, quantized per 1x128 group of each row exactly as
 * quantize_fp8_groups quantizes a bf16 input, inside the product's epilogue
 * (the pages' Blackwell path offers a quantize-to-FP8 epilogue with per-row
 * output scale factors: deepgemm-rust README, key techniques, "Epilogues";
 * here at 1x128 granularity with FP32 scales, the activation recipe of the
 * next linear).  The result is bit-identical to fp8_gemm_nt followed by
 * quantize_fp8_groups on its output.
 *
 * a_e4m3, sa, sa_ld, b_e4m3, sb, m, n, k: as fp8_gemm_nt.
 * q_e4m3  [m][n] E4M3 output.
 * sd      [n/128][sd_ld] float32 output, MN-major (the layout of sa, so q and
 *         sd feed the next fp8_gemm_nt as its A operand).
 * d_bf16  [m][n] bfloat16 output of the same product, or NULL.
 * Requirements: as fp8_gemm_nt, plus n % 128 == 0, sd_ld % 4 == 0 and
 * sd_ld >= m.  Uses the tile kernels for every m (no decode form). */
int fp8_gemm_nt_fp8_out(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                        void* q_e4m3, float* sd, int64_t sd_ld, void* d_bf16, int64_t m, int64_t n, int64_t k,
                        void* stream);

/* M-grouped contiguous variant for mixture-of-experts layers (deepgemm-rust
 * README, "What's implemented", m_grouped_fp8_gemm_nt_contiguous row: the
 * tokens of all experts concatenated, 128-row group alignment; "Quick start",
 * grouped example for the shapes of b and sfb).
 *
 * a_e4m3     [m][k] E4M3: the rows of all groups, each group starting at a
 *            multiple of 128 rows and padded to a multiple of 128.
 * sa         [k/128][sa_ld] float32 MN-major scales of a.
 * m_indices  [m] int32: the group of each row, or -1 for a padding row.  Each
 *            128-row block is computed with the group of its first row and
 *            skipped when that is negative or >= num_groups.  The contents
 *            are device data and never read on the host.
 * b_e4m3     [num_groups][n][k] E4M3 (equivalently (num_groups*n) x k).
 * sb         [num_groups][ceil(n/128)][k/128] float32.
 * d_bf16     [m][n] bfloat16 output; rows whose m_indices entry is -1 are
 *            unspecified.
 * Requirements: m % 128 == 0, num_groups >= 1, n >= 0, k > 0 and
 * k % 128 == 0, sa_ld % 4 == 0, sa_ld >= m. */
int m_grouped_fp8_gemm_nt_contiguous(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                                     const void* b_e4m3, const float* sb, int32_t num_groups, void* d_bf16,
                                     int64_t m, int64_t n, int64_t k, void* stream);

/* M-grouped masked variant for mixture-of-experts layers at decode time
 * (deepgemm-rust README, "What's implemented", m_grouped_fp8_gemm_nt_masked
 * row: the same kernel with a masked_m scheduler, for a DeepEP-style dispatch
 * output, with expected_m guiding the schedule and no host synchronisation).
 * Every group owns max_m rows of a dispatch buffer, of which only the first
 * masked_m[g] are real; the counts are device data, never read on the host.
 *
 * a_e4m3     [num_groups][max_m][k] E4M3: group g's row r is buffer row
 *            g * max_m + r.
 * sa         [k/128][sa_ld] float32: the MN-major scales of the buffer viewed
 *            as one (num_groups * max_m) x k matrix, i.e. the group folded
 *            into the scale column (what quantize_fp8_groups writes for it,
 *            and quantize_fp8_groups_masked for its real rows only).
 * masked_m   [num_groups] int32: rows of each group to compute (values
 *            outside [0, max_m] are clamped to it).
 * b_e4m3     [num_groups][n][k] E4M3; sb [num_groups][ceil(n/128)][k/128].
 * expected_m host-side hint: the typical count, used only to choose the tile
 *            (<= 0: assume max_m).  Any value gives the same results.
 * d_bf16     [num_groups][max_m][n] bfloat16 output; rows r >= masked_m[g]
 *            of group g are not written.
 * Requirements: num_groups >= 1, max_m >= 0 and max_m % 4 == 0, n >= 0,
 * k > 0 and k % 128 == 0, sa_ld % 4 == 0, sa_ld >= num_groups * max_m. */
int m_grouped_fp8_gemm_nt_masked(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                 const void* b_e4m3, const float* sb, int32_t num_groups, int64_t max_m,
                                 int64_t expected_m, void* d_bf16, int64_t n, int64_t k, void* stream);

/* The masked product with a workspace (the same row of the deepgemm-rust
 * README; its kernel notes name persistent tile scheduling and a tile order
 * for the SM count), for dispatches too small to fill the GPU.  Where the
 * expected live tiles -- num_groups * ceil(expected_m / 128) tiles of 128
 * rows, times the plan's column tiles -- fill at most a quarter of the
 * compute units, one workgroup per compute unit walks the live tiles (those
 * whose rows lie below their group's count, in group order), and when the
 * last round of tiles would leave compute units idle, each of that round's
 * tiles is split along K into up to 8 parts whose FP32 partials meet in the
 * workspace; otherwise the call runs m_grouped_fp8_gemm_nt_masked.  The
 * parts are summed in a fixed order by whichever arrives last, so the
 * results are deterministic; a split tile's sum of parts rounds differently
 * from the unsplit form (within the same parity bar), and which tiles split
 * depends on the live tile count and the device's compute units.  No
 * workgroup waits on another.  FGFP8_MASKED_SPLIT=1 (0) forces (forbids)
 * the walk whatever expected_m says.
 *
 * workspace  device memory, 256-byte aligned, of workspace_bytes >=
 *            m_grouped_fp8_gemm_nt_masked_workspace_bytes(...); zero-filled
 *            before its first use, and every call leaves it so when it
 *            completes.  Calls that may overlap in time must not share it.  A
 *            smaller workspace (or NULL with 0 bytes) runs
 *            m_grouped_fp8_gemm_nt_masked.
 * Other arguments and requirements: as m_grouped_fp8_gemm_nt_masked. */
int m_grouped_fp8_gemm_nt_masked_ws(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                    const void* b_e4m3, const float* sb, int32_t num_groups, int64_t max_m,
                                    int64_t expected_m, void* d_bf16, int64_t n, int64_t k, void* workspace,
                                    int64_t workspace_bytes, void* stream);
/* Bytes of workspace m_grouped_fp8_gemm_nt_masked_ws uses: 1 KB of counters
 * and 256 FP32 slots of one 128 x 256 tile (32 MiB + 1 KB); 0 for invalid
 * arguments.  Host-only. */
int64_t m_grouped_fp8_gemm_nt_masked_workspace_bytes(int32_t num_groups, int64_t max_m, int64_t n, int64_t k);

/* quantize_fp8_groups over the same dispatch buffer, reading the counts on
 * the device: rows r < masked_m[g] of each group g (clamped to [0, max_m])
 * are quantized exactly as quantize_fp8_groups quantizes them (codes and
 * scales bit for bit), the other rows are neither read nor written.  The
 * masked product never reads those rows, so the pair quantizes only what
 * the dispatch delivered (deepgemm-rust README, "What's implemented",
 * m_grouped_fp8_gemm_nt_masked row: a dispatch buffer whose per-group
 * counts stay on the device, with no host synchronisation).
 *
 * x_bf16    [num_groups][max_m][k] bfloat16 (read).
 * masked_m  [num_groups] int32 on the device.
 * q_e4m3    [num_groups][max_m][k] E4M3; sa [k/128][sa_ld] float32 with
 *           group g's row r in column g * max_m + r (the layout the masked
 *           product takes).  Rows past a group's count keep their contents.
 * Requirements: num_groups >= 1, max_m >= 0 and max_m % 4 == 0, k > 0 and
 * k % 128 == 0, sa_ld % 4 == 0, sa_ld >= num_groups * max_m; pointers
 * 16-byte aligned. */
int quantize_fp8_groups_masked(const void* x_bf16, const int32_t* masked_m, int32_t num_groups, int64_t max_m,
                               int64_t k, void* q_e4m3, float* sa, int64_t sa_ld, void* stream);

/* The linear as the pages run it (Linnet "Backend plugins" page,
 * _BlockProduct.execute: round the bf16 input per 1x128 group, then
 * fp8_gemm_nt with the stored weight): D = quantize_groups(x) . B^T.
 *
 * For m <= 4 (k <= 32768) this is a single kernel that quantizes x into LDS
 * inside every workgroup while the weight stream is in flight (decode: the
 * activation-quantize step must not cost a launch of its own; the AReno FP8
 * decode pull request measured the separate quantize chain holding a decode
 * linear at ~1.2x until it was fused).  For 4 < m <= 16 on wide weights
 * (n of about 12288 and more, so that workgroups of three 16-column slabs
 * still cover every CU) it is one kernel that quantizes all m rows into LDS,
 * where m * k/128 <= 512 with q_e4m3/sa NULL and <= 256 with them given (past
 * that the separate quantize launch is cheaper than every workgroup redoing
 * the quantization).  Otherwise, for 4 < m <= 16 (or k > 32768), with
 * q_e4m3/sa NULL it is a single kernel that quantizes x in registers, each
 * wave its own K range; with q_e4m3/sa given it runs quantize_fp8_groups and
 * fp8_gemm_nt.  fgfp8_describe_linear names the path.  Every path is
 * bit-identical to quantize_fp8_groups followed by fp8_gemm_nt.  Above 16
 * rows it runs those two calls.
 *
 * x_bf16  [m][k] bfloat16, input.
 * b_e4m3  [n][k] E4M3 and sb [ceil(n/128)][k/128] float32: the stored weight
 *         (as written by quantize_fp8_blocks).
 * d_bf16  [m][n] bfloat16, output.
 * q_e4m3, sa, sa_ld: the quantized activation [m][k] and its MN-major scales
 *         [k/128][sa_ld], exactly as quantize_fp8_groups writes them.
 *         Optional (both NULL) when m <= 16; required as workspace otherwise.
 * Requirements: m >= 0, n >= 0, k > 0 and k % 128 == 0; if q_e4m3 is given,
 * sa_ld % 4 == 0 and sa_ld >= m. */
int fp8_linear_nt(const void* x_bf16, int64_t m, int64_t k, const void* b_e4m3, const float* sb, int64_t n,
                  void* d_bf16, void* q_e4m3, float* sa, int64_t sa_ld, void* stream);

/* UE8M0 recipe: power-of-two scales (the Blackwell path of the pages keeps
 * its scale factors as UE8M0 powers of two and bridges FP32 scales to them:
 * deepgemm-rust README, key techniques and the note on the SM100 device API).
 * A different recipe from the calls above -- each scale is fl32(amax/448)
 * rounded up to a power of two within [2^-127, 2^127] (1 for a zero group),
 * the element E4M3(x / s) -- with the same layouts and requirements.
 * quantize_fp8_groups_ue8m0 / quantize_fp8_blocks_ue8m0: as the FP32-scale
 * quantizers.  fp8_gemm_nt_ue8m0: as fp8_gemm_nt, for operands whose every
 * scale is such a power of two (only the exponent field of each scale is
 * read); the matrix cores apply the scales and accumulate across the K
 * chunks, so no FP32 promotion is needed.  Results agree with fp8_gemm_nt on
 * the same operands up to FP32 summation order. */
int quantize_fp8_groups_ue8m0(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, float* sa, int64_t sa_ld,
                              void* stream);
int quantize_fp8_blocks_ue8m0(const void* w_bf16, int64_t n, int64_t k, void* q_e4m3, float* sb, void* stream);
int fp8_gemm_nt_ue8m0(const void* a_e4m3, const float* sa, int64_t sa_ld, const void* b_e4m3, const float* sb,
                      void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream);

/* The MXFP8 recipe: one power-of-two scale per 1x32 block along K, on both
 * operands (deepgemm-rust README, "Full recipes": gran-32 scale factors on
 * either side; the scales are UE8M0 powers of two, as on the Blackwell
 * path's block-scaled MMA).  The scale of a block is the UE8M0 rule of
 * quantize_fp8_groups_ue8m0 over its 32 values; the element is
 * E4M3(x / s).  Scales are stored as E8M0 codes (exponent + 127), the four
 * of a 128-column chunk packed in one int32 (byte j = block 4c + j),
 * MN-major: s[c * s_ld + row].
 *
 * quantize_fp8_mx: x [m][k] bf16 -> q [m][k] E4M3 and s int32 [k/128][s_ld];
 * k % 128 == 0, s_ld % 4 == 0, s_ld >= m.  The same call quantizes a weight
 * [n][k] (one scale per 1x32 block of each weight row, i.e. per output
 * column). */
int quantize_fp8_mx(const void* x_bf16, int64_t m, int64_t k, void* q_e4m3, int32_t* s, int64_t s_ld, void* stream);

/* D[m][n] = sum over 32-blocks b of 2^(ea[m][b]-127) * 2^(eb[n][b]-127) *
 * sum_{k in b} A[m][k] B[n][k], with A's scales sa [k/128][sa_ld] and B's
 * sb [k/128][sb_ld] from quantize_fp8_mx.  The matrix cores apply the scales
 * per 32-block (v_mfma_scale) and accumulate across all of K in FP32; no
 * per-chunk promotion.  bf16 out; sb_ld % 4 == 0, sb_ld >= n. */
int fp8_gemm_nt_mx(const void* a_e4m3, const int32_t* sa, int64_t sa_ld, const void* b_e4m3, const int32_t* sb,
                   int64_t sb_ld, void* d_bf16, int64_t m, int64_t n, int64_t k, void* stream);

/* The FP8 mixture-of-experts layer around the grouped product, step by step,
 * with no device-to-host synchronisation (deepgemm-rust README, "What's
 * implemented", moe_fp8_layer row: histogram -> offsets -> gather -> grouped
 * GEMM -> SiLU.mul -> grouped GEMM -> weighted combine).  With tokens T,
 * slots per token topk, experts G, hidden size H and expert width I:
 *   moe_route_contiguous   topk_idx -> layout (counts, m_indices, rows)
 *   moe_gather_quantize    x [T][H] -> A1 (E4M3 [m_pad_max][H], scales)
 *   m_grouped_fp8_gemm_nt_contiguous  A1 x W1 [G][2I][H] -> h [m_pad_max][2I]
 *   silu_mul_quantize      h -> A2 = quantize(bf16(silu(h[:, :I]) * h[:, I:]))
 *     (or both at once: moe_gate_up_silu_quantize  A1 x W1 -> A2, no h)
 *   m_grouped_fp8_gemm_nt_contiguous  A2 x W2 [G][H][I] -> y [m_pad_max][H]
 *   moe_combine            y -> out [T][H]
 * Every buffer is sized by m_pad_max = moe_max_padded_rows(T, topk, G), an
 * upper bound of the padded row count; rows past the real count carry group
 * -1 and are skipped by the grouped product. */

/* Upper bound of the padded rows: roundup(T*topk + G*127, 128) (or -1 on
 * bad arguments).  Host-only. */
int64_t moe_max_padded_rows(int64_t tokens, int32_t topk, int32_t num_experts);
/* Bytes of device workspace moe_route_contiguous needs (or -1).  Host-only. */
int64_t moe_route_workspace_bytes(int64_t tokens, int32_t num_experts);

/* Routing layout.  topk_idx [tokens][topk] int32, the experts of each token
 * (values outside [0, num_experts) drop that slot).  Outputs (device):
 * counts [num_experts] pairs per expert; m_indices [m_pad_max] the expert of
 * each row or -1 (expert e owns rows starts[e] .. starts[e] + counts[e] - 1,
 * starts 128-aligned, experts in order); token_of_row [m_pad_max] the token of
 * each row or -1; row_of [tokens][topk] the row of each pair or -1.  Within an
 * expert, pairs are ordered by (token, slot).  workspace: device scratch of
 * workspace_bytes >= moe_route_workspace_bytes(tokens, num_experts).
 * Requirements: 1 <= topk <= 8, 1 <= num_experts <= 2048, m_pad_max a
 * multiple of 128 and >= moe_max_padded_rows(tokens, topk, num_experts). */
int moe_route_contiguous(const int32_t* topk_idx, int64_t tokens, int32_t topk, int32_t num_experts, int32_t* counts,
                         int32_t* m_indices, int32_t* token_of_row, int32_t* row_of, int64_t m_pad_max,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* moe_route_contiguous without a workspace argument, for callers that
 * cannot allocate device memory (code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation).  Same arguments (minus
 * workspace and workspace_bytes), same requirements and the same outputs,
 * bit for bit.  The routing workspace is a fixed device array inside the
 * library, one per device, of moe_route_noalloc_max_workspace_bytes() bytes
 * (4 MiB), held from the first call on a device until the process ends; no
 * call allocates or frees anything.  Problems whose
 * moe_route_workspace_bytes(tokens, num_experts) exceeds that size are
 * rejected with FGFP8_EINVAL (e.g. 256 experts allow up to ~1M tokens).
 * Every call on one device shares the array and leaves its contents behind
 * (nothing in it needs to start at zero: each call writes every entry it
 * reads).  Calls that overlap in time on one device -- on different streams,
 * or from different host threads -- therefore race and give undefined
 * results: serialize them (one stream, or events). */
int moe_route_contiguous_noalloc(const int32_t* topk_idx, int64_t tokens, int32_t topk, int32_t num_experts,
                                 int32_t* counts, int32_t* m_indices, int32_t* token_of_row, int32_t* row_of,
                                 int64_t m_pad_max, void* stream);
/* The size of the fixed routing workspace above, in bytes.  Host-only. */
int64_t moe_route_noalloc_max_workspace_bytes(void);

/* Row r of the layout = x[token_of_row[r]] (a zero row for an index outside
 * [0, tokens)), quantized exactly as quantize_fp8_groups.  x [tokens][k] bf16;
 * q [m_pad_max][k] E4M3; sa [k/128][sa_ld], sa_ld >= m_pad_max, sa_ld % 4 == 0;
 * k % 128 == 0. */
int moe_gather_quantize(const void* x_bf16, int64_t tokens, int64_t k, const int32_t* token_of_row, int64_t m_pad_max,
                        void* q_e4m3, float* sa, int64_t sa_ld, void* stream);

/* moe_gather_quantize for the layout moe_route_contiguous writes, by token:
 * each token's row of x is read and quantized once and its codes and scales
 * are written to every row row_of[t][j] (j < topk) it was routed to; rows
 * r < m_pad_max whose token_of_row entry lies outside [0, tokens) get zero
 * codes and scale 1 (a zero row, quantized).  With row_of and token_of_row
 * the inverse maps the routing writes, q and sa equal what
 * moe_gather_quantize writes, byte for byte: a row's codes depend on its
 * values only.  It reads x once instead of once per routed slot.
 * x [tokens][k] bf16; row_of [tokens][topk] int32; token_of_row [m_pad_max]
 * int32; q [m_pad_max][k] E4M3; sa [k/128][sa_ld], sa_ld >= m_pad_max,
 * sa_ld % 4 == 0.  Requirements: 1 <= topk <= 8, k % 128 == 0. */
int moe_gather_quantize_tokens(const void* x_bf16, int64_t tokens, int64_t k, int32_t topk, const int32_t* row_of,
                               const int32_t* token_of_row, int64_t m_pad_max, void* q_e4m3, float* sa, int64_t sa_ld,
                               void* stream);

/* act[r][c] = bf16(silu(h[r][c]) * h[r][inter + c]) in FP32 (silu(g) =
 * g / (1 + exp(-g)), the gate half first), quantized per 1x128 group as
 * quantize_fp8_groups: q [m][inter], sa [inter/128][sa_ld].  Rows whose
 * m_indices entry is negative are zero rows.  h [m][2*inter] bf16. */
int silu_mul_quantize(const void* h_bf16, int64_t m, int64_t inter, const int32_t* m_indices, void* q_e4m3, float* sa,
                      int64_t sa_ld, void* stream);

/* The two steps above in one kernel (the gate_up product with SiLU-times-up
 * and the activation quantizer in its epilogue; h never reaches memory):
 * q [m][inter] and sq [inter/128][sq_ld] are exactly what
 * m_grouped_fp8_gemm_nt_contiguous(a, sa, sa_ld, m_indices, w1, sb1,
 * num_groups, h) followed by silu_mul_quantize(h, m, inter, m_indices, q, sq,
 * sq_ld) write, bit for bit, on every 128-row block whose first row's group
 * lies in [0, num_groups); a block whose first row is outside that range
 * (padding) gets zero codes and scale 1, as silu_mul_quantize gives rows of
 * group -1.  w1 [num_groups][2*inter][k] E4M3 (the gate rows, then the up
 * rows) with sb1 [num_groups][2*inter/128][k/128] from the block quantizer;
 * a [m][k], sa [k/128][sa_ld] as for the grouped product.  Requirements:
 * m % 128 == 0, k % 128 == 0, inter % 128 == 0, (inter + 128) * k < 2^31,
 * sa_ld and sq_ld multiples of 4 and >= m. */
int moe_gate_up_silu_quantize(const void* a_e4m3, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                              const void* w1_e4m3, const float* sb1, int32_t num_groups, void* q_e4m3, float* sq,
                              int64_t sq_ld, int64_t m, int64_t inter, int64_t k, void* stream);

/* out[t][c] = bf16(sum_{j < topk} topk_weights[t][j] * y[row_of[t][j]][c]),
 * summed in FP32 in slot order; slots whose row lies outside [0, y_rows) are
 * skipped.  y [y_rows][hdim] bf16, row_of and topk_weights [tokens][topk],
 * out [tokens][hdim] bf16, hdim % 8 == 0, 1 <= topk <= 8. */
int moe_combine(const void* y_bf16, int64_t y_rows, int64_t hdim, const int32_t* row_of, const float* topk_weights,
                int64_t tokens, int32_t topk, void* out_bf16, void* stream);

/* Message for the most recent non-zero status returned on the calling thread
 * (thread-local; the pointer stays valid until the next failing call on that
 * thread).  Returns "" if no call has failed. */
const char* fgfp8_last_error(void);

/* Writes a NUL-terminated description of the kernel configuration that
 * fp8_gemm_nt would use for (m, n, k) into buf (at most len bytes, truncated)
 * and returns FGFP8_OK; host-only, enqueues nothing, touches no device.
 * Mirrors the pages' habit of printing every tile decision next to the
 * number it produced (deepgemm-rust README, "Benchmark").  For m > 16 the
 * environment variable FGFP8_GEMM_TILE, set to one of the tile names
 * (tile256x256_w4x2, tile256x192_w4x3, tile256x128_w4x2, tile128x256_w2x4,
 * tile128x128_w2x2), forces that tile in fp8_gemm_nt (tuning and tests; the
 * FP8-output call takes tile256x256_w4x2 for tile256x192_w4x3); other values
 * are ignored.  FGFP8_SPLITK=1 (0) forces (forbids) the K-split plan of
 * fp8_gemm_nt_ws for k >= 256.  FGFP8_PERSISTENT=1 (0) forces (forbids)
 * the persistent tile walk of fp8_gemm_nt (bf16 output, FP32 scales) and
 * m_grouped_fp8_gemm_nt_contiguous for k >= 256: one workgroup per compute
 * unit, the K pipeline continuing across tiles, same results bit for bit.
 * By default it is taken where it measured faster: two or more rounds of
 * 256x256 tiles in fp8_gemm_nt, and two or more rounds of tiles at
 * k <= 4096 in the grouped call (the description then ends in
 * "persistent"); every other tile is a workgroup of its own.  FGFP8_DECODE_XQ
 * (any value) makes fp8_linear_nt's fused path use the register-quantizing
 * kernel at every m <= 16 (tests; same bits).  FGFP8_DECODE_SLABS=1|3 sets
 * the 16-column weight slabs per workgroup of the m <= 16 product (by
 * default 3 for m > 4 where the shape allows, else 1; the description then
 * ends in "slabs=3"; same values either way).  FGFP8_MASKED_TILE, set to
 * tile128x256_w2x4 or tile128x128_w2x2, forces that tile in
 * m_grouped_fp8_gemm_nt_masked in place of the one expected_m selects
 * (tuning and tests; same values).  FGFP8_MASKED_SPLIT=1 (0) forces (forbids)
 * the split walk of m_grouped_fp8_gemm_nt_masked_ws.  FGFP8_PRINT_CONFIG=1
 * prints each call's kernel choice to stderr. */
int fgfp8_describe_gemm(int64_t m, int64_t n, int64_t k, char* buf, int64_t len);

/* The kernel m_grouped_fp8_gemm_nt_contiguous runs for an m x n x k call
 * (m the padded row count, a multiple of 128): "tile128x512_w2x4" (8 waves
 * of 64x128, one workgroup per 128-row block and 512 columns; its scales
 * are loaded into registers) or "tile128x256_w2x4" (8 waves of 64x64),
 * followed by " persistent" when the 128x256 tiles are walked by one
 * workgroup per compute unit.  The tile with fewer CU-rounds times tile area
 * over its measured efficiency is taken; FGFP8_GROUPED_TILE, set to one of
 * the two names, forces it (tuning and tests; same values either way).
 * Without it, K <= 1024 takes 128x256 (its walk is ahead there).  K of
 * 2^23 or more always takes 128x256 (the wide tile's 512-row weight panel
 * would pass 32-bit buffer offsets).
 * Writes a NUL-terminated string of at most len bytes into buf.  Host-only.
 * FGFP8_EINVAL for a null buffer or a bad shape. */
int fgfp8_describe_grouped(int64_t m, int64_t n, int64_t k, char* buf, int64_t len);

/* The path fp8_linear_nt takes for an m x n x k call, act_out non-zero when
 * the caller passes q_e4m3/sa: "fused act-quant + decode_splitk_slab16
 * split=S slabs=L form=F" (F = lds4, lds16 or registers, as described at
 * fp8_linear_nt) or "quantize_fp8_groups + " and fgfp8_describe_gemm's text.
 * Writes a NUL-terminated string of at most len bytes into buf.  Host-only.
 * FGFP8_EINVAL for a null buffer, a bad shape, or m > 16 with act_out == 0
 * (fp8_linear_nt needs the workspace there). */
int fgfp8_describe_linear(int64_t m, int64_t n, int64_t k, int act_out, char* buf, int64_t len);

/* Measurement aid: reads `bytes` of device memory at src once (bytes a
 * multiple of 32768), with nothing else to do -- the practical ceiling of
 * the HBM-bound calls at a given size (the decode product reads its weight
 * once per call).  Each thread stores one 16-byte XOR of what it read into
 * out (out_bytes >= 4096; the grid is at most out_bytes / 4096 workgroups of
 * 256 threads), so that no load is dropped.  Pointers 16-byte aligned. */
int fgfp8_stream_read(const void* src, int64_t bytes, void* out, int64_t out_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FGFP8_H_ */
