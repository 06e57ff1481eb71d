// Host-side launchers of the gfx950 kernels (no validation here: the C ABI
// layer checks every argument before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgfp8 {

hipError_t launch_quantize_groups(const void* x, int64_t m, int64_t k, void* q, float* sa, int64_t sa_ld,
                                  hipStream_t stream, bool ue8m0 = false);
// MX recipe: per-1x32 power-of-two scales, E8M0 codes packed four to an
// int32, s int32 [k/128][s_ld].
// The groups quantizer over a dispatch buffer [num_groups][max_m][k]: rows
// r < masked_m[g] (clamped to [0, max_m]) of group g only; max_m % 4 == 0.
hipError_t launch_quantize_groups_masked(const void* x, const int32_t* masked_m, int32_t num_groups, int64_t max_m,
                                         int64_t k, void* q, float* sa, int64_t sa_ld, hipStream_t stream);
hipError_t launch_quantize_mx(const void* x, int64_t m, int64_t k, void* q, int32_t* s, int64_t s_ld,
                              hipStream_t stream);
hipError_t launch_quantize_blocks(const void* w, int64_t n, int64_t k, void* q, float* sb, hipStream_t stream,
                                  bool ue8m0 = false);

// Kernel configurations of the dense product.
enum GemmKind : int {
  kGemmTile256x256 = 0,  // 256x256 workgroup tile, 8 waves of 64x128
  kGemmTile128x256 = 1,  // 128x256, 8 waves of 64x64
  kGemmTile256x128 = 2,  // 256x128, 8 waves of 64x64
  kGemmTile128x128 = 3,  // 128x128, 4 waves of 64x64
  kGemmDecode = 4,       // M <= 16: 16-column slabs, K split across waves
  kGemmTile256x192 = 5,  // 256x192, 12 waves of 64x64
  kGemmTile256x256SplitK2 = 6,  // 256x256 tiles, K split over two workgroups (needs a workspace)
  kGemmTile128x512 = 7,  // 128x512, 8 waves of 64x128, scales in registers (grouped product)
};

struct GemmPlan {
  GemmKind kind;
  int split;  // decode: waves per 16-column slab (K split)
};

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k);
const char* gemm_kind_name(GemmKind kind);
// The plan when a workspace may be used: plan_gemm's, or the K-split 256x256
// tiles where those fill the compute units and whole tiles would not.
GemmPlan plan_gemm_ws(int64_t m, int64_t n, int64_t k);
// Workspace bytes of the K-split plan for (m, n, k) (0 for other plans):
// 2 ints per 256x256 tile (zero between calls), padded to 256 bytes, then
// one 256x256 FP32 partial per tile.
int64_t gemm_splitk_workspace_bytes(int64_t m, int64_t n);
hipError_t launch_gemm_splitk(const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb, void* d,
                              int64_t m, int64_t n, int64_t k, void* workspace, hipStream_t stream);

hipError_t launch_gemm(const GemmPlan& plan, const void* a, const float* sa, int64_t sa_ld, const void* b,
                       const float* sb, void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// UE8M0 recipe (every scale a power of two): the tile kernels let the matrix
// core apply the scales and accumulate across chunks (no FP32 promotion);
// decode shapes use the decode kernel, exact for such scales.
hipError_t launch_gemm_ue8m0(const GemmPlan& plan, const void* a, const float* sa, int64_t sa_ld, const void* b,
                             const float* sb, void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// FP8-output product (n % 128 == 0): q = quantize_groups(bf16(A . B^T)) per
// 1x128 group of each row with MN-major scales sd [n/128][sd_ld]; d (bf16)
// optional.  Tile kernels only; plan_tiles gives the tile for any m.
// MX product: packed E8M0 scale words sa int32 [k/128][sa_ld] (A rows) and
// sb int32 [k/128][sb_ld] (B rows, i.e. output columns).
hipError_t launch_gemm_mx(GemmKind kind, const void* a, const int32_t* sa, int64_t sa_ld, const void* b,
                          const int32_t* sb, int64_t sb_ld, void* d, int64_t m, int64_t n, int64_t k,
                          hipStream_t stream);
GemmKind plan_tiles(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_fp8out(GemmKind kind, const void* a, const float* sa, int64_t sa_ld, const void* b,
                              const float* sb, void* q, float* sd, int64_t sd_ld, void* d, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream);

// Decode-shaped products (M <= 16): K split over ks waves per 16-column slab.
// Decode plan: waves per slab (the K split) and slabs per workgroup.
struct DecodePlan {
  int ks, slabs;
};
DecodePlan decode_plan(int64_t m, int64_t n, int64_t k);
int decode_split(int64_t m, int64_t n, int64_t k);
hipError_t launch_decode(int ks, const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb,
                         void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream);
// Fused activation quantization + product: one kernel for M <= kFusedMaxM
// (any K).  Up to kFusedLdsMaxM rows it quantizes into LDS and beats the two
// launches; above that the register form is slower than them, so it runs
// only when the caller gives no workspace for the two-launch path.
constexpr int64_t kFusedMaxM = 16;
constexpr int64_t kFusedLdsMaxM = 4;
constexpr int64_t kFusedLdsMaxK = 32768;  // 4 x K bytes of LDS per workgroup
// Whether the fused call at 4 < M <= 16 quantizes into LDS too (three slabs
// per workgroup and few enough quantize tasks per lane; act_out: the caller
// also wants the quantized activation, so the two-launch path is the
// alternative).
bool decode_fused_wide(int64_t m, int64_t n, int64_t k, bool act_out);
hipError_t launch_decode_fused(const void* x, const void* b, const float* sb, void* d, int64_t m, int64_t n,
                               int64_t k, void* q_out, float* sa_out, int64_t sa_out_ld, hipStream_t stream);

// Whether a product with this K runs the persistent tile walk.
bool use_persistent(int64_t tiles, int64_t k, bool grouped, bool measured_tile);
// Whether fp8_gemm_nt (bf16 output, FP32 scales) runs this plan's tiles as the persistent walk.
bool plan_persistent(const GemmPlan& plan, int64_t m, int64_t n, int64_t k);
// The grouped product's tile (kGemmTile128x512 or kGemmTile128x256).
GemmKind plan_grouped_gemm(int64_t m, int64_t n, int64_t k);
bool plan_grouped_walk(int64_t m, int64_t n, int64_t k);
hipError_t launch_grouped_gemm(const void* a, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                               const void* b, const float* sb, int32_t num_groups, void* d, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream);

// The MoE gate_up product fused with SiLU-times-up and the 1x128 activation
// quantizer: w1 [G][2*inter][k] (gate rows, then up rows), sb1
// [G][2*inter/128][k/128]; writes q [m][inter] (E4M3) and sq [inter/128][sq_ld].
hipError_t launch_grouped_gemm_silu(const void* a, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                                    const void* w1, const float* sb1, int32_t num_groups, void* q, float* sq,
                                    int64_t sq_ld, int64_t m, int64_t inter, int64_t k, hipStream_t stream);

// Masked grouped product: a 128-row tile chosen from the expected rows per
// group (a host-side hint; the per-group counts stay on the device).
GemmKind plan_masked(int32_t num_groups, int64_t max_m, int64_t expected_m, int64_t n);
hipError_t launch_masked_gemm(GemmKind kind, const void* a, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                              const void* b, const float* sb, int32_t num_groups, int64_t max_m, void* d, int64_t n,
                              int64_t k, hipStream_t stream);
// The masked product over a workspace of masked_split_workspace_bytes():
// one workgroup per CU walks the live tiles, the last round's tiles split
// along K when it would leave CUs idle.  The workspace is zero before the
// first call; each call leaves it so.
int64_t masked_split_workspace_bytes();
// Whether that form pays for this call (from the expected rows per group).
bool masked_split_walk(GemmKind kind, int32_t num_groups, int64_t max_m, int64_t expected_m, int64_t n);
hipError_t launch_masked_gemm_split(GemmKind kind, const void* a, const float* sa, int64_t sa_ld,
                                    const int32_t* masked_m, const void* b, const float* sb, int32_t num_groups,
                                    int64_t max_m, void* d, int64_t n, int64_t k, void* workspace, hipStream_t stream);

// Streaming read (measurement aid): bytes (a multiple of
// stream_read_unit_bytes()) of src read once; out receives one 16-byte XOR
// per thread of a grid of at most out_bytes / 4096 workgroups.
int64_t stream_read_unit_bytes();
hipError_t launch_stream_read(const void* src, int64_t bytes, void* out, int64_t out_bytes, hipStream_t stream);

// Mixture-of-experts layer steps around the grouped product.
int64_t moe_route_workspace_bytes(int64_t tokens, int experts);
hipError_t launch_moe_route(const int32_t* topk_idx, int64_t tokens, int topk, int experts, int32_t* counts,
                            int32_t* m_indices, int32_t* token_of_row, int32_t* row_of, int64_t m_pad_max,
                            void* workspace, hipStream_t stream);
// The fixed routing workspace of the allocation-free routing call: its size
// in bytes, and its device address on the current device (looked up once per
// device).  Every call on a device shares it.
int64_t moe_route_scratch_bytes();
hipError_t moe_route_scratch(void** out);
// The same rows, each token's row read and quantized once and written to
// the rows row_of[t][j]; rows no token maps to get zero codes and scale 1.
hipError_t launch_moe_gather_quantize_tokens(const void* x, int64_t tokens, int64_t k, int topk,
                                             const int32_t* row_of, const int32_t* token_of_row, int64_t m_pad_max,
                                             void* q, float* sa, int64_t sa_ld, hipStream_t stream);
hipError_t launch_moe_gather_quantize(const void* x, int64_t tokens, int64_t k, const int32_t* token_of_row,
                                      int64_t m_pad_max, void* q, float* sa, int64_t sa_ld, hipStream_t stream);
hipError_t launch_moe_silu_mul_quantize(const void* h, int64_t m, int64_t inter, const int32_t* m_indices, void* q,
                                        float* sa, int64_t sa_ld, hipStream_t stream);
hipError_t launch_moe_combine(const void* y, int64_t y_rows, int64_t hdim, const int32_t* row_of, const float* w,
                              int64_t tokens, int topk, void* out, hipStream_t stream);

}  // namespace fgfp8
