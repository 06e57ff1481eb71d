// The FP8 mixture-of-experts layer around the grouped product, with no
// device-to-host synchronisation (deepgemm-rust README, "What's implemented",
// moe_fp8_layer row: histogram -> offsets -> gather -> grouped GEMM ->
// SiLU.mul -> grouped GEMM -> weighted combine):
//
//   route      per-expert counts of the routed (token, slot) pairs, 128-row
//              aligned group offsets, and each pair's row in the contiguous
//              layout (tokens of an expert in ascending order);
//   gather     the routed rows of x, quantized per 1x128 group (exactly the
//              arithmetic of quantize_fp8_groups) into the layout;
//   (grouped product, gate_up)
//   silu_mul   act = bf16(silu(gate) * up) per row, quantized per 1x128 group;
//   (grouped product, down)
//   combine    out[t] = bf16(sum_j w[t][j] * y[row(t, j)]), the slots j in
//              order, in FP32.
//
// The routing buffers cover an upper bound of rows (m_pad_max); rows past the
// real padded count carry group -1 and are skipped by the grouped product, so
// no count ever has to reach the host.

#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace fgfp8 {

constexpr int kRouteThreads = 256;  // tokens per routing block

// ------------------------------------------------------------------ route
// Pass 1: per-block per-expert pair counts.
__global__ __launch_bounds__(kRouteThreads) void moe_count_kernel(const int32_t* __restrict__ topk_idx,
                                                                  int64_t tokens, int topk, int experts,
                                                                  int32_t* __restrict__ block_counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < experts; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  if (t < tokens) {
    for (int j = 0; j < topk; j++) {
      const int e = topk_idx[t * topk + j];
      if (e >= 0 && e < experts) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < experts; e += blockDim.x) block_counts[(int64_t)blockIdx.x * experts + e] = cnt[e];
}

// Pass 2 (one workgroup): totals, 128-aligned group starts, and each block's
// first row per expert (block_counts is turned into block bases in place).
__global__ __launch_bounds__(256) void moe_offsets_kernel(int32_t* __restrict__ block_counts, int nblocks,
                                                          int experts, int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ starts) {
  // every thread owns experts e = threadIdx.x + 256 i; the exclusive scan of
  // the padded totals runs over the experts in order in LDS.  The block
  // counts are read kBatch blocks at a time (independent loads), first to
  // sum them, then again to write each block's offset, so a thread waits
  // for memory once per batch rather than once per block.
  constexpr int kBatch = 8;
  extern __shared__ int32_t padded[];
  for (int e = threadIdx.x; e < experts; e += blockDim.x) {
    int32_t run = 0;
    for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
      int32_t c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; i++) c[i] = b0 + i < nblocks ? block_counts[(int64_t)(b0 + i) * experts + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; i++) run += c[i];
    }
    counts[e] = run;
    padded[e] = (run + 127) / 128 * 128;
  }
  __syncthreads();
  {
    // exclusive scan of padded[] over the experts: thread t takes the
    // contiguous run e0 .. e1 - 1 (at most 8 experts for 2048), a wave
    // shuffle scan and the four wave totals give the run's first offset
    __shared__ int32_t wave_total[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int per = (experts + 255) / 256;
    const int e0 = threadIdx.x * per < experts ? threadIdx.x * per : experts;
    const int e1 = e0 + per < experts ? e0 + per : experts;
    int32_t local = 0;
    for (int e = e0; e < e1; e++) local += padded[e];
    int32_t incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int32_t off = incl - local;
    for (int w = 0; w < wave; w++) off += wave_total[w];
    for (int e = e0; e < e1; e++) {
      const int32_t p = padded[e];
      padded[e] = off;
      off += p;
    }
  }
  __syncthreads();
  // each block's first row for expert e: the expert's start plus the
  // expert's pairs in the blocks before it
  for (int e = threadIdx.x; e < experts; e += blockDim.x) {
    int32_t run = padded[e];
    starts[e] = run;
    for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
      int32_t c[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; i++) c[i] = b0 + i < nblocks ? block_counts[(int64_t)(b0 + i) * experts + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; i++) {
        if (b0 + i < nblocks) block_counts[(int64_t)(b0 + i) * experts + e] = run;
        run += c[i];
      }
    }
  }
}

// Pass 3: every row of the layout gets its group (or -1) and, for now, no
// token.
__global__ void moe_rows_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ starts,
                                int experts, int64_t m_pad_max, int32_t* __restrict__ m_indices,
                                int32_t* __restrict__ token_of_row) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= m_pad_max) return;
  // last expert whose start is <= r (starts ascend)
  int lo = 0, hi = experts - 1, e = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) / 2;
    if (starts[mid] <= r) {
      e = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  m_indices[r] = (e >= 0 && r < (int64_t)starts[e] + counts[e]) ? e : -1;
  token_of_row[r] = -1;
}

// Pass 4: each pair's row = its block's base for the expert + the number of
// the block's earlier pairs routed to the same expert, pairs ordered by
// (token, slot): an exclusive prefix over the wave's lanes of each lane's
// pair count for the expert (bit-plane ballots; a count is at most 8), a
// prefix over the block's waves through LDS, and the earlier slots of the
// same token.  An expert's tokens thus keep their ascending order.
__global__ __launch_bounds__(kRouteThreads) void moe_assign_kernel(const int32_t* __restrict__ topk_idx,
                                                                   int64_t tokens, int topk, int experts,
                                                                   const int32_t* __restrict__ block_bases,
                                                                   int32_t* __restrict__ row_of,
                                                                   int32_t* __restrict__ token_of_row) {
  extern __shared__ int32_t wave_counts[];  // [4 waves][experts]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * kRouteThreads + threadIdx.x;
  const bool live = t < tokens;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int my_e[8], my_rank[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    my_e[j] = (live && j < topk) ? topk_idx[t * topk + j] : -1;
    my_rank[j] = 0;
  }
  for (int e = 0; e < experts; e++) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) c += my_e[j] == e ? 1 : 0;
    int prefix = 0, total = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint64_t mask = __ballot((c >> b) & 1);
      prefix += __popcll(mask & below) << b;
      total += __popcll(mask) << b;
    }
    if (lane == 0) wave_counts[wave * experts + e] = total;
    int seen = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      if (my_e[j] == e) {
        my_rank[j] = prefix + seen;
        seen++;
      }
    }
  }
  __syncthreads();
  if (!live) return;
  for (int j = 0; j < topk; j++) {
    const int e = my_e[j];
    if (e < 0 || e >= experts) {
      row_of[t * topk + j] = -1;
      continue;
    }
    int before = 0;
    for (int w = 0; w < wave; w++) before += wave_counts[w * experts + e];
    const int32_t row = block_bases[(int64_t)blockIdx.x * experts + e] + before + my_rank[j];
    row_of[t * topk + j] = row;
    token_of_row[row] = (int32_t)t;
  }
}

int64_t moe_route_workspace_bytes(int64_t tokens, int experts) {
  const int64_t nblocks = (tokens + kRouteThreads - 1) / kRouteThreads;
  return nblocks * experts * 4 + (int64_t)experts * 4;
}

// ------------------------------------------- routing without allocation
// A fixed routing workspace for callers that cannot allocate device memory:
// the per-256-token-block expert counts and the group starts of
// launch_moe_route live in this array.  Each device that runs the library
// holds its own copy (kRouteScratchInts int32, 4 MiB) until the process
// ends.  Host code never passes the symbol itself to a kernel: its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept in g_route_scratch.
constexpr int64_t kRouteScratchInts = int64_t(1) << 20;
static __device__ __align__(256) int32_t scratch[kRouteScratchInts];

int64_t moe_route_scratch_bytes() { return kRouteScratchInts * 4; }

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_route_scratch[kScratchDevices];
}  // namespace

hipError_t moe_route_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_route_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_route_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_moe_route(const int32_t* topk_idx, int64_t tokens, int topk, int experts, int32_t* counts,
                            int32_t* m_indices, int32_t* token_of_row, int32_t* row_of, int64_t m_pad_max,
                            void* workspace, hipStream_t stream) {
  const int nblocks = (int)((tokens + kRouteThreads - 1) / kRouteThreads);
  int32_t* block_counts = static_cast<int32_t*>(workspace);
  int32_t* starts = block_counts + (int64_t)nblocks * experts;
  if (nblocks > 0) {
    hipLaunchKernelGGL(moe_count_kernel, dim3(nblocks), dim3(kRouteThreads), experts * 4, stream, topk_idx, tokens,
                       topk, experts, block_counts);
  }
  hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(256), experts * 4, stream, block_counts, nblocks, experts,
                     counts, starts);
  hipLaunchKernelGGL(moe_rows_kernel, dim3((uint32_t)((m_pad_max + 255) / 256)), dim3(256), 0, stream, counts,
                     starts, experts, m_pad_max, m_indices, token_of_row);
  if (nblocks > 0) {
    hipLaunchKernelGGL(moe_assign_kernel, dim3(nblocks), dim3(kRouteThreads), 4 * experts * 4, stream, topk_idx,
                       tokens, topk, experts, block_counts, row_of, token_of_row);
  }
  return hipGetLastError();
}

// ------------------------------------------------ gather + quantize, act
// One wave quantizes 4 rows x 4 groups (as quantize_groups_kernel).  GATHER:
// row r of the layout reads x[token_of_row[r]] (a row of zeros for an index
// outside [0, tokens)).
// SILU: row r reads gate = h[r][col] and up = h[r][inter + col] (bf16) and
// forms bf16(silu(gate) * up) in FP32 first; rows of group -1 are zeros.
template <bool SILU>
__global__ __launch_bounds__(256) void moe_quantize_kernel(const uint16_t* __restrict__ src, int64_t src_rows,
                                                           const int32_t* __restrict__ sel, int64_t m, int64_t k,
                                                           int64_t src_ld, uint8_t* __restrict__ q,
                                                           float* __restrict__ sa, int64_t sa_ld,
                                                           int64_t group_quads, int64_t total_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;  // wave-uniform
  const int64_t r0 = (blk / group_quads) * 4;
  const int64_t g = (blk % group_quads) * 4 + (lane >> 4);
  const bool g_ok = g < k / kGroup;
  const int64_t col = g * kGroup + (lane & 15) * 8;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t r = r0 + i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (!g_ok || r >= m) continue;
    const int32_t s = sel[r];
    if (s < 0 || (!SILU && s >= src_rows)) continue;
    if (!SILU) {
      v[i] = *reinterpret_cast<const uint4*>(src + (int64_t)s * src_ld + col);
    } else {
      const uint4 gt = *reinterpret_cast<const uint4*>(src + r * src_ld + col);
      const uint4 up = *reinterpret_cast<const uint4*>(src + r * src_ld + k + col);
      const uint32_t gw[4] = {gt.x, gt.y, gt.z, gt.w}, uw[4] = {up.x, up.y, up.z, up.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float g0 = bf16_lo(gw[e]), g1 = bf16_hi(gw[e]);
        const float a0 = silu_mul_f32(g0, bf16_lo(uw[e]));
        const float a1 = silu_mul_f32(g1, bf16_hi(uw[e]));
        o[e] = pack_bf16x2(a0, a1);
      }
      v[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t amax_bits = row16_max_u32(absmax8_bits(v[i]));
    s[i] = group_scale(__uint_as_float(amax_bits));
    const double r = 1.0 / (double)s[i];
    const uint2 o = quantize8(v[i], r);
    if (g_ok && r0 + i < m) *reinterpret_cast<uint2*>(q + (r0 + i) * k + col) = o;
  }
  if (g_ok && (lane & 15) == 0) {
    float* dst = sa + g * sa_ld + r0;
    if (r0 + 4 <= m) {
      *reinterpret_cast<float4*>(dst) = make_float4(s[0], s[1], s[2], s[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (r0 + i < m) dst[i] = s[i];
    }
  }
}

static hipError_t launch_moe_quantize(bool silu, const void* src, int64_t src_rows, const int32_t* sel, int64_t m,
                                      int64_t k,
                                      int64_t src_ld, void* q, float* sa, int64_t sa_ld, hipStream_t stream) {
  const int64_t group_quads = (k / kGroup + 3) / 4;
  const int64_t total = (m + 3) / 4 * group_quads;
  const dim3 grid((uint32_t)((total + 3) / 4)), block(256);
  if (silu)
    hipLaunchKernelGGL(moe_quantize_kernel<true>, grid, block, 0, stream, static_cast<const uint16_t*>(src), src_rows,
                       sel, m, k, src_ld, static_cast<uint8_t*>(q), sa, sa_ld, group_quads, total);
  else
    hipLaunchKernelGGL(moe_quantize_kernel<false>, grid, block, 0, stream, static_cast<const uint16_t*>(src), src_rows,
                       sel, m, k, src_ld, static_cast<uint8_t*>(q), sa, sa_ld, group_quads, total);
  return hipGetLastError();
}

hipError_t launch_moe_gather_quantize(const void* x, int64_t tokens, int64_t k, const int32_t* token_of_row,
                                      int64_t m_pad_max, void* q, float* sa, int64_t sa_ld, hipStream_t stream) {
  return launch_moe_quantize(false, x, tokens, token_of_row, m_pad_max, k, k, q, sa, sa_ld, stream);
}

hipError_t launch_moe_silu_mul_quantize(const void* h, int64_t m, int64_t inter, const int32_t* m_indices, void* q,
                                        float* sa, int64_t sa_ld, hipStream_t stream) {
  return launch_moe_quantize(true, h, m, m_indices, m, inter, 2 * inter, q, sa, sa_ld, stream);
}

// ------------------------------------------- gather + quantize, by token
// The same rows as the gather above when row_of and token_of_row are the
// inverse maps the routing writes, but each token's row of x is read and
// quantized once: a wave quantizes 4 tokens x 4 groups (as
// quantize_groups_kernel) and writes every token's codes and scales to each
// row row_of[t][j] it was routed to.  A row's codes depend on its values
// only, so every copy holds the bytes the row-major gather writes.  The
// rows no token maps to (padding, and the rows past the real count) are
// written by moe_zero_rows_kernel below.
__global__ __launch_bounds__(256) void moe_gather_tokens_kernel(const uint16_t* __restrict__ x, int64_t tokens,
                                                                int64_t k, const int32_t* __restrict__ row_of,
                                                                int topk, int64_t m_pad_max, uint8_t* __restrict__ q,
                                                                float* __restrict__ sa, int64_t sa_ld,
                                                                int64_t group_quads, int64_t total_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= total_blocks) return;  // wave-uniform
  const int64_t t0 = (blk / group_quads) * 4;
  const int64_t g = (blk % group_quads) * 4 + (lane >> 4);
  const bool g_ok = g < k / kGroup;
  const int64_t col = g * kGroup + (lane & 15) * 8;
  // the rows of the wave's (up to) 4 tokens: lane i * topk + j holds row_of[t0 + i][j]
  const int64_t nidx = (tokens - t0 < 4 ? tokens - t0 : 4) * topk;
  const int32_t my_row = lane < nidx ? row_of[t0 * topk + lane] : -1;
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; i++)
    v[i] = (g_ok && t0 + i < tokens) ? *reinterpret_cast<const uint4*>(x + (t0 + i) * k + col) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (t0 + i >= tokens) break;  // uniform
    const uint32_t amax_bits = row16_max_u32(absmax8_bits(v[i]));
    const float s = group_scale(__uint_as_float(amax_bits));
    const double r = 1.0 / (double)s;
    const uint2 o = quantize8(v[i], r);
    for (int j = 0; j < topk; j++) {
      const int32_t row = __builtin_amdgcn_readlane(my_row, i * topk + j);
      if (row < 0 || row >= m_pad_max) continue;  // a dropped slot; uniform
      if (g_ok) {
        *reinterpret_cast<uint2*>(q + (int64_t)row * k + col) = o;
        if ((lane & 15) == 0) sa[g * sa_ld + row] = s;
      }
    }
  }
}

// Rows r < m_pad_max whose token_of_row entry lies outside [0, tokens): a
// zero row quantized -- zero codes, scale 1 (the all-zero group's scale).
// A wave takes 64 rows and one 1 KB column slice of them (blockIdx.y): it
// finds its zero rows with one ballot and writes each row's slice with one
// 16-byte store per lane, and the scales of its share of the K groups with
// lane i holding row i (one coalesced store per group).  The zero rows bunch
// up (each group's padding and the whole tail past the real count), so
// splitting the columns over waves keeps one wave from writing 64 whole rows
// in a row, and the MN-major scales are written a group column at a time
// rather than a row at a time (measured on the 8192-token layer's ~4000 zero
// rows of 7 KB: 26 us for 64 whole rows per wave with per-row scale stores,
// 17 us with column slices, 11 us with the scales by column as well).
__global__ __launch_bounds__(256) void moe_zero_rows_kernel(const int32_t* __restrict__ token_of_row, int64_t tokens,
                                                            int64_t k, int64_t m_pad_max, uint8_t* __restrict__ q,
                                                            float* __restrict__ sa, int64_t sa_ld) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int64_t r = r0 + lane;
  bool zero = false;
  if (r < m_pad_max) {
    const int32_t t = token_of_row[r];
    zero = t < 0 || t >= tokens;
  }
  uint64_t mask = __ballot(zero);
  const int64_t kb = k / kGroup;
  const int64_t c16 = (int64_t)blockIdx.y * 64 + lane;  // this lane's 16-byte column slot
  if (mask == 0) return;  // uniform
  const int64_t per = (kb + gridDim.y - 1) / gridDim.y, c0 = (int64_t)blockIdx.y * per;
  if (zero)
    for (int64_t c = c0; c < c0 + per && c < kb; c++) sa[c * sa_ld + r] = 1.0f;
  while (mask != 0) {  // uniform
    const int b = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int64_t row = r0 + b;
    if (c16 < k / 16) reinterpret_cast<uint4*>(q + row * k)[c16] = make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_moe_gather_quantize_tokens(const void* x, int64_t tokens, int64_t k, int topk,
                                             const int32_t* row_of, const int32_t* token_of_row, int64_t m_pad_max,
                                             void* q, float* sa, int64_t sa_ld, hipStream_t stream) {
  if (m_pad_max > 0)
    hipLaunchKernelGGL(moe_zero_rows_kernel, dim3((uint32_t)((m_pad_max + 255) / 256), (uint32_t)((k / 16 + 63) / 64)),
                       dim3(256), 0, stream, token_of_row, tokens, k, m_pad_max, static_cast<uint8_t*>(q), sa, sa_ld);
  const int64_t group_quads = (k / kGroup + 3) / 4;
  const int64_t total = (tokens + 3) / 4 * group_quads;
  if (total > 0)
    hipLaunchKernelGGL(moe_gather_tokens_kernel, dim3((uint32_t)((total + 3) / 4)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), tokens, k, row_of, topk, m_pad_max,
                       static_cast<uint8_t*>(q), sa, sa_ld, group_quads, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// One workgroup per token; each thread sums 8 columns over the token's slots
// in order (FP32), then rounds to bf16.  Slots whose row lies outside
// [0, y_rows) are skipped.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ y, int64_t y_rows, int64_t hdim,
                                                          const int32_t* __restrict__ row_of,
                                                          const float* __restrict__ w, int topk,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < hdim; c += (int64_t)blockDim.x * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < topk; j++) {
      const int32_t r = row_of[t * topk + j];
      if (r < 0 || r >= y_rows) continue;
      const float wj = w[t * topk + j];
      const uint4 v = *reinterpret_cast<const uint4*>(y + (int64_t)r * hdim + c);
      const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        acc[2 * e] = __builtin_fmaf(wj, bf16_lo(vw[e]), acc[2 * e]);
        acc[2 * e + 1] = __builtin_fmaf(wj, bf16_hi(vw[e]), acc[2 * e + 1]);
      }
    }
    *reinterpret_cast<uint4*>(out + t * hdim + c) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                               pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

hipError_t launch_moe_combine(const void* y, int64_t y_rows, int64_t hdim, const int32_t* row_of, const float* w,
                              int64_t tokens, int topk, void* out, hipStream_t stream) {
  if (tokens > 0)
    hipLaunchKernelGGL(moe_combine_kernel, dim3((uint32_t)tokens), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(y), y_rows, hdim, row_of, w, topk, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace fgfp8
