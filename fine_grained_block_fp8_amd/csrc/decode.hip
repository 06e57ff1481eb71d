// Decode-shaped block-scaled FP8 products (M <= 16): a stream over the weight.
//
// Same definition as the dense product (deepgemm-rust README, "What's
// implemented" table, fp8_gemm_nt row; per-128-block scale promotion), but
// with at most 16 activation rows the work is bound by reading B (N*K bytes)
// from HBM: every decoded token streams the whole weight from memory again
// (AReno FP8 decode pull request, Summary).  A workgroup owns 16 output
// columns -- one 16-row slab of B, contiguous in memory -- and its KS waves
// split K into contiguous chunk ranges.  Each wave issues the loads of all
// its chunks (two 16-byte loads per lane per chunk, straight into MFMA
// fragment registers) before doing anything else, so the whole weight stream
// is in flight at once; then it forms one 16x16x128 MFMA per chunk with a
// zero accumulator and promotes it with sa * sb in FP32.  The KS partial
// tiles are summed through LDS in wave order.
//
// The fused variant takes the bf16 activation (M <= 4; decode_xq_kernel below
// covers M <= 16) and quantizes it per 1x128 group into LDS inside every
// workgroup, with exactly the arithmetic of quantize_fp8_groups, while the
// weight loads are in flight: one launch per decode linear instead of two (the
// pages' decode path spent its time in the per-call activation-quantize chain
// until that was fused into one kernel: AReno pull request, commit notes on
// fusing the activation quantize).  All variants share the chunk order and the
// reduction order, so their outputs are bit-identical.

#include <atomic>
#include <cstdlib>
#include <cstring>

#include "common.hpp"
#include "kernels.hpp"

namespace fgfp8 {

// Chunks of one wave held in registers at a time.  With KS <= 4 (the split
// of the wide shapes, N = 12288 at K = 4096: 768 slabs, three workgroups per
// CU) a wave holds 8 chunks and stays within 168 VGPRs, so three waves fit
// per SIMD; with KS = 8 (two waves per SIMD) it holds 12.  The A fragments of
// the non-fused form take registers too: it holds 8.  KS = 16 (N = 4096 at
// K = 12288: four waves per SIMD, 128 VGPRs) holds 6.
// With S = 3 slabs per workgroup a chunk brings three slabs' weight
// fragments: 4 chunks at a time (<= 8 waves, two per SIMD).
template <int KS, bool FUSED, int S = 1>
constexpr int decode_max_chunks() { return S > 1 ? 4 : (KS >= 16 ? 6 : (FUSED && KS >= 8 ? 12 : 8)); }
constexpr int kFusedMaxRows = (int)kFusedLdsMaxM;

__device__ __forceinline__ v8i_t frag_of(uint4 lo, uint4 hi) {
  v8i_t f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

__device__ __forceinline__ v4f_t mfma_fp8_dec(const v8i_t& x, const v8i_t& y) {
  const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// S slabs per workgroup (1 or 3): the workgroup owns 16 S consecutive output
// columns, and each wave's activation fragments of a chunk serve all S
// slabs' MFMAs, so the activation is read (or, fused, quantized) once per
// S slabs.  Every output takes the same chunks, promotions and wave-order
// reduction whatever S is, so the result does not depend on S.
//
// FUSED = false: A is E4M3 [M][K] with scales sa [K/128][sa_ld] in global
// memory.  FUSED = true: X is bf16 [M][K] (M <= MR), quantized here; if q_out
// is non-null, the quantized activation and its scales are written out too
// (q_out [M][K], sa_out [K/128][sa_out_ld]), each (row, group) task by
// workgroup task % gridDim.x, so that no workgroup carries all the writes
// (one writer made it the launch's last workgroup: +1.5 us at M = 16).  XA:
// activation loads per lane issued ahead of the weight stream (loads complete
// in issue order, so one issued after the stream can only be used once the
// whole stream has arrived): 3 covers M = 1; 12 covers M <= 4 at the common
// K; 16 covers the three-slab form's M * K/128 <= 512.
//
// MR: the activation rows the fused form's LDS holds (4, or 16 for the
// three-slab form at 4 < M <= 16; see launch_decode_fused).
template <int KS, bool FUSED, int XA = 3, int S = 1, int MR = kFusedMaxRows>
__global__ __launch_bounds__(KS * 64) void decode_kernel(const void* __restrict__ Ain, const float* __restrict__ SA,
                                                         int64_t sa_ld, const uint8_t* __restrict__ B,
                                                         const float* __restrict__ SB, uint16_t* __restrict__ D,
                                                         int M, int64_t N, int K, uint8_t* __restrict__ q_out,
                                                         float* __restrict__ sa_out, int64_t sa_out_ld) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int64_t nw = (int64_t)blockIdx.x * 16 * S;  // the workgroup's first column
  const int KB = K / kGroup;
  const int per = (KB + KS - 1) / KS;
  const int c_begin = wave * per;
  const int c_end = c_begin + per < KB ? c_begin + per : KB;
  rsrc_t rb[S], rsb[S];
#pragma unroll
  for (int sl = 0; sl < S; sl++) {
    const int64_t n0 = nw + 16 * sl;  // slabs past N get empty resources: every load reads zeros
    const uint32_t b_rows = (uint32_t)(N - n0 <= 0 ? 0 : (N - n0 < 16 ? N - n0 : 16));
    rb[sl] = make_rsrc(B + (b_rows ? n0 : 0) * K, b_rows * (uint32_t)K);
    rsb[sl] = make_rsrc(SB + (b_rows ? n0 / kGroup : 0) * KB, b_rows ? (uint32_t)KB * 4u : 0u);
  }
  const uint32_t off = (uint32_t)li * (uint32_t)K + (uint32_t)lg * 32u;
  const bool row_ok = li < M;

  // LDS: [red: S x KS x 64 x 16 B][FUSED: qa MR x K bytes][FUSED: scales KB x MR floats]
  v4f_t* red = reinterpret_cast<v4f_t*>(smem);
  uint8_t* qa = smem + S * KS * 64 * 16;
  float* qs = reinterpret_cast<float*>(qa + MR * K);

  // Every operand of a batch of chunks is requested before any is used, so
  // a wave waits for memory once per batch, not once per chunk: the B
  // fragments, the weight scales of the batch (one per lane, broadcast with
  // readlane) and, without fusion, the A fragments and activation scales.
  // Every load is issued unconditionally, as a buffer load: one past the end
  // of its operand (a chunk beyond the batch, a row beyond M) gets an offset
  // outside the resource and returns zeros without touching memory.  The
  // number of loads in flight is then the same on every path, so the
  // compiler waits for exactly the load an instruction needs -- a branch
  // around a load would make it wait for all of them (the whole weight
  // stream) before the first use.
  constexpr uint32_t kOob = 0x80000000u;
  constexpr int MAXC = decode_max_chunks<KS, FUSED, S>();
  v4f_t acc[S];
#pragma unroll
  for (int sl = 0; sl < S; sl++) acc[sl] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
  uint4 b0[MAXC][S], b1[MAXC][S], a0[FUSED ? 1 : MAXC], a1[FUSED ? 1 : MAXC];
  float sav[FUSED ? 1 : MAXC];
  float sbv[S];
  // the non-fused form's activation and its scales (M rows; scale column li
  // of chunk kb at kb * sa_ld + li)
  const rsrc_t ra = make_rsrc(FUSED ? nullptr : Ain, FUSED ? 0u : (uint32_t)M * (uint32_t)K);
  const rsrc_t rsa = make_rsrc(FUSED ? nullptr : SA, FUSED ? 0u : (uint32_t)((int64_t)KB * sa_ld * 4));
  // Small operands first: requests queue in order behind the weight stream,
  // so anything issued after it would arrive only when the stream has.
  auto issue = [&](int cb, int nc) {
#pragma unroll
    for (int sl = 0; sl < S; sl++)
      sbv[sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rsb[sl], lane < nc ? (uint32_t)(cb + lane) * 4u : kOob, 0, 0));
    if (!FUSED) {
      // A fragments and scales, every load issued (rows >= M and chunks past
      // the batch get out-of-range offsets and read zeros), so that the
      // compiler waits for each chunk's own loads rather than for the whole
      // batch before the first MFMA.
#pragma unroll
      for (int u = 0; u < MAXC; u++) {
        const bool ok = row_ok && u < nc;
        const uint32_t o = ok ? (uint32_t)li * (uint32_t)K + (uint32_t)(cb + u) * 128u + (uint32_t)lg * 32u : kOob;
        a0[u] = load_rsrc16(ra, o);
        a1[u] = load_rsrc16(ra, ok ? o + 16u : kOob);
        sav[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rsa, ok ? ((uint32_t)(cb + u) * (uint32_t)sa_ld + (uint32_t)li) * 4u : kOob, 0, 0));
      }
    }
#pragma unroll
    for (int u = 0; u < MAXC; u++) {
      const uint32_t o = u < nc ? off + (uint32_t)(cb + u) * 128u : kOob;
#pragma unroll
      for (int sl = 0; sl < S; sl++) {
        b0[u][sl] = load_rsrc16(rb[sl], o);
        b1[u][sl] = load_rsrc16(rb[sl], u < nc ? o + 16u : kOob);
      }
    }
  };
  // One MFMA per chunk into alternating partial registers, each promoted
  // after the next MFMA is issued (so the MFMAs do not wait on each other);
  // chunks are added to acc in order.
  auto compute = [&](int cb, int nc) {
    v4f_t part[2][S];
    float scl[2][S];
#pragma unroll
    for (int u = 0; u <= MAXC; u++) {
      if (u < nc) {
        const int kb = cb + u;
        v8i_t af;
        float sa_u;
        if (FUSED) {
          if (row_ok) {
            const uint8_t* p = qa + li * K + kb * kGroup + lg * 32;
            af = frag_of(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 16));
            sa_u = qs[kb * MR + li];
          } else {
            af = frag_of(make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0));
            sa_u = 0.0f;
          }
        } else {
          af = frag_of(a0[u], a1[u]);
          sa_u = sav[u];
        }
#pragma unroll
        for (int sl = 0; sl < S; sl++) {
          part[u & 1][sl] = mfma_fp8_dec(frag_of(b0[u][sl], b1[u][sl]), af);
          scl[u & 1][sl] =
              sa_u * __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sbv[sl]), u));
        }
        if (!FUSED) {  // registers are scarcer here: promote at once
#pragma unroll
          for (int sl = 0; sl < S; sl++) {
            const v4f_t& p = part[u & 1][sl];
            const float sc = scl[u & 1][sl];
            acc[sl][0] = __builtin_fmaf(p[0], sc, acc[sl][0]);
            acc[sl][1] = __builtin_fmaf(p[1], sc, acc[sl][1]);
            acc[sl][2] = __builtin_fmaf(p[2], sc, acc[sl][2]);
            acc[sl][3] = __builtin_fmaf(p[3], sc, acc[sl][3]);
          }
        }
      }
      if (FUSED && u > 0 && u - 1 < nc) {
#pragma unroll
        for (int sl = 0; sl < S; sl++) {
          const v4f_t& p = part[(u - 1) & 1][sl];
          const float sc = scl[(u - 1) & 1][sl];
          acc[sl][0] = __builtin_fmaf(p[0], sc, acc[sl][0]);
          acc[sl][1] = __builtin_fmaf(p[1], sc, acc[sl][1]);
          acc[sl][2] = __builtin_fmaf(p[2], sc, acc[sl][2]);
          acc[sl][3] = __builtin_fmaf(p[3], sc, acc[sl][3]);
        }
      }
    }
  };

  int cb = c_begin;
  int nc = c_end - cb < MAXC ? c_end - cb : MAXC;
  if (FUSED) {
    // Every wave helps quantize the activation into LDS (16 lanes per (row,
    // group), as quantize_fp8_groups).  The first kXAhead activation loads of
    // each lane go out before the weight loads, and the quantization runs
    // while the weight stream is in flight.
    constexpr int kXAhead = XA;
    const uint16_t* X = static_cast<const uint16_t*>(Ain);
    const int tasks = M * KB, step = KS * 4, part = threadIdx.x & 15, t0 = (int)(threadIdx.x >> 4);
    const rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
    uint4 xv[kXAhead];
#pragma unroll
    for (int i = 0; i < kXAhead; i++) {
      const int task = t0 + i * step;
      const int m = task / KB, g = task - m * KB;
      xv[i] = load_rsrc16(rx, task < tasks ? (uint32_t)(m * K + g * kGroup + part * 8) * 2u : kOob);
    }
    issue(cb, nc);  // even with nc == 0 (every load out of range): no branch around loads
    auto quantize_task = [&](int task, const uint4& v) {
      const int m = task / KB, g = task - m * KB;
      const uint32_t amax_bits = row16_max_u32(absmax8_bits(v));
      const float s = group_scale(__uint_as_float(amax_bits));
      const double r = 1.0 / (double)s;
      const uint2 o = quantize8(v, r);
      *reinterpret_cast<uint2*>(qa + m * K + g * kGroup + part * 8) = o;
      if (part == 0) qs[g * MR + m] = s;
      if (q_out != nullptr && (uint32_t)task % gridDim.x == blockIdx.x) {
        *reinterpret_cast<uint2*>(q_out + (int64_t)m * K + g * kGroup + part * 8) = o;
        if (part == 0) sa_out[(int64_t)g * sa_out_ld + m] = s;
      }
    };
#pragma unroll
    for (int i = 0; i < kXAhead; i++) {
      const int task = t0 + i * step;
      if (task < tasks) quantize_task(task, xv[i]);
    }
    for (int task = t0 + kXAhead * step; task < tasks; task += step) {
      const int m = task / KB, g = task - m * KB;
      quantize_task(task, *reinterpret_cast<const uint4*>(X + (int64_t)m * K + g * kGroup + part * 8));
    }
    __syncthreads();
  } else {
    issue(cb, nc);
  }
  while (nc > 0) {
    compute(cb, nc);
    cb += nc;
    nc = c_end - cb < MAXC ? c_end - cb : MAXC;
    if (nc > 0) issue(cb, nc);
  }
#pragma unroll
  for (int sl = 0; sl < S; sl++) red[(sl * KS + wave) * 64 + lane] = acc[sl];
  __syncthreads();
  // wave sl % KS sums slab sl's KS partials in wave order
#pragma unroll
  for (int sl = 0; sl < S; sl++) {
    if (wave != sl % KS) continue;  // wave-uniform
    v4f_t s = red[(sl * KS) * 64 + lane];
#pragma unroll
    for (int w = 1; w < KS; w++) {
      const v4f_t o = red[(sl * KS + w) * 64 + lane];
      s[0] += o[0]; s[1] += o[1]; s[2] += o[2]; s[3] += o[3];
    }
    // lane (li, lg): output row li, columns n0 + 4*lg .. n0 + 4*lg + 3
    const int64_t n0 = nw + 16 * sl;
    if (row_ok && n0 < N) {
      const int64_t c0 = n0 + 4 * lg;
      uint16_t* drow = D + (int64_t)li * N;
      if ((N % 4) == 0 && c0 + 4 <= N) {
        *reinterpret_cast<uint2*>(drow + c0) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (c0 + r < N) drow[c0 + r] = (uint16_t)bf16_rne(s[r]);
      }
    }
  }
}

// Fused act-quant + product for M <= 16, with the activation quantized in
// registers instead of LDS.  Lane (li, lg) of a wave needs, per chunk kb of
// its K range, the A fragment bytes of row li at K positions kb*128 + 32*lg
// .. +32 (the same lane layout as the weight fragments).  It loads those 32
// bf16 values itself; a 1x128 group of row li lies on the four lanes li +
// 16*lg, so its amax is two lane exchanges, and the lane then encodes its
// 32 values with the group's scale: exactly quantize_fp8_groups'
// arithmetic (amax, s = fl32(amax/448), E4M3(fl32(x/s))), so the product is
// bit-identical to quantize_fp8_groups followed by the decode product (same
// chunk ranges, promotion order and reduction order).  Rows >= M load
// nothing (out-of-range buffer offsets) and contribute zeros.  Nothing is
// held per workgroup, so M and K are not bound by LDS; each wave requests
// MAXC chunks at a time -- per chunk the four activation loads, then the two
// weight loads (requests complete in issue order, so a chunk's activation
// is usable once the previous chunk's weights have arrived).  If q_out is
// non-null, workgroup 0 also writes the quantized activation and scales.
template <int KS, int MAXC>
__global__ __launch_bounds__(KS * 64) void decode_xq_kernel(const uint16_t* __restrict__ X,
                                                            const uint8_t* __restrict__ B,
                                                            const float* __restrict__ SB, uint16_t* __restrict__ D,
                                                            int M, int64_t N, int K, uint8_t* __restrict__ q_out,
                                                            float* __restrict__ sa_out, int64_t sa_out_ld) {
  __shared__ v4f_t red[KS * 64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int KB = K / kGroup;
  const int per = (KB + KS - 1) / KS;
  const int c_begin = wave * per;
  const int c_end = c_begin + per < KB ? c_begin + per : KB;
  const uint32_t b_rows = (uint32_t)(N - n0 < 16 ? N - n0 : 16);
  const rsrc_t rb = make_rsrc(B + n0 * K, b_rows * (uint32_t)K);
  const uint32_t off = (uint32_t)li * (uint32_t)K + (uint32_t)lg * 32u;
  const bool row_ok = li < M;
  const rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t xoff = off * 2u;  // bytes of bf16 row li, K position 32*lg
  const rsrc_t rsb = make_rsrc(SB + (n0 / kGroup) * KB, (uint32_t)KB * 4u);
  const bool writer = q_out != nullptr && blockIdx.x == 0;
  constexpr uint32_t kOob = 0x80000000u;

  v4f_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  uint4 xv[MAXC][4], b0[MAXC], b1[MAXC];
  float sbv = 0.0f;
  // Every load is issued unconditionally (out-of-range offsets read zeros
  // without touching memory), so the compiler waits for exactly the load
  // each instruction needs.
  auto issue = [&](int cb, int nc) {
    sbv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rsb, lane < nc ? (uint32_t)(cb + lane) * 4u : kOob, 0, 0));
#pragma unroll
    for (int u = 0; u < MAXC; u++) {
      const bool live = u < nc;
      const uint32_t xo = live && row_ok ? xoff + (uint32_t)(cb + u) * 256u : kOob;
#pragma unroll
      for (int j = 0; j < 4; j++) xv[u][j] = load_rsrc16(rx, xo == kOob ? kOob : xo + 16u * j);
      const uint32_t o = live ? off + (uint32_t)(cb + u) * 128u : kOob;
      b0[u] = load_rsrc16(rb, o);
      b1[u] = load_rsrc16(rb, live ? o + 16u : kOob);
    }
  };
  auto compute = [&](int cb, int nc) {
    v4f_t part[2];
    float scl[2];
#pragma unroll
    for (int u = 0; u <= MAXC; u++) {
      if (u < nc) {
        const int kb = cb + u;
        uint32_t am = max(max(absmax8_bits(xv[u][0]), absmax8_bits(xv[u][1])),
                          max(absmax8_bits(xv[u][2]), absmax8_bits(xv[u][3])));
        am = max(am, (uint32_t)__shfl_xor((int)am, 16));
        am = max(am, (uint32_t)__shfl_xor((int)am, 32));
        const float s = group_scale(__uint_as_float(am));
        const double r = 1.0 / (double)s;
        const uint2 q0 = quantize8(xv[u][0], r), q1 = quantize8(xv[u][1], r);
        const uint2 q2 = quantize8(xv[u][2], r), q3 = quantize8(xv[u][3], r);
        const uint4 lo = make_uint4(q0.x, q0.y, q1.x, q1.y), hi = make_uint4(q2.x, q2.y, q3.x, q3.y);
        if (writer && row_ok) {
          uint8_t* qp = q_out + (int64_t)li * K + (int64_t)kb * kGroup + lg * 32;
          *reinterpret_cast<uint4*>(qp) = lo;
          *reinterpret_cast<uint4*>(qp + 16) = hi;
          if (lg == 0) sa_out[(int64_t)kb * sa_out_ld + li] = s;
        }
        part[u & 1] = mfma_fp8_dec(frag_of(b0[u], b1[u]), frag_of(lo, hi));
        scl[u & 1] = (row_ok ? s : 0.0f) *
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sbv), u));
      }
      if (u > 0 && u - 1 < nc) {
        const v4f_t& p = part[(u - 1) & 1];
        const float sc = scl[(u - 1) & 1];
        acc[0] = __builtin_fmaf(p[0], sc, acc[0]);
        acc[1] = __builtin_fmaf(p[1], sc, acc[1]);
        acc[2] = __builtin_fmaf(p[2], sc, acc[2]);
        acc[3] = __builtin_fmaf(p[3], sc, acc[3]);
      }
    }
  };
  int cb = c_begin;
  int nc = c_end - cb < MAXC ? c_end - cb : MAXC;
  issue(cb, nc);  // even with nc <= 0 (every load out of range): no branch around loads
  while (nc > 0) {
    compute(cb, nc);
    cb += nc;
    nc = c_end - cb < MAXC ? c_end - cb : MAXC;
    if (nc > 0) issue(cb, nc);
  }
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    v4f_t sum = red[lane];
#pragma unroll
    for (int w = 1; w < KS; w++) {
      const v4f_t o = red[w * 64 + lane];
      sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
    }
    if (row_ok) {
      const int64_t c0 = n0 + 4 * lg;
      uint16_t* drow = D + (int64_t)li * N;
      if ((N % 4) == 0 && c0 + 4 <= N) {
        *reinterpret_cast<uint2*>(drow + c0) = make_uint2(pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (c0 + r < N) drow[c0 + r] = (uint16_t)bf16_rne(sum[r]);
      }
    }
  }
}

// K split (1..16 waves per slab): enough waves in flight to cover HBM
// latency, and at most 12 chunks per wave on the common shapes.  Where eight
// waves would each take more than 8 chunks (K > 8192 on a narrow N), sixteen
// waves of 128 VGPRs (four per SIMD) shorten every wave's serial tail:
// measured at N = 4096, K = 12288, 13.6 -> 12.9 us at M = 1 and 17.3 -> 15.6
// us at M = 4 (graph replay).
//
// Slabs per workgroup: 3 where more than 4 activation rows make the
// activation's fragments as costly as the weight's (each slab workgroup
// re-reads all M rows from L2) and the shape allows -- K <= 16384, so that
// three slabs' reduction space (and the fused form's activation) fits in
// LDS, and a split of 8 waves, since with 16 three slabs' fragments do not
// fit the 128 VGPRs of four waves per SIMD -- else 1.  The split is then
// planned over the workgroups instead of the slabs.  Measured (graph replay
// over 8 weight sets, N = 12288, K = 4096): M = 16 19.5 -> 18.4 us per call;
// at M = 1 and 4 three slabs lose (11.4 -> 14.6 and 14.4 -> 16.0 us).
// Three slabs also need a workgroup for every CU: at N = 2048, K = 4096, M =
// 16 the 43 three-slab workgroups took 13.7 us against 10.8 for 128 of one.
// FGFP8_DECODE_SLABS=1|3 forces the choice (tests, tuning).  The fused
// forms and the two-launch path take the same plan for the same M, so they
// stay bit-identical.
constexpr int64_t kDecodeCUs = 256;

static int split_for(int64_t units, int64_t kb) {
  int ks = 4;
  while (ks < 8 && (units * ks < 2048 || (kb + ks - 1) / ks > 12)) ks *= 2;
  if (ks == 8 && (kb + 7) / 8 > 8) ks = 16;
  while (ks > 1 && (kb + ks - 1) / ks < 2) ks /= 2;
  return ks;
}

DecodePlan decode_plan(int64_t m, int64_t n, int64_t k) {
  const int64_t slabs = (n + 15) / 16, kb = k / kGroup;
  const char* force = getenv("FGFP8_DECODE_SLABS");
  const bool three = force != nullptr ? strcmp(force, "3") == 0 : m > kFusedLdsMaxM && (slabs + 2) / 3 >= kDecodeCUs;
  if (three && k <= 16384) {
    const int ks = split_for((slabs + 2) / 3, kb);
    if (ks == 8) return {ks, 3};
  }
  return {split_for(slabs, kb), 1};
}

int decode_split(int64_t m, int64_t n, int64_t k) { return decode_plan(m, n, k).ks; }

template <int KS, bool FUSED, int XA, int S, int MR>
static hipError_t allow_lds() {
  // The fused variant holds the quantized activation (MR x K bytes) in
  // LDS; allow dynamic LDS beyond the 64 KB default, once per kernel and
  // device (devices beyond the table set it on every call).
  static std::atomic<bool> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done[dev].load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<KS, FUSED, XA, S, MR>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess && cached) done[dev].store(true, std::memory_order_relaxed);
  return e;
}

template <int KS, bool FUSED, int XA = 3, int S = 1, int MR = kFusedMaxRows>
static hipError_t launch_decode_ks(const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb,
                                   void* d, int64_t m, int64_t n, int64_t k, uint8_t* q_out, float* sa_out,
                                   int64_t sa_out_ld, hipStream_t stream) {
  size_t lds = (size_t)S * KS * 64 * 16;
  if (FUSED) lds += (size_t)MR * k + (size_t)(k / kGroup) * MR * 4;
  if (lds > 64 * 1024) {
    const hipError_t e = allow_lds<KS, FUSED, XA, S, MR>();
    if (e != hipSuccess) return e;
  }
  const int64_t wgs = ((n + 15) / 16 + S - 1) / S;
  hipLaunchKernelGGL((decode_kernel<KS, FUSED, XA, S, MR>), dim3((uint32_t)wgs), dim3(KS * 64), lds, stream, a, sa, sa_ld,
                     static_cast<const uint8_t*>(b), sb, static_cast<uint16_t*>(d), (int)m, n, (int)k, q_out, sa_out,
                     sa_out_ld);
  return hipGetLastError();
}

template <bool FUSED, int XA = 3>
static hipError_t launch_decode_t(int ks, const void* a, const float* sa, int64_t sa_ld, const void* b,
                                  const float* sb, void* d, int64_t m, int64_t n, int64_t k, uint8_t* q_out,
                                  float* sa_out, int64_t sa_out_ld, hipStream_t stream) {
  if (decode_plan(m, n, k).slabs == 3) {
    if (ks == 8) return launch_decode_ks<8, FUSED, XA, 3>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
  }
  switch (ks) {
    case 1: return launch_decode_ks<1, FUSED, XA>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 2: return launch_decode_ks<2, FUSED, XA>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 4: return launch_decode_ks<4, FUSED, XA>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 8: return launch_decode_ks<8, FUSED, XA>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    default: return launch_decode_ks<16, FUSED, XA>(a, sa, sa_ld, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
  }
}

hipError_t launch_decode(int ks, const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb,
                         void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  return launch_decode_t<false>(ks, a, sa, sa_ld, b, sb, d, m, n, k, nullptr, nullptr, 0, stream);
}

template <int KS, int MAXC>
static hipError_t launch_decode_xq_ks(const void* x, const void* b, const float* sb, void* d, int64_t m, int64_t n,
                                      int64_t k, uint8_t* q_out, float* sa_out, int64_t sa_out_ld,
                                      hipStream_t stream) {
  hipLaunchKernelGGL((decode_xq_kernel<KS, MAXC>), dim3((uint32_t)((n + 15) / 16)), dim3(KS * 64), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(b), sb, static_cast<uint16_t*>(d),
                     (int)m, n, (int)k, q_out, sa_out, sa_out_ld);
  return hipGetLastError();
}

// Four chunks per request batch (140 VGPRs: three waves per SIMD; three
// chunks at KS = 16, whose four waves per SIMD allow 128).  Measured against
// 6 and 8 chunks and other splits: four is fastest at both decode shapes.
// The split is decode_split's, so the result is bit-identical to the
// two-launch path.
static hipError_t launch_decode_xq(int ks, const void* x, const void* b, const float* sb, void* d, int64_t m,
                                   int64_t n, int64_t k, uint8_t* q_out, float* sa_out, int64_t sa_out_ld,
                                   hipStream_t stream) {
  switch (ks) {
    case 1: return launch_decode_xq_ks<1, 4>(x, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 2: return launch_decode_xq_ks<2, 4>(x, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 4: return launch_decode_xq_ks<4, 4>(x, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    case 8: return launch_decode_xq_ks<8, 4>(x, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
    default: return launch_decode_xq_ks<16, 3>(x, b, sb, d, m, n, k, q_out, sa_out, sa_out_ld, stream);
  }
}

// The three-slab form with all M <= 16 rows quantized into LDS: each
// workgroup's 32 lanes-of-16 take the M * K/128 quantize tasks, and every
// lane's share must go out in one batch of kWideAhead loads ahead of the
// weight stream (a load issued after the stream would arrive only with it).
// Every workgroup redoes the whole quantization, and that costs more than
// the separate quantize launch once a lane has more than 8 tasks: measured
// (graph replay over 8 weight sets, N = 12288, K = 4096), the two-launch path
// against this form took 17.9 / 16.4 us at M = 5, 18.3 / 17.2 at M = 6,
// 18.1 / 17.8 at M = 8, 18.4 / 19.8 at M = 12 and 18.6 / 22.0 at M = 16.
// Without a workspace for the two-launch path it is compared with the
// register form instead, which it beats at every such M (20.5 against 30.8
// us at M = 16).
constexpr int kWideRows = 16, kWideAhead = 16;

bool decode_fused_wide(int64_t m, int64_t n, int64_t k, bool act_out) {
  if (m <= kFusedMaxRows || m > kWideRows || getenv("FGFP8_DECODE_XQ") != nullptr) return false;
  // LDS: three slabs' sums (24 KB), 16 x K activation bytes and their
  // scales; K <= 8192 keeps them within 160 KB (the 8-wave split of three
  // slabs implies it too: more than 64 chunks take 16 waves)
  if (k > 8192) return false;
  const DecodePlan p = decode_plan(m, n, k);
  const int64_t per_lane = (m * (k / kGroup) + 8 * 4 - 1) / (8 * 4);
  return p.slabs == 3 && p.ks == 8 && per_lane <= (act_out ? 8 : kWideAhead);
}

hipError_t launch_decode_fused(const void* x, const void* b, const float* sb, void* d, int64_t m, int64_t n,
                               int64_t k, void* q_out, float* sa_out, int64_t sa_out_ld, hipStream_t stream) {
  const int ks = decode_split(m, n, k);
  if (decode_fused_wide(m, n, k, q_out != nullptr))
    return launch_decode_ks<8, true, kWideAhead, 3, kWideRows>(x, nullptr, 0, b, sb, d, m, n, k,
                                                               static_cast<uint8_t*>(q_out), sa_out, sa_out_ld,
                                                               stream);
  // Test override: FGFP8_DECODE_XQ forces the register form at any M.
  if (m > kFusedMaxRows || k > kFusedLdsMaxK || getenv("FGFP8_DECODE_XQ") != nullptr)
    return launch_decode_xq(ks, x, b, sb, d, m, n, k, static_cast<uint8_t*>(q_out), sa_out, sa_out_ld, stream);
  // Activation quantize tasks (row, 128-group) per lane: M * K/128 over the
  // workgroup's KS * 4 lanes-of-16.  When more than three, issue up to 12
  // ahead of the weight stream.
  const int64_t per_lane = (m * (k / kGroup) + ks * 4 - 1) / (ks * 4);
  uint8_t* q = static_cast<uint8_t*>(q_out);
  if (per_lane > 3 && per_lane <= 12)
    return launch_decode_t<true, 12>(ks, x, nullptr, 0, b, sb, d, m, n, k, q, sa_out, sa_out_ld, stream);
  return launch_decode_t<true>(ks, x, nullptr, 0, b, sb, d, m, n, k, q, sa_out, sa_out_ld, stream);
}

}  // namespace fgfp8
