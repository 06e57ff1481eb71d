// Shared device helpers for the gfx950 kernels of libfgfp8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgfp8 {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kGroup = 128;       // K elements per scale group / per 128-wide K chunk
constexpr float kE4m3Max = 448.0f;

// Raw buffer resource (gfx9 word 3: 32-bit data format, no swizzle, stride 0).
// Any load whose byte range is not inside [0, num_bytes) returns zeros.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

// Whole-wave 16-byte global->LDS copy: lane L's 16 bytes (at voffset) land at
// lds_wave_base + 16 * L.  lds_wave_base must be wave-uniform.
__device__ __forceinline__ void load_lds16(rsrc_t r, void* lds_wave_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ uint4 load_rsrc16(rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

// float -> bfloat16 bits, round to nearest even, two at a time with gfx950's
// v_cvt_pk_bf16_f32 (one instruction per pair; checked on the device to equal
// the bit-level round-half-to-even for every non-NaN float32, denormals
// included; a NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_rne(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Maximum over the 16 lanes of each DPP row (lanes 16r .. 16r+15), returned to
// every lane of the row: two quad permutations, then the half-row and row
// mirrors.  Unsigned compare; callers pass magnitudes' bit patterns, whose
// integer order is their value order.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return v;
}

// Scale of a group from its largest magnitude: fl32(amax / 448) (a correctly
// rounded float division), or 1 for an all-zero group.
__device__ __forceinline__ float group_scale(float amax) { return amax == 0.0f ? 1.0f : amax / kE4m3Max; }

// Power-of-two (UE8M0) scale: group_scale rounded up to the next power of
// two, within the E8M0 range [2^-127, 2^127].  2^-127 is the float32
// subnormal 0x00400000, so its exponent field (0) is again the E8M0 code.
__device__ __forceinline__ float group_scale_ue8m0(float amax) {
  const uint32_t b = __float_as_uint(group_scale(amax));
  const uint32_t e = b >> 23, man = b & 0x7fffffu;
  uint32_t out;
  if (e == 0) {
    out = man <= 0x400000u ? 0x400000u : 0x800000u;  // (0, 2^-127] -> 2^-127, (2^-127, 2^-126) -> 2^-126
  } else {
    uint32_t f = e + (man != 0u ? 1u : 0u);
    if (f > 254u) f = 254u;
    out = f << 23;
  }
  return __uint_as_float(out);
}

// The E8M0 code of a power-of-two float32 scale (its exponent field; the
// mantissa of a non-power-of-two is ignored).
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// fl32(x / s) for every float32 x given r = 1/s in double.  x * r carries a
// relative error below 2^-52, while a float32 quotient x/s with a normal
// result is never within 2^-49 (relative) of a float32 rounding boundary
// without lying on one, and never lies on one; so rounding x * r to float
// gives the correctly rounded quotient.  Quotients in the float32 subnormal
// range may differ, but every such value encodes to an E4M3 zero of the same
// sign either way.
__device__ __forceinline__ float div_by_scale(float x, double r) { return (float)((double)x * r); }

// Four float32 values -> four E4M3 bytes (byte i = value i): saturate to
// +-448, then the hardware round-to-nearest-even conversion (which itself
// does not saturate).
__device__ __forceinline__ uint32_t e4m3x4(float y0, float y1, float y2, float y3) {
  y0 = __builtin_amdgcn_fmed3f(y0, -kE4m3Max, kE4m3Max);
  y1 = __builtin_amdgcn_fmed3f(y1, -kE4m3Max, kE4m3Max);
  y2 = __builtin_amdgcn_fmed3f(y2, -kE4m3Max, kE4m3Max);
  y3 = __builtin_amdgcn_fmed3f(y3, -kE4m3Max, kE4m3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// The MoE layer's activation: silu(g) * u = g / (1 + e^-g) * u, each step in
// FP32, for the bf16 gate and up projections g and u (the caller rounds the
// result to bf16).  One definition for the standalone kernel and the fused
// gate_up epilogue, so that the two agree bit for bit.
__device__ __forceinline__ float silu_mul_f32(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Largest |value| bit pattern among the 8 bf16 in a 16-byte word (as the
// float32 bit pattern, i.e. shifted into the high half).
__device__ __forceinline__ uint32_t absmax8_bits(uint4 v) {
  uint32_t m = v.x & 0x7fffu;
  m = max(m, (v.x >> 16) & 0x7fffu);
  m = max(m, v.y & 0x7fffu);
  m = max(m, (v.y >> 16) & 0x7fffu);
  m = max(m, v.z & 0x7fffu);
  m = max(m, (v.z >> 16) & 0x7fffu);
  m = max(m, v.w & 0x7fffu);
  m = max(m, (v.w >> 16) & 0x7fffu);
  return m << 16;
}

// Quantize 8 bf16 (one 16-byte word) with r = 1/s: 8 E4M3 bytes.
__device__ __forceinline__ uint2 quantize8(uint4 v, double r) {
  uint2 o;
  o.x = e4m3x4(div_by_scale(bf16_lo(v.x), r), div_by_scale(bf16_hi(v.x), r), div_by_scale(bf16_lo(v.y), r),
               div_by_scale(bf16_hi(v.y), r));
  o.y = e4m3x4(div_by_scale(bf16_lo(v.z), r), div_by_scale(bf16_hi(v.z), r), div_by_scale(bf16_lo(v.w), r),
               div_by_scale(bf16_hi(v.w), r));
  return o;
}

}  // namespace fgfp8
