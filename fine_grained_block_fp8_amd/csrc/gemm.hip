// Block-scaled FP8 products for gfx950: the dense fp8_gemm_nt, its M-grouped
// contiguous variant, and a streaming form for decode-shaped M <= 16.
//
// Definition (deepgemm-rust README, "What's implemented" table, fp8_gemm_nt
// row and the kernel notes on per-128-block scale promotion):
//   D[m][n] = sum_kb sa[kb][m] * sb[n/128][kb] * P(m, n, kb),
//   P(m, n, kb) = sum_{k in chunk kb} a[m][k] * b[n][k]   (FP8 x FP8, FP32 sum)
// P of a 16x16 output tile and one 128-wide chunk is exactly one
// v_mfma_f32_16x16x128_f8f6f4 with a zero accumulator; the scale product is
// then applied in FP32 registers, acc = fma(P, sa*sb, acc) ("promotion").
//
// Operand roles: the MFMA's first operand is a 16-row slice of B and its
// second a 16-row slice of A, so lane l of the 4-register result holds one
// row of A (l % 16) and four columns of B.  That makes the promotion scale
// sa[row] * sb[block] a single per-lane value for the whole 16x16 tile.
// Within a wave tile of NT 16-column MFMA tiles, MFMA tile t's column c is
// mapped to a wave column chosen so that each 16-byte store of the epilogue
// writes 8 consecutive columns and the four lanes of a row cover 64
// contiguous bytes.  The B tile is stored in LDS with its columns permuted
// to match, so that every MFMA tile reads 16 consecutive LDS rows, exactly
// like the A fragments.

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fgfp8 {

// ------------------------------------------------------------ tile configs
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  // LDS stages of the K loop: chunk kb + STAGES - 1 is copied while chunk kb
  // is multiplied, so a copy has STAGES - 1 chunk times to arrive.
  static constexpr int STAGES = STAGES_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  // Waves that copy the K chunks into LDS (the first COPY_WAVES).  With 8 or
  // 12 waves only waves 0-3, one per SIMD, copy: waves w, w + 4 (and w + 8)
  // share a SIMD, and its arbiter favours the older wave, which reaches the
  // barrier ~30% sooner; giving it all the copy issue shortens the others'
  // chunk (measured, bit-identical results: +2-3% on the 256x256 shapes, +2%
  // on 256x128 and 256x192, +4% on the grouped 128x256 product).
  static constexpr int COPY_WAVES = WAVES >= 8 ? 4 : WAVES;
  static constexpr int TM = BM / WAVES_M;  // wave tile rows
  static constexpr int TN = BN / WAVES_N;  // wave tile columns (inside one 128-column scale block)
  static constexpr int MT = TM / 16;
  static constexpr int NT = TN / 16;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  // One stage's scales: the tile's activation scales (<= 256 floats, or
  // packed E8M0 words of the MX recipe) at +0, and at +1024 the weight
  // scales: one 4-byte slot per lane of the copy, slot j holding the scale
  // of the tile's column block j, or (MX) the tile's BN packed E8M0 words.
  // Tiles whose stages leave no room for the scale area (128x512: two
  // stages of 80 KB fill the 160 KB) keep their scales in registers: each
  // wave loads the activation scales of its rows and the weight scale of its
  // column block for the next chunk with vector loads (gemm_tile), and the
  // LDS holds operand stages only.
  static constexpr bool REG_SCALES = STAGES * (A_BYTES + B_BYTES) + STAGES * 2048 + WAVES * TM * 4 > 160 * 1024;
  static constexpr int S_BYTES = REG_SCALES ? 0 : 1024 + 1024;
  static constexpr int SB_IN_S = 1024;
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = STAGES * A_BYTES;
  static constexpr int S_OFF = B_OFF + STAGES * B_BYTES;
  // FP8-output epilogue: one float per (wave, row) for the partner-wave amax
  // exchange of 64-column wave tiles.
  static constexpr int EPI_OFF = S_OFF + STAGES * S_BYTES;
  static constexpr int LDS = EPI_OFF + (REG_SCALES ? 0 : WAVES * TM * 4);
  static_assert(TN == 64 || TN == 128, "a wave tile spans 64 or 128 columns of one scale block");
  static_assert(TM % 16 == 0 && BM % 8 == 0 && BN % 8 == 0, "tile shape");
  // The copies of a chunk are 8-row segments dealt to the copying waves in
  // turn; an uneven deal (some waves copy one segment fewer) needs the
  // vmcnt(0) wait of the two-stage loop, which does not count copies.
  static_assert(((BM / 8) % COPY_WAVES == 0 && (BN / 8) % COPY_WAVES == 0) || STAGES == 2,
                "segments divide evenly among waves");
  static_assert(REG_SCALES || BM * 4 <= SB_IN_S, "one wave loads a stage's activation scales");
  static_assert(REG_SCALES || BN * 4 <= S_BYTES - SB_IN_S, "one wave loads a stage's MX weight scales");
  static_assert(STAGES == 2 || STAGES == 3, "two or three stages");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Two waves per SIMD (8 per workgroup) hide each other's LDS and barrier
// stalls; the 64x128 and 64x64 wave tiles keep the FP32 accumulators in
// architectural VGPRs, where the promotion FMAs can reach them.  Tiles whose
// stage is at most 48 KB take three stages (a longer prefetch distance, which
// matters when B streams from HBM rather than the last-level cache, as the
// per-expert weights of the grouped product do); 256x256 fits two.
using Tile256x256 = Tile<256, 256, 4, 2, 2>;
// 256x192 with 12 waves (3 per SIMD) of 64x64: 2048 x 6144 is exactly 256
// such tiles, one per CU.  n0 is a multiple of 64, so every 64-column wave
// tile still lies inside one 128-column scale block.
using Tile256x192 = Tile<256, 192, 4, 3, 2>;
using Tile128x256 = Tile<128, 256, 2, 4, 3>;
using Tile256x128 = Tile<256, 128, 4, 2, 3>;
using Tile128x128 = Tile<128, 128, 2, 2, 3>;
// The grouped product's wide tile: 128 rows (the experts' alignment unit, so
// no tile straddles two experts) by 512 columns, 8 waves of 64x128 -- the
// 256x256 tile's wave tiles, LDS fragment bytes per FLOP and stage size
// (plus 16 KB), where 128x256 tiles need 64x64 wave tiles.
using Tile128x512 = Tile<128, 512, 2, 4, 2>;
static_assert(Tile128x512::REG_SCALES && Tile128x512::LDS == 160 * 1024, "two 80 KB stages, scales in registers");
static_assert(!Tile256x256::REG_SCALES && !Tile256x192::REG_SCALES && !Tile128x256::REG_SCALES &&
                  !Tile256x128::REG_SCALES && !Tile128x128::REG_SCALES,
              "the other tiles stage their scales through LDS");

// LDS layout of a K chunk: row r of a tile is 128 bytes (8 slots of 16
// bytes); logical slot c of row r is stored at slot c ^ swz(r).  Fragment
// reads always cover 16 consecutive rows (a 16-row-aligned group) per
// instruction, and swz depends only on r mod 16, so a fragment's address is
// a per-lane base plus a compile-time offset (2 KB per 16-row tile, 32 KB per
// stage) -- no address arithmetic in the main loop.  With (r ^ r>>3) over the
// low four bits the 16-row reads run at ~85% of the conflict-free
// ds_read_b128 rate on gfx950 (measured), well above what the loop needs.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Output column of MFMA tile t, position c (c = 4*lg + r for output lane
// (li, lg), register r), within a wave's TN-column region: the lane's 4*NT
// values j = NT*r + t go to columns 32*(j/8) + 8*lg + (j%8), so the four lanes
// of a row together write 64 contiguous bytes per 16-byte store.
template <class C>
__device__ __forceinline__ int wave_col(int c, int t) {
  const int j = C::NT * (c & 3) + t;
  return 32 * (j >> 3) + 8 * (c >> 2) + (j & 7);
}

// LDS row rho of the B tile holds tile column b_col_of_row(rho): within each
// wave's TN-column region, row 16*t + c holds wave_col(c, t), so MFMA tile t
// reads the 16 consecutive rows 16t .. 16t+15.
template <class C>
__device__ __forceinline__ int b_col_of_row(int rho) {
  const int w = rho / C::TN, rl = rho % C::TN;
  return w * C::TN + wave_col<C>(rl & 15, rl >> 4);
}

// The copying waves (Tile::COPY_WAVES of them) copy chunk kb of the A tile
// and the B tile into one LDS stage with direct global->LDS buffer loads (1
// KB = 8 LDS rows per wave instruction; rows past the matrix edge read as
// zero): wave w copies segments w, w + COPY_WAVES, ... of A and of B (with 12
// waves the 32 A segments of a 256-row tile fall unevenly: waves 8-11 copy
// one fewer).  Wave 0 copies the activation scales and wave 1 the weight
// scales of the tile's column blocks.  voff[] holds the per-lane byte offsets of those
// segments for chunk 0; the chunk's column offset is the scalar offset of
// each load.  Staging the weight scales through LDS keeps scalar memory loads
// out of the loop: their completion shares a counter with the LDS reads and
// would force every fragment read of the chunk to drain before the first
// MFMA.
template <class C>
struct StageLoader {
  static constexpr int CW = C::COPY_WAVES;
  static constexpr int A_SEGS = C::BM / 8, B_SEGS = C::BN / 8;
  static constexpr int AN = (A_SEGS + CW - 1) / CW, BN_ = (B_SEGS + CW - 1) / CW, NSEG = AN + BN_;
  static constexpr bool EVEN = A_SEGS % CW == 0 && B_SEGS % CW == 0;
  static_assert(NSEG + 1 < 16 || C::STAGES == 2, "a chunk's copies must fit the 4-bit vmcnt field used by the waits");
  // 256x256: segment i of a wave lies a multiple of K bytes past its first A
  // (or B) segment, with the same swizzle, so one vector offset per operand
  // serves all of them and the difference goes in the scalar offset.  In A,
  // segment i is 8 * CW * i rows further; in B (LDS rows permuted as
  // b_col_of_row: within a 128-column wave region, row 16 t + c holds column
  // 32 (c & 3) + 8 (c >> 2) + t) it is col_delta(i) columns further.
  static constexpr bool SOFF = C::BM == 256 && C::BN == 256 && C::TN == 128 && C::NT == 8 && 128 % (8 * CW) == 0;
  static constexpr int col_delta(int i) { return 128 * ((8 * CW * i) / 128) + ((8 * CW * i) % 128) / 16; }
  uint8_t* lds;
  rsrc_t ra, rb, rs, rsb;
  const uint32_t* voff;
  uint32_t sa_ld_bytes, vsb;
  int wave, lane;
  // 0: the weight-scale copy is one 4-byte block scale per lane; else the MX
  // recipe's packed words, 16 bytes per lane, rows sb_row_bytes apart per chunk.
  uint32_t sb_row_bytes = 0;
  uint32_t kdim = 0;  // K (bytes per operand row)
  __device__ __forceinline__ bool copier() const { return wave < CW; }
  // Segment i (< NSEG; copying waves only) of chunk kb into `stage`; segment
  // NSEG is the scales (waves 0 and 1).
  __device__ __forceinline__ void issue(int i, int stage, int kb) const {
    const uint32_t koff = (uint32_t)kb * 128u;
    if (i < AN) {
      if (EVEN || wave + CW * i < A_SEGS)  // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void_t*)(lds + C::A_OFF + stage * C::A_BYTES + (wave + CW * i) * 1024), 16,
            SOFF ? voff[0] : voff[i], SOFF ? koff + (uint32_t)(8 * CW * i) * kdim : koff, 0, 0);
    } else if (i < NSEG) {
      if (EVEN || wave + CW * (i - AN) < B_SEGS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_t*)(lds + C::B_OFF + stage * C::B_BYTES + (wave + CW * (i - AN)) * 1024), 16,
            SOFF ? voff[AN] : voff[i], SOFF ? koff + (uint32_t)col_delta(i - AN) * kdim : koff, 0, 0);
    } else if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lds + C::S_OFF + stage * C::S_BYTES), 16,
                                               (uint32_t)lane * 16u, (uint32_t)kb * sa_ld_bytes, 0, 0);
    else if (wave == 1 && sb_row_bytes == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void_t*)(lds + C::S_OFF + stage * C::S_BYTES + C::SB_IN_S),
                                               4, vsb, (uint32_t)kb * 4u, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void_t*)(lds + C::S_OFF + stage * C::S_BYTES + C::SB_IN_S),
                                               16, vsb, (uint32_t)kb * sb_row_bytes, 0, 0);
  }
  __device__ __forceinline__ void all(int stage, int kb) const {
    if (copier()) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < NSEG; i++) issue(i, stage, kb);
    }
    if constexpr (!C::REG_SCALES) issue(NSEG, stage, kb);
  }
};

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every outstanding global->LDS copy (vmcnt(0)) and would drain the
// copies of the chunks ahead, reducing three stages to two.  The K loop
// orders LDS traffic itself (explicit vmcnt waits for the copies; every
// fragment read of a stage is consumed by an MFMA before the barrier after
// which the stage is refilled); the empty asm statements keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The matrix core takes K positions [16*lg, 16*lg + 16) of row li from a
// lane's first four fragment registers and [64 + 16*lg, 64 + 16*lg + 16) from
// its last four (fitted on gfx950 from the per-32-block scale each K byte
// receives).  Logical LDS slot c of a row therefore holds the chunk's 16-byte
// K segment k_segment(c): slots 2*lg and 2*lg + 1, which a lane reads, hold
// segments lg and lg + 4.  The eight lanes copying a row still read its 128
// contiguous bytes, in another lane order.
__device__ __forceinline__ int k_segment(int c) { return (c >> 1) | ((c & 1) << 2); }

// up_rows (the fused gate_up tile only): B rows of tile columns >= 128 lie
// up_rows further on (the up half of the weight).
template <class C>
__device__ __forceinline__ void stage_offsets(uint32_t* voff, uint32_t K, int wave, int lane, uint32_t up_rows = 0) {
  // the loader's counts: rounded up, so that an uneven deal still gives
  // every wave AN A-offsets followed by BN_ B-offsets
  constexpr int AN = StageLoader<C>::AN, BN_ = StageLoader<C>::BN_;
  const int r8 = lane >> 3, cs = lane & 7;
#pragma unroll
  for (int i = 0; i < AN; i++) {
    const int rho = (wave + C::COPY_WAVES * i) * 8 + r8;
    voff[i] = (uint32_t)rho * K + (k_segment(cs ^ swz(rho)) << 4);
  }
#pragma unroll
  for (int i = 0; i < BN_; i++) {
    const int rho = (wave + C::COPY_WAVES * i) * 8 + r8;
    const uint32_t col = (uint32_t)b_col_of_row<C>(rho);
    voff[AN + i] = (col + (col >= (uint32_t)kGroup ? up_rows : 0u)) * K + (k_segment(cs ^ swz(rho)) << 4);
  }
}

// LDS byte offsets of the two 16-byte slots lane (li, lg) reads for a
// 16x16x128 MFMA fragment of rows base_row .. base_row+15 (base_row a
// multiple of 16, so the swizzle depends on li only): logical slots 2*lg and
// 2*lg + 1, which hold K segments lg and lg + 4 (k_segment above), so the
// instruction's K order is the memory order.  Reading slots lg and lg + 4
// directly instead halves the measured ds_read_b128 rate on gfx950.  Adding
// 2048 selects the next 16-row tile, adding an operand-tile size the other
// stage.
struct FragAddr {
  uint32_t lo, hi;
};
__device__ __forceinline__ FragAddr frag_addr(uint32_t region, int base_row, int li, int lg) {
  const uint32_t row = region + (uint32_t)(base_row + li) * 128u;
  return {row + (uint32_t)(((2 * lg) ^ swz(li)) << 4), row + (uint32_t)(((2 * lg + 1) ^ swz(li)) << 4)};
}
__device__ __forceinline__ v8i_t read_frag(const uint8_t* lds, const FragAddr& a, uint32_t cst) {
  const uint4 lo = *reinterpret_cast<const uint4*>(lds + a.lo + cst);
  const uint4 hi = *reinterpret_cast<const uint4*>(lds + a.hi + cst);
  v8i_t f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

__device__ __forceinline__ v4f_t mfma_fp8(const v8i_t& x, const v8i_t& y) {
  const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// acc += p * s, one FMA per element (single rounding).
__device__ __forceinline__ void promote(v4f_t& acc, const v4f_t& p, float s) {
  acc[0] = __builtin_fmaf(p[0], s, acc[0]);
  acc[1] = __builtin_fmaf(p[1], s, acc[1]);
  acc[2] = __builtin_fmaf(p[2], s, acc[2]);
  acc[3] = __builtin_fmaf(p[3], s, acc[3]);
}

// B fragment of column tile t for lane c = li: LDS row 16*t + c of the wave's
// region, which holds wave column wave_col(c, t).  acc[mt][t][r] of output
// lane (li, lg) is therefore wave column wave_col(4*lg + r, t).
template <class C>
__device__ __forceinline__ v8i_t read_b(const uint8_t* lds, const FragAddr& ba, int stage, int t) {
  return read_frag(lds, ba, (uint32_t)(stage * C::B_BYTES + 2048 * t));
}

// A fragments and promotion scales (sa[row] * sb) of one chunk.
template <class C>
__device__ __forceinline__ void read_a(const uint8_t* lds, const FragAddr& aa, uint32_t sa_addr, uint32_t sb_addr,
                                       int stage, v8i_t (&af)[C::MT], float (&sc)[C::MT]) {
  const float sbv = *reinterpret_cast<const float*>(lds + sb_addr + stage * C::S_BYTES);
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    af[mt] = read_frag(lds, aa, (uint32_t)(stage * C::A_BYTES + 2048 * mt));
    sc[mt] = *reinterpret_cast<const float*>(lds + sa_addr + stage * C::S_BYTES + 64 * mt) * sbv;
  }
}

// Column tiles [T0, T1) of a chunk, software-pipelined two MFMAs deep: MFMA i
// is issued, then the FP32 promotion of MFMA i-2's partial runs on the VALU
// (independent of MFMAs i-1 and i, so they overlap), and the B fragment of
// the next column tile is read one tile ahead (from LDS, or from registers
// when PRE).  Each accumulator still takes its chunks' promotions in chunk
// order, so the schedule does not change a bit of the result.
template <class C, int T0, int T1, bool PRE, bool LD>
__device__ __forceinline__ void mfma_tiles(const uint8_t* lds, const FragAddr& ba, int stage, int load_stage,
                                           const v8i_t (&af)[C::MT], const float (&sc)[C::MT], const v8i_t* pre,
                                           v4f_t (&acc)[C::MT][C::NT], const StageLoader<C>& ld, int next_kb) {
  // With LD (copying waves), the next chunk's global->LDS copies (NSEG
  // instructions per wave) are spread over the first half of the column
  // tiles, so that no wave stalls for long on a full vector-memory queue,
  // and they land well before the next barrier even when the weight streams
  // from HBM: spread over all the tiles, the copying waves of gate_up waited
  // ~880 ticks per chunk for their last copies with the weights rotating
  // through more than the last-level cache (183.6 us), against ~470 over the
  // first half (177.9 us; the same 170-171 us with the weight cache-resident).
  constexpr int NL = StageLoader<C>::NSEG;
  constexpr int HALF = (T1 - T0) / 2 > 0 ? (T1 - T0) / 2 : 1;
  constexpr int PER = (NL + HALF - 1) / HALF;
  constexpr int N_MFMA = (T1 - T0) * C::MT;
  v8i_t bfr[2];
  v4f_t part[3];
  bfr[0] = PRE ? pre[0] : read_b<C>(lds, ba, stage, T0);
#pragma unroll
  for (int i = 0; i < N_MFMA; i++) {
    const int u = i / C::MT, mt = i % C::MT, t = T0 + u;
    if (LD && mt == 0) {
#pragma unroll
      for (int q = 0; q < PER; q++)
        if (u * PER + q < NL) ld.issue(u * PER + q, load_stage, next_kb);
    }
    if (mt == 0 && t + 1 < T1) bfr[(u + 1) & 1] = PRE ? pre[u + 1] : read_b<C>(lds, ba, stage, t + 1);
    part[i % 3] = mfma_fp8(bfr[u & 1], af[mt]);
    if (i > 1) {
      const int pu = (i - 2) / C::MT, pm = (i - 2) % C::MT;
      promote(acc[pm][T0 + pu], part[(i - 2) % 3], sc[pm]);
    }
    // Keep the written order: MFMA i is issued before the promotion of
    // partial i-2, whose MFMA has finished by then, so the promotion needs
    // no wait states and the wave issues MFMAs back to back (promoting i-1
    // instead costs ~100 cycles of hazard waits per chunk; measured +1-2% on
    // the 256x256 shapes).
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i > 1) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (N_MFMA > 1)
    promote(acc[(N_MFMA - 2) % C::MT][T0 + (N_MFMA - 2) / C::MT], part[(N_MFMA - 2) % 3], sc[(N_MFMA - 2) % C::MT]);
  promote(acc[C::MT - 1][T1 - 1], part[(N_MFMA - 1) % 3], sc[C::MT - 1]);
}

// UE8M0 recipe: with power-of-two scales the scaling is exact, so the
// matrix core applies it -- v_mfma_scale takes one E8M0 exponent per operand
// row and 32-wide K block (lane l supplies row l % 16, block l / 16; here the
// four blocks of a row share one exponent), and the product accumulates across chunks in the
// MFMA accumulator itself: acc = MFMA(B, A, acc) * 2^(eb + ea), with no FP32
// promotion.  Per chunk, a lane's A exponent is that of its row's scale and
// the B exponent that of the wave's column block (uniform).
template <class C>
__device__ __forceinline__ void read_a_ue8m0(const uint8_t* lds, const FragAddr& aa, uint32_t sa_addr,
                                             uint32_t sb_addr, int stage, v8i_t (&af)[C::MT], int (&ea)[C::MT],
                                             int& eb) {
  eb = e8m0_of(*reinterpret_cast<const float*>(lds + sb_addr + stage * C::S_BYTES));
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    af[mt] = read_frag(lds, aa, (uint32_t)(stage * C::A_BYTES + 2048 * mt));
    ea[mt] = e8m0_of(*reinterpret_cast<const float*>(lds + sa_addr + stage * C::S_BYTES + 64 * mt));
  }
}

template <class C, bool LD>
__device__ __forceinline__ void mfma_tiles_ue8m0(const uint8_t* lds, const FragAddr& ba, int stage, int load_stage,
                                                 const v8i_t (&af)[C::MT], const int (&ea)[C::MT], int eb,
                                                 v4f_t (&acc)[C::MT][C::NT], const StageLoader<C>& ld, int next_kb) {
  constexpr int NL = StageLoader<C>::NSEG;
  constexpr int HALF = C::NT / 2 > 0 ? C::NT / 2 : 1;
  constexpr int PER = (NL + HALF - 1) / HALF;
  constexpr int N_MFMA = C::NT * C::MT;
  v8i_t bfr[2];
  bfr[0] = read_b<C>(lds, ba, stage, 0);
#pragma unroll
  for (int i = 0; i < N_MFMA; i++) {
    const int u = i / C::MT, mt = i % C::MT;
    if (mt == 0) {
#pragma unroll
      for (int q = 0; q < PER; q++)
        if (LD && u * PER + q < NL) ld.issue(u * PER + q, load_stage, next_kb);
      if (u + 1 < C::NT) bfr[(u + 1) & 1] = read_b<C>(lds, ba, stage, u + 1);
    }
    acc[mt][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[u & 1], af[mt], acc[mt][u], 0, 0, 0, eb, 0,
                                                                  ea[mt]);
  }
}

// MX recipe: one E8M0 scale per operand row and 32-wide K block, which is
// exactly what v_mfma_scale takes per lane (lane i + 16b supplies row i,
// K block b, i.e. K [32b, 32b + 32) of the chunk in memory order, which the
// staging order above keeps).  A lane's A scale is byte lg of its
// row's packed word; its B scale for column tile t is byte lg of the packed
// word of the tile column its B fragment row holds (ebo[t], a byte offset
// into the stage's weight-scale area).  The product accumulates across all
// of K in the MFMA accumulator: no FP32 promotion.
template <class C>
__device__ __forceinline__ void read_a_mx(const uint8_t* lds, const FragAddr& aa, uint32_t sa_addr, int stage,
                                          int lg, v8i_t (&af)[C::MT], int (&ea)[C::MT]) {
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    af[mt] = read_frag(lds, aa, (uint32_t)(stage * C::A_BYTES + 2048 * mt));
    const uint32_t w = *reinterpret_cast<const uint32_t*>(lds + sa_addr + stage * C::S_BYTES + 64 * mt);
    ea[mt] = (int)((w >> (8 * lg)) & 0xffu);
  }
}

template <class C>
__device__ __forceinline__ int read_eb_mx(const uint8_t* lds, const uint32_t (&ebo)[C::NT], int stage, int t, int lg) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(lds + ebo[t] + stage * C::S_BYTES);
  return (int)((w >> (8 * lg)) & 0xffu);
}

template <class C, bool LD>
__device__ __forceinline__ void mfma_tiles_mx(const uint8_t* lds, const FragAddr& ba, const uint32_t (&ebo)[C::NT],
                                              int stage, int load_stage, int lg, const v8i_t (&af)[C::MT],
                                              const int (&ea)[C::MT], v4f_t (&acc)[C::MT][C::NT],
                                              const StageLoader<C>& ld, int next_kb) {
  constexpr int NL = StageLoader<C>::NSEG;
  constexpr int HALF = C::NT / 2 > 0 ? C::NT / 2 : 1;
  constexpr int PER = (NL + HALF - 1) / HALF;
  constexpr int N_MFMA = C::NT * C::MT;
  v8i_t bfr[2];
  int ebr[2];
  bfr[0] = read_b<C>(lds, ba, stage, 0);
  ebr[0] = read_eb_mx<C>(lds, ebo, stage, 0, lg);
#pragma unroll
  for (int i = 0; i < N_MFMA; i++) {
    const int u = i / C::MT, mt = i % C::MT;
    if (mt == 0) {
#pragma unroll
      for (int q = 0; q < PER; q++)
        if (LD && u * PER + q < NL) ld.issue(u * PER + q, load_stage, next_kb);
      if (u + 1 < C::NT) {
        bfr[(u + 1) & 1] = read_b<C>(lds, ba, stage, u + 1);
        ebr[(u + 1) & 1] = read_eb_mx<C>(lds, ebo, stage, u + 1, lg);
      }
    }
    acc[mt][u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[u & 1], af[mt], acc[mt][u], 0, 0, 0,
                                                                  ebr[u & 1], 0, ea[mt]);
  }
}

// The 8 values of epilogue slot s of an MFMA row tile, rounded to bf16 and
// packed in column order (see the epilogue).
template <class C>
__device__ __forceinline__ uint4 pack8(const v4f_t (&a)[C::NT], int s) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int j0 = 8 * s + 2 * e, j1 = j0 + 1;
    w[e] = pack_bf16x2(a[j0 % C::NT][j0 / C::NT], a[j1 % C::NT][j1 / C::NT]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Where a tile's results go: bf16 D (d, optional when q is given) and, for
// the FP8-output form, E4M3 Q with its MN-major 1x128 scales (sd, sd_ld).
struct TileOut {
  uint16_t* d;
  uint8_t* q;
  float* sd;
  int64_t sd_ld;
};

// The bf16 output is a separate __restrict__ parameter (d == out.d): inlining
// a function with a noalias pointer argument tags every memory access of the
// tile body with alias metadata, and without any such metadata the
// wait-count pass treats each LDS read as a possible reader of every
// in-flight global->LDS copy and drains all of them (vmcnt(0)) before it,
// which serialises the K pipeline.  The pipeline orders those copies before
// the reads itself (explicit vmcnt waits and a barrier per K block).  The
// codegen test checks the count of full drains per kernel.
// The fused gate_up tile of the MoE layer (SILU): tile columns [0, 128) are
// gate rows gate_block*128 .. of the weight and [128, 256) the matching up
// rows, up_rows further on (b points at the gate block); the epilogue writes
// the 1x128-quantized activation bf16(silu(gate) * up) of act columns
// col0 .. col0 + 127 into q [M][ld] (the tile's output parameter) with
// scales sq [ld/128][sq_ld], zero for rows whose m_indices entry is negative.
struct GateUp {
  uint32_t up_rows = 0;
  int64_t gate_block = 0, up_block = 0;
  float* sq = nullptr;
  int64_t sq_ld = 0, col0 = 0, ld = 0;
  const int32_t* m_indices = nullptr;
};

// Epilogue of the fused gate_up tile (waves wn = 0, 1 hold the gate half,
// wn = 2, 3 the up half, with the same fragment geometry: value (mt, t, r)
// of lane L of gate wave (wm, h) and of up wave (wm, 2 + h) belong to the
// same activation column).  Every wave runs the same barriers.
//  1. The up waves store their bf16-rounded values in LDS by position (the
//     stages are free once every wave is past its last fragment read).
//  2. The gate waves form bf16(silu(bf16(gate)) * up) with silu_mul_f32,
//     zero for rows whose m_indices entry is negative -- the standalone
//     silu_mul_quantize kernel's values, bit for bit.
//  3. Each row's 128 activation columns lie on gate waves 0 and 1: their
//     amax meet through LDS, then each lane quantizes 8-column runs with the
//     activation quantizer's arithmetic and stores codes and the scale.
template <class C>
__device__ __forceinline__ void silu_epilogue(uint8_t* lds, v4f_t (&acc)[C::MT][C::NT], const GateUp& gu,
                                              uint8_t* q, int64_t m0, int wave, int wm, int wn, int lane) {
  static_assert(C::BM == 128 && C::BN == 256 && C::TN == 64 && C::WAVES_N == 4, "gate waves 0-1, up waves 2-3");
  constexpr int VALS = C::MT * C::NT * 4, WORDS = VALS / 8;
  const int li = lane & 15, lg = lane >> 4;
  uint4* xch = reinterpret_cast<uint4*>(lds);  // [slot][word][lane], 8 KB per slot
  const int slot = wm + C::WAVES_M * (wn & 1);
  // value v of a lane: acc[v / (4 NT)][(v / 4) % NT][v % 4]
  __syncthreads();  // every wave is past its last fragment read
  if (wn >= 2) {
#pragma unroll
    for (int i = 0; i < WORDS; i++) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int v0 = 8 * i + 2 * e, v1 = v0 + 1;
        w[e] = pack_bf16x2(acc[v0 / (C::NT * 4)][(v0 / 4) % C::NT][v0 % 4],
                           acc[v1 / (C::NT * 4)][(v1 / 4) % C::NT][v1 % 4]);
      }
      xch[(slot * WORDS + i) * 64 + lane] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();
  uint32_t am[C::MT];
  if (wn < 2) {
    bool live[C::MT];
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++) live[mt] = gu.m_indices[m0 + wm * C::TM + 16 * mt + li] >= 0;
#pragma unroll
    for (int i = 0; i < WORDS; i++) {
      const uint4 u = xch[(slot * WORDS + i) * 64 + lane];
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int v = 8 * i + e, mt = v / (C::NT * 4), t = (v / 4) % C::NT, r = v % 4;
        const float g = __uint_as_float(bf16_rne(acc[mt][t][r]) << 16);
        const float up = (e & 1) ? bf16_hi(uw[e >> 1]) : bf16_lo(uw[e >> 1]);
        const float act = __uint_as_float(bf16_rne(silu_mul_f32(g, up)) << 16);
        acc[mt][t][r] = live[mt] ? act : 0.0f;
      }
    }
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++) {
      uint32_t m_ = 0;
#pragma unroll
      for (int s = 0; s < C::NT / 2; s++) m_ = max(m_, absmax8_bits(pack8<C>(acc[mt], s)));
      m_ = max(m_, (uint32_t)__shfl_xor((int)m_, 16));
      m_ = max(m_, (uint32_t)__shfl_xor((int)m_, 32));
      am[mt] = m_;
    }
    uint32_t* ex = reinterpret_cast<uint32_t*>(lds + C::EPI_OFF);
    if (lg == 0) {
#pragma unroll
      for (int mt = 0; mt < C::MT; mt++) ex[wave * C::TM + 16 * mt + li] = am[mt];
    }
  }
  __syncthreads();
  if (wn < 2) {
    const uint32_t* ex = reinterpret_cast<const uint32_t*>(lds + C::EPI_OFF);
    const int partner = wm + C::WAVES_M * (wn ^ 1);
    const int64_t cw = gu.col0 + wn * C::TN;
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++) {
      const int64_t row = m0 + wm * C::TM + 16 * mt + li;
      const float sc = group_scale(__uint_as_float(max(am[mt], ex[partner * C::TM + 16 * mt + li])));
      const double r = 1.0 / (double)sc;
#pragma unroll
      for (int s = 0; s < C::NT / 2; s++) {
        const int64_t c0 = cw + 32 * s + 8 * lg;
        *reinterpret_cast<uint2*>(q + row * gu.ld + c0) = quantize8(pack8<C>(acc[mt], s), r);
      }
      if (lg == 0 && wn == 0) gu.sq[(gu.col0 / kGroup) * gu.sq_ld + row] = sc;
    }
  }
}

// bf16 epilogue of a wave tile: lane (li, lg) owns rows m0 + wm*TM + 16*mt
// + li; its values j = 8*s + e (s < NT/2, e < 8) go to column n0 + wn*TN +
// 32*s + 8*lg + e, held in acc[mt][j % NT][j / NT], rounded to bf16 (RNE)
// and stored as 16-byte words where the row is aligned and in range.
template <class C, int MT0 = 0, int MT1 = C::MT>
__device__ __forceinline__ void store_bf16(uint16_t* __restrict__ d, const v4f_t (&acc)[C::MT][C::NT], int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int wm, int wn, int li, int lg) {
  const bool vec = (N % 8) == 0;
#pragma unroll
  for (int mt = MT0; mt < MT1; mt++) {
    const int64_t row = m0 + wm * C::TM + 16 * mt + li;
    if (row >= M) continue;
    uint16_t* drow = d + row * N;
#pragma unroll
    for (int s = 0; s < C::NT / 2; s++) {
      const int64_t c0 = n0 + wn * C::TN + 32 * s + 8 * lg;
      if (vec && c0 + 8 <= N) {
        *reinterpret_cast<uint4*>(drow + c0) = pack8<C>(acc[mt], s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int j = 8 * s + e;
          if (c0 + e < N) drow[c0 + e] = (uint16_t)bf16_rne(acc[mt][j % C::NT][j / C::NT]);
        }
      }
    }
  }
}

// K split over two workgroups per output tile (fp8_gemm_nt with a
// workspace, for shapes whose 256x256 tiles would leave half the compute
// units idle).  Each workgroup sums the chunks kb0 .. kb1 - 1 of its tile in
// FP32 as gemm_tile does; the two partial sums then meet through the
// workspace: the first workgroup of the pair to finish (an atomic arrival
// count) writes its partial and raises the tile's ready flag; the second
// waits for the flag -- it only waits on a workgroup that has already
// arrived, so the wait always ends -- adds the partial to its own
// (acc0 + acc1, a single FP32 addition, the same bits whichever finished
// first), rounds to bf16, stores, and sets the counter and the flag back
// to zero for the next call.
struct SplitK {
  int kb0 = 0, kb1 = 0;     // chunk range; kb1 == 0: all of K
  float* partial = nullptr;  // the tile's FP32 slot, BM * BN floats (n-way: parts consecutive slots)
  int* arrive = nullptr;     // the tile's arrival count (0 between calls)
  int* ready = nullptr;      // the tile's partial-ready flag (0 between calls; pair form only)
  int parts = 1, part = 0;   // n-way form: this workgroup sums part `part` of `parts`
};

// Longest wait for the partner's partial (s_sleep 2 units, ~128 cycles
// each): far beyond the partner's few-microsecond store, a bound that turns
// a broken invariant into an unwritten output tile instead of a hang.
constexpr int kSplitSpinLimit = 1 << 24;

// Cache policy of the partial's stores and loads: system scope (sc0 sc1),
// so that they write through to and read from memory -- the two workgroups
// of a tile may sit on different XCDs, whose L2 caches are not coherent with
// each other -- without the whole-cache writeback and invalidation an
// agent-scope fence costs.
constexpr int kSysCoherent = 1 | 16;

template <class C, int MT0>
__device__ __forceinline__ void add_store_rows(rsrc_t rp, uint32_t base, v4f_t (&acc)[C::MT][C::NT],
                                               uint16_t* __restrict__ d, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                               int wm, int wn, int li, int lg) {
  constexpr int R = 2;  // rows of MFMA tiles per batch: 2 * NT loads in flight
  if constexpr (MT0 < C::MT) {
    v4f_t p[R][C::NT];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
      for (int t = 0; t < C::NT; t++)
        p[r][t] = __builtin_bit_cast(v4f_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rp, base + (uint32_t)((MT0 + r) * C::NT + t) * 1024u, 0, kSysCoherent));
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
      for (int t = 0; t < C::NT; t++) acc[MT0 + r][t] += p[r][t];
    store_bf16<C, MT0, MT0 + R>(d, acc, M, N, m0, n0, wm, wn, li, lg);
    __builtin_amdgcn_sched_barrier(0);
    add_store_rows<C, MT0 + R>(rp, base, acc, d, M, N, m0, n0, wm, wn, li, lg);
  }
}

template <class C>
__device__ __forceinline__ void split_fixup(uint8_t* lds, v4f_t (&acc)[C::MT][C::NT], const SplitK& sk,
                                            uint16_t* __restrict__ d, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                            int wave, int wm, int wn, int lane) {
  int* shared = reinterpret_cast<int*>(lds);
  __syncthreads();  // every wave is past its last fragment read: LDS is free
  if (threadIdx.x == 0)
    shared[0] = __hip_atomic_fetch_add(sk.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  const bool first = shared[0] == 0;
  // lane's j-th 4-float group at float4 index (wave * MT * NT + j) * 64 +
  // lane of the tile's slot: each wave store or load moves 1 KB of
  // consecutive bytes
  const rsrc_t rp = make_rsrc(sk.partial, (uint32_t)(C::BM * C::BN * 4));
  const uint32_t base = ((uint32_t)wave * (C::MT * C::NT) * 64u + (uint32_t)lane) * 16u;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  if (first) {
#pragma unroll
    for (int j = 0; j < C::MT * C::NT; j++)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[j / C::NT][j % C::NT]), rp,
                                             base + (uint32_t)j * 1024u, 0, kSysCoherent);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial has reached memory
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(sk.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return;
  }
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(sk.ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == 0 && spins < kSplitSpinLimit) {
      __builtin_amdgcn_s_sleep(2);
      spins++;
    }
    shared[1] = spins < kSplitSpinLimit;
  }
  __syncthreads();
  // No partial within the bound (a broken invariant): the tile is left
  // unwritten rather than the workgroup hanging.
  if (shared[1] == 0) return;  // uniform
  if (threadIdx.x == 0) {
    __hip_atomic_store(sk.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(sk.ready, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  // one row of MFMA tiles at a time: its partial is loaded, added and stored
  // as bf16 before the next row's loads, so that the partial and all of acc
  // are never live at once
  const int li = lane & 15, lg = lane >> 4;
  add_store_rows<C, 0>(rp, base, acc, d, M, N, m0, n0, wm, wn, li, lg);
}

// n-way form: the tile's parts summed in a fixed order, p_0 + p_1 + ... +
// p_{parts-1}, one row of MFMA tiles at a time, this workgroup's own part
// (index own) taken from its registers and every other part loaded from its
// slot; the bits do not depend on which part arrived last.
template <class C, int MT0>
__device__ __forceinline__ void load_part_rows(rsrc_t rp, uint32_t off, const v4f_t (&acc)[C::MT][C::NT], bool own,
                                               v4f_t (&p)[2][C::NT]) {
  if (own) {  // uniform
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int t = 0; t < C::NT; t++) p[r][t] = acc[MT0 + r][t];
  } else {
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int t = 0; t < C::NT; t++)
        p[r][t] = __builtin_bit_cast(v4f_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rp, off + (uint32_t)((MT0 + r) * C::NT + t) * 1024u, 0, kSysCoherent));
  }
}

template <class C, int MT0>
__device__ __forceinline__ void sum_store_rows(rsrc_t rp, uint32_t base, int parts, int own,
                                               v4f_t (&acc)[C::MT][C::NT], uint16_t* __restrict__ d, int64_t M,
                                               int64_t N, int64_t m0, int64_t n0, int wm, int wn, int li, int lg) {
  constexpr uint32_t kSlot = (uint32_t)(C::BM * C::BN * 4);
  if constexpr (MT0 < C::MT) {
    static_assert(C::MT % 2 == 0, "rows of MFMA tiles go in pairs");
    v4f_t sum[2][C::NT];
    load_part_rows<C, MT0>(rp, base, acc, own == 0, sum);
    for (int i = 1; i < parts; i++) {
      v4f_t p[2][C::NT];
      load_part_rows<C, MT0>(rp, (uint32_t)i * kSlot + base, acc, own == i, p);
#pragma unroll
      for (int r = 0; r < 2; r++)
#pragma unroll
        for (int t = 0; t < C::NT; t++) sum[r][t] += p[r][t];
    }
#pragma unroll
    for (int r = 0; r < 2; r++)
#pragma unroll
      for (int t = 0; t < C::NT; t++) acc[MT0 + r][t] = sum[r][t];
    store_bf16<C, MT0, MT0 + 2>(d, acc, M, N, m0, n0, wm, wn, li, lg);
    __builtin_amdgcn_sched_barrier(0);
    sum_store_rows<C, MT0 + 2>(rp, base, parts, own, acc, d, M, N, m0, n0, wm, wn, li, lg);
  }
}

// n-way K split without waiting: every part stores its FP32 partial to its
// own slot (system scope, written through to memory), and only then counts
// its arrival; the part that arrives last -- every other part's slot already
// in memory -- sums the parts in index order, rounds and stores the tile,
// and resets the count for the next call.  No workgroup ever waits on
// another, so the protocol cannot hang whatever the residency.  parts == 1:
// the plain bf16 store.
template <class C>
__device__ __forceinline__ void split_fixup_n(uint8_t* lds, v4f_t (&acc)[C::MT][C::NT], const SplitK& sk,
                                              uint16_t* __restrict__ d, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                              int wave, int wm, int wn, int lane) {
  const int li = lane & 15, lg = lane >> 4;
  if (sk.parts <= 1) {
    store_bf16<C>(d, acc, M, N, m0, n0, wm, wn, li, lg);
    return;
  }
  constexpr uint32_t kSlot = (uint32_t)(C::BM * C::BN * 4);
  const rsrc_t rp = make_rsrc(sk.partial, (uint32_t)sk.parts * kSlot);
  // the slot layout of split_fixup: 1 KB of consecutive bytes per wave store
  const uint32_t base = ((uint32_t)wave * (C::MT * C::NT) * 64u + (uint32_t)lane) * 16u;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int j = 0; j < C::MT * C::NT; j++)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[j / C::NT][j % C::NT]), rp,
                                           (uint32_t)sk.part * kSlot + base + (uint32_t)j * 1024u, 0, kSysCoherent);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of the part has reached memory
  int* shared = reinterpret_cast<int*>(lds);
  __syncthreads();  // every wave's share stored; every wave past its last fragment read (LDS free)
  if (threadIdx.x == 0)
    shared[0] = __hip_atomic_fetch_add(sk.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  if (shared[0] != sk.parts - 1) return;  // uniform: another part finishes the tile
  if (threadIdx.x == 0) __hip_atomic_store(sk.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  sum_store_rows<C, 0>(rp, base, sk.parts, sk.part, acc, d, M, N, m0, n0, wm, wn, li, lg);
}

// ROWSKIP (the masked product, whose tiles are often partly filled): a wave
// whose rows all lie past M skips its fragment reads and MFMAs and only
// issues its copies, and the waves are laid out row-half-major (wm = wave /
// WAVES_N), so that waves w and w + 4 -- which share a SIMD -- belong to
// different row halves and a skipping wave leaves its SIMD to the other.
// The results are the same bits.
template <class C, bool FP8OUT = false, bool UE8M0 = false, bool MX = false, bool SILU = false, bool ROWSKIP = false,
          int SPLIT = 0>
__device__ __forceinline__ void gemm_tile(uint8_t* lds, const uint8_t* a, const uint8_t* b, const float* sa,
                                          const float* sb_base, uint16_t* __restrict__ d, const TileOut& out,
                                          int64_t M, int64_t N, int K, int64_t sa_ld, int64_t m0, int64_t n0,
                                          int64_t sb_ld = 0, const GateUp& gu = GateUp{}, const SplitK& sk = SplitK{}) {
  // the FP8-output and SiLU epilogues pair waves as wave = wm + WAVES_M * wn
  static_assert(!ROWSKIP || (!FP8OUT && !UE8M0 && !MX && !SILU), "row skipping is for the bf16 FP32-scale tile");
  static_assert(!C::REG_SCALES || (C::STAGES == 2 && !FP8OUT && !UE8M0 && !MX && !SILU && !ROWSKIP && SPLIT == 0),
                "register scales: the two-stage bf16 FP32-scale tile");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = ROWSKIP ? wave / C::WAVES_N : wave % C::WAVES_M;
  const int wn = ROWSKIP ? wave % C::WAVES_N : wave / C::WAVES_M;
  const int KB = K / kGroup;
  const uint32_t a_rows = (uint32_t)(M - m0 < C::BM ? M - m0 : C::BM);
  const uint32_t b_rows = SILU ? gu.up_rows + (uint32_t)C::BN : (uint32_t)(N - n0 < C::BN ? N - n0 : C::BN);
  const rsrc_t ra = make_rsrc(a, a_rows * (uint32_t)K);
  const rsrc_t rb = make_rsrc(b, b_rows * (uint32_t)K);
  const rsrc_t rs = make_rsrc(sa + m0, (uint32_t)(((int64_t)KB * sa_ld - m0) * 4));
  // Weight scales: lane j of wave 1 copies the scale of column block
  // n0/128 + j (clamped to the last block: a wave entirely past N never
  // stores its results).
  const int64_t nblocks = (N + kGroup - 1) / kGroup;
  int64_t nb_lane = n0 / kGroup + lane;
  if (nb_lane >= nblocks) nb_lane = nblocks - 1;
  if constexpr (SILU) nb_lane = lane == 0 ? gu.gate_block : gu.up_block;
  // MX: lane j copies the packed words of columns n0 + 4j .. n0 + 4j + 3 of
  // chunk kb (sb_base[kb * sb_ld + column]).
  const rsrc_t rsb = MX ? make_rsrc(sb_base + n0, (uint32_t)(((int64_t)KB * sb_ld - n0) * 4))
                        : make_rsrc(sb_base, (uint32_t)(nblocks * KB * 4));
  const uint32_t vsb = MX ? (uint32_t)lane * 16u : (uint32_t)(nb_lane * KB * 4);

  v4f_t acc[C::MT][C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; i++)
#pragma unroll
    for (int j = 0; j < C::NT; j++) acc[i][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};

  const int li = lane & 15, lg = lane >> 4;
  v8i_t af[C::MT];
  float sc[C::MT];
  uint32_t voff[StageLoader<C>::NSEG];
  stage_offsets<C>(voff, (uint32_t)K, wave, lane, SILU ? gu.up_rows : 0u);
  const StageLoader<C> loader{lds, ra, rb, rs, rsb, voff, (uint32_t)(sa_ld * 4), vsb, wave, lane,
                              MX ? (uint32_t)(sb_ld * 4) : 0u, (uint32_t)K};
  // MX: byte offsets of the packed weight-scale word each lane's B fragment
  // row refers to, per column tile.
  uint32_t ebo[C::NT];
  if constexpr (MX) {
#pragma unroll
    for (int t = 0; t < C::NT; t++)
      ebo[t] = C::S_OFF + C::SB_IN_S + (uint32_t)(wn * C::TN + wave_col<C>(li, t)) * 4u;
  }
  const FragAddr aa = frag_addr(C::A_OFF, wm * C::TM, li, lg);
  const FragAddr ba = frag_addr(C::B_OFF, wn * C::TN, li, lg);
  const uint32_t sa_addr = C::S_OFF + (uint32_t)(wm * C::TM + li) * 4u;
  // The stage's slot j holds column block n0/128 + j (n0 is a multiple of 64).
  const uint32_t sb_addr =
      C::S_OFF + C::SB_IN_S + (uint32_t)((n0 + wn * C::TN) / kGroup - n0 / kGroup) * 4u;
  // One chunk: wait for this wave's copies of chunk kb, barrier (every
  // wave's copies have landed, and the stage chunk kb - 1 occupied is no
  // longer read), then compute chunk kb while filling that stage with chunk
  // kb + STAGES - 1.  Near the end the copy repeats the last chunk (valid
  // addresses, into a stage that is not read again), so the loop body has no
  // branch.  Copies return in issue order, so "chunk kb has landed" is "at
  // most the copies of the chunks after it are outstanding": none with two
  // stages; with three, one chunk's NSEG segments plus the scale copy that
  // waves 0 and 1 issue.
  // The loop is written once per copying role (CP: this wave issues
  // segment copies), chosen once per wave, so that the loop itself has no
  // branch around the copies.
  const int kb0 = SPLIT ? sk.kb0 : 0, kb1 = SPLIT ? sk.kb1 : KB;
  // REG_SCALES: this wave's scales of the next chunk -- its rows' activation
  // scales (row wm*TM + 16 mt + li: the rows of its promotions) and its
  // column block's weight scale -- loaded one chunk ahead; the two-stage
  // loop's vmcnt(0) at the top of a chunk covers them.  Rows past M read
  // whatever the scale buffer holds there, as the LDS copy does; their
  // outputs are never stored.
  float sa_nx[C::MT], sb_nx = 0.0f;
  const int64_t nb_wave = (n0 + wn * C::TN) / kGroup < nblocks ? (n0 + wn * C::TN) / kGroup : nblocks - 1;
  auto load_scales = [&](int kb) {
    if constexpr (C::REG_SCALES) {
#pragma unroll
      for (int mt = 0; mt < C::MT; mt++)
        sa_nx[mt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rs, (uint32_t)(wm * C::TM + 16 * mt + li) * 4u, (uint32_t)kb * (uint32_t)(sa_ld * 4), 0));
      sb_nx = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsb, (uint32_t)(nb_wave * KB + kb) * 4u, 0, 0));
    }
  };
  loader.all(0, kb0);
  load_scales(kb0);
  if (C::STAGES == 3) loader.all(1, kb0 + 1 < kb1 ? kb0 + 1 : kb0);
  auto k_loop = [&](auto cp) {
  constexpr bool CP = decltype(cp)::value;
  int stage = 0;
  for (int kb = kb0; kb < kb1; kb++) {
    const int load_stage = stage == 0 ? C::STAGES - 1 : stage - 1;
    const int next = kb + C::STAGES - 1 < kb1 ? kb + C::STAGES - 1 : kb1 - 1;
    if (C::STAGES == 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    } else if (wave < 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | (StageLoader<C>::NSEG + 1));  // vmcnt(NSEG + 1)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70 | StageLoader<C>::NSEG);  // vmcnt(NSEG)
    }
    barrier_no_fence();
    if constexpr (C::REG_SCALES) {
      // the products first, so that the next chunk's loads reuse the same
      // registers (no loop-carried copies, whose waits would drain the copies)
#pragma unroll
      for (int mt = 0; mt < C::MT; mt++) sc[mt] = sa_nx[mt] * sb_nx;
      load_scales(next);
#pragma unroll
      for (int mt = 0; mt < C::MT; mt++) af[mt] = read_frag(lds, aa, (uint32_t)(stage * C::A_BYTES + 2048 * mt));
      mfma_tiles<C, 0, C::NT, false, CP>(lds, ba, stage, load_stage, af, sc, nullptr, acc, loader, next);
      stage = stage + 1 == C::STAGES ? 0 : stage + 1;
      continue;
    }
    if (wave < 2) loader.issue(StageLoader<C>::NSEG, load_stage, next);  // scales
    if constexpr (MX) {
      int ea[C::MT];
      read_a_mx<C>(lds, aa, sa_addr, stage, lg, af, ea);
      mfma_tiles_mx<C, CP>(lds, ba, ebo, stage, load_stage, lg, af, ea, acc, loader, next);
    } else if constexpr (UE8M0) {
      int ea[C::MT], eb;
      read_a_ue8m0<C>(lds, aa, sa_addr, sb_addr, stage, af, ea, eb);
      mfma_tiles_ue8m0<C, CP>(lds, ba, stage, load_stage, af, ea, eb, acc, loader, next);
    } else if (ROWSKIP && (uint32_t)(wm * C::TM) >= a_rows) {  // uniform: this wave's rows are all past M
      if (CP) {
#pragma unroll
        for (int i = 0; i < StageLoader<C>::NSEG; i++) loader.issue(i, load_stage, next);
      }
    } else {
      read_a<C>(lds, aa, sa_addr, sb_addr, stage, af, sc);
      mfma_tiles<C, 0, C::NT, false, CP>(lds, ba, stage, load_stage, af, sc, nullptr, acc, loader, next);
    }
    stage = stage + 1 == C::STAGES ? 0 : stage + 1;
  }
  };
  if constexpr (C::COPY_WAVES == C::WAVES) {
    k_loop(std::true_type{});
  } else {
    if (loader.copier()) k_loop(std::true_type{});  // wave-uniform
    else k_loop(std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy into LDS outlives the loop

  if constexpr (SILU) {
    // the codes go through d, the tile's __restrict__ output (see below)
    silu_epilogue<C>(lds, acc, gu, reinterpret_cast<uint8_t*>(d), m0, wave, wm, wn, lane);
    return;
  }

  if constexpr (SPLIT == 1) {
    split_fixup<C>(lds, acc, sk, d, M, N, m0, n0, wave, wm, wn, lane);
    return;
  } else if constexpr (SPLIT == 2) {
    split_fixup_n<C>(lds, acc, sk, d, M, N, m0, n0, wave, wm, wn, lane);
    return;
  }

  // Epilogue: bf16 (store_bf16), or the FP8 output below.
  if constexpr (!FP8OUT) {
    store_bf16<C>(d, acc, M, N, m0, n0, wm, wn, li, lg);
    return;
  } else {
  // FP8 output (N % 128 == 0): the bf16 values above, quantized per 1x128
  // group of each row exactly as quantize_fp8_groups quantizes a bf16
  // input -- amax over the group, s = fl32(amax/448) (1 for a zero group),
  // E4M3(fl32(x / s)) -- so the result equals that call applied to the bf16
  // output, bit for bit.  A row's group is spread over the four lanes li +
  // 16 lg of a wave (TN = 128), or of two partner waves wn, wn ^ 1 (TN = 64,
  // amax exchanged through LDS).
  uint32_t am[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    uint32_t m_ = 0;
#pragma unroll
    for (int s = 0; s < C::NT / 2; s++) m_ = max(m_, absmax8_bits(pack8<C>(acc[mt], s)));
    m_ = max(m_, (uint32_t)__shfl_xor((int)m_, 16));
    m_ = max(m_, (uint32_t)__shfl_xor((int)m_, 32));
    am[mt] = m_;
  }
  if constexpr (C::TN == 64) {
    uint32_t* ex = reinterpret_cast<uint32_t*>(lds + C::EPI_OFF);
    if (lg == 0) {
#pragma unroll
      for (int mt = 0; mt < C::MT; mt++) ex[wave * C::TM + 16 * mt + li] = am[mt];
    }
    __syncthreads();
    const int partner = wm + C::WAVES_M * (wn ^ 1);
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++) am[mt] = max(am[mt], ex[partner * C::TM + 16 * mt + li]);
  }
  const int64_t cw = n0 + wn * C::TN;  // first column of this wave
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    const int64_t row = m0 + wm * C::TM + 16 * mt + li;
    if (row >= M || cw >= N) continue;
    const float sc = group_scale(__uint_as_float(am[mt]));
    const double r = 1.0 / (double)sc;
#pragma unroll
    for (int s = 0; s < C::NT / 2; s++) {
      const int64_t c0 = cw + 32 * s + 8 * lg;
      const uint4 w = pack8<C>(acc[mt], s);
      *reinterpret_cast<uint2*>(out.q + row * N + c0) = quantize8(w, r);
      if (d != nullptr) *reinterpret_cast<uint4*>(d + row * N + c0) = w;
    }
    if (lg == 0 && (C::TN == 128 || (wn & 1) == 0)) out.sd[(cw / kGroup) * out.sd_ld + row] = sc;
  }
  }
}

// Block -> tile order.  Consecutive workgroup ids are dispatched round-robin
// over the 8 XCDs; remapping gives each XCD a contiguous run of tiles, and the
// run is walked in bands of 8 tile rows so that the tiles an XCD has in
// flight share A and B panels in its L2.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  int v = bid;
  if ((nblocks & 7) == 0) v = (bid & 7) * (nblocks >> 3) + (bid >> 3);
  constexpr int kBand = 8;
  const int per_band = kBand * tiles_n;
  const int band = v / per_band;
  const int first = band * kBand;
  const int rows = tiles_m - first < kBand ? tiles_m - first : kBand;
  const int r = v - band * per_band;
  tm = first + r % rows;
  tn = r / rows;
}

// ------------------------------------------------------------- persistent
// tile_coords over a tile count padded to a multiple of 8: false for an id
// past the tiles_m x tiles_n tiles.
__device__ __forceinline__ bool tile_coords_padded(int t, int t_pad, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int v = (t & 7) * (t_pad >> 3) + (t >> 3);
  if (v >= tiles_m * tiles_n) return false;
  constexpr int kBand = 8;
  const int per_band = kBand * tiles_n;
  const int band = v / per_band;
  const int first = band * kBand;
  const int rows = tiles_m - first < kBand ? tiles_m - first : kBand;
  const int r = v - band * per_band;
  tm = first + r % rows;
  tn = r / rows;
  return true;
}

// One output tile of a persistent walk: its corner and operand bases.
struct TileRef {
  int64_t m0, n0;
  const uint8_t* a;   // A + m0 * K
  const uint8_t* b;   // B (of the tile's group) + n0 * K
  const float* sb;    // weight scales of the tile's group
};

// Dense tiles: every id below tiles_m x tiles_n is a tile.
struct DenseTiles {
  const uint8_t* A;
  const uint8_t* B;
  const float* SB;
  int64_t K;
  int tiles_m, tiles_n, t_pad, bm, bn;
  __device__ __forceinline__ bool get(int t, TileRef& r) const {
    int tm, tn;
    if (!tile_coords_padded(t, t_pad, tiles_m, tiles_n, tm, tn)) return false;
    r.m0 = (int64_t)tm * bm;
    r.n0 = (int64_t)tn * bn;
    r.a = A + r.m0 * K;
    r.b = B + r.n0 * K;
    r.sb = SB;
    return true;
  }
};

// Grouped tiles: 128-row blocks of a 128-aligned group layout; a block whose
// first row is padding (-1 or out of range) is not a tile.
struct GroupedTiles {
  const uint8_t* A;
  const uint8_t* B;
  const float* SB;
  const int32_t* m_indices;
  int64_t M, N, K;
  int num_groups, tiles_m, tiles_n, t_pad;
  __device__ __forceinline__ bool get(int t, TileRef& r) const {
    int tm, tn;
    if (!tile_coords_padded(t, t_pad, tiles_m, tiles_n, tm, tn)) return false;
    r.m0 = (int64_t)tm * 128;
    // A scalar load (constant address space, uniform address): a vector load
    // here would make its use wait for every copy in flight, the next tile's
    // prefetch included.
    const int g = ((const __attribute__((address_space(4))) int32_t*)m_indices)[r.m0];
    if (g < 0 || g >= num_groups) return false;
    r.n0 = (int64_t)tn * 256;
    r.a = A + r.m0 * K;
    r.b = B + (int64_t)g * N * K + r.n0 * K;
    const int64_t KB = K / kGroup, NB = (N + kGroup - 1) / kGroup;
    r.sb = SB + (int64_t)g * NB * KB;
    return true;
  }
};

// The first tile id >= t (stepping by the grid) that is a tile, or t_pad.
template <class Src>
__device__ __forceinline__ int next_tile(const Src& src, int t, TileRef& r) {
  for (; t < src.t_pad; t += (int)gridDim.x)
    if (src.get(t, r)) return t;
  return src.t_pad;
}

template <class C>
__device__ __forceinline__ StageLoader<C> tile_loader(uint8_t* lds, const TileRef& t, const float* sa, int64_t sa_ld,
                                                      int64_t M, int64_t N, int K, const uint32_t* voff, int wave,
                                                      int lane) {
  const int KB = K / kGroup;
  const uint32_t a_rows = (uint32_t)(M - t.m0 < C::BM ? M - t.m0 : C::BM);
  const uint32_t b_rows = (uint32_t)(N - t.n0 < C::BN ? N - t.n0 : C::BN);
  const int64_t nblocks = (N + kGroup - 1) / kGroup;
  int64_t nb_lane = t.n0 / kGroup + lane;
  if (nb_lane >= nblocks) nb_lane = nblocks - 1;
  return StageLoader<C>{lds,
                        make_rsrc(t.a, a_rows * (uint32_t)K),
                        make_rsrc(t.b, b_rows * (uint32_t)K),
                        make_rsrc(sa + t.m0, (uint32_t)(((int64_t)KB * sa_ld - t.m0) * 4)),
                        make_rsrc(t.sb, (uint32_t)(nblocks * KB * 4)),
                        voff,
                        (uint32_t)(sa_ld * 4),
                        (uint32_t)(nb_lane * KB * 4),
                        wave,
                        lane,
                        0u,
                        (uint32_t)K};
}

__device__ __forceinline__ TileRef select_tile(bool first, const TileRef& x, const TileRef& y) {
  TileRef r = y;
  if (first) r = x;
  return r;
}

// The bf16 results of a finished tile, packed while the next tile starts.
template <class C>
__device__ __forceinline__ void store_packed(uint16_t* __restrict__ d, const uint4 (&w)[C::MT][C::NT / 2],
                                             int64_t M, int64_t N, int64_t m0, int64_t n0, int wm, int wn, int li,
                                             int lg) {
  const bool vec = (N % 8) == 0;
#pragma unroll
  for (int mt = 0; mt < C::MT; mt++) {
    const int64_t row = m0 + wm * C::TM + 16 * mt + li;
    if (row >= M) continue;
    uint16_t* drow = d + row * N;
#pragma unroll
    for (int s = 0; s < C::NT / 2; s++) {
      const int64_t c0 = n0 + wn * C::TN + 32 * s + 8 * lg;
      if (vec && c0 + 8 <= N) {
        *reinterpret_cast<uint4*>(drow + c0) = w[mt][s];
      } else {
        const uint32_t v[4] = {w[mt][s].x, w[mt][s].y, w[mt][s].z, w[mt][s].w};
#pragma unroll
        for (int e = 0; e < 8; e++)
          if (c0 + e < N) drow[c0 + e] = (uint16_t)(e & 1 ? v[e / 2] >> 16 : v[e / 2] & 0xffff);
      }
    }
  }
}

// Persistent walk over the tiles of `src`: workgroup w takes tiles w, w + G,
// w + 2G, ... (G = the grid, a multiple of 8, so every tile of a workgroup
// falls in its XCD's run).  The K pipeline runs on across tiles: during the
// last STAGES - 1 chunks of a tile the copies already fetch the first chunks
// of the next one, so no tile starts with an empty pipeline.  A finished
// tile's results are rounded and packed to registers, and (three stages)
// stored after the next chunk's barrier; the chunk after that waits for every
// outstanding memory operation (the stores included) before its barrier.
// With two stages every chunk already starts with that wait, so the results
// are stored as soon as they are packed.  Needs
// K / 128 >= STAGES - 1.  Per output element the arithmetic is that of
// gemm_tile, so the results are bit-identical.
template <class C, class Src>
__device__ __forceinline__ void gemm_persistent(uint8_t* lds, const Src& src, const float* sa, int64_t sa_ld,
                                                uint16_t* __restrict__ d, int64_t M, int64_t N, int K) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int li = lane & 15, lg = lane >> 4;
  const int KB = K / kGroup;
  const int G = (int)gridDim.x;

  static_assert(!C::REG_SCALES, "the walk stages its scales through LDS");
  TileRef cur, nxt;
  int t = next_tile(src, (int)blockIdx.x, cur);
  if (t >= src.t_pad) return;  // uniform, before any barrier
  int tn_ = next_tile(src, t + G, nxt);
  bool has_next = tn_ < src.t_pad;
  if (!has_next) nxt = cur;

  uint32_t voff[StageLoader<C>::NSEG];
  stage_offsets<C>(voff, (uint32_t)K, wave, lane);
  const FragAddr aa = frag_addr(C::A_OFF, wm * C::TM, li, lg);
  const FragAddr ba = frag_addr(C::B_OFF, wn * C::TN, li, lg);
  const uint32_t sa_addr = C::S_OFF + (uint32_t)(wm * C::TM + li) * 4u;
  static_assert(C::BN % kGroup == 0, "the walk takes tiles of whole 128-column blocks");
  const uint32_t sb_addr = C::S_OFF + C::SB_IN_S + (uint32_t)((wn * C::TN) / kGroup) * 4u;

  v4f_t acc[C::MT][C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; i++)
#pragma unroll
    for (int j = 0; j < C::NT; j++) acc[i][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
  v8i_t af[C::MT];
  float sc[C::MT];
  uint4 pend[C::MT][C::NT / 2];
  int64_t pend_m0 = 0, pend_n0 = 0;

  {
    const StageLoader<C> l0 = tile_loader<C>(lds, cur, sa, sa_ld, M, N, K, voff, wave, lane);
    l0.all(0, 0);
    if (C::STAGES == 3) l0.all(1, 1);
  }
  int pending = 0;  // three stages: 1 = packed results to store, 2 = their stores in flight
  int stage = 0, kb = 0;
  // written once per copying role, as gemm_tile's loop
  auto walk = [&](auto cp) {
  constexpr bool CP = decltype(cp)::value;
  while (true) {
    const int load_stage = stage == 0 ? C::STAGES - 1 : stage - 1;
    // The chunk this iteration copies: STAGES - 1 ahead, in this tile or the
    // next (the last tile repeats its last chunk into a stage never read).
    const int q = kb + C::STAGES - 1;
    const bool in_cur = q < KB || !has_next;
    const int next_kb = q < KB ? q : (has_next ? q - KB : KB - 1);
    const StageLoader<C> ld = tile_loader<C>(lds, select_tile(in_cur, cur, nxt), sa, sa_ld, M, N, K, voff, wave,
                                             lane);
    if (C::STAGES == 2 || pending == 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      if (pending == 2) pending = 0;
    } else if (wave < 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | (StageLoader<C>::NSEG + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70 | StageLoader<C>::NSEG);
    }
    barrier_no_fence();
    if (pending == 1) {
      store_packed<C>(d, pend, M, N, pend_m0, pend_n0, wm, wn, li, lg);
      pending = 2;
    }
    if (wave < 2) ld.issue(StageLoader<C>::NSEG, load_stage, next_kb);  // scales
    read_a<C>(lds, aa, sa_addr, sb_addr, stage, af, sc);
    mfma_tiles<C, 0, C::NT, false, CP>(lds, ba, stage, load_stage, af, sc, nullptr, acc, ld, next_kb);
    stage = stage + 1 == C::STAGES ? 0 : stage + 1;
    if (kb + 1 < KB) {
      kb++;
      continue;
    }
    // Tile done: pack its results (two stages: store them at once, the next
    // chunk drains every outstanding operation anyway), start the next tile.
#pragma unroll
    for (int mt = 0; mt < C::MT; mt++) {
#pragma unroll
      for (int s2 = 0; s2 < C::NT / 2; s2++) pend[mt][s2] = pack8<C>(acc[mt], s2);
#pragma unroll
      for (int j = 0; j < C::NT; j++) acc[mt][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
    }
    if constexpr (C::STAGES == 2) {
      store_packed<C>(d, pend, M, N, cur.m0, cur.n0, wm, wn, li, lg);
    } else {
      pend_m0 = cur.m0;
      pend_n0 = cur.n0;
      pending = 1;
    }
    if (!has_next) break;
    cur = nxt;
    t = tn_;
    tn_ = next_tile(src, t + G, nxt);
    has_next = tn_ < src.t_pad;
    if (!has_next) nxt = cur;
    kb = 0;
  }
  };
  if constexpr (C::COPY_WAVES == C::WAVES) {
    walk(std::true_type{});
  } else {
    if (wave < C::COPY_WAVES) walk(std::true_type{});  // wave-uniform
    else walk(std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no copy into LDS outlives the loop
  if constexpr (C::STAGES == 3) store_packed<C>(d, pend, M, N, pend_m0, pend_n0, wm, wn, li, lg);
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_nt_persistent_kernel(DenseTiles src, const float* __restrict__ SA,
                                                                        uint16_t* __restrict__ D, int64_t M,
                                                                        int64_t N, int K, int64_t sa_ld) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  gemm_persistent<C>(lds, src, SA, sa_ld, D, M, N, K);
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_nt_persistent_kernel(GroupedTiles src,
                                                                                const float* __restrict__ SA,
                                                                                uint16_t* __restrict__ D, int64_t M,
                                                                                int64_t N, int K, int64_t sa_ld) {
  static_assert(C::BM == 128 && C::BN == 256, "grouped tiles are 128x256");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  gemm_persistent<C>(lds, src, SA, sa_ld, D, M, N, K);
}

template <class C, bool FP8OUT, bool UE8M0, bool MX = false>
__global__ __launch_bounds__(C::THREADS) void gemm_nt_kernel(const uint8_t* __restrict__ A, const float* __restrict__ SA,
                                                             const uint8_t* __restrict__ B,
                                                             const float* __restrict__ SB, TileOut out, int64_t M,
                                                             int64_t N, int K, int64_t sa_ld, int tiles_m,
                                                             int tiles_n, int64_t sb_ld = 0) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  gemm_tile<C, FP8OUT, UE8M0, MX>(lds, A + m0 * K, B + n0 * K, SA, SB, out.d, out, M, N, K, sa_ld, m0, n0, sb_ld);
}

// K split in two (SplitK): workgroups b and b + tiles share output tile b
// (the same XCD when tiles % 8 == 0), summing chunks [0, KB/2) and
// [KB/2, KB).  ws_counters holds 2 * tiles ints (arrival counts, then
// ready flags; zero between calls), ws_partials tiles * BM * BN floats.
template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_nt_splitk_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const uint8_t* __restrict__ B,
    const float* __restrict__ SB, uint16_t* __restrict__ D, int64_t M, int64_t N, int K, int64_t sa_ld, int tiles_m,
    int tiles_n, int* __restrict__ ws_counters, float* __restrict__ ws_partials) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  const int tiles = tiles_m * tiles_n;
  const int half = (int)blockIdx.x / tiles, t = (int)blockIdx.x - half * tiles;
  int tm, tn;
  tile_coords(t, tiles, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  const int KB = K / kGroup, kbh = KB / 2;
  SplitK sk;
  sk.kb0 = half == 0 ? 0 : kbh;
  sk.kb1 = half == 0 ? kbh : KB;
  sk.partial = ws_partials + (size_t)t * (C::BM * C::BN);
  sk.arrive = ws_counters + t;
  sk.ready = ws_counters + tiles + t;
  gemm_tile<C, false, false, false, false, false, 1>(lds, A + m0 * K, B + n0 * K, SA, SB, D,
                                                        TileOut{D, nullptr, nullptr, 0}, M, N, K, sa_ld, m0, n0, 0,
                                                        GateUp{}, sk);
}

// Grouped: every BM-row block lies inside one group (groups start at
// multiples of 128 rows and BM = 128); its group is m_indices of its first
// row, and a block of padding (-1) is skipped.
template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_nt_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const int32_t* __restrict__ m_indices,
    const uint8_t* __restrict__ B, const float* __restrict__ SB, uint16_t* __restrict__ D, int64_t M, int64_t N,
    int K, int64_t sa_ld, int num_groups, int tiles_m, int tiles_n) {
  static_assert(C::BM == 128, "grouped blocks are the 128-row alignment unit");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  const int g = __builtin_amdgcn_readfirstlane(m_indices[m0]);
  if (g < 0 || g >= num_groups) return;  // padding; uniform across the workgroup, before any barrier
  const int64_t KB = K / kGroup, NB = (N + kGroup - 1) / kGroup;
  gemm_tile<C>(lds, A + m0 * K, B + (int64_t)g * N * K + n0 * K, SA, SB + (int64_t)g * NB * KB, D,
               TileOut{D, nullptr, nullptr, 0}, M, N, K, sa_ld, m0, n0);
}

// The MoE layer's gate_up product with SiLU-times-up and the activation
// quantizer in its epilogue.  w1 [G][2I][K] holds the gate rows, then the up
// rows, and sb1 [G][2I/128][K/128] their block scales.  Tile (tm, j) takes
// the 128 rows m0 = 128 tm and gate block j with up block j, and writes the
// quantized activation's columns 128 j .. 128 j + 127.  A padding block (its
// first row's group outside [0, G)) writes zero codes and scale 1, what the
// standalone kernel writes for rows of group -1.
template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_silu_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const int32_t* __restrict__ m_indices,
    const uint8_t* __restrict__ B, const float* __restrict__ SB, uint8_t* __restrict__ Q, float* __restrict__ SQ,
    int64_t sq_ld, int64_t M, int64_t I, int K, int64_t sa_ld, int num_groups, int tiles_m, int tiles_n) {
  static_assert(C::BM == 128 && C::BN == 2 * kGroup, "a tile is one gate block and one up block");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  int tm, j;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, j);
  const int64_t m0 = (int64_t)tm * C::BM, col0 = (int64_t)j * kGroup;
  const int g = __builtin_amdgcn_readfirstlane(m_indices[m0]);
  if (g < 0 || g >= num_groups) {  // uniform across the workgroup, before any barrier
    for (int i = threadIdx.x; i < C::BM * 8; i += C::THREADS)  // 128 rows x 8 runs of 16 bytes
      *reinterpret_cast<uint4*>(Q + (m0 + i / 8) * I + col0 + (i % 8) * 16) = make_uint4(0, 0, 0, 0);
    for (int i = threadIdx.x; i < C::BM; i += C::THREADS) SQ[(int64_t)j * sq_ld + m0 + i] = 1.0f;
    return;
  }
  const int64_t KB = K / kGroup;
  GateUp gu;
  gu.up_rows = (uint32_t)(I - kGroup);
  gu.gate_block = j;
  gu.up_block = I / kGroup + j;
  gu.sq = SQ;
  gu.sq_ld = sq_ld;
  gu.col0 = col0;
  gu.ld = I;
  gu.m_indices = m_indices;
  // Q travels as the tile's __restrict__ output parameter d.
  gemm_tile<C, false, false, false, true>(lds, A + m0 * K, B + (int64_t)g * 2 * I * K + col0 * K, SA,
                                          SB + (int64_t)g * (2 * I / kGroup) * KB, reinterpret_cast<uint16_t*>(Q),
                                          TileOut{nullptr, nullptr, nullptr, 0}, M, 2 * I, K, sa_ld, m0, 0, 0, gu);
}

// Masked: group g owns rows [g*max_m, g*max_m + max_m) of A and D (a
// dispatch buffer with a fixed stride per group), of which only the first
// masked_m[g] are real.  The grid covers every group's max_m rows; a block
// reads its group's count on the device (no host synchronisation) and exits
// when its rows are all past it.  Rows past the count read as zero and are
// never stored.  A count outside [0, max_m] is clamped to it.
template <class C>
__global__ __launch_bounds__(C::THREADS) void masked_gemm_nt_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const int32_t* __restrict__ masked_m,
    const uint8_t* __restrict__ B, const float* __restrict__ SB, uint16_t* __restrict__ D, int64_t max_m, int64_t N,
    int K, int64_t sa_ld, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  const int per_group = tiles_m * tiles_n;
  const int g = blockIdx.x / per_group;
  int tm, tn;
  tile_coords(blockIdx.x - g * per_group, per_group, tiles_m, tiles_n, tm, tn);
  int rows = __builtin_amdgcn_readfirstlane(masked_m[g]);
  rows = rows < 0 ? 0 : (rows > max_m ? (int)max_m : rows);
  if ((int64_t)tm * C::BM >= rows) return;  // uniform across the workgroup, before any barrier
  const int64_t base = (int64_t)g * max_m;
  const int64_t m0 = base + (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
  const int64_t KB = K / kGroup, NB = (N + kGroup - 1) / kGroup;
  gemm_tile<C, false, false, false, false, true>(lds, A + m0 * K, B + (int64_t)g * N * K + n0 * K, SA,
                                                SB + (int64_t)g * NB * KB, D, TileOut{D, nullptr, nullptr, 0},
                                                base + rows, N, K, sa_ld, m0, n0);
}

// The masked product over a workspace.  Its live tiles -- row tiles below
// each group's count, in group order, column tile fastest -- are dealt
// round-robin to one workgroup per compute unit (G of them).  When the last
// round would hold r < G tiles, those r tiles are split along K into s =
// min(G / r, kMaskedMaxParts, K / 128) parts each, so that the last round
// spreads over r * s workgroups instead of leaving G - r CUs idle; their
// parts meet through split_fixup_n (slots: s per split tile, at most G;
// counters: one per split tile).  The counts stay on the device: every
// workgroup derives the tile list from them.
constexpr int kMaskedMaxParts = 8;
constexpr int kMaskedMaxGrid = 256;  // slots and counters the workspace holds

__device__ __forceinline__ int masked_rows(const int32_t* masked_m, int g, int64_t max_m) {
  const int rows = masked_m[g];
  return rows < 0 ? 0 : (rows > max_m ? (int)max_m : rows);
}

// Live tiles of the first g groups for every g at once: lane l of the
// returned chunk scan holds the live tiles of groups g0 .. g0 + l.
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void masked_gemm_nt_split_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ SA, const int32_t* __restrict__ masked_m,
    const uint8_t* __restrict__ B, const float* __restrict__ SB, uint16_t* __restrict__ D, int64_t max_m, int64_t N,
    int K, int64_t sa_ld, int num_groups, int tiles_n, int* __restrict__ counters, float* __restrict__ partials) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  const int lane = threadIdx.x & 63;
  const int G = (int)gridDim.x;
  const int KB = K / kGroup;
  const int64_t NB = (N + kGroup - 1) / kGroup;
  // the first 64 groups' live tiles stay in registers (lane = group); more
  // groups are rescanned from memory
  const int rows0 = lane < num_groups ? masked_rows(masked_m, lane, max_m) : 0;
  const int lt0 = (rows0 + C::BM - 1) / C::BM * tiles_n;
  const int incl0 = wave_inclusive_sum(lt0, lane);
  int live = __shfl(incl0, 63, 64);
  for (int g0 = 64; g0 < num_groups; g0 += 64) {
    const int g = g0 + lane;
    const int lt = g < num_groups ? (masked_rows(masked_m, g, max_m) + C::BM - 1) / C::BM * tiles_n : 0;
    live += __shfl(wave_inclusive_sum(lt, lane), 63, 64);
  }
  const int rem = live % G;
  int parts = rem ? G / rem : 1;
  parts = parts < kMaskedMaxParts ? parts : kMaskedMaxParts;
  parts = parts < KB ? parts : KB;
  if (parts < 2) parts = 1;
  const int full = parts > 1 ? live - rem : live;
  const int items = full + (parts > 1 ? rem * parts : 0);
  for (int it = (int)blockIdx.x; it < items; it += G) {  // uniform
    int tile = it, part = 0;
    if (it >= full) {
      tile = full + (it - full) / parts;
      part = (it - full) % parts;
    }
    // the tile's group: the first whose inclusive live count passes it
    int g = 0, local = 0, before = 0;
    for (int g0 = 0; g0 < num_groups; g0 += 64) {
      const int gl = g0 + lane;
      const int lt =
          g0 == 0 ? lt0 : (gl < num_groups ? (masked_rows(masked_m, gl, max_m) + C::BM - 1) / C::BM * tiles_n : 0);
      const int incl = g0 == 0 ? incl0 : wave_inclusive_sum(lt, lane);
      const uint64_t hit = __ballot(before + incl > tile);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        g = g0 + l;
        local = tile - before - (__shfl(incl, l, 64) - __shfl(lt, l, 64));
        break;
      }
      before += __shfl(incl, 63, 64);
    }
    g = __builtin_amdgcn_readfirstlane(g);
    const int rows = __builtin_amdgcn_readfirstlane(g < 64 ? __shfl(rows0, g, 64) : masked_rows(masked_m, g, max_m));
    local = __builtin_amdgcn_readfirstlane(local);
    const int tm = local / tiles_n, tn = local - (local / tiles_n) * tiles_n;
    const int64_t base = (int64_t)g * max_m;
    const int64_t m0 = base + (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    SplitK sk;
    sk.kb0 = 0;
    sk.kb1 = KB;
    if (it >= full) {
      const int q = tile - full;
      sk.parts = parts;
      sk.part = part;
      sk.kb0 = part * KB / parts;
      sk.kb1 = (part + 1) * KB / parts;
      sk.partial = partials + (size_t)q * parts * (C::BM * C::BN);
      sk.arrive = counters + q;
    }
    __syncthreads();  // every wave is past the previous tile's last LDS read
    gemm_tile<C, false, false, false, false, true, 2>(lds, A + m0 * K, B + (int64_t)g * N * K + n0 * K, SA,
                                                      SB + (int64_t)g * NB * KB, D, TileOut{D, nullptr, nullptr, 0},
                                                      base + rows, N, K, sa_ld, m0, n0, 0, GateUp{}, sk);
  }
}

// ------------------------------------------------------------ host side
namespace {
struct Candidate {
  GemmKind kind;
  int bm, bn;
  double eff;  // outputs per CU per unit time relative to the 256x256 tile
};
// Calibrated from the time of one round of tiles (every CU busy with one
// tile, K = 4096, forced tiles over 45 LLM-like shapes on one box): 256x256
// 57.0 us, 256x192 46.7, 256x128 35.0, 128x256 34.7, 128x128 27.7.  With
// these the plan picks a tile within 2.3% of the fastest on every one of
// those shapes (0.1% over all of them); the earlier figures, taken on
// 8192^3 alone, left it up to 12% slower (2.2% over all).
constexpr Candidate kCandidates[] = {
    {kGemmTile256x256, 256, 256, 1.00},
    {kGemmTile256x192, 256, 192, 0.91},  // 12 waves; 2048 x 6144 is 256 tiles, one per CU
    {kGemmTile256x128, 256, 128, 0.81},
    {kGemmTile128x256, 128, 256, 0.82},
    {kGemmTile128x128, 128, 128, 0.51},
};
constexpr int kCUs = 256;
}  // namespace

GemmPlan plan_gemm(int64_t m, int64_t n, int64_t k) {
  if (m <= 16) return {kGemmDecode, decode_split(m, n, k)};
  // Tuning and test override: FGFP8_GEMM_TILE=<tile name> forces a tile.
  if (const char* force = getenv("FGFP8_GEMM_TILE")) {
    for (const Candidate& c : kCandidates)
      if (strcmp(force, gemm_kind_name(c.kind)) == 0) return {c.kind, 0};
  }
  GemmPlan best{kGemmTile256x256, 0};
  double best_cost = 1e300;
  for (const Candidate& c : kCandidates) {
    const int64_t tiles = ((m + c.bm - 1) / c.bm) * ((n + c.bn - 1) / c.bn);
    const int64_t rounds = (tiles + kCUs - 1) / kCUs;
    const double cost = (double)rounds * c.bm * c.bn / c.eff;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = {c.kind, 0};
    }
  }
  return best;
}

// K split over two workgroups per 256x256 tile: where 256x256 tiles would
// fill at most half the compute units (so both halves of every tile run in
// one round) and each half keeps at least 32 chunks (measured on M = 2048,
// N = 4096: 5% faster than 256x128 tiles at K = 12288, 17% slower at
// K = 4096, where the exchange of the partial sums is not amortised).  Tuning and test
// override: FGFP8_SPLITK=0|1 (1 forces it for k >= 256).
GemmPlan plan_gemm_ws(int64_t m, int64_t n, int64_t k) {
  const GemmPlan base = plan_gemm(m, n, k);
  if (base.kind == kGemmDecode) return base;
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  bool split = 2 * tiles <= kCUs && k >= 64 * kGroup;
  if (const char* force = getenv("FGFP8_SPLITK")) split = strcmp(force, "0") != 0 && k >= 2 * kGroup;
  return split ? GemmPlan{kGemmTile256x256SplitK2, 2} : base;
}

int64_t gemm_splitk_workspace_bytes(int64_t m, int64_t n) {
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  return (2 * tiles * 4 + 255) / 256 * 256 + tiles * 256 * 256 * 4;
}

hipError_t launch_gemm_splitk(const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb, void* d,
                              int64_t m, int64_t n, int64_t k, void* workspace, hipStream_t stream) {
  using C = Tile256x256;
  const int tiles_m = (int)((m + C::BM - 1) / C::BM), tiles_n = (int)((n + C::BN - 1) / C::BN);
  const int tiles = tiles_m * tiles_n;
  int* counters = static_cast<int*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + (2 * (int64_t)tiles * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL(gemm_nt_splitk_kernel<C>, dim3(2u * (uint32_t)tiles), dim3(C::THREADS), 0, stream,
                     static_cast<const uint8_t*>(a), sa, static_cast<const uint8_t*>(b), sb, static_cast<uint16_t*>(d), m,
                     n, (int)k, sa_ld, tiles_m, tiles_n, counters, partials);
  return hipGetLastError();
}

const char* gemm_kind_name(GemmKind kind) {
  switch (kind) {
    case kGemmTile256x256: return "tile256x256_w4x2";
    case kGemmTile256x192: return "tile256x192_w4x3";
    case kGemmTile128x256: return "tile128x256_w2x4";
    case kGemmTile256x128: return "tile256x128_w4x2";
    case kGemmTile128x128: return "tile128x128_w2x2";
    case kGemmDecode: return "decode_splitk_slab16";
    case kGemmTile256x256SplitK2: return "tile256x256_w4x2_splitk2";
    case kGemmTile128x512: return "tile128x512_w2x4";
  }
  return "?";
}

// Persistent walk (gemm_persistent) or one workgroup per tile.  The walk
// runs the K pipeline on from one tile into the next, which pays where a
// launch takes two or more rounds of tiles: measured with identical bits
// (A/B interleaved on one box), 256x256 tiles 1-6% faster (2048 x 24576 x
// 4096 169.1 against 172.7 us, 8192^3 425.8 against 433.2, 16384^2 x 8192
// 1725 against 1747, most at short K: 8192 x 8192 x 1024 71.5 against 75.8),
// the grouped product 7% faster at K = 2048 (627 against 674 us) and 3% at
// K = 1024, but 1% slower at K = 7168, and one round of tiles 5% slower (o
// at M = 2048).  So: two or more rounds, the 256x256 tile for the dense
// product (the only one measured there) and K <= 4096 for the grouped one.
// Tuning and test override: FGFP8_PERSISTENT=0|1.  The walk needs K >= 256
// (two chunks per tile keep a finished tile's stores ahead of the next pack).
bool use_persistent(int64_t tiles, int64_t k, bool grouped, bool measured_tile) {
  if (k < 2 * kGroup) return false;
  if (const char* force = getenv("FGFP8_PERSISTENT")) return strcmp(force, "0") != 0;
  return tiles >= 2 * kCUs && measured_tile && (!grouped || k <= 4096);
}

bool plan_persistent(const GemmPlan& plan, int64_t m, int64_t n, int64_t k) {
  // launch_tile's rule: tiles of whole 128-column blocks only
  int bm = 0, bn = 0;
  switch (plan.kind) {
    case kGemmTile256x256: bm = 256, bn = 256; break;
    case kGemmTile256x128: bm = 256, bn = 128; break;
    case kGemmTile128x256: bm = 128, bn = 256; break;
    case kGemmTile128x128: bm = 128, bn = 128; break;
    default: return false;
  }
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  return use_persistent(tiles, k, false, bm == 256 && bn == 256);
}

// Compute units of the current device (queried once per device).
static int device_cus() {
  static std::atomic<int> cus[64];  // per device; 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = kCUs;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of a persistent launch: one per compute unit (the tiles' LDS
// allows one per CU), a multiple of 8, at most the padded tile count.
static int persistent_grid(int t_pad) {
  const int n = device_cus();
  int g = n / 8 * 8;
  if (g < 8) g = 8;
  return g < t_pad ? g : t_pad;
}

template <class C>
static hipError_t launch_tile(const void* a, const float* sa, int64_t sa_ld, const void* b, const float* sb,
                              const TileOut& out, int64_t m, int64_t n, int64_t k, hipStream_t stream,
                              bool ue8m0 = false) {
  const int tiles_m = (int)((m + C::BM - 1) / C::BM), tiles_n = (int)((n + C::BN - 1) / C::BN);
  const dim3 grid((uint32_t)tiles_m * tiles_n), block(C::THREADS);
  const uint8_t *pa = static_cast<const uint8_t*>(a), *pb = static_cast<const uint8_t*>(b);
  // The persistent walk and the FP8-output epilogue take tiles whose
  // column blocks align with 128 (the epilogue pairs waves wn, wn ^ 1).
  constexpr bool kAligned = C::BN % kGroup == 0;
  if constexpr (kAligned) {
    if (!ue8m0 && out.q == nullptr &&
        use_persistent((int64_t)tiles_m * tiles_n, k, false, C::BM == 256 && C::BN == 256)) {
      const int t_pad = (tiles_m * tiles_n + 7) / 8 * 8;
      const DenseTiles src{pa, pb, sb, k, tiles_m, tiles_n, t_pad, C::BM, C::BN};
      hipLaunchKernelGGL(gemm_nt_persistent_kernel<C>, dim3((uint32_t)persistent_grid(t_pad)), block, 0, stream, src,
                         sa, out.d, m, n, (int)k, sa_ld);
      return hipGetLastError();
    }
  }
  if (ue8m0) {
    hipLaunchKernelGGL((gemm_nt_kernel<C, false, true>), grid, block, 0, stream, pa, sa, pb, sb, out, m, n, (int)k,
                       sa_ld, tiles_m, tiles_n);
  } else if (out.q != nullptr) {
    if constexpr (!kAligned) return hipErrorInvalidValue;
    else
      hipLaunchKernelGGL((gemm_nt_kernel<C, true, false>), grid, block, 0, stream, pa, sa, pb, sb, out, m, n, (int)k,
                         sa_ld, tiles_m, tiles_n);
  } else
    hipLaunchKernelGGL((gemm_nt_kernel<C, false, false>), grid, block, 0, stream, pa, sa, pb, sb, out, m, n, (int)k,
                       sa_ld, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& plan, const void* a, const float* sa, int64_t sa_ld, const void* b,
                       const float* sb, void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const TileOut out{static_cast<uint16_t*>(d), nullptr, nullptr, 0};
  switch (plan.kind) {
    case kGemmTile256x256SplitK2:  // without a workspace: whole tiles
    case kGemmTile256x256: return launch_tile<Tile256x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile256x192: return launch_tile<Tile256x192>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile128x256: return launch_tile<Tile128x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile256x128: return launch_tile<Tile256x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile128x128: return launch_tile<Tile128x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmDecode: return launch_decode(plan.split, a, sa, sa_ld, b, sb, d, m, n, k, stream);
    case kGemmTile128x512: break;  // the grouped product's tile only
  }
  return hipErrorInvalidValue;
}

GemmKind plan_masked(int32_t num_groups, int64_t max_m, int64_t expected_m, int64_t n) {
  // Tiles of 128 rows (the smallest that keeps two waves per SIMD); the
  // column width from the expected work: rounds of 256 CUs over
  // num_groups * ceil(expected_m / 128) row tiles, as in plan_gemm.
  // Tuning and test override: FGFP8_MASKED_TILE=<tile name> (a 128-row tile).
  if (const char* force = getenv("FGFP8_MASKED_TILE")) {
    for (const Candidate& c : kCandidates)
      if (c.bm == 128 && strcmp(force, gemm_kind_name(c.kind)) == 0) return c.kind;
  }
  const int64_t em = expected_m > 0 && expected_m < max_m ? expected_m : max_m;
  const int64_t row_tiles = (int64_t)num_groups * ((em + 127) / 128);
  GemmKind best = kGemmTile128x256;
  double best_cost = 1e300;
  for (const Candidate& c : kCandidates) {
    if (c.bm != 128) continue;
    const int64_t tiles = row_tiles * ((n + c.bn - 1) / c.bn);
    const double cost = (double)((tiles + kCUs - 1) / kCUs) * c.bm * c.bn / c.eff;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = c.kind;
    }
  }
  return best;
}

template <class C>
static hipError_t launch_masked_tile(const void* a, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                     const void* b, const float* sb, int32_t num_groups, int64_t max_m, void* d,
                                     int64_t n, int64_t k, hipStream_t stream) {
  const int tiles_m = (int)((max_m + C::BM - 1) / C::BM), tiles_n = (int)((n + C::BN - 1) / C::BN);
  hipLaunchKernelGGL(masked_gemm_nt_kernel<C>, dim3((uint32_t)num_groups * tiles_m * tiles_n), dim3(C::THREADS), 0,
                     stream, static_cast<const uint8_t*>(a), sa, masked_m, static_cast<const uint8_t*>(b), sb,
                     static_cast<uint16_t*>(d), max_m, n, (int)k, sa_ld, tiles_m, tiles_n);
  return hipGetLastError();
}

// Whether the workspace form walks the tiles with the last round split: only
// where the expected live tiles (num_groups * ceil(expected_m / 128) column
// tiles of the plan) fill at most a quarter of the CUs.  Measured (N = 4096,
// K = 7168, A/B on one box): 32 live tiles 26.4 against 45.8 us, 64 tiles
// 38.2 against 46.2, but 128 tiles 65.3 against 47.6 -- from about half the
// CUs on, the plain launch already streams the weights at the HBM rate, and
// the split's partial round trips only add bytes -- and from 256 tiles on
// within -4% .. +12% of the plain launch (1024 tokens top-4 over 32 experts,
// Zipf: 271 against 266 us).  Tuning and test override:
// FGFP8_MASKED_SPLIT=0|1.
bool masked_split_walk(GemmKind kind, int32_t num_groups, int64_t max_m, int64_t expected_m, int64_t n) {
  if (const char* force = getenv("FGFP8_MASKED_SPLIT")) return strcmp(force, "0") != 0;
  const int64_t bn = kind == kGemmTile128x128 ? 128 : 256;
  const int64_t em = expected_m > 0 && expected_m < max_m ? expected_m : max_m;
  const int64_t tiles = (int64_t)num_groups * ((em + 127) / 128) * ((n + bn - 1) / bn);
  int cus = device_cus();
  cus = cus < kMaskedMaxGrid ? cus : kMaskedMaxGrid;
  return tiles * 4 <= cus;
}

int64_t masked_split_workspace_bytes() {
  // counters, then kMaskedMaxGrid slots of the widest 128-row tile
  return (int64_t)kMaskedMaxGrid * 4 + (int64_t)kMaskedMaxGrid * 128 * 256 * 4;
}

template <class C>
static hipError_t launch_masked_split_tile(const void* a, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                                           const void* b, const float* sb, int32_t num_groups, int64_t max_m, void* d,
                                           int64_t n, int64_t k, void* workspace, hipStream_t stream) {
  static_assert(C::BM * C::BN <= 128 * 256, "a slot holds one 128x256 tile");
  const int tiles_n = (int)((n + C::BN - 1) / C::BN);
  int grid = device_cus();
  grid = grid < kMaskedMaxGrid ? grid : kMaskedMaxGrid;
  int* counters = static_cast<int*>(workspace);
  float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + (int64_t)kMaskedMaxGrid * 4);
  hipLaunchKernelGGL(masked_gemm_nt_split_kernel<C>, dim3((uint32_t)grid), dim3(C::THREADS), 0, stream,
                     static_cast<const uint8_t*>(a), sa, masked_m, static_cast<const uint8_t*>(b), sb,
                     static_cast<uint16_t*>(d), max_m, n, (int)k, sa_ld, (int)num_groups, tiles_n, counters, partials);
  return hipGetLastError();
}

hipError_t launch_masked_gemm_split(GemmKind kind, const void* a, const float* sa, int64_t sa_ld,
                                    const int32_t* masked_m, const void* b, const float* sb, int32_t num_groups,
                                    int64_t max_m, void* d, int64_t n, int64_t k, void* workspace,
                                    hipStream_t stream) {
  switch (kind) {
    case kGemmTile128x256:
      return launch_masked_split_tile<Tile128x256>(a, sa, sa_ld, masked_m, b, sb, num_groups, max_m, d, n, k,
                                                   workspace, stream);
    case kGemmTile128x128:
      return launch_masked_split_tile<Tile128x128>(a, sa, sa_ld, masked_m, b, sb, num_groups, max_m, d, n, k,
                                                   workspace, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_masked_gemm(GemmKind kind, const void* a, const float* sa, int64_t sa_ld, const int32_t* masked_m,
                              const void* b, const float* sb, int32_t num_groups, int64_t max_m, void* d, int64_t n,
                              int64_t k, hipStream_t stream) {
  switch (kind) {
    case kGemmTile128x256:
      return launch_masked_tile<Tile128x256>(a, sa, sa_ld, masked_m, b, sb, num_groups, max_m, d, n, k, stream);
    case kGemmTile128x128:
      return launch_masked_tile<Tile128x128>(a, sa, sa_ld, masked_m, b, sb, num_groups, max_m, d, n, k, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_fp8out(GemmKind kind, const void* a, const float* sa, int64_t sa_ld, const void* b,
                              const float* sb, void* q, float* sd, int64_t sd_ld, void* d, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  const TileOut out{static_cast<uint16_t*>(d), static_cast<uint8_t*>(q), sd, sd_ld};
  switch (kind) {
    case kGemmTile256x192:  // the epilogue's 1x128 groups need 128-aligned column blocks
    case kGemmTile256x256: return launch_tile<Tile256x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile128x256: return launch_tile<Tile128x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile256x128: return launch_tile<Tile256x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    case kGemmTile128x128: return launch_tile<Tile128x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_ue8m0(const GemmPlan& plan, const void* a, const float* sa, int64_t sa_ld, const void* b,
                             const float* sb, void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const TileOut out{static_cast<uint16_t*>(d), nullptr, nullptr, 0};
  switch (plan.kind) {
    case kGemmTile256x256SplitK2:
    case kGemmTile256x256: return launch_tile<Tile256x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream, true);
    case kGemmTile256x192: return launch_tile<Tile256x192>(a, sa, sa_ld, b, sb, out, m, n, k, stream, true);
    case kGemmTile128x256: return launch_tile<Tile128x256>(a, sa, sa_ld, b, sb, out, m, n, k, stream, true);
    case kGemmTile256x128: return launch_tile<Tile256x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream, true);
    case kGemmTile128x128: return launch_tile<Tile128x128>(a, sa, sa_ld, b, sb, out, m, n, k, stream, true);
    // decode shapes: the promote path is exact for power-of-two scales
    case kGemmDecode: return launch_decode(plan.split, a, sa, sa_ld, b, sb, d, m, n, k, stream);
    case kGemmTile128x512: break;
  }
  return hipErrorInvalidValue;
}

template <class C>
static hipError_t launch_tile_mx(const void* a, const int32_t* sa, int64_t sa_ld, const void* b, const int32_t* sb,
                                 int64_t sb_ld, void* d, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const int tiles_m = (int)((m + C::BM - 1) / C::BM), tiles_n = (int)((n + C::BN - 1) / C::BN);
  const TileOut out{static_cast<uint16_t*>(d), nullptr, nullptr, 0};
  // The packed int32 scale words travel through the float-typed scale
  // pointers of the tile body, which only copies them as bytes.
  hipLaunchKernelGGL((gemm_nt_kernel<C, false, false, true>), dim3((uint32_t)tiles_m * tiles_n), dim3(C::THREADS), 0,
                     stream, static_cast<const uint8_t*>(a), reinterpret_cast<const float*>(sa),
                     static_cast<const uint8_t*>(b), reinterpret_cast<const float*>(sb), out, m, n, (int)k, sa_ld,
                     tiles_m, tiles_n, sb_ld);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(GemmKind kind, const void* a, const int32_t* sa, int64_t sa_ld, const void* b,
                          const int32_t* sb, int64_t sb_ld, void* d, int64_t m, int64_t n, int64_t k,
                          hipStream_t stream) {
  switch (kind) {
    case kGemmTile256x256: return launch_tile_mx<Tile256x256>(a, sa, sa_ld, b, sb, sb_ld, d, m, n, k, stream);
    case kGemmTile256x192: return launch_tile_mx<Tile256x192>(a, sa, sa_ld, b, sb, sb_ld, d, m, n, k, stream);
    case kGemmTile128x256: return launch_tile_mx<Tile128x256>(a, sa, sa_ld, b, sb, sb_ld, d, m, n, k, stream);
    case kGemmTile256x128: return launch_tile_mx<Tile256x128>(a, sa, sa_ld, b, sb, sb_ld, d, m, n, k, stream);
    case kGemmTile128x128: return launch_tile_mx<Tile128x128>(a, sa, sa_ld, b, sb, sb_ld, d, m, n, k, stream);
    default: return hipErrorInvalidValue;
  }
}

GemmKind plan_tiles(int64_t m, int64_t n, int64_t k) {
  const GemmPlan p = plan_gemm(m > 16 ? m : 17, n, k);
  return p.kind == kGemmDecode ? kGemmTile128x128 : p.kind;
}

hipError_t launch_grouped_gemm_silu(const void* a, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                                    const void* w1, const float* sb1, int32_t num_groups, void* q, float* sq,
                                    int64_t sq_ld, int64_t m, int64_t inter, int64_t k, hipStream_t stream) {
  using C = Tile128x256;
  const int tiles_m = (int)(m / C::BM), tiles_n = (int)(inter / kGroup);
  hipLaunchKernelGGL(grouped_gemm_silu_kernel<C>, dim3((uint32_t)tiles_m * tiles_n), dim3(C::THREADS), 0, stream,
                     static_cast<const uint8_t*>(a), sa, m_indices, static_cast<const uint8_t*>(w1), sb1,
                     static_cast<uint8_t*>(q), sq, sq_ld, m, inter, (int)k, sa_ld, (int)num_groups, tiles_m, tiles_n);
  return hipGetLastError();
}

// The grouped product's tile: 128x512 or 128x256, whichever costs fewer
// rounds of 256 CUs times tile area over its measured efficiency (outputs per
// CU per unit time, relative to the dense 256x256 tile).  The wide tile
// reads a chunk's fragments with the 256x256 tile's LDS bytes per FLOP, but
// here the experts' weights stream from HBM, and a 128-row block reads its
// expert's whole weight whatever the tile width, so both tiles move the same
// weight bytes per FLOP.  Measured (interleaved A/B, one box): the 32-expert
// product at K = 7168, N = 4096 1107.9-1109.2 us against 1106.2-1108.5 us for
// 128x256; the MoE layer's down product (K = 2048, N = 7168) 630.1-630.6 us
// against 645.0-645.5 for 128x256 in the persistent walk, hence 0.84.  At
// K <= 1024 the walk, which hides each tile's pipeline fill behind the last
// one's chunks, is ahead (M_pad = 34944 over 32 experts: N = 14336 758-764 us
// against 789-795 for 128x512; N = 4096 223 against 224-225), so those shapes
// keep 128x256 tiles.  Tuning and test override: FGFP8_GROUPED_TILE=<tile name>.
constexpr double kEff128x512 = 0.84;
GemmKind plan_grouped_gemm(int64_t m, int64_t n, int64_t k) {
  // The wide tile's weight panel (512 rows of K bytes) is addressed with
  // 32-bit buffer offsets: beyond 2^23 - 128 it would wrap, so such K takes
  // the 128x256 tile (256 K < 2^32 for every K the calls accept), forced or not.
  if (512 * k >= (int64_t(1) << 32)) return kGemmTile128x256;
  if (const char* force = getenv("FGFP8_GROUPED_TILE")) {
    if (strcmp(force, gemm_kind_name(kGemmTile128x512)) == 0) return kGemmTile128x512;
    if (strcmp(force, gemm_kind_name(kGemmTile128x256)) == 0) return kGemmTile128x256;
  }
  if (k <= 1024) return kGemmTile128x256;
  const int64_t blocks = m / 128;
  auto cost = [&](int64_t bn, double eff) {
    const int64_t tiles = blocks * ((n + bn - 1) / bn);
    return (double)((tiles + kCUs - 1) / kCUs) * (double)(128 * bn) / eff;
  };
  return cost(512, kEff128x512) < cost(256, 0.82) ? kGemmTile128x512 : kGemmTile128x256;
}

// Whether the grouped product runs the persistent walk (128x256 tiles only).
bool plan_grouped_walk(int64_t m, int64_t n, int64_t k) {
  if (plan_grouped_gemm(m, n, k) != kGemmTile128x256) return false;
  return use_persistent((m / 128) * ((n + 255) / 256), k, true, true);
}

hipError_t launch_grouped_gemm(const void* a, const float* sa, int64_t sa_ld, const int32_t* m_indices,
                               const void* b, const float* sb, int32_t num_groups, void* d, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream) {
  if (plan_grouped_gemm(m, n, k) == kGemmTile128x512) {
    using W = Tile128x512;
    const int tiles_m = (int)(m / W::BM), tiles_n = (int)((n + W::BN - 1) / W::BN);
    hipLaunchKernelGGL(grouped_gemm_nt_kernel<W>, dim3((uint32_t)tiles_m * tiles_n), dim3(W::THREADS), 0, stream,
                       static_cast<const uint8_t*>(a), sa, m_indices, static_cast<const uint8_t*>(b), sb,
                       static_cast<uint16_t*>(d), m, n, (int)k, sa_ld, (int)num_groups, tiles_m, tiles_n);
    return hipGetLastError();
  }
  using C = Tile128x256;
  const int tiles_m = (int)(m / C::BM), tiles_n = (int)((n + C::BN - 1) / C::BN);
  if (plan_grouped_walk(m, n, k)) {
    const int t_pad = (tiles_m * tiles_n + 7) / 8 * 8;
    const GroupedTiles src{static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b), sb, m_indices, m, n, k,
                           (int)num_groups, tiles_m, tiles_n, t_pad};
    hipLaunchKernelGGL(grouped_gemm_nt_persistent_kernel<C>, dim3((uint32_t)persistent_grid(t_pad)),
                       dim3(C::THREADS), 0, stream, src, sa, static_cast<uint16_t*>(d), m, n, (int)k, sa_ld);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(grouped_gemm_nt_kernel<C>, dim3((uint32_t)tiles_m * tiles_n), dim3(C::THREADS), 0, stream,
                     static_cast<const uint8_t*>(a), sa, m_indices, static_cast<const uint8_t*>(b), sb,
                     static_cast<uint16_t*>(d), m, n, (int)k, sa_ld, (int)num_groups, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace fgfp8
