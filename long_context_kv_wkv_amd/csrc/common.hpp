// Device-side helpers shared by the Compressor kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "compressor.h"

namespace cmp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kRmsEps = 1e-6f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 on raw 16-bit codes
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 by the hardware conversion (v_cvt_pk_bf16_f32, two values
// per instruction): round to nearest even; a NaN stays a quiet NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------------------
// Column order of the fused weight panel.
//
// The panel has N = 2*coff*D rows (one per projected column).  It is cut into
// groups of 128 columns; a group holds 128 / (2*coff) channels, in 32-column
// blocks: block q of a group carries variant v = q % (2*coff) of channels
// [sub*32, sub*32 + 32) of the group, sub = q / (2*coff).  Variant v < coff
// is kv of channel set v; variant coff + v is the score of set v.  So one
// 32-wide MFMA column block holds 32 consecutive channels of one variant, and
// the 2*coff variants of a channel sit in the same lane of neighbouring blocks.
// ---------------------------------------------------------------------------
//
// Memory layout of the panel (bf16): fragment-major.  Column block cb (32
// panel columns) and k-step ks (16 values of K) form one 1 KiB fragment at
// element offset ((cb * (K/16) + ks) * 64 + lane) * 8; lane l holds column
// cb*32 + l%32, K values ks*16 + (l/32)*8 .. +8 - exactly the B operand of
// one 32x32x16 MFMA.  Consecutive k-steps of a block are contiguous, so a
// wave streaming one block reads one contiguous run of HBM.
__host__ __device__ __forceinline__ size_t panel_offset(int col, int k, int K) {
  const int cb = col >> 5, ks = k >> 4;
  const int lane = (col & 31) + 32 * ((k >> 3) & 1);
  return (((size_t)cb * (K >> 4) + ks) * 64 + lane) * 8 + (k & 7);
}

__host__ __device__ __forceinline__ int packed_col(int is_score, int cset, int c, int coff) {
  const int nv = 2 * coff;
  const int cpg = 128 / nv;                 // channels per 128-column group
  const int g = c / cpg, rem = c % cpg;
  const int sub = rem >> 5, i = rem & 31;
  const int v = is_score ? coff + cset : cset;
  return g * 128 + (sub * nv + v) * 32 + i;
}

// ---------------------------------------------------------------------------
// Per-request plan record (int32 x 8) kept in the workspace.
// ---------------------------------------------------------------------------
//   START  s_b, first position of this call's tokens    NTOK  n_b
//   END    e_b = s_b + n_b                              ROW0  packed row of s_b
//   NWIN   windows completed in this call               NROWS ceil(n_b / r)
//   OUT0   first output row of request b
//   FIRST  first position the request's GEMM tiles cover (window-aligned,
//          one window earlier for ratio 4: the halo)
//   TILE0  index of the request's first M-tile           NTILE its M-tiles
enum PlanField {
  PL_START = 0, PL_NTOK, PL_END, PL_ROW0, PL_NWIN, PL_NROWS, PL_OUT0, PL_FIRST, PL_TILE0, PL_NTILE,
  PL_WIDTH = 12
};

// Static configuration passed by value to kernels.
struct Cfg {
  int ratio, coff, D, H, N, rope, rotate, bs, nblocks, stride;
  int bm;   // prefill GEMM tile rows (256, or 128 for short calls)
};

// Ring slot of position p, and its (block, row) through a table row.
// Returns false (and sets *bad) if the table entry is out of range.
__device__ __forceinline__ bool state_row(const Cfg& cf, const int32_t* __restrict__ table, int b,
                                          int p, long* row_index) {
  const int q = p % (cf.coff * cf.ratio);
  const int blk = table[(long)b * cf.stride + q / cf.bs];
  if (blk < 0 || blk >= cf.nblocks) return false;
  *row_index = (long)blk * cf.bs + (q % cf.bs);
  return true;
}

// v of lane (this lane) ^ M, M a power of two below 64, by register permutes
// only (no LDS): DPP quad permutes for M = 1, 2, row shifts for 4, a row
// rotate for 8, v_permlane16_swap / v_permlane32_swap for 16 and 32.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);          // row_shl:4, from i + 4
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);          // row_shr:4, from i - 4
    return __int_as_float((threadIdx.x & 4) ? dn : up);
  } else if constexpr (M == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  } else {
    static_assert(M == 32, "lane_xor: M in 1, 2, 4, ..., 32");
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void set_error(uint32_t* err, uint32_t bits) {
  if (bits) atomicOr(err, bits);
}

}  // namespace cmp
