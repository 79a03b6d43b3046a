// Quantised write of compressed rows into a paged FP8 cache: the step after
// the Compressor that stores its rows into the Lightning Indexer / Sparse
// Flash Attention compressed caches, which may hold float8 ([PyPTO]
// DeepSeek-V4 整网集成方式).  The page names the step and the cache dtype
// only; the format (OCP E4M3), the scaling (one fp32 scale per 128 channels,
// amax / 448) and the placement (row i to slot slot_mapping[i], -1 = none)
// are the plainest reading of that sentence.
//
// HBM-bound: per 128-channel block, 256 B of bf16 in, 128 B of codes and a
// 4-byte scale out.  A 16-lane group (one DPP row) takes a block, 8 channels
// per lane (one 16-byte load); its absmax is a 4-step DPP reduction inside
// the row.  Each group takes EPL_GROUP_BLOCKS consecutive blocks with every
// load issued before the first reduction.  q = x * (448 / amax) in fp32
// (correctly rounded division, clamped to +-448) and the hardware conversion
// v_cvt_pk_fp8_f32 (round to nearest even) gives the codes.
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int EPL_THREADS = 256;
constexpr int EPL_BLOCK = 128;          // channels per scale
constexpr int EPL_GROUP_BLOCKS = 4;     // blocks per 16-lane group
constexpr float EPL_E4M3_MAX = 448.f;

// n_blocks = rows * nblk_row < 2^31 (checked on the host).
__global__ __launch_bounds__(EPL_THREADS) void epilog_kernel(
    const uint16_t* __restrict__ rows, int n_blocks, int nblk_row,
    const int32_t* __restrict__ slot_mapping, uint8_t* __restrict__ cache,
    float* __restrict__ scale, long num_slots, uint32_t* __restrict__ err) {
  const int sub = threadIdx.x & 15;
  const int g0 = (blockIdx.x * (EPL_THREADS / 16) + (threadIdx.x >> 4)) * EPL_GROUP_BLOCKS;
  if (g0 >= n_blocks) return;            // whole 16-lane groups leave together
  const int D = nblk_row * EPL_BLOCK;
  // (row, block) of the group's blocks: one division, then steps; blocks past
  // the last one repeat it (their results are not stored)
  int rw[EPL_GROUP_BLOCKS], bkj[EPL_GROUP_BLOCKS];
  {
    int row = g0 / nblk_row, bk = g0 - row * nblk_row;
#pragma unroll
    for (int j = 0; j < EPL_GROUP_BLOCKS; ++j) {
      const bool past = g0 + j >= n_blocks;
      rw[j] = past ? (n_blocks - 1) / nblk_row : row;
      bkj[j] = past ? nblk_row - 1 : bk;
      if (++bk == nblk_row) {
        bk = 0;
        ++row;
      }
    }
  }
  // loads of every block first
  uint4 raw[EPL_GROUP_BLOCKS];
  int slot[EPL_GROUP_BLOCKS];
#pragma unroll
  for (int j = 0; j < EPL_GROUP_BLOCKS; ++j) {
    slot[j] = slot_mapping[rw[j]];
    raw[j] = *reinterpret_cast<const uint4*>(rows + (long)rw[j] * D + bkj[j] * EPL_BLOCK + sub * 8);
  }
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < EPL_GROUP_BLOCKS; ++j) {
    if (g0 + j >= n_blocks) break;       // uniform in the group
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, lane_xor<1>(amax));
    amax = fmaxf(amax, lane_xor<2>(amax));
    amax = fmaxf(amax, lane_xor<4>(amax));
    amax = fmaxf(amax, lane_xor<8>(amax));
    const float inv = amax > 0.f ? __fdiv_rn(EPL_E4M3_MAX, amax) : 0.f;
    const float sc = __fdiv_rn(amax, EPL_E4M3_MAX);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(v[i] * inv, -EPL_E4M3_MAX), EPL_E4M3_MAX);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
    const int s = slot[j];
    if (s == -1) continue;
    if (s < -1 || s >= num_slots) {
      bad |= CMP_DEVERR_SLOT;
      continue;
    }
    *reinterpret_cast<uint2*>(cache + (long)s * D + bkj[j] * EPL_BLOCK + sub * 8) =
        make_uint2(uint32_t(lo), uint32_t(hi));
    if (sub == 0) scale[(long)s * nblk_row + bkj[j]] = sc;
  }
  if (bad && sub == 0 && err) atomicOr(err, bad);
}

}  // namespace cmp
