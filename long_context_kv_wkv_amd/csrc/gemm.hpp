// Prefill projection: P[T, N] (fp32) = X[T, H] (bf16) . Wp[N, H]^T (bf16).
//
// This is the fused "[kv, score] = X @ [W_kv, W_gate]" step ([CANN] 计算公式
// step 1; [AscendC] 具体计算流程 矩阵乘法), both weight matrices in one panel so
// a single pass over X produces every projected column.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, each wave a
// 128 x 128 sub-tile = 4 x 4 blocks of the 32x32x16 bf16 MFMA, accumulators
// in AGPRs), K step 64, two 64 KiB LDS stages filled by direct-to-LDS copies
// (global_load_lds_dwordx4: no staging registers, no ds_write).
//  * X tile: row-major in LDS, 128 B per row, 16-byte chunks XOR-swizzled by
//    (row & 7) ^ ((row >> 3) & 1) so fragment reads are bank-conflict free
//    whether LDS serves 8 or 16 lanes per cycle.  A copy instruction covers 8
//    rows x 128 B (one cache line per row); each lane fetches the logical chunk
//    the swizzle places at its LDS slot.
//  * Panel tile: fragment-major like the panel in HBM (1 KiB per MFMA B
//    fragment), copied and read lane-contiguously.
// Per K step the 16 copies of the next tile are interleaved one per two MFMAs
// in the first half of the step, while the second half's fragments are read;
// the second half's MFMAs then cover the copies' latency before the single
// wait + barrier of the step.  (Measured on MI355X: the copy stream, not the
// MFMA rate, bounds this kernel; bursts of copies stall issue, deeper stage
// counts lower the copy rate.)
//
// The tile schedule and the epilogue live in pool.hpp (the GEMM never writes
// the projection to HBM: its epilogue pools windows straight from the
// accumulators).
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GM_BM = 256, GM_BN = 256, GM_BK = 64;
constexpr int GM_THREADS = 256;
constexpr int GM_STAGES = 2;
constexpr int GM_STAGE_BYTES = (GM_BM + GM_BN) * GM_BK * 2;   // 64 KiB
constexpr int GM_LDS_BYTES = GM_STAGES * GM_STAGE_BYTES;     // 128 KiB

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
// byte offset of 16-byte chunk `chunk` of row `row` in a 128-byte-row tile
__device__ __forceinline__ int swz(int row, int chunk) {
  return (row << 7) + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

// ---------------------------------------------------------------------------
// Main loop of one 256 x 256 tile: acc[i][j] (wave (wm, wn), 32x32 block i of
// its 128 rows, block j of its 128 columns) += X[rows] . Wp[n0 .. n0+256)^T.
// arow[j] is the packed X row that this lane's j-th copy instruction reads:
// tile row ((wave * 8 + j) * 8 + lane / 8); rows outside the tensor must be
// clamped by the caller to any valid row (their results are not used).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gemm_mainloop(f32x16 (&acc)[4][4], uint8_t* smem,
                                              const uint16_t* __restrict__ X,
                                              const uint16_t* __restrict__ W, int K, int n0,
                                              const int (&arow)[8]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // A copies: instruction j of wave w fills tile rows r0 = (8w + j) * 8 .. +8;
  // lane l lands at LDS byte r0*128 + 16 l, i.e. row r0 + l/8, physical chunk
  // l%8, so it fetches the logical chunk that the swizzle places there.
  const uint16_t* asrc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (wave * 8 + j) * 8 + (lane >> 3);
    const int kc = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
    asrc[j] = X + (size_t)arow[j] * K + kc * 8;
  }
  // B copies: fragment f = 8w + j of the stage is (column block f / 4, k-step f % 4)
  const size_t ksteps = (size_t)(K >> 4);
  const uint16_t* bsrc = W + ((((size_t)(n0 >> 5) + 2 * wave) * ksteps) * 64 + lane) * 8;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int KT = K / GM_BK;
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | 0x0f70)
#define BARRIER() asm volatile("s_barrier" ::: "memory")
  {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dma16(asrc[j], smem + (wave * 8 + j) * 1024);
      dma16(bsrc + ((size_t)(j >> 2) * ksteps + (j & 3)) * 512, smem + 32768 + (wave * 8 + j) * 1024);
    }
  }
  WAIT_VM(0);
  BARRIER();
  for (int kt = 0; kt < KT; ++kt) {
    // the next tile's copies go to the other stage, which every wave finished
    // reading before the last barrier (the last iteration re-copies tile
    // KT-1 there; nothing reads it)
    const int kn = min(kt + 1, KT - 1);
    uint8_t* stn = smem + ((kt + 1) & 1) * GM_STAGE_BYTES;
    const uint8_t* sa = smem + (kt & 1) * GM_STAGE_BYTES;
    const uint8_t* sb = sa + 32768;
    bf16x8 a[4][4], b[4][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[kk][i] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 128 + i * 32 + lrow, kk * 2 + lhalf));
        b[kk][i] = *reinterpret_cast<const bf16x8*>(sb + ((wn * 4 + i) * 4 + kk) * 1024 + lane * 16);
      }
    __builtin_amdgcn_sched_barrier(0);
    // first half: all copies of the next tile interleaved with 32 MFMAs, and
    // the second half's fragments read from LDS
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dma16(asrc[j] + kn * GM_BK, stn + (wave * 8 + j) * 1024);
      dma16(bsrc + ((size_t)(j >> 2) * ksteps + (kn * GM_BK >> 4) + (j & 3)) * 512,
            stn + 32768 + (wave * 8 + j) * 1024);
    }
#pragma unroll
    for (int kk = 2; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[kk][i] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 128 + i * 32 + lrow, kk * 2 + lhalf));
        b[kk][i] = *reinterpret_cast<const bf16x8*>(sb + ((wn * 4 + i) * 4 + kk) * 1024 + lane * 16);
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], b[kk][j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one copy
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 2; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk][i], b[kk][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    WAIT_VM(0);
    BARRIER();
  }
#undef WAIT_VM
#undef BARRIER
}

}  // namespace cmp
