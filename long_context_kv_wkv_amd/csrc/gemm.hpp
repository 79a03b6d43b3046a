// Prefill projection: P[T, N] (fp32) = X[T, H] (bf16) . Wp[N, H]^T (bf16).
//
// This is the fused "[kv, score] = X @ [W_kv, W_gate]" step ([CANN] 计算公式
// step 1; [AscendC] 具体计算流程 矩阵乘法), both weight matrices in one panel so
// a single pass over X produces every projected column.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, each wave a
// 128 x 128 sub-tile = 4 x 4 blocks of the 32x32x16 bf16 MFMA, accumulators
// in AGPRs), K step 32, four 32 KiB LDS stages filled by direct-to-LDS copies
// (global_load_lds_dwordx4: no staging registers, no ds_write).
//  * X tile: row-major in LDS, 64 B per row, 16-byte chunks XOR-swizzled by
//    ((row >> 1) ^ (row >> 2)) & 3 so fragment reads are bank conflict free
//    whether LDS serves 8 or 16 lanes per cycle.  A copy instruction covers
//    16 rows x 64 B; each lane fetches the logical chunk the swizzle places
//    at its LDS slot.
//  * Panel tile: fragment-major like the panel in HBM (1 KiB per MFMA B
//    fragment), copied and read lane-contiguously.
// Copies run three K steps ahead of the MFMAs: on MI355X one step of MFMA
// work (~0.5 us) is shorter than the latency of a batch of copies (~1.2 us
// measured), so fewer stages leave the MFMAs waiting; the stage count is
// what 128 KiB of LDS holds at this K step.  The 8 copies of a step are
// interleaved one per two MFMAs in its first half.
//
// Workgroups are persistent (one per CU, each walking a run of tiles): the
// last three K steps of a tile issue the copies of the first three steps of
// the workgroup's next tile, so the next tile's stages are in flight while
// the epilogue of the current one runs and the MFMAs restart without a
// pipeline fill.
//
// The tile schedule and the epilogue live in pool.hpp (the GEMM never writes
// the projection to HBM: its epilogue pools windows straight from the
// accumulators).
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GM_BM = 256, GM_BN = 256, GM_BK = 32;
constexpr int GM_THREADS = 256;
constexpr int GM_STAGES = 4;
constexpr int GM_STAGE_BYTES = (GM_BM + GM_BN) * GM_BK * 2;   // 32 KiB
constexpr int GM_LDS_BYTES = GM_STAGES * GM_STAGE_BYTES;     // 128 KiB
constexpr int GM_A_COPIES = GM_BM * GM_BK * 2 / 1024 / 4;     // X copies per wave and stage
constexpr int GM_A_ROWS = 1024 / (GM_BK * 2);                 // X rows per copy instruction

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
// byte offset of 16-byte chunk `chunk` of row `row` in a 64-byte-row tile
__device__ __forceinline__ int swz(int row, int chunk) {
  return (row << 6) + ((chunk ^ (((row >> 1) ^ (row >> 2)) & 3)) << 4);
}
// Tile row that copy instruction j of `wave` fills for `lane`.
__device__ __forceinline__ int gm_copy_row(int wave, int lane, int j) {
  return (wave * GM_A_COPIES + j) * GM_A_ROWS + lane / (GM_BK / 8);
}

// ---------------------------------------------------------------------------
// K loop of one 256 x 256 tile: acc[i][j] (wave (wm, wn), 32x32 block i of
// its 128 rows, block j of its 128 columns) = X[rows] . Wp[n0 .. n0+256)^T.
// K % 128 == 0 (so the K step count is a multiple of the 4 stages).
//
// Schedule of a K step (32 MFMAs per wave in 8 groups of 4): each group
// issues one copy of step kt+3 and two LDS fragment reads.  The first half's
// MFMAs use k-step 0 of the stage while k-step 1 is read, the second half's
// use k-step 1 while the next stage's k-step 0 is read, and the single
// barrier of the step sits between the halves, so no LDS read latency is
// exposed.  The copy unit takes a 1 KiB copy every few tens of cycles and a
// wave cannot issue past a copy it has not accepted, so the waves place
// their copy at different MFMAs of the group (wave w after MFMA w): copies
// from the lock-stepped waves reach the unit one after another instead of
// together.  Every group is fenced so the compiler keeps this order.
// ---------------------------------------------------------------------------
#define GM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | 0x0f70)
// s_waitcnt vmcnt(12) lgkmcnt(0)
#define GM_WAIT_VM12_LGKM0() __builtin_amdgcn_s_waitcnt((12 & 0xf) | ((12 >> 4) << 14) | 0x0070)
#define GM_BARRIER() asm volatile("s_barrier" ::: "memory")

// Copy sources of one tile: this lane's X rows (one per X copy instruction)
// and its panel fragments.
struct GmSrc {
  const uint16_t* a[GM_A_COPIES];
  const uint16_t* b;
};

// arow[j] is the X row that this lane's j-th copy instruction reads (tile row
// gm_copy_row(wave, lane, j)); rows outside the tensor must be clamped by the
// caller to any valid row (their results are not used).
__device__ __forceinline__ GmSrc gm_sources(const uint16_t* __restrict__ X,
                                            const uint16_t* __restrict__ W, int K, int n0,
                                            const int (&arow)[GM_A_COPIES]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  GmSrc src;
  // X copies: instruction j of wave w fills tile rows r0 = (4w + j) * 16 ..
  // +16; lane l lands at LDS byte r0*64 + 16 l, i.e. row r0 + l/4, physical
  // chunk l%4, so it fetches the logical chunk the swizzle places there.
#pragma unroll
  for (int j = 0; j < GM_A_COPIES; ++j) {
    const int row = gm_copy_row(wave, lane, j);
    const int kc = (lane & 3) ^ (((row >> 1) ^ (row >> 2)) & 3);
    src.a[j] = X + (size_t)arow[j] * K + kc * 8;
  }
  // panel copies: fragment f = 4w + j of a stage is (column block f / 2,
  // k-step f % 2)
  src.b = W + ((((size_t)(n0 >> 5) + 2 * wave) * (size_t)(K >> 4)) * 64 + lane) * 8;
  return src;
}

// The copies of steps 0 .. 2 of a tile into stages 0 .. 2 (the first tile of
// a workgroup; later tiles get theirs from the previous tile's last steps).
__device__ __forceinline__ void gm_prologue(uint8_t* smem, const GmSrc& src, size_t ksteps) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    uint8_t* st = smem + t * GM_STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dma16(src.a[j] + t * GM_BK, st + (wave * 4 + j) * 1024);
      dma16(src.b + ((size_t)(j >> 1) * ksteps + t * 2 + (j & 1)) * 512,
            st + 16384 + (wave * 4 + j) * 1024);
    }
  }
}

// The K loop of one tile.  Step kt copies step kt+3 of this tile, or, in the
// last three steps, step kt+3-KT of the next tile (has_next) or a re-copy of
// step KT-1 into a stage nothing reads any more; so the next tile's first
// stages are in flight while this tile's epilogue runs.  KT % 4 == 0 keeps
// the stage of step kt at kt % 4 in every tile.
template <int P>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4][4], uint8_t* smem, const GmSrc& cur,
                                          const GmSrc& nxt, bool has_next, size_t ksteps,
                                          int KT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // step 0's stage has landed once at most the 16 newest memory operations
  // are outstanding (copies of steps 1 and 2, or the previous epilogue's
  // stores, which come after them)
  GM_WAIT_VM(16);
  GM_BARRIER();
  // Fragments: a0/b0 = k-step 0 of the current stage, a1/b1 = k-step 1.
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] = *reinterpret_cast<const bf16x8*>(smem + swz(wm * 128 + i * 32 + lrow, lhalf));
    b0[i] = *reinterpret_cast<const bf16x8*>(smem + 16384 + ((wn * 4 + i) * 2) * 1024 + lane * 16);
  }
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* sa = smem + (kt & 3) * GM_STAGE_BYTES;
    const uint8_t* sb = sa + 16384;
    const uint8_t* na = smem + ((kt + 1) & 3) * GM_STAGE_BYTES;
    const uint8_t* nb = na + 16384;
    // copies of step kt+3 go to the stage of step kt-1, which every wave
    // finished reading before the previous step's barrier
    const bool to_next = kt + 3 >= KT;
    const bool from_next = to_next && has_next;
    const int kn = to_next ? (has_next ? kt + 3 - KT : KT - 1) : kt + 3;
    uint8_t* st = smem + ((kt + 3) & 3) * GM_STAGE_BYTES;
    const uint16_t* bk = (from_next ? nxt.b : cur.b) + (size_t)kn * 2 * 512;
    // first half: copies 0-3 (X rows), reads of a1/b1, MFMAs of a0 x b0
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_barrier(0);
      a1[g] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 128 + g * 32 + lrow, 2 + lhalf));
      b1[g] = *reinterpret_cast<const bf16x8*>(sb + ((wn * 4 + g) * 2 + 1) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j == P) {
          __builtin_amdgcn_sched_barrier(0);
          dma16((from_next ? nxt.a[g] : cur.a[g]) + kn * GM_BK, st + (wave * 4 + g) * 1024);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[g][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[g], b0[j], acc[g][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // step kt+1's stage: this wave's copies are done when only the 12 issued
    // after them (step kt+2's and half of step kt+3's) are outstanding, and
    // the barrier publishes every wave's (a bare barrier: a workgroup fence
    // would wait for every copy)
    GM_WAIT_VM12_LGKM0();
    GM_BARRIER();
    // second half: copies 4-7 (panel fragments), reads of the next a0/b0,
    // MFMAs of a1 x b1
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_barrier(0);
      a0[g] = *reinterpret_cast<const bf16x8*>(na + swz(wm * 128 + g * 32 + lrow, lhalf));
      b0[g] = *reinterpret_cast<const bf16x8*>(nb + ((wn * 4 + g) * 2) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j == P) {
          __builtin_amdgcn_sched_barrier(0);
          dma16(bk + ((size_t)(g >> 1) * ksteps + (g & 1)) * 512, st + 16384 + (wave * 4 + g) * 1024);
          __builtin_amdgcn_sched_barrier(0);
        }
        acc[g][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[g], b1[j], acc[g][j], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One tile's K loop with the wave's copy position (see the schedule above).
__device__ __forceinline__ void gemm_tile_any(f32x16 (&acc)[4][4], uint8_t* smem,
                                              const GmSrc& cur, const GmSrc& nxt, bool has_next,
                                              size_t ksteps, int KT) {
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: gemm_tile<0>(acc, smem, cur, nxt, has_next, ksteps, KT); break;
    case 1: gemm_tile<1>(acc, smem, cur, nxt, has_next, ksteps, KT); break;
    case 2: gemm_tile<2>(acc, smem, cur, nxt, has_next, ksteps, KT); break;
    default: gemm_tile<3>(acc, smem, cur, nxt, has_next, ksteps, KT); break;
  }
}

// Every copy has landed (before the workgroup ends: no copy may write its
// LDS after that).
__device__ __forceinline__ void gm_drain() {
  GM_WAIT_VM(0);
  GM_BARRIER();
}

#undef GM_WAIT_VM
#undef GM_WAIT_VM12_LGKM0
#undef GM_BARRIER

}  // namespace cmp
