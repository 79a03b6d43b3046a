// Prefill projection: P[T, N] (fp32) = X[T, H] (bf16) . Wp[N, H]^T (bf16).
//
// This is the fused "[kv, score] = X @ [W_kv, W_gate]" step ([CANN] 计算公式
// step 1; [AscendC] 具体计算流程 矩阵乘法), both weight matrices in one panel so
// a single pass over X produces every projected column.
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2, each wave a
// 128 x 128 sub-tile = 4 x 4 blocks of the 32x32x16 bf16 MFMA), K step 64,
// two LDS stages of 64 KiB.  X is read row-major (128 contiguous bytes per
// row and K tile); the panel is fragment-major, so each 64-thread group reads
// one contiguous 1 KiB fragment.  LDS rows are
// 128 bytes; the 16-byte chunk index is XOR-swizzled with (row & 7) so eight
// lanes reading eight rows hit eight distinct bank groups.
//
// Workgroup order: the hardware deals workgroups round-robin to the 8 XCDs
// (workgroup i to XCD i % 8).  Tile ids are remapped so each XCD owns a
// contiguous run of tiles, N-fastest: the 8 N-tiles of an M-block (which
// share that block's X rows) run together on one XCD and share its L2.
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GM_BM = 256, GM_BN = 256, GM_BK = 64;
constexpr int GM_THREADS = 256;
constexpr int GM_STAGE_BYTES = (GM_BM + GM_BN) * GM_BK * 2;   // 64 KiB

__device__ __forceinline__ int swz(int row, int chunk) { return (row << 7) + ((chunk ^ (row & 7)) << 4); }

template <bool kStoreP>
__global__ __launch_bounds__(GM_THREADS, 1) void gemm_proj_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ P, int T,
    int N, int K, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order
  const int nwg = gridDim.x;
  const int per_xcd = nwg >> 3;
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= tiles_m * tiles_n) return;
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int m0 = tm * GM_BM, n0 = tn * GM_BN;

  // X (row-major): chunk i of a thread is row (tid >> 3) + 32 i, 16-byte
  // column chunk tid & 7 (the same for every i).
  const int row0 = tid >> 3, kc = tid & 7;
  const int soff = swz(row0, kc);          // + i * 4096 for chunk i
  const int last_row = T - 1;
  // Panel (fragment-major): chunk i of a thread is column block n0/32 + i,
  // k-step (tid >> 6) of the 4 in the K tile, fragment lane tid & 63, i.e.
  // panel column n0 + 32 i + (tid & 31), 16-byte K chunk 2*(tid >> 6) + ((tid >> 5) & 1).
  const int bl = tid & 63, bks = tid >> 6;
  const int brow = bl & 31, bkc = 2 * bks + (bl >> 5);
  const int sboff = swz(brow, bkc);        // + i * 4096 for chunk i
  const size_t ksteps = (size_t)(K >> 4);
  const uint16_t* gb = W + (((size_t)(n0 >> 5) * ksteps + bks) * 64 + bl) * 8;
  const size_t bstep = ksteps * 64 * 8;    // next column block

  const size_t kcol = (size_t)kc * 8;
  const uint16_t* ga[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ga[i] = X + (size_t)min(m0 + row0 + 32 * i, last_row) * K + kcol;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = K / GM_BK;
  uint4 ra[8], rb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ra[i] = *reinterpret_cast<const uint4*>(ga[i]);
    rb[i] = *reinterpret_cast<const uint4*>(gb + i * bstep);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    *reinterpret_cast<uint4*>(smem + soff + i * 4096) = ra[i];
    *reinterpret_cast<uint4*>(smem + GM_BM * GM_BK * 2 + sboff + i * 4096) = rb[i];
  }
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    // prefetch the next K tile (the last iteration re-reads the final tile
    // into the idle stage, which nothing reads afterwards)
    const int k0 = min(kt + 1, KT - 1) * GM_BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(ga[i] + k0);
      rb[i] = *reinterpret_cast<const uint4*>(gb + i * bstep + (size_t)(k0 >> 4) * 512);
    }
    const uint8_t* sa = smem + (kt & 1) * GM_STAGE_BYTES;
    const uint8_t* sb = sa + GM_BM * GM_BK * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[4], b[4];
      const int ch = kk * 2 + lhalf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 128 + i * 32 + lrow, ch));
        b[i] = *reinterpret_cast<const bf16x8*>(sb + swz(wn * 128 + i * 32 + lrow, ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    {
      uint8_t* da = smem + ((kt + 1) & 1) * GM_STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<uint4*>(da + soff + i * 4096) = ra[i];
        *reinterpret_cast<uint4*>(da + GM_BM * GM_BK * 2 + sboff + i * 4096) = rb[i];
      }
    }
    __syncthreads();
  }

  if constexpr (kStoreP) {
    // 32x32 accumulator layout: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 128 + j * 32 + lrow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
          if (row < T) P[(size_t)row * N + col] = acc[i][j][r];
        }
      }
  }
}

}  // namespace cmp
