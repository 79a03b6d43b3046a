// Prefill projection: P[T, N] (fp32) = X[T, H] (bf16) . Wp[N, H]^T (bf16).
//
// This is the fused "[kv, score] = X @ [W_kv, W_gate]" step ([CANN] 计算公式
// step 1; [AscendC] 具体计算流程 矩阵乘法), both weight matrices in one panel so
// a single pass over X produces every projected column.
//
// Tiling: 256 x 256 output tile per workgroup of 8 waves, two per SIMD (4 x
// 2, each wave a 64 x 128 sub-tile = 2 x 4 blocks of the 32x32x16 bf16 MFMA,
// 128 accumulator registers).  With one wave per SIMD (128 x 128 sub-tiles)
// a wave that waits for the load unit to accept a copy leaves the SIMD's
// matrix core idle; with two, the other wave's MFMAs fill that time (3%
// faster at the 128K C4A shape, although every wave now reads half of a
// fragment set it shares with three others).  K step 32, operands staged in
// LDS by direct-to-LDS copies (global_load_lds_dwordx4: no staging
// registers, no ds_write), all 160 KiB of the CU's LDS.  Calls too short to
// give every CU a 256-row tile run 4 MFMA waves (2 x 2) on 128 x 256 tiles
// instead (same wave sub-tile, 112 KiB of LDS), so that the chip fills; their
// copies are issued by 4 more waves that do nothing else (one per SIMD
// beside the MFMA wave), since a wave that issues a copy waits until the
// CU's load unit accepts it and a lone MFMA wave per SIMD would leave its
// matrix core idle for that time:
//  * X: three 32 KiB buffers, each two K steps (256 rows x 128 B), so every
//    copy fetches whole 128-byte cache lines (8 rows x 128 B per copy
//    instruction).  Rows are row-major with their 16-byte chunks
//    XOR-swizzled by (row & 7) ^ ((row >> 3) & 1), which keeps fragment
//    reads bank conflict free whether LDS serves 8 or 16 lanes per cycle;
//    each lane fetches the logical chunk the swizzle places at its LDS slot.
//  * Panel: four 16 KiB stages of one K step, fragment-major like the panel
//    in HBM (1 KiB per MFMA B fragment), copied and read lane-contiguously.
// Copies run three K steps ahead of the MFMAs (the X buffers: two to four):
// on MI355X one step of MFMA work (~0.5 us) is shorter than the latency of a
// batch of copies (~1.2 us measured), so fewer stages leave the MFMAs
// waiting.  Each wave issues 4 copies per step (a copy wave of the 4-wave
// shape 6: the same panel copied by half as many waves).
//
// Workgroups are persistent (one per CU, each walking a run of tiles): the
// last three K steps of a tile issue the copies of the first three steps of
// the workgroup's next tile, so the next tile's stages are in flight while
// the epilogue of the current one runs and the MFMAs restart without a
// pipeline fill.  The X buffers rotate across tiles (the buffer of a tile's
// first K-step pair is passed in).
//
// The tile schedule and the epilogue live in pool.hpp (the GEMM never writes
// the projection to HBM: its epilogue pools windows straight from the
// accumulators).
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GM_BN = 256, GM_BK = 32;
constexpr int GM_WROWS = 64;                                   // rows of a wave's sub-tile
constexpr int GM_W_STAGE_BYTES = GM_BN * GM_BK * 2;            // 16 KiB
constexpr int GM_X_OFF = 4 * GM_W_STAGE_BYTES;                 // panel stages first
constexpr int GM_A_COPIES = 4;                                 // X copies per wave and buffer
constexpr int GM_A_ROWS = 1024 / (2 * GM_BK * 2);              // X rows per copy instruction (8)

// The two tile shapes, by MFMA wave count WV: 8 waves (4 row-waves x 2) make
// a 256 x 256 tile; 4 waves (2 x 2) a 128 x 256 tile, with 4 copy waves
// beside them.  The wave sub-tile (64 x 128) and the per-role X copies are
// the same.
template <int WV>
struct Gm {
  static constexpr int COPIERS = WV == 4 ? 4 : 0;              // copy-only waves
  static constexpr int THREADS = 64 * (WV + COPIERS);
  static constexpr int BM = 32 * WV;                           // tile rows
  static constexpr int NWM = BM / GM_WROWS;                    // row-waves
  static constexpr int X_BUF_BYTES = BM * 2 * GM_BK * 2;       // BM rows x two K steps
  static constexpr int LDS_BYTES = GM_X_OFF + 3 * X_BUF_BYTES; // 160 / 112 KiB
  static constexpr int WC = 16 / WV;                           // panel copies per role and step
  static_assert(X_BUF_BYTES / 1024 / WV == GM_A_COPIES, "X copies per wave");
};
// What a wave of the K loop does: copy and multiply (8-wave shape), only
// multiply, or only copy (the two halves of the 4-wave shape).  A copy role
// r in 0 .. WV-1 names the share of the copies the wave issues.
enum GmMode { GM_ALL, GM_MFMA, GM_COPY };

// LDS the epilogue may use between two tiles: the panel stage of a tile's
// last K step, which nothing reads or fills until the next tile's first step.
constexpr int GM_IDLE_OFF = 3 * GM_W_STAGE_BYTES;
constexpr int GM_IDLE_BYTES = GM_W_STAGE_BYTES;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
__device__ __forceinline__ int swz_bits(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// Tile row that X copy instruction j of copy role `role` fills for `lane`.
__device__ __forceinline__ int gm_copy_row(int role, int lane, int j) {
  return (role * GM_A_COPIES + j) * GM_A_ROWS + (lane >> 3);
}

// ---------------------------------------------------------------------------
// K loop of one BM x 256 tile: acc[i][j] (wave (wm, wn), 32x32 block i of
// its 64 rows, block j of its 128 columns) = X[rows] . Wp[n0 .. n0+256)^T.
// K % 128 == 0 (so the K step count is a multiple of the 4 panel stages).
//
// Schedule of a K step (8 MFMAs per wave and k-step, in 4 groups of 2): each
// group reads the next k-step's panel fragment (and, in two of them, its X
// fragment).  The first half's MFMAs use k-step 0 of the step while k-step
// 1 is read, the second half's use k-step 1 while the next step's k-step 0
// is read, and the single barrier of the step sits between the halves, so
// no LDS read latency is exposed.  The first half issues 2 X copies (a
// quarter of the buffer two K-step pairs ahead: step 2c issues the first
// half of pair c+2, step 2c+1 the second), the second half the WC panel
// copies of step kt+3 (8 waves: wave w copies column block w of the tile;
// 4 waves: blocks 2w and 2w+1, one copy per MFMA group).  The copy
// unit takes a 1 KiB copy every few tens of cycles and a wave cannot issue
// past a copy it has not accepted, so waves on different SIMDs place their
// copies at different MFMAs (P = wave % 4; other placements measured the
// same).  Every group is fenced so the compiler keeps this order.
// ---------------------------------------------------------------------------
#define GM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | 0x0f70)
// s_waitcnt vmcnt(n) lgkmcnt(0)
#define GM_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 0xf) | (((n) >> 4) << 14) | 0x0070)
#define GM_BARRIER() asm volatile("s_barrier" ::: "memory")

// Copy sources of one tile: a uniform base for X (the tile's first row) and
// one for the wave's panel column block, and this lane's byte offsets from
// the X base (the copies take the scalar-base address form, so the bases
// live in scalar registers).
struct GmSrc {
  const uint8_t* x;
  const uint8_t* w;
  uint32_t a[GM_A_COPIES];
};

// arow[j] is the X row that this lane's j-th copy instruction reads (tile row
// gm_copy_row(role, lane, j)); rows outside the tensor must be clamped by the
// caller to any valid row (their results are not used).  arow0 (uniform)
// <= every arow[j] and arow[j] - arow0 < the tile rows.
template <int WV>
__device__ __forceinline__ GmSrc gm_sources(const uint16_t* __restrict__ X,
                                            const uint16_t* __restrict__ W, int K, int n0,
                                            const int (&arow)[GM_A_COPIES], int arow0, int role) {
  const int lane = threadIdx.x & 63;
  GmSrc src;
  // X copies: instruction j of role w fills buffer rows r0 = (4w + j) * 8 ..
  // +8; lane l lands at LDS byte r0*128 + 16 l, i.e. row r0 + l/8, physical
  // chunk l%8, so it fetches the logical chunk the swizzle places there.
#pragma unroll
  for (int j = 0; j < GM_A_COPIES; ++j) {
    const int row = gm_copy_row(role, lane, j);
    const int kc = (lane & 7) ^ swz_bits(row);
    src.a[j] = (uint32_t)(((size_t)(arow[j] - arow0) * K + kc * 8) * 2);
  }
  src.x = reinterpret_cast<const uint8_t*>(X + (size_t)__builtin_amdgcn_readfirstlane(arow0) * K);
  // panel copies: role w copies column blocks w*WC/2 .. (fragments (block,
  // k-step) of a stage); lane offsets come from gm_woff
  const int wv = __builtin_amdgcn_readfirstlane(role);
  src.w = reinterpret_cast<const uint8_t*>(
      W + (((size_t)(n0 >> 5) + wv * (Gm<WV>::WC / 2)) * (size_t)(K >> 4)) * 512);
  return src;
}

template <int WV>
__device__ __forceinline__ uint8_t* gm_xbuf(uint8_t* smem, int buf) {
  return smem + GM_X_OFF + buf * Gm<WV>::X_BUF_BYTES;
}
// Byte offset of this wave's panel copy c of K step t (column block c / 2
// of the wave's, k-step c % 2; a column block is ksteps fragments of 1 KiB).
__device__ __forceinline__ uint32_t gm_woff(int c, int t, int ksteps) {
  return (uint32_t)((((c >> 1) * ksteps + t * 2 + (c & 1)) << 10) + (threadIdx.x & 63) * 16);
}
// Quarter q of copy role `role`'s X copies of K-step pair c into buffer xb.
__device__ __forceinline__ void gm_xcopy(const GmSrc& src, int c, int q, uint8_t* xb, int role) {
#pragma unroll
  for (int g = 0; g < 2; ++g)
    dma16(src.x + (src.a[2 * q + g] + (uint32_t)c * (4 * GM_BK)),
          xb + (role * GM_A_COPIES + 2 * q + g) * 1024);
}
// Copy role `role`'s panel copies of K step t into stage st.
template <int WV>
__device__ __forceinline__ void gm_wcopy(const GmSrc& src, int t, uint8_t* st, int ksteps,
                                         int role) {
  constexpr int WC = Gm<WV>::WC;
#pragma unroll
  for (int c = 0; c < WC; ++c) dma16(src.w + gm_woff(c, t, ksteps), st + (role * WC + c) * 1024);
}

// The copies of steps 0 .. 2 of a workgroup's first tile (pairs 0 and 1 into
// X buffers 0 and 1, steps 0 .. 2 into panel stages 0 .. 2), in the order the
// steady state issues them; later tiles get theirs from the previous tile's
// last steps.
template <int WV>
__device__ __forceinline__ void gm_prologue(uint8_t* smem, const GmSrc& src, int ksteps,
                                            int role) {
  gm_xcopy(src, 0, 0, gm_xbuf<WV>(smem, 0), role);
  gm_xcopy(src, 0, 1, gm_xbuf<WV>(smem, 0), role);
  gm_wcopy<WV>(src, 0, smem, ksteps, role);
  gm_xcopy(src, 1, 0, gm_xbuf<WV>(smem, 1), role);
  gm_wcopy<WV>(src, 1, smem + GM_W_STAGE_BYTES, ksteps, role);
  gm_xcopy(src, 1, 1, gm_xbuf<WV>(smem, 1), role);
  gm_wcopy<WV>(src, 2, smem + 2 * GM_W_STAGE_BYTES, ksteps, role);
}

// The K loop of one tile; xrot = X buffer of its K-step pair 0.  Step kt
// copies panel step kt+3 and half of X pair kt/2+2 of this tile, or, past
// the tile's end, those of the next tile (has_next) or re-copies of the last
// ones into a stage or buffer nothing reads any more; so the next tile's
// first stages are in flight while this tile's epilogue runs.  KT % 4 == 0
// keeps the panel stage of step kt at kt % 4 in every tile; the X buffers
// continue their rotation into the next tile.  MODE: what this wave does
// (GmMode); role: its share of the copies; every mode passes the same
// barriers.
template <int WV, int P, int MODE>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[2][4], uint8_t* smem, const GmSrc& cur,
                                          const GmSrc& nxt, bool has_next, int KT, int xrot,
                                          int ksteps, int role) {
  constexpr int WC = Gm<WV>::WC;
  constexpr bool COPY = MODE != GM_MFMA, MUL = MODE != GM_COPY;
  // outstanding copies allowed at the mid-step wait (step kt-1's and the
  // first half of step kt's) and at the tile start (pair 1's, steps 1 and 2)
  constexpr int VM_MID = 2 + WC + 2, VM_START = 4 + 2 * WC;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int KC = KT >> 1;
  if constexpr (MUL) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
  // step 0's stage and pair 0 have landed once at most the VM_START newest
  // memory operations are outstanding (copies of pair 1 and steps 1 and 2,
  // or the previous epilogue's stores, which come after them); a wave that
  // issues no copies waits for none
  if constexpr (COPY) GM_WAIT_VM(VM_START);
  GM_BARRIER();
  // X buffers of pairs kc, kc + 1, kc + 2
  int xb0 = xrot, xb1 = xrot == 2 ? 0 : xrot + 1, xb2 = xrot == 0 ? 2 : xrot - 1;
  // this lane's A fragment row (block 0) and its swizzle; block i adds i*4096
  const int arow_off = (wm * GM_WROWS + lrow) << 7;
  const int asw = swz_bits(lrow);
  // Fragments: a0/b0 = k-step 0 of the current step, a1/b1 = k-step 1.
  bf16x8 a0[2], b0[4], a1[2], b1[4];
  if constexpr (MUL) {
    const uint8_t* xa = gm_xbuf<WV>(smem, xb0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a0[i] = *reinterpret_cast<const bf16x8*>(xa + arow_off + ((lhalf ^ asw) << 4) + i * 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b0[j] = *reinterpret_cast<const bf16x8*>(smem + ((wn * 4 + j) * 2) * 1024 + lane * 16);
  }
  for (int kc = 0; kc < KC; ++kc) {
    const uint8_t* xa = gm_xbuf<WV>(smem, xb0);
    const uint8_t* xn = gm_xbuf<WV>(smem, xb1);
    uint8_t* xc = gm_xbuf<WV>(smem, xb2);
    // X pair kc+2 goes to the buffer of pair kc-1, which every wave finished
    // reading before the barrier of step 2kc-1
    const bool xto_next = kc + 2 >= KC;
    const int xkn = xto_next ? (has_next ? kc + 2 - KC : KC - 1) : kc + 2;
    const GmSrc& xs = xto_next && has_next ? nxt : cur;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kt = 2 * kc + p;
      const uint8_t* sb = smem + (kt & 3) * GM_W_STAGE_BYTES;
      const uint8_t* nb = smem + ((kt + 1) & 3) * GM_W_STAGE_BYTES;
      const uint8_t* na = p == 0 ? xa : xn;
      // panel step kt+3 goes to the stage of step kt-1, which every wave
      // finished reading before the previous step's barrier
      const bool to_next = kt + 3 >= KT;
      const bool from_next = to_next && has_next;
      const int kn = to_next ? (has_next ? kt + 3 - KT : KT - 1) : kt + 3;
      uint8_t* st = smem + ((kt + 3) & 3) * GM_W_STAGE_BYTES;
      const uint8_t* bk = from_next ? nxt.w : cur.w;
      const int q1 = ((4 * p + 2 + lhalf) ^ asw) << 4;       // k-step 1 of this step
      const int qn = ((4 * (1 - p) + lhalf) ^ asw) << 4;     // k-step 0 of the next
      // first half: X copies, reads of a1/b1, MFMAs of a0 x b0
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MUL) {
          b1[g] = *reinterpret_cast<const bf16x8*>(sb + ((wn * 4 + g) * 2 + 1) * 1024 + lane * 16);
          if (g < 2) a1[g] = *reinterpret_cast<const bf16x8*>(xa + arow_off + q1 + g * 4096);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if (COPY && (g & 1) == (P >> 1) && i == (P & 1)) {
            __builtin_amdgcn_sched_barrier(0);
            const int j = 2 * p + (g >> 1);
            dma16(xs.x + (xs.a[j] + (uint32_t)xkn * (4 * GM_BK)),
                  xc + (role * GM_A_COPIES + j) * 1024);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (MUL)
            acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[g], acc[i][g], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // step kt+1's panel stage and X pair: this wave's copies are done when
      // only the VM_MID issued after them (step kt-1's and the first half of
      // step kt's) are outstanding, and the barrier publishes every wave's (a
      // bare barrier: a workgroup fence would wait for every copy)
      if constexpr (COPY)
        GM_WAIT_VM_LGKM0(VM_MID);
      else
        __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0)
      GM_BARRIER();
      // second half: panel copies, reads of the next a0/b0, MFMAs of a1 x b1
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MUL) {
          b0[g] = *reinterpret_cast<const bf16x8*>(nb + ((wn * 4 + g) * 2) * 1024 + lane * 16);
          if (g < 2) a0[g] = *reinterpret_cast<const bf16x8*>(na + arow_off + qn + g * 4096);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          // WC = 2: copy g / 2 at two of the slots; WC = 4: copy g in every group
          if (COPY && (WC == 4 || (g & 1) == (P >> 1)) && i == (P & 1)) {
            __builtin_amdgcn_sched_barrier(0);
            const int c = WC == 4 ? g : g >> 1;
            dma16(bk + gm_woff(c, kn, ksteps), st + (role * WC + c) * 1024);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (MUL)
            acc[i][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[g], acc[i][g], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int t = xb0;
    xb0 = xb1;
    xb1 = xb2;
    xb2 = t;
  }
}

// One tile's K loop in role MODE: a wave of the 8-wave shape copies and
// multiplies, with its copy position P = wave % 4 (see the schedule above);
// in the 4-wave shape waves 0..3 multiply and waves 4..7 issue the copies of
// roles 0..3.
template <int WV, int MODE>
__device__ __forceinline__ void gemm_tile_any(f32x16 (&acc)[2][4], uint8_t* smem,
                                              const GmSrc& cur, const GmSrc& nxt, bool has_next,
                                              int KT, int xrot, int ksteps, int role) {
  if constexpr (MODE != GM_ALL) {
    gemm_tile<WV, 0, MODE>(acc, smem, cur, nxt, has_next, KT, xrot, ksteps, role);
  } else {
    switch (role & 3) {
      case 0: gemm_tile<WV, 0, GM_ALL>(acc, smem, cur, nxt, has_next, KT, xrot, ksteps, role); break;
      case 1: gemm_tile<WV, 1, GM_ALL>(acc, smem, cur, nxt, has_next, KT, xrot, ksteps, role); break;
      case 2: gemm_tile<WV, 2, GM_ALL>(acc, smem, cur, nxt, has_next, KT, xrot, ksteps, role); break;
      default: gemm_tile<WV, 3, GM_ALL>(acc, smem, cur, nxt, has_next, KT, xrot, ksteps, role); break;
    }
  }
}

// Every copy has landed (before the workgroup ends: no copy may write its
// LDS after that).
__device__ __forceinline__ void gm_drain() {
  GM_WAIT_VM(0);
  GM_BARRIER();
}

#undef GM_WAIT_VM
#undef GM_WAIT_VM_LGKM0
#undef GM_BARRIER

}  // namespace cmp
