// Prefill kernels other than the projection GEMM: request plan, window
// pooling, post-processing (RMSNorm, RoPE, Hadamard), state write-back.
#pragma once
#include "common.hpp"

namespace cmp {

// ---------------------------------------------------------------------------
// Setup of a prefill call: one launch of four independent parts.
//  * workgroup 0 plans the call (per-request start, length, windows, output
//    rows and GEMM tiles), writes the call's error word and clears the
//    GEMM's tile queue heads;
//  * the next D*D/2048 workgroups (rotate only) check the Hadamard matrix
//    and copy it to the MFMA fragment order;
//  * for ratios of 8 and more, R/4 workgroups copy Ape transposed
//    ([channel][slot]), so that the GEMM epilogue reads the Ape of 4
//    consecutive slots with one load;
//  * the rest stage the ring rows of positions before each request's first
//    token (read once here, before the GEMM stores any state row).
// No part reads another's output, so they need no ordering inside the
// launch; every later kernel of the call sees all four.
// ---------------------------------------------------------------------------
constexpr int SETUP_THREADS = 256;

// Request b of a call, from cu_seqlens / seqused / start_pos, with the
// argument checks of the plan (the planning workgroup and the staging
// workgroups decode a request the same way):
//   n_b = seqused[b] (or the slot length), s_b = start_pos[b] (or 0);
//   an inconsistent slot, n or s makes the request empty and sets a bit.
struct PReq {
  int s, n, row0;
  uint32_t bad;
};
__device__ __forceinline__ PReq prefill_request(int b, int B, int T,
                                                const int32_t* __restrict__ cu_seqlens,
                                                const int32_t* __restrict__ seqused,
                                                const int32_t* __restrict__ start_pos) {
  PReq q{0, 0, 0, 0u};
  int c0, c1;
  if (cu_seqlens) { c0 = cu_seqlens[b]; c1 = cu_seqlens[b + 1]; }
  else { const int S = T / B; c0 = b * S; c1 = c0 + S; }
  if (c0 < 0 || c1 < c0 || c1 > T) { q.bad |= CMP_DEVERR_SEQLEN; c0 = 0; c1 = 0; }
  const int slot = c1 - c0;
  int n = seqused ? seqused[b] : slot;
  if (n < 0 || n > slot) { q.bad |= CMP_DEVERR_SEQLEN; n = n < 0 ? 0 : slot; }
  int s = start_pos ? start_pos[b] : 0;
  if (s < 0 || s > 0x7fffffff - n) { q.bad |= CMP_DEVERR_START_POS; s = 0; n = 0; }
  q.s = s;
  q.n = n;
  q.row0 = c0;
  return q;
}

// First position the GEMM tiles of a request starting at s cover (window
// aligned, one window earlier for ratio 4: the halo of staged rows)
__device__ __forceinline__ int prefill_first(int s, int ratio, int coff) {
  return ratio * (s / ratio) - (coff - 1) * ratio;
}

// Plan: per-request start / length / windows / output rows, computed on the
// device (no host synchronisation); also writes this call's error word.
//   n_b   = seqused[b] (or the slot length)        e_b = s_b + n_b
//   c_b   = floor(e_b / r) - floor(s_b / r)        windows completed here
//   u_b   = ceil(n_b / r)                          output rows owned
//   o_b   = sum_{b' < b} u_b'                      first output row
// Windows complete when (start_pos + i + 1) % ratio == 0 ([PyPTO]
// 数值精度与验证要点), which is what c_b counts.  Rows per request and their
// placement are the output layout documented in compressor.h.
// One workgroup; B is walked in chunks of SETUP_THREADS with a carried offset.
__device__ __forceinline__ void plan_block(
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, int B, int T, int ratio, int coff, int tile_rows,
    int out_rows, int32_t* __restrict__ plan, int32_t* __restrict__ tile_count,
    uint32_t* __restrict__ err) {
  __shared__ int scan[SETUP_THREADS];
  __shared__ int scan2[SETUP_THREADS];
  __shared__ uint32_t s_err;
  __shared__ int s_carry, s_tcarry;
  const int tid = threadIdx.x;
  const int halo = (coff - 1) * ratio;
  if (tid == 0) { s_err = 0; s_carry = 0; s_tcarry = 0; }
  __syncthreads();
  uint32_t my_err = 0;
  for (int base = 0; base < B; base += SETUP_THREADS) {
    const int b = base + tid;
    PReq q{0, 0, 0, 0u};
    if (b < B) q = prefill_request(b, B, T, cu_seqlens, seqused, start_pos);
    my_err |= q.bad;
    const int s = q.s, n = q.n;
    const int u = (n + ratio - 1) / ratio;
    // GEMM tiles: tile_rows positions each from the window start r*floor(s/r)
    // until e is covered; staged state rows start `halo` positions earlier
    const int first = prefill_first(s, ratio, coff);
    const int over = s + n - (first + halo) - tile_rows;
    const int ntile = n == 0 ? 0 : 1 + (over > 0 ? (over + tile_rows - 1) / tile_rows : 0);
    scan[tid] = u;
    scan2[tid] = ntile;
    __syncthreads();
    for (int off = 1; off < SETUP_THREADS; off <<= 1) {     // inclusive scans
      const int v = tid >= off ? scan[tid - off] : 0;
      const int v2 = tid >= off ? scan2[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      scan2[tid] += v2;
      __syncthreads();
    }
    if (b < B) {
      const int e = s + n;
      int32_t* rec = plan + (long)b * PL_WIDTH;
      rec[PL_START] = s;
      rec[PL_NTOK] = n;
      rec[PL_END] = e;
      rec[PL_ROW0] = q.row0;
      rec[PL_NWIN] = e / ratio - s / ratio;
      rec[PL_NROWS] = u;
      rec[PL_OUT0] = s_carry + scan[tid] - u;
      rec[PL_FIRST] = first;
      rec[PL_TILE0] = s_tcarry + scan2[tid] - ntile;
      rec[PL_NTILE] = ntile;
    }
    __syncthreads();
    if (tid == SETUP_THREADS - 1) { s_carry += scan[tid]; s_tcarry += scan2[tid]; }
    __syncthreads();
  }
  if (my_err) atomicOr(&s_err, my_err);
  __syncthreads();
  if (tid == 0) {
    uint32_t e = s_err;
    if (s_carry > out_rows) e |= CMP_DEVERR_OUT_ROWS;
    *err = e;                                       // this call's error word
    tile_count[0] = s_tcarry;
  }
  if (tid >= 1 && tid <= 8) tile_count[tid] = 0;   // the GEMM's per-XCD tile queues
}

// Request owning output row `row` (largest b with o_b <= row), or -1.
__device__ __forceinline__ int find_request(const int32_t* __restrict__ plan, int B, int row) {
  int lo = 0, hi = B - 1, ans = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (plan[(long)mid * PL_WIDTH + PL_OUT0] <= row) { ans = mid; lo = mid + 1; }
    else hi = mid - 1;
  }
  return ans;
}

// Does output row `row` hold a window?  (Request b's k-th completed window
// is row o_b + k; every other row is +0.)
__device__ __forceinline__ bool row_has_window(const int32_t* __restrict__ plan, int B, int row) {
  const int b = find_request(plan, B, row);
  if (b < 0) return false;
  const int32_t* rec = plan + (long)b * PL_WIDTH;
  return row - rec[PL_OUT0] < rec[PL_NWIN];
}

// ---------------------------------------------------------------------------
// Post-processing of PR (32 or 16) output rows per workgroup: RMSNorm (eps 1e-6, fp32,
// times the weight), interleaved RoPE on channels [D-64, D) ([PyPTO]
// 压缩窗口与状态更新 / 算子级辅助函数), then either the bf16 store or, with
// rotate, out = y @ Had as a bf16 MFMA product (K = D) against the matrix in
// fragment-major order (hadamard_pack_block).  Rows without a window are +0.
// Pairs (2i, 2i+1) of the rotary slice rotate together: the even element with
// cos/sin column i, the odd one with column 32 + i.
//
// Each wave normalises PR / 4 rows in batches of 4 (all loads of a batch in
// flight before the first reduction).  Calls whose 32-row grid would not
// give every CU a workgroup take 16-row workgroups: one batch per wave, so
// each workgroup waits for one load round after its plan lookups instead of
// two (8192-token C128A call, 64 rows: 9.0 -> 6.8 us); with more rows than
// that the extra workgroups' plan lookups cost more (128K C4A call, 32768
// rows: 36.6 -> 42.6 us with 16-row workgroups).  When Had is a scaled Sylvester matrix
// (no hadamard_pack_block flag is set) the product is the fast
// Walsh-Hadamard transform of the fp32 row in registers (log2 D butterfly
// stages: within a lane, then across lanes), times Had[0][0]: no matrix
// reads.  Otherwise the MFMA product reads each Had fragment once per
// 32-column block of a wave, four k-steps ahead of its use, and stores each
// block's rows as it completes.  Both paths keep the register demand low enough for four waves
// per SIMD (with 64-row tiles and every output block's accumulators live,
// the kernel needed 384 registers per wave: one wave per SIMD, and half of
// the workgroups of a 32768-row call waited for a second round).
// ---------------------------------------------------------------------------
constexpr int POST_ROWS = 32;                    // rows of the LDS tile (the most per workgroup)
constexpr int POST_BATCH = 4;

// N consecutive bf16 rotary columns, loaded as one piece
template <int N>
struct __attribute__((aligned(2 * N))) RopeCols {
  uint16_t v[N];
};

// LDS byte offset of the 16-byte chunk `ch` of tile row `lr` (rows of D bf16,
// D * 2 a multiple of 256): 16 consecutive rows at one chunk index hit 16
// distinct bank groups
template <int D>
__device__ __forceinline__ int post_lds(int lr, int ch) {
  return lr * D * 2 + ((ch ^ (lr & 15)) << 4);
}

// One butterfly stage of the transform across lanes: lane pairs (l, l ^ M),
// the lower lane keeping a + b, the upper one a - b (a from the lower lane).
template <int M, int CPL>
__device__ __forceinline__ void fwht_lanes(float (&y)[CPL], int lane) {
  const float sgn = (lane & M) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) y[i] = fmaf(sgn, y[i], lane_xor<M>(y[i]));
}

template <int CPL, int PR>
__global__ __launch_bounds__(256, 4) void post_kernel(
    Cfg cf, const float* __restrict__ pooled, const float* __restrict__ split,
    const int32_t* __restrict__ plan, int B, int out_rows,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ hadF,
    const uint32_t* __restrict__ had_flags, int nhad, uint16_t* __restrict__ out) {
  constexpr int D = CPL * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [64][D] bf16, swizzled
  static_assert(PR == 16 || PR == 32, "rows per workgroup");
  __shared__ int32_t row_live[PR];
  // per row of the workgroup: bit 0 holds a window, bit 1 a window split
  // between GEMM tiles, bits 2.. that window's second tile
  __shared__ int32_t row_info[PR];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_base = blockIdx.x * PR;
  if ((int)threadIdx.x < PR) {                    // every row's plan lookup at once
    const int row = row_base + threadIdx.x;
    int info = 0;
    const int rb = row < out_rows ? find_request(plan, B, row) : -1;
    if (rb >= 0) {
      const int32_t* rrec = plan + (long)rb * PL_WIDTH;
      const int k = row - rrec[PL_OUT0];
      if (k < rrec[PL_NWIN]) {
        info = 1;
        // windows per GEMM tile: tile rows / 4 (a power of two)
        const int wsh = __builtin_ctz(cf.bm >> 2);
        if (cf.coff == 2 && k > 0 && (k & ((1 << wsh) - 1)) == 0)
          info |= 2 | ((rrec[PL_TILE0] + (k >> wsh)) << 2);
      }
    }
    row_info[threadIdx.x] = info;
  }
  // any Hadamard-check workgroup that found the matrix not a scaled
  // Sylvester matrix (nhad <= 128 flags, one per thread)
  const int general = __syncthreads_or(cf.rotate && (int)threadIdx.x < nhad &&
                                       had_flags[threadIdx.x] != 0);
  const int c0 = lane * CPL;
  const int rope0 = D - cf.rope, half = cf.rope / 2;
  const bool rope_lane = c0 >= rope0;
  const int pr0 = rope_lane ? (c0 - rope0) >> 1 : 0;
  float g[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) g[i] = bf2f(gamma[c0 + i]);
  const bool fwht = cf.rotate && !general;
  const float hscale = cf.rotate ? bf2f(hadF[0]) : 0.f;   // Had[0][0]

#pragma unroll 1
  for (int bt = 0; bt < PR / 4 / POST_BATCH; ++bt) {
    const int lr0 = wave * (PR / 4) + bt * POST_BATCH;
    // loads of the whole batch first (rows clamped into the buffers);
    // rope lanes also take cos/sin columns pr (even element) and half + pr
    // (odd element) of their pairs
    // (CPL / 2 consecutive bf16 columns per load: [0] cos pr, [1] cos half+pr,
    // [2] sin pr, [3] sin half+pr)
    float y[POST_BATCH][CPL];
    RopeCols<CPL / 2> rt[POST_BATCH][4];
#pragma unroll
    for (int q = 0; q < POST_BATCH; ++q) {
      const int rr = min(row_base + lr0 + q, out_rows - 1);
      const float* src = pooled + (size_t)rr * D + c0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[q][i] = src[i];
      if (rope_lane) {
        const uint16_t* cr = cosv + (size_t)rr * cf.rope + pr0;
        const uint16_t* sr = sinv + (size_t)rr * cf.rope + pr0;
        rt[q][0] = *reinterpret_cast<const RopeCols<CPL / 2>*>(cr);
        rt[q][1] = *reinterpret_cast<const RopeCols<CPL / 2>*>(cr + half);
        rt[q][2] = *reinterpret_cast<const RopeCols<CPL / 2>*>(sr);
        rt[q][3] = *reinterpret_cast<const RopeCols<CPL / 2>*>(sr + half);
      }
    }
    bool live[POST_BATCH];
    float ss[POST_BATCH];
#pragma unroll
    for (int q = 0; q < POST_BATCH; ++q) {
      const int info = row_info[lr0 + q];
      live[q] = (info & 1) != 0;
      if (info & 2) {
        // a window split between two GEMM tiles: first channel set from the
        // previous tile, second set from this one
        const int mt = info >> 2;
        const float* pa = split + (size_t)(mt - 1) * 6 * D + c0;
        const float* pb = split + (size_t)mt * 6 * D + 3 * D + c0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          float ma = pa[i], la = pa[D + i], xa = pa[2 * D + i];
          float mb = pb[i], lb = pb[D + i], xb = pb[2 * D + i];
          if (la == 0.f) { ma = mb; }
          if (lb == 0.f) { mb = ma; }
          const float mn = fmaxf(ma, mb);
          const float sa = la == 0.f ? 0.f : __expf(ma - mn), sb = lb == 0.f ? 0.f : __expf(mb - mn);
          const float l = la * sa + lb * sb;
          y[q][i] = l > 0.f ? (xa * sa + xb * sb) / l : 0.f;
        }
      }
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        if (!live[q]) y[q][i] = 0.f;
        acc += y[q][i] * y[q][i];
      }
      ss[q] = acc;
    }
#pragma unroll
    for (int q = 0; q < POST_BATCH; ++q) {
      ss[q] += lane_xor<32>(ss[q]);
      ss[q] += lane_xor<16>(ss[q]);
      ss[q] += lane_xor<8>(ss[q]);
      ss[q] += lane_xor<4>(ss[q]);
      ss[q] += lane_xor<2>(ss[q]);
      ss[q] += lane_xor<1>(ss[q]);
    }
#pragma unroll
    for (int q = 0; q < POST_BATCH; ++q) {
      const int lr = lr0 + q;
      const float inv = rsqrtf(ss[q] / float(D) + kRmsEps);
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[q][i] = y[q][i] * inv * g[i];
      if (rope_lane) {
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
          const float e = y[q][i], o = y[q][i + 1];
          y[q][i] = e * bf2f(rt[q][0].v[i / 2]) - o * bf2f(rt[q][2].v[i / 2]);
          y[q][i + 1] = o * bf2f(rt[q][1].v[i / 2]) + e * bf2f(rt[q][3].v[i / 2]);
        }
      }
      if (fwht) {
        // y . Had = Had[0][0] * WHT(y): butterflies over channel bit b, bits
        // below log2(CPL) inside the lane, the others against lane ^ 2^j
#pragma unroll
        for (int h = 1; h < CPL; h <<= 1)
#pragma unroll
          for (int i = 0; i < CPL; ++i)
            if ((i & h) == 0) {
              const float a = y[q][i], b = y[q][i + h];
              y[q][i] = a + b;
              y[q][i + h] = a - b;
            }
        fwht_lanes<1>(y[q], lane);
        fwht_lanes<2>(y[q], lane);
        fwht_lanes<4>(y[q], lane);
        fwht_lanes<8>(y[q], lane);
        fwht_lanes<16>(y[q], lane);
        fwht_lanes<32>(y[q], lane);
#pragma unroll
        for (int i = 0; i < CPL; ++i) y[q][i] *= hscale;
      }
      uint32_t pk[CPL / 2];
#pragma unroll
      for (int i = 0; i < CPL; i += 2) pk[i / 2] = live[q] ? pack_bf2(y[q][i], y[q][i + 1]) : 0u;
      if (cf.rotate && !fwht) {
        if constexpr (CPL == 8)
          *reinterpret_cast<uint4*>(smem + post_lds<D>(lr, lane)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        else
          *reinterpret_cast<uint32_t*>(smem + post_lds<D>(lr, lane >> 2) + (lane & 3) * 4) = pk[0];
        if (lane == 0) row_live[lr] = live[q];
      } else if (row_base + lr < out_rows) {
        uint16_t* dst = out + (size_t)(row_base + lr) * D + c0;
        if constexpr (CPL == 8)
          *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        else
          *reinterpret_cast<uint32_t*>(dst) = pk[0];
      }
    }
  }
  if (!cf.rotate || fwht) return;
  __syncthreads();

  // out[PR, D] = Y . Had (one 32-row MFMA block; with PR = 16 its rows 16 ..
  // 31 read LDS that no row of this workgroup filled and are not stored,
  // and rows of the product do not mix); wave w owns output columns [w*D/4,
  // (w+1)*D/4), walked one 32-column block at a time (few accumulators live:
  // the kernel's register demand sets how many waves share a SIMD on every
  // path).  The tile is only read, so each block's rows go straight out: 32
  // lanes write 64 contiguous bytes of one row per store.
  constexpr int RB = POST_ROWS / 32;        // 32-row blocks of the LDS tile
  constexpr int NB = D / 128;               // 32-column blocks per wave
  constexpr int KS = D / 16;                // k-steps
  constexpr int PF = KS < 4 ? KS : 4;       // k-steps of Had fragments in flight
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int cb0 = wave * NB;
#pragma unroll 1
  for (int j = 0; j < NB; ++j) {
    const uint16_t* hsrc = hadF + ((size_t)(cb0 + j) * KS * 64 + lane) * 8;   // fragment (cb, 0)
    f32x16 acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    bf16x8 bq[PF];
#pragma unroll
    for (int pf = 0; pf < PF; ++pf) bq[pf] = *reinterpret_cast<const bf16x8*>(hsrc + (size_t)pf * 512);
    static_assert(KS % PF == 0, "k-steps in whole prefetch rounds");
#pragma unroll 1
    for (int k0 = 0; k0 < KS; k0 += PF) {
#pragma unroll
      for (int pf = 0; pf < PF; ++pf) {
        const int kk = k0 + pf;
        const int ch = kk * 2 + lhalf;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + post_lds<D>(i * 32 + lrow, ch));
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[pf], acc[i], 0, 0, 0);
        }
        if (kk + PF < KS) bq[pf] = *reinterpret_cast<const bf16x8*>(hsrc + (size_t)(kk + PF) * 512);
      }
    }
    // element r of block i is tile row i*32 + 8*(r/4) + 4*lhalf + r%4
    const int col = (cb0 + j) * 32 + lrow;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        const int row = row_base + lr;
        if (lr < PR && row < out_rows)
          out[(size_t)row * D + col] = row_live[lr] ? f2bf(acc[i][r]) : uint16_t(0);
      }
  }
}

// Had (D x D bf16, row k, column n) in the fragment-major order of the MFMA B
// operand: fragment (column block cb, k-step kk) is 64 lanes x 8 values, lane
// l holding column cb*32 + l%32 and rows kk*16 + 8*(l/32) .. +8.  One thread
// per lane piece; D*D/8 pieces, 256 per workgroup.  The same pass checks
// whether Had is the Sylvester matrix times a constant, Had[k][n] =
// Had[0][0] * (-1)^popcount(k & n) bit for bit, with Had[0][0] finite and
// non-zero: workgroup `wg` writes flag[wg] = 1 if its pieces hold any other
// value, else 0, and post_kernel multiplies by the matrix instead of running
// the fast transform when any flag is set.
__device__ __forceinline__ void hadamard_pack_block(int wg, const uint16_t* __restrict__ had,
                                                    uint16_t* __restrict__ hadF, int D,
                                                    uint32_t* __restrict__ had_flags) {
  __shared__ int any_general;
  if (threadIdx.x == 0) any_general = 0;
  __syncthreads();
  const int o = wg * 256 + threadIdx.x;
  const int lane = o & 63, f = o >> 6;
  const int ks = D / 16;
  const int cb = f / ks, kk = f - cb * ks;
  const int n = cb * 32 + (lane & 31), k0 = kk * 16 + 8 * (lane >> 5);
  const uint32_t h00 = had[0];
  bool sylvester = (h00 & 0x7FFFu) != 0 && (h00 & 0x7F80u) != 0x7F80u;
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = had[(size_t)(k0 + e) * D + n];
    const uint32_t want = (__popc((uint32_t)((k0 + e) & n)) & 1) ? (h00 ^ 0x8000u) : h00;
    sylvester = sylvester && v[e] == want;
  }
  *reinterpret_cast<uint4*>(hadF + (size_t)o * 8) =
      make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  if (!sylvester) any_general = 1;
  __syncthreads();
  if (threadIdx.x == 0) had_flags[wg] = any_general ? 1u : 0u;
}

// Staging of ring row j of request b: position p = first_b + j, when
// 0 <= p < s_b, into row j of the request's staging area (kv row of coff*D,
// then the score row).  A table entry outside the pool skips the row; the
// GEMM reports it (its first tile of the request checks the same entries).
__device__ __forceinline__ void prefix_block(const Cfg& cf, int j, int b, int B, int T,
                                             const int32_t* __restrict__ cu_seqlens,
                                             const int32_t* __restrict__ seqused,
                                             const int32_t* __restrict__ start_pos,
                                             const float* __restrict__ kv_state,
                                             const float* __restrict__ score_state,
                                             const int32_t* __restrict__ kv_tab,
                                             const int32_t* __restrict__ st_tab,
                                             float* __restrict__ staging) {
  const PReq q = prefill_request(b, B, T, cu_seqlens, seqused, start_pos);
  const int p = prefill_first(q.s, cf.ratio, cf.coff) + j;
  if (q.n == 0 || p < 0 || p >= q.s) return;
  const int cD = cf.coff * cf.D;
  long rk, rs;
  if (!state_row(cf, kv_tab, b, p, &rk) || !state_row(cf, st_tab, b, p, &rs)) return;
  float* dst = staging + ((size_t)b * cf.coff * cf.ratio + j) * 2 * cD;
  for (int i = threadIdx.x; i < cD; i += blockDim.x) {
    dst[i] = kv_state[rk * cD + i];
    dst[cD + i] = score_state[rs * cD + i];
  }
}

// The setup launch: workgroup 0 plans, workgroups [1, 1 + nhad) pack the
// Hadamard matrix (nhad = 0 without rotate), the rest stage ring rows,
// coff*r per request.
// Slots 4j .. 4j+3 of Ape (fp32 [ratio, coff*D], coff = 1 here) into
// apet[c][4j .. 4j+3] for every channel c.
__device__ __forceinline__ void ape_transpose_block(const Cfg& cf, int j, const float* __restrict__ ape,
                                                    float* __restrict__ apet) {
  const int cD = cf.coff * cf.D;
  for (int c = threadIdx.x; c < cD; c += SETUP_THREADS) {
    float4 v;
    v.x = ape[(size_t)(4 * j + 0) * cD + c];
    v.y = ape[(size_t)(4 * j + 1) * cD + c];
    v.z = ape[(size_t)(4 * j + 2) * cD + c];
    v.w = ape[(size_t)(4 * j + 3) * cD + c];
    *reinterpret_cast<float4*>(apet + (size_t)c * cf.ratio + 4 * j) = v;
  }
}

__global__ __launch_bounds__(SETUP_THREADS) void setup_kernel(
    Cfg cf, const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, int B, int T, int out_rows,
    int32_t* __restrict__ plan, int32_t* __restrict__ tile_count, uint32_t* __restrict__ err,
    const uint16_t* __restrict__ had, uint16_t* __restrict__ hadF,
    uint32_t* __restrict__ had_flags, int nhad, const float* __restrict__ ape,
    float* __restrict__ apet, int napet, const float* __restrict__ kv_state,
    const float* __restrict__ score_state, const int32_t* __restrict__ kv_tab,
    const int32_t* __restrict__ st_tab, float* __restrict__ staging) {
  const int g = blockIdx.x;
  if (g == 0) {
    plan_block(cu_seqlens, seqused, start_pos, B, T, cf.ratio, cf.coff, cf.bm, out_rows, plan,
               tile_count, err);
  } else if (g <= nhad) {
    hadamard_pack_block(g - 1, had, hadF, cf.D, had_flags);
  } else if (g <= nhad + napet) {
    ape_transpose_block(cf, g - 1 - nhad, ape, apet);
  } else {
    const int i = g - 1 - nhad - napet, per = cf.coff * cf.ratio;
    prefix_block(cf, i % per, i / per, B, T, cu_seqlens, seqused, start_pos, kv_state,
                 score_state, kv_tab, st_tab, staging);
  }
}

// ---------------------------------------------------------------------------
// Weight packing and pool fills.
// ---------------------------------------------------------------------------
// Column n of the panel projects one wkv / wgate row (order of packed_col);
// its K values are scattered into the fragment-major layout of panel_offset
// in 16-byte pieces (8 consecutive K values stay together).
__global__ __launch_bounds__(256) void pack_weights_kernel(Cfg cf, const uint16_t* __restrict__ wkv,
                                                          const uint16_t* __restrict__ wgate,
                                                          uint16_t* __restrict__ wp) {
  const int n = blockIdx.x;
  const int nv = 2 * cf.coff, cpg = 128 / nv;
  const int g = n >> 7, q = (n & 127) >> 5, i = n & 31;
  const int v = q % nv, sub = q / nv;
  const int c = g * cpg + sub * 32 + i;
  const bool is_score = v >= cf.coff;
  const int cs = is_score ? v - cf.coff : v;
  const uint16_t* src = (is_score ? wgate : wkv) + (size_t)(cs * cf.D + c) * cf.H;
  for (int k = threadIdx.x * 8; k < cf.H; k += blockDim.x * 8)
    *reinterpret_cast<uint4*>(wp + panel_offset(n, k, cf.H)) =
        *reinterpret_cast<const uint4*>(src + k);
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, long n, float v) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = v;
}

// Refill the ring blocks named by table rows rows[0..n): kv 0, score -inf.
// Workgroup (j, i) refills entry j of table row rows[i]; a row index outside
// [0, table_rows) or an entry outside [0, num_blocks) is skipped and reported.
__global__ __launch_bounds__(256) void reset_rows_kernel(Cfg cf, float* __restrict__ kv_state,
                                                        float* __restrict__ score_state,
                                                        const int32_t* __restrict__ kv_tab,
                                                        const int32_t* __restrict__ st_tab,
                                                        const int32_t* __restrict__ rows,
                                                        int table_rows, uint32_t* __restrict__ err) {
  const int rb = rows[blockIdx.y];
  const int j = blockIdx.x;
  if (rb < 0 || rb >= table_rows) {
    if (j == 0 && threadIdx.x == 0 && err) atomicOr(err, CMP_DEVERR_TABLE);
    return;
  }
  const int kb = kv_tab[(long)rb * cf.stride + j], sb = st_tab[(long)rb * cf.stride + j];
  const bool kok = kb >= 0 && kb < cf.nblocks, sok = sb >= 0 && sb < cf.nblocks;
  if ((!kok || !sok) && threadIdx.x == 0 && err) atomicOr(err, CMP_DEVERR_TABLE);
  const long blk = (long)cf.bs * cf.coff * cf.D;
  if (kok)
    for (long i = threadIdx.x; i < blk; i += blockDim.x) kv_state[kb * blk + i] = 0.f;
  if (sok)
    for (long i = threadIdx.x; i < blk; i += blockDim.x) score_state[sb * blk + i] = -INFINITY;
}

}  // namespace cmp
