// Prefill kernels other than the projection GEMM: request plan, window
// pooling, post-processing (RMSNorm, RoPE, Hadamard), state write-back.
#pragma once
#include "common.hpp"

namespace cmp {

// ---------------------------------------------------------------------------
// Plan: per-request start / length / windows / output rows, computed on the
// device from cu_seqlens, seqused and start_pos (no host synchronisation).
// Also clears the error word of this call.
//   n_b   = seqused[b] (or the slot length)        e_b = s_b + n_b
//   c_b   = floor(e_b / r) - floor(s_b / r)        windows completed here
//   u_b   = ceil(n_b / r)                          output rows owned
//   o_b   = sum_{b' < b} u_b'                      first output row
// Windows complete when (start_pos + i + 1) % ratio == 0 ([PyPTO]
// 数值精度与验证要点), which is what c_b counts.  Rows per request and their
// placement are the output layout documented in compressor.h.
// One workgroup of 1024 threads; B is walked in chunks with a carried offset.
// ---------------------------------------------------------------------------
constexpr int PLAN_THREADS = 1024;

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, int B, int T, int ratio, int coff, int tile_rows,
    int out_rows, int32_t* __restrict__ plan, int32_t* __restrict__ tile_count,
    uint32_t* __restrict__ err) {
  __shared__ int scan[PLAN_THREADS];
  __shared__ int scan2[PLAN_THREADS];
  __shared__ uint32_t s_err;
  __shared__ int s_carry, s_tcarry;
  const int tid = threadIdx.x;
  const int halo = (coff - 1) * ratio;
  if (tid == 0) { s_err = 0; s_carry = 0; s_tcarry = 0; }
  __syncthreads();
  uint32_t my_err = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + tid;
    int s = 0, n = 0, row0 = 0;
    if (b < B) {
      int c0, c1;
      if (cu_seqlens) { c0 = cu_seqlens[b]; c1 = cu_seqlens[b + 1]; }
      else { const int S = T / B; c0 = b * S; c1 = c0 + S; }
      if (c0 < 0 || c1 < c0 || c1 > T) { my_err |= CMP_DEVERR_SEQLEN; c0 = 0; c1 = 0; }
      const int slot = c1 - c0;
      n = seqused ? seqused[b] : slot;
      if (n < 0 || n > slot) { my_err |= CMP_DEVERR_SEQLEN; n = n < 0 ? 0 : slot; }
      s = start_pos ? start_pos[b] : 0;
      if (s < 0 || s > 0x7fffffff - n) { my_err |= CMP_DEVERR_START_POS; s = 0; n = 0; }
      row0 = c0;
    }
    const int u = (n + ratio - 1) / ratio;
    // GEMM tiles: tile_rows positions each from the window start r*floor(s/r)
    // until e is covered; staged state rows start `halo` positions earlier
    const int first = ratio * (s / ratio) - halo;
    const int over = s + n - (first + halo) - tile_rows;
    const int ntile = n == 0 ? 0 : 1 + (over > 0 ? (over + tile_rows - 1) / tile_rows : 0);
    scan[tid] = u;
    scan2[tid] = ntile;
    __syncthreads();
    for (int off = 1; off < PLAN_THREADS; off <<= 1) {     // inclusive scans
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
      rec[PL_ROW0] = row0;
      rec[PL_NWIN] = e / ratio - s / ratio;
      rec[PL_NROWS] = u;
      rec[PL_OUT0] = s_carry + scan[tid] - u;
      rec[PL_FIRST] = first;
      rec[PL_TILE0] = s_tcarry + scan2[tid] - ntile;
      rec[PL_NTILE] = ntile;
    }
    __syncthreads();
    if (tid == PLAN_THREADS - 1) { s_carry += scan[tid]; s_tcarry += scan2[tid]; }
    __syncthreads();
  }
  if (my_err) atomicOr(&s_err, my_err);
  __syncthreads();
  if (tid == 0) {
    uint32_t e = s_err;
    if (s_carry > out_rows) e |= CMP_DEVERR_OUT_ROWS;
    *err = e;                                       // this call's error word
    *tile_count = s_tcarry;
  }
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
// Post-processing of 64 pooled rows per workgroup: RMSNorm (eps 1e-6, fp32,
// times the weight), interleaved RoPE on channels [D-64, D) ([PyPTO]
// 压缩窗口与状态更新 / 算子级辅助函数), then either the bf16 store or, with
// rotate, out = y @ Had as a bf16 MFMA product (K = D) against the
// transposed matrix HadT[n][k] = Had[k][n].  Rows without a window are +0.
// Pairs (2i, 2i+1) of the rotary slice rotate together: the even element with
// cos/sin column i, the odd one with column 32 + i.
// ---------------------------------------------------------------------------
constexpr int POST_ROWS = 64;

template <int CPL>
__global__ __launch_bounds__(256) void post_kernel(
    Cfg cf, const float* __restrict__ pooled, const float* __restrict__ split,
    const int32_t* __restrict__ plan, int B, int out_rows,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ hadT,
    uint16_t* __restrict__ out) {
  constexpr int D = CPL * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // [64][D] bf16, swizzled
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_base = blockIdx.x * POST_ROWS;
  const int c0 = lane * CPL;
  const int rope0 = D - cf.rope;
  float g[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) g[i] = bf2f(gamma[c0 + i]);

  for (int rr = 0; rr < POST_ROWS / 4; ++rr) {
    const int lr = wave * (POST_ROWS / 4) + rr;
    const int row = row_base + lr;
    if (row >= out_rows) break;
    float y[CPL];
    const int rb = find_request(plan, B, row);
    const int32_t* rrec = plan + (long)(rb < 0 ? 0 : rb) * PL_WIDTH;
    const int k = row - rrec[PL_OUT0];
    const bool live = rb >= 0 && k < rrec[PL_NWIN];
    if (live) {
      float ss = 0.f;
      if (cf.coff == 2 && k > 0 && (k & 63) == 0) {
        // a window split between two GEMM tiles: first channel set from the
        // previous tile, second set from this one
        const int mt = rrec[PL_TILE0] + (k >> 6);
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
          y[i] = l > 0.f ? (xa * sa + xb * sb) / l : 0.f;
          ss += y[i] * y[i];
        }
      } else {
        const float* src = pooled + (size_t)row * D + c0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) { y[i] = src[i]; ss += y[i] * y[i]; }
      }
      ss = wave_sum(ss);
      const float inv = rsqrtf(ss / float(D) + kRmsEps);
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[i] = y[i] * inv * g[i];
      if (c0 >= rope0) {
        const uint16_t* cr = cosv + (size_t)row * cf.rope;
        const uint16_t* sr = sinv + (size_t)row * cf.rope;
        const int half = cf.rope / 2;
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
          const int pr = (c0 + i - rope0) >> 1;
          const float e = y[i], o = y[i + 1];
          y[i] = e * bf2f(cr[pr]) - o * bf2f(sr[pr]);
          y[i + 1] = o * bf2f(cr[half + pr]) + e * bf2f(sr[half + pr]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[i] = 0.f;
    }
    if (!cf.rotate) {
      uint16_t* dst = out + (size_t)row * D + c0;
#pragma unroll
      for (int i = 0; i < CPL; i += 2)
        *reinterpret_cast<uint32_t*>(dst + i) = live ? pack_bf2(y[i], y[i + 1]) : 0u;
    } else {
      // LDS tile row lr (D*2 bytes, a multiple of 256): 16-byte chunk ch at
      // ((ch ^ (lr & 15)) * 16), so 16 consecutive rows read at one chunk
      // index hit 16 distinct bank groups
#pragma unroll
      for (int i = 0; i < CPL; i += 2) {
        const int c = c0 + i;
        const int ch = c >> 3, within = c & 7;
        *reinterpret_cast<uint32_t*>(smem + lr * D * 2 + ((ch ^ (lr & 15)) << 4) + within * 2) =
            pack_bf2(y[i], y[i + 1]);
      }
    }
  }
  if (!cf.rotate) return;
  __syncthreads();

  // out[64, D] = Y[64, D] . Had; wave w owns output columns [w*D/4, (w+1)*D/4)
  constexpr int NB = D / 128;               // 32-column blocks per wave
  const int lrow = lane & 31, lhalf = lane >> 5;
  f32x16 acc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nbase = wave * (D / 4);
  for (int kk = 0; kk < D / 16; ++kk) {
    const int ch = kk * 2 + lhalf;
    bf16x8 a[2], bb[NB];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = i * 32 + lrow;
      a[i] = *reinterpret_cast<const bf16x8*>(smem + rr * D * 2 + ((ch ^ (rr & 15)) << 4));
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bb[j] = *reinterpret_cast<const bf16x8*>(hadT + (size_t)(nbase + j * 32 + lrow) * D + ch * 8);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bb[j], acc[i][j], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
      const int row = row_base + lr;
      if (row >= out_rows) continue;
      const bool live = row_has_window(plan, B, row);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int col = nbase + j * 32 + lrow;
        out[(size_t)row * D + col] = live ? f2bf(acc[i][j][r]) : uint16_t(0);
      }
    }
}

// HadT[n][k] = Had[k][n] (D x D bf16), through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             uint16_t* __restrict__ outT, int D) {
  __shared__ uint16_t tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 8 rows per pass
  for (int y = ty; y < 32; y += 8) tile[y][tx] = in[(size_t)(by + y) * D + bx + tx];
  __syncthreads();
  for (int y = ty; y < 32; y += 8) outT[(size_t)(bx + y) * D + by + tx] = tile[tx][y];
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
__global__ __launch_bounds__(256) void reset_rows_kernel(Cfg cf, float* __restrict__ kv_state,
                                                        float* __restrict__ score_state,
                                                        const int32_t* __restrict__ kv_tab,
                                                        const int32_t* __restrict__ st_tab,
                                                        const int32_t* __restrict__ rows) {
  const int rb = rows[blockIdx.y];
  const int used = (cf.coff * cf.ratio + cf.bs - 1) / cf.bs;
  const int j = blockIdx.x;
  if (j >= used) return;
  const int kb = kv_tab[(long)rb * cf.stride + j], sb = st_tab[(long)rb * cf.stride + j];
  const long blk = (long)cf.bs * cf.coff * cf.D;
  if (kb >= 0 && kb < cf.nblocks)
    for (long i = threadIdx.x; i < blk; i += blockDim.x) kv_state[kb * blk + i] = 0.f;
  if (sb >= 0 && sb < cf.nblocks)
    for (long i = threadIdx.x; i < blk; i += blockDim.x) score_state[sb * blk + i] = -INFINITY;
}

}  // namespace cmp
