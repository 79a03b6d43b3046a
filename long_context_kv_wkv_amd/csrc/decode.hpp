// Decode kernels: one token per request.
//
// The projection of B <= 64 tokens streams the whole weight panel from HBM
// once, so it is bound by HBM bandwidth, not by the matrix cores.  It is split
// over output columns and K so that every CU streams its own slice: a
// workgroup owns 32 panel columns and one K range that its 4 waves divide;
// each wave multiplies its x fragments (rows = tokens) by the weight
// fragments it loads straight from HBM with the 32x32x16 bf16 MFMA.  The 4
// waves reduce through LDS and the workgroup writes one fp32 partial per K
// range; the tail kernel sums the K ranges in a fixed order (deterministic).
//
// The Triton-Ascend article (性能优化 / Decode) made the same observation for
// its hardware: decode must split along output columns and use a larger K
// step per loop so that more cores take part.
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GV_THREADS = 256;

template <int NRB>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ partial,
    int B, int N, int K, int steps_per_wave, int32_t* __restrict__ counters, int ncounters,
    uint32_t* __restrict__ err) {
  __shared__ float red[4][NRB * 16][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    // this call's error word and the tail kernel's arrival counters
    for (int i = tid; i < ncounters; i += GV_THREADS) counters[i] = 0;
    if (tid == 0) *err = 0;
  }
  const int i = lane & 31, h = lane >> 5;
  const int n = blockIdx.x * 32 + i;
  const int kbeg = (blockIdx.y * 4 + wave) * steps_per_wave * 16 + h * 8;
  const uint16_t* wp = W + (size_t)n * K + kbeg;
  const uint16_t* xp[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) xp[rb] = X + (size_t)min(rb * 32 + i, B - 1) * K + kbeg;

  f32x16 acc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[rb][r] = 0.f;

  for (int s = 0; s < steps_per_wave; s += 8) {
    bf16x8 wf[8], xf[NRB][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) wf[u] = *reinterpret_cast<const bf16x8*>(wp + (s + u) * 16);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int u = 0; u < 8; ++u) xf[rb][u] = *reinterpret_cast<const bf16x8*>(xp[rb] + (s + u) * 16);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[rb][u], wf[u], acc[rb], 0, 0, 0);
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][rb * 16 + r][lane] = acc[rb][r];
  __syncthreads();
  // fixed-order sum of the 4 waves; element (reg, lane) -> (row, column)
  for (int e = tid; e < NRB * 16 * 64; e += GV_THREADS) {
    const int reg = e >> 6, ln = e & 63;
    const float v = red[0][reg][ln] + red[1][reg][ln] + red[2][reg][ln] + red[3][reg][ln];
    const int rb = reg >> 4, r = reg & 15;
    const int row = rb * 32 + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
    const int col = blockIdx.x * 32 + (ln & 31);
    if (row < B) partial[((size_t)blockIdx.y * B + row) * N + col] = v;
  }
}

// ---------------------------------------------------------------------------
// Decode tail.  Workgroup (b, slice) handles 64 channels of request b:
//  1. sums the K-range partials of its columns (fixed order) and adds Ape to
//     the scores of the token at position s = start_pos[b];
//  2. if the token completes window w = (s+1)/r - 1, pools the window's slots
//     for its channels: the token itself from step 1, earlier positions from
//     the state ring, negative positions as padding ([PyPTO]
//     压缩窗口与状态更新; [CANN] 计算公式) - the 4 waves split the slots and
//     merge their running (max, sum, weighted sum) in a fixed order;
//  3. stores the token's kv / score rows into ring slot s mod (coff*r) when
//     the token is still needed (every case but a completed C128A window);
//     the slot written is never one the window reads;
//  4. the last workgroup of request b to arrive (atomic counter, release /
//     acquire fences) runs RMSNorm, RoPE and the optional Hadamard product on
//     the whole row and writes output row o_b (or +0 when no window closes).
// Workgroup B * D/64 zero-fills the rows after the last request's.
// ---------------------------------------------------------------------------
constexpr int TL_THREADS = 256;

__global__ __launch_bounds__(TL_THREADS) void decode_tail_kernel(
    Cfg cf, const float* __restrict__ partial, int KS, int B, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, const float* __restrict__ ape,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ had, uint16_t* __restrict__ out,
    int out_rows, float* __restrict__ pooled, int32_t* __restrict__ counters,
    uint32_t* __restrict__ err) {
  __shared__ float cur[2][2][64];          // [kv | score][set][channel]
  __shared__ float mer[4][3][64];          // per-wave (max, sum, weighted sum)
  __shared__ float yv[512];
  __shared__ float red[TL_THREADS / 64];
  __shared__ int s_flag, s_o;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int D = cf.D, r = cf.ratio, coff = cf.coff, cD = coff * D;
  const int nslices = D / 64;

  auto count_before = [&](int upto) -> int {   // sum of n_b' for b' < upto
    int acc = 0;
    if (!seqused) return upto;
    for (int j = tid; j < upto; j += TL_THREADS) {
      const int v = seqused[j];
      acc += (v == 1) ? 1 : 0;
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    __syncthreads();
    if (lane == 0) red[wave] = float(acc);
    __syncthreads();
    int tot = 0;
    for (int w = 0; w < TL_THREADS / 64; ++w) tot += int(red[w]);
    __syncthreads();
    return tot;
  };

  if (blockIdx.x == B * nslices) {              // rows after the last request's
    const int total = count_before(B);
    if (total > out_rows && tid == 0) set_error(err, CMP_DEVERR_OUT_ROWS);
    for (long i = (long)total * D + tid; i < (long)out_rows * D; i += TL_THREADS) out[i] = 0;
    return;
  }
  const int b = blockIdx.x / nslices, slice = blockIdx.x - b * nslices;
  const int c = slice * 64 + lane;
  int n = seqused ? seqused[b] : 1;
  int s = start_pos ? start_pos[b] : 0;
  uint32_t bad = 0;
  if (n < 0 || n > 1) { bad |= CMP_DEVERR_SEQLEN; n = 0; }
  if (s < 0 || s == 0x7fffffff) { bad |= CMP_DEVERR_START_POS; n = 0; s = 0; }

  // 1. the token's projected row for this slice
  if (n && tid < 2 * coff * 64) {
    const int v = tid >> 6;
    const int is_score = v >= coff, cs = is_score ? v - coff : v;
    const int col = packed_col(is_score, cs, c, coff);
    float sum = 0.f;
    for (int ks = 0; ks < KS; ++ks) sum += partial[((size_t)ks * B + b) * cf.N + col];
    if (is_score) sum += ape[(long)(s % r) * cD + cs * D + c];
    cur[is_score][cs][lane] = sum;
  }
  __syncthreads();
  const int e = s + n;
  const bool completing = n && (e % r == 0);

  // 2. pooling of this slice
  if (completing) {
    const int w = e / r - 1;
    float m = -INFINITY, l = 0.f, a = 0.f;
    for (int j = wave; j < coff * r; j += 4) {
      const int cs = (coff == 2) ? (j >= r) : 0;
      const int p = (coff == 2) ? (w - 1 + cs) * r + (j - cs * r) : w * r + j;
      if (p < 0) continue;
      float kv, z;
      if (p == s) { kv = cur[0][cs][lane]; z = cur[1][cs][lane]; }
      else {
        long rk, rs;
        if (!state_row(cf, kv_tab, b, p, &rk) || !state_row(cf, st_tab, b, p, &rs)) {
          bad |= CMP_DEVERR_TABLE;
          continue;
        }
        kv = kv_state[rk * cD + cs * D + c];
        z = score_state[rs * cD + cs * D + c];
      }
      if (z == -INFINITY) continue;
      const float mn = fmaxf(m, z);
      const float sc = __expf(m - mn), pe = __expf(z - mn);
      l = l * sc + pe;
      a = a * sc + pe * kv;
      m = mn;
    }
    mer[wave][0][lane] = m;
    mer[wave][1][lane] = l;
    mer[wave][2][lane] = a;
    __syncthreads();
    if (wave == 0) {
      float M = -INFINITY;
      for (int q = 0; q < 4; ++q) M = fmaxf(M, mer[q][0][lane]);
      float L = 0.f, A = 0.f;
      for (int q = 0; q < 4; ++q) {
        if (mer[q][1][lane] == 0.f) continue;
        const float sc = __expf(mer[q][0][lane] - M);
        L += mer[q][1][lane] * sc;
        A += mer[q][2][lane] * sc;
      }
      pooled[(size_t)b * D + c] = L > 0.f ? A / L : 0.f;
    }
  }

  // 3. state row of the token
  if (n && tid < 2 * coff * 64) {
    const int lo = max(s, r * (e / r) - (coff - 1) * r);
    if (lo <= s) {
      const int v = tid >> 6;
      const int is_score = v >= coff, cs = is_score ? v - coff : v;
      long ri;
      if (state_row(cf, is_score ? st_tab : kv_tab, b, s, &ri))
        (is_score ? score_state : kv_state)[ri * cD + cs * D + c] = cur[is_score][cs][lane];
      else
        bad |= CMP_DEVERR_TABLE;
    }
  }
  if (bad) set_error(err, bad);

  // 4. last arriver of request b finishes the row.  Every thread releases its
  // own stores device-wide before the barrier; the arrival is counted after it.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&counters[b], 1);
    s_flag = (old == nslices - 1);
  }
  __syncthreads();
  if (!s_flag) return;
  __threadfence();                             // acquire the other slices' rows
  const int o = count_before(b);
  if (!n) return;
  if (o >= out_rows) {
    if (tid == 0) set_error(err, CMP_DEVERR_OUT_ROWS);
    return;
  }
  uint16_t* orow = out + (size_t)o * D;
  if (!completing) {
    for (int i = tid; i < D; i += TL_THREADS) orow[i] = 0;
    return;
  }
  // RMSNorm over D channels: thread t owns channels 2t, 2t+1 (t < D/2)
  const bool own = 2 * tid < D;
  float y0 = 0.f, y1 = 0.f;
  if (own) {
    y0 = pooled[(size_t)b * D + 2 * tid];
    y1 = pooled[(size_t)b * D + 2 * tid + 1];
  }
  float ss = y0 * y0 + y1 * y1;
  for (int of = 32; of > 0; of >>= 1) ss += __shfl_xor(ss, of, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = 0.f;
  for (int q = 0; q < TL_THREADS / 64; ++q) ss += red[q];
  const float inv = rsqrtf(ss / float(D) + kRmsEps);
  if (own) {
    const int ch = 2 * tid;
    y0 = y0 * inv * bf2f(gamma[ch]);
    y1 = y1 * inv * bf2f(gamma[ch + 1]);
    const int rope0 = D - cf.rope;
    if (ch >= rope0) {
      const int pr = (ch - rope0) >> 1, half = cf.rope / 2;
      const uint16_t* cr = cosv + (size_t)o * cf.rope;
      const uint16_t* sr = sinv + (size_t)o * cf.rope;
      const float ev = y0, od = y1;
      y0 = ev * bf2f(cr[pr]) - od * bf2f(sr[pr]);
      y1 = od * bf2f(cr[half + pr]) + ev * bf2f(sr[half + pr]);
    }
    if (!cf.rotate) {
      *reinterpret_cast<uint32_t*>(orow + ch) = pack_bf2(y0, y1);
    } else {
      yv[ch] = y0;
      yv[ch + 1] = y1;
    }
  }
  if (!cf.rotate) return;
  __syncthreads();
  // out[j] = sum_i y[i] * Had[i][j]; thread t owns columns 2t, 2t+1
  if (own) {
    float o0 = 0.f, o1 = 0.f;
    for (int i = 0; i < D; ++i) {
      const uint32_t hv = *reinterpret_cast<const uint32_t*>(had + (size_t)i * D + 2 * tid);
      o0 += yv[i] * bf2f(uint16_t(hv & 0xffffu));
      o1 += yv[i] * bf2f(uint16_t(hv >> 16));
    }
    *reinterpret_cast<uint32_t*>(orow + 2 * tid) = pack_bf2(o0, o1);
  }
}

}  // namespace cmp
