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

// One run of U k16-steps: every weight and x fragment of the run is loaded
// before the first MFMA of the run, so a wave keeps U * (1 + NRB) 16-byte
// loads per lane in flight (the scheduler is fenced so it cannot interleave
// them with the MFMAs to save registers).
template <int U, int NRB>
__device__ __forceinline__ void gemv_run(const uint16_t* __restrict__ wp,
                                         const uint16_t* const* __restrict__ xp, int s,
                                         f32x16* acc) {
  bf16x8 wf[U], xf[NRB][U];
#pragma unroll
  for (int u = 0; u < U; ++u) wf[u] = *reinterpret_cast<const bf16x8*>(wp + (s + u) * 512);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int u = 0; u < U; ++u) xf[rb][u] = *reinterpret_cast<const bf16x8*>(xp[rb] + (s + u) * 16);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[rb][u], wf[u], acc[rb], 0, 0, 0);
}

template <int NRB>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ partial,
    int B, int N, int K, int steps_per_wave, uint32_t* __restrict__ err) {
  __shared__ float red[4][NRB * 16][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *err = 0;   // this call's error word
  const int i = lane & 31, h = lane >> 5;
  const int kstep0 = (blockIdx.y * 4 + wave) * steps_per_wave;
  const int kbeg = kstep0 * 16 + h * 8;
  // fragment (column block blockIdx.x, k-step kstep0 + u) is 1 KiB contiguous
  const uint16_t* wp = W + (((size_t)blockIdx.x * (K >> 4) + kstep0) * 64 + lane) * 8;
  const uint16_t* xp[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) xp[rb] = X + (size_t)min(rb * 32 + i, B - 1) * K + kbeg;

  f32x16 acc[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[rb][r] = 0.f;

  int s = 0;
  for (; s + 16 <= steps_per_wave; s += 16) gemv_run<16, NRB>(wp, xp, s, acc);
  if (s < steps_per_wave) gemv_run<8, NRB>(wp, xp, s, acc);
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
// Decode tail: one workgroup per request b, thread c owns channel c.
//  1. the token's kv and score of channel c in every channel set: the K-range
//     partials summed in a fixed order, Ape added to the score of position
//     s = start_pos[b];
//  2. if the token completes window w = (s+1)/r - 1: pool the window's slots
//     ([PyPTO] 压缩窗口与状态更新; [CANN] 计算公式 steps 3-5) - the token
//     itself from step 1, earlier positions from the state ring, negative
//     positions as padding - then RMSNorm, RoPE on the last 64 channels and
//     the optional Hadamard product, stored to output row o_b; otherwise
//     output row o_b is +0 ([PyPTO] 返回值说明);
//  3. store the token's kv / score into ring slot s mod (coff*r) unless a
//     C128A window just closed (no later window pools it).  That slot is never
//     one the window reads, so reads and the write do not race.
// Workgroup B zero-fills the rows after the last request's.
// ---------------------------------------------------------------------------
constexpr int TL_THREADS = 512;

template <int R, int COFF>
__global__ __launch_bounds__(TL_THREADS) void decode_tail_kernel(
    Cfg cf, const float* __restrict__ partial, int KS, int B, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, const float* __restrict__ ape,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ had, uint16_t* __restrict__ out,
    int out_rows, uint32_t* __restrict__ err) {
  __shared__ float red[TL_THREADS / 64];
  __shared__ float yv[512];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int D = cf.D, cD = COFF * D;

  // block-wide sum (every thread of the workgroup must call it)
  auto block_sum = [&](float v) -> float {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < TL_THREADS / 64; ++q) t += red[q];
    return t;
  };
  // output rows used by requests [0, upto): each carries at most one token
  auto rows_before = [&](int upto) -> int {
    if (!seqused) return upto;
    float cnt = 0.f;
    for (int j = tid; j < upto; j += TL_THREADS) cnt += (seqused[j] == 1) ? 1.f : 0.f;
    return int(block_sum(cnt));
  };

  if (blockIdx.x == B) {                         // rows after the last request's
    const int total = rows_before(B);
    if (total > out_rows && tid == 0) set_error(err, CMP_DEVERR_OUT_ROWS);
    for (long i = (long)total * D + tid; i < (long)out_rows * D; i += TL_THREADS) out[i] = 0;
    return;
  }
  const int b = blockIdx.x;
  int n = seqused ? seqused[b] : 1;
  int s = start_pos ? start_pos[b] : 0;
  uint32_t bad = 0;
  if (n < 0 || n > 1) { bad |= CMP_DEVERR_SEQLEN; n = 0; }
  if (s < 0 || s == 0x7fffffff) { bad |= CMP_DEVERR_START_POS; n = 0; s = 0; }
  const int o = rows_before(b);
  if (bad && tid == 0) set_error(err, bad);
  if (n == 0) return;
  if (o >= out_rows) {
    if (tid == 0) set_error(err, CMP_DEVERR_OUT_ROWS);
    return;
  }
  const int e = s + 1;
  const bool completing = (e % R) == 0;
  const int c = tid;
  const bool own = c < D;

  // 1. the token's projected values of channel c
  float kvc[COFF], zc[COFF];
#pragma unroll
  for (int cs = 0; cs < COFF; ++cs) { kvc[cs] = 0.f; zc[cs] = 0.f; }
  if (own) {
    const float* pb = partial + (size_t)b * cf.N;
    const size_t kstride = (size_t)B * cf.N;
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) {
      const int ck = packed_col(0, cs, c, COFF), cz = packed_col(1, cs, c, COFF);
      for (int ks = 0; ks < KS; ++ks) {
        kvc[cs] += pb[ks * kstride + ck];
        zc[cs] += pb[ks * kstride + cz];
      }
      zc[cs] += ape[(long)(s % R) * cD + cs * D + c];
    }
  }
  uint32_t tbad = 0;

  if (completing) {
    // 2. pooling of channel c over the window's slots
    float pooled = 0.f;
    if (own) {
      const int w = e / R - 1;
      float m = -INFINITY, l = 0.f, a = 0.f;
#pragma unroll 8
      for (int j = 0; j < COFF * R; ++j) {
        const int cs = (COFF == 2) ? (j >= R) : 0;
        const int p = (COFF == 2) ? (w - 1 + cs) * R + (j - cs * R) : w * R + j;
        if (p < 0) continue;
        float kv, z;
        if (p == s) {
          kv = kvc[cs];
          z = zc[cs];
        } else {
          long rk, rs;
          if (!state_row(cf, kv_tab, b, p, &rk) || !state_row(cf, st_tab, b, p, &rs)) {
            tbad |= CMP_DEVERR_TABLE;
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
      pooled = l > 0.f ? a / l : 0.f;
    }
    // RMSNorm over the D channels
    const float ss = block_sum(own ? pooled * pooled : 0.f);
    const float inv = rsqrtf(ss / float(D) + kRmsEps);
    float y = own ? pooled * inv * bf2f(gamma[c < D ? c : 0]) : 0.f;
    // RoPE: pair (2i, 2i+1) of the trailing rope slice, partner via lane ^ 1
    const float partner = __shfl_xor(y, 1, 64);
    const int rope0 = D - cf.rope;
    if (own && c >= rope0) {
      const int pr = (c - rope0) >> 1, half = cf.rope / 2;
      const uint16_t* cr = cosv + (size_t)o * cf.rope;
      const uint16_t* sr = sinv + (size_t)o * cf.rope;
      y = (c & 1) == 0 ? y * bf2f(cr[pr]) - partner * bf2f(sr[pr])
                       : y * bf2f(cr[half + pr]) + partner * bf2f(sr[half + pr]);
    }
    uint16_t* orow = out + (size_t)o * D;
    if (!cf.rotate) {
      if (own) orow[c] = f2bf(y);
    } else {
      if (own) yv[c] = y;
      __syncthreads();
      if (own) {
        float acc = 0.f;
#pragma unroll 8
        for (int i2 = 0; i2 < D; ++i2) acc += yv[i2] * bf2f(had[(size_t)i2 * D + c]);
        orow[c] = f2bf(acc);
      }
    }
  } else if (own) {
    out[(size_t)o * D + c] = 0;
  }

  // 3. the token's state row
  const int lo = max(s, R * (e / R) - (COFF - 1) * R);
  if (own && lo <= s) {
    long rk, rs;
    const bool okk = state_row(cf, kv_tab, b, s, &rk);
    const bool oks = state_row(cf, st_tab, b, s, &rs);
    if (okk && oks) {
#pragma unroll
      for (int cs = 0; cs < COFF; ++cs) {
        kv_state[rk * cD + cs * D + c] = kvc[cs];
        score_state[rs * cD + cs * D + c] = zc[cs];
      }
    } else {
      tbad |= CMP_DEVERR_TABLE;
    }
  }
  if (tbad) set_error(err, tbad);
}

}  // namespace cmp
