// Decode kernels: at most 4 tokens per request, at most 64 packed rows.
//
// The projection of B <= 64 tokens streams the whole weight panel from HBM
// once, so it is bound by HBM bandwidth, not by the matrix cores.  It is split
// over output columns and K so that every CU streams its own slice: a
// workgroup owns 32 panel columns (or, for single-row-block calls with two
// channel sets, 64: two column blocks that share the staged x rows) and one
// K range that its 8 waves divide; each wave multiplies its x fragments
// (rows = tokens) by the weight fragments it loads straight from HBM with the
// 32x32x16 bf16 MFMA.  The 8 waves reduce through LDS and the workgroup
// writes one fp32 partial per K range and column; the tail kernel sums the K
// ranges in a fixed order (deterministic).
//
// The K split: the H/16 k-steps are cut into 8 * KS nearly equal wave ranges
// (KS K ranges of 8 waves), so any H that is a multiple of 512 is covered
// whole; KS is chosen for about 512 single-block GEMV workgroups (two per
// CU), or about one pair workgroup per CU, with 4 to 8 k-steps per wave.  All of a wave's loads are issued before its first MFMA:
// with more loads in flight per wave than one round of HBM latency covers,
// a second round per wave only adds its latency (measured: 7 steps per wave
// over 512 workgroups streams the 29 MB C4A panel in 8.5 us of graph time
// against 9.0 us for 8 steps over 448).
//
// The Triton-Ascend article (性能优化 / Decode) made the same observation for
// its hardware: decode must split along output columns and use a larger K
// step per loop so that more cores take part.
#pragma once
#include "common.hpp"

namespace cmp {

constexpr int GV_THREADS = 512;                // 8 waves

typedef __attribute__((address_space(3))) void dec_lds_t;
typedef __attribute__((address_space(1))) void dec_glb_t;

// One run of U k16-steps of a wave, steps s .. s+U-1 of its n (steps at or
// beyond n load step n-1 again and skip their MFMA, so every run issues the
// same number of loads).  The x rows of the run go to the wave's own LDS
// region by direct-to-LDS copies that each cover whole 16-byte-chunk runs of
// rows (a row of the run is U*32 contiguous bytes), then the panel fragments
// of the run are loaded (1 KiB contiguous each, for each of the CBW column
// blocks); once the copies have landed, the x fragments are read from LDS
// and the MFMAs run, each x fragment for all CBW blocks.  Row t, chunk
// c sits at t*U*32 + ((c ^ (t & m)) * 16), m = min(2U, 16) - 1 (the swizzle
// never leaves the row's 2U chunks): the fragment reads (32 rows at one
// chunk index) spread over the banks.  Rows >= B repeat row B-1 (their
// results are not used).  NT: the panel loads carry the non-temporal
// (streaming) hint; every panel byte is read once per call.
template <int U, int NRB, bool NT, int CBW = 1>
__device__ __forceinline__ void gemv_run(const uint16_t* __restrict__ wp, size_t cbstride,
                                         const uint16_t* __restrict__ xk, int K, int B, int s,
                                         int n, uint8_t* xl, f32x16 (*acc)[NRB]) {
  constexpr int CPR = 2 * U;             // 16-byte chunks per row of the run
  constexpr int RPI = 64 / CPR;          // rows per copy instruction
  constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;   // chunk swizzle mask: stays inside the row
  static_assert(U >= 1 && U <= 32 && (U & (U - 1)) == 0, "run length: a power of two");
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < NRB * U; ++j) {
    const int t = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ (t & SWZ);
    const int ks = min(s + (c >> 1), n - 1);
    __builtin_amdgcn_global_load_lds(
        (dec_glb_t*)(xk + (size_t)min(t, B - 1) * K + ks * 16 + (c & 1) * 8),
        (dec_lds_t*)(xl + j * 1024), 16, 0, 0);
  }
  // the run's panel fragments of each of the CBW column blocks (cbstride
  // elements apart)
  bf16x8 wf[CBW][U];
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bf16x8* src =
          reinterpret_cast<const bf16x8*>(wp + cb * cbstride + min(s + u, n - 1) * 512);
      wf[cb][u] = NT ? __builtin_nontemporal_load(src) : *src;
    }
  // the copies were issued first: when only the CBW * U panel loads are
  // outstanding, they have landed
  constexpr int NL = CBW * U;
  __builtin_amdgcn_s_waitcnt((NL & 0xf) | ((NL >> 4) << 14) | 0x0f70);
  __builtin_amdgcn_sched_barrier(0);
  // every MFMA runs (a branch around the steps past n would let the compiler
  // sink their panel loads into it, one round trip at a time); those steps
  // multiply a zero x fragment
  const bf16x8 zero = {};
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int t = rb * 32 + (lane & 31);
      const int c = 2 * u + (lane >> 5);
      bf16x8 xf = *reinterpret_cast<const bf16x8*>(xl + t * CPR * 16 + ((c ^ (t & SWZ)) << 4));
      xf = s + u < n ? xf : zero;
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
        acc[cb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, wf[cb][u], acc[cb][rb], 0, 0, 0);
    }
  }
  // the next run's copies overwrite the region: every read must be done
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
}

// K range [k0, k1) of wave range v of 8 * KS: nearly equal shares of the KT
// k-steps (lengths differ by at most one).
__host__ __device__ __forceinline__ void dec_wave_range(int v, int KS, int KT, int* k0, int* k1) {
  const int nr = 8 * KS;                // v * KT <= 8 * 20 * 640: no overflow
  *k0 = v * KT / nr;
  *k1 = (v + 1) * KT / nr;
}

// ---------------------------------------------------------------------------
// Requests of a decode call: request b owns packed rows [cu[b], cu[b] + n_b)
// of x (cu = cu_seqlens, or one row per request when it is NULL), n_b =
// seqused[b] (or the slot length) tokens at positions s_b .. s_b + n_b - 1,
// with n_b <= DEC_MAX_TOK ([PyPTO] 参数说明: S of a decode call is small).
// Invalid values set an error bit and make the request empty.
// ---------------------------------------------------------------------------
constexpr int DEC_MAX_TOK = 4;
constexpr int DEC_MAX_WIN = 2;               // windows a request completes: <= ceil(4 / 2)

struct DecReq {
  int s, n, row0;
  uint32_t bad;
};
// Checks of request b's fields (cu[b], cu[b + 1], seqused[b], start_pos[b],
// loaded by the caller; absent arrays take their defaults here)
__device__ __forceinline__ DecReq dec_check(int b, int T, bool has_cu, bool has_su, int c0, int c1,
                                            int nu, int s) {
  DecReq q{0, 0, 0, 0u};
  if (!has_cu) { c0 = b; c1 = b + 1; }
  if (c0 < 0 || c1 < c0 || c1 > T) { q.bad |= CMP_DEVERR_SEQLEN; return q; }
  const int n = has_su ? nu : c1 - c0;
  if (n < 0 || n > c1 - c0 || n > DEC_MAX_TOK) { q.bad |= CMP_DEVERR_SEQLEN; return q; }
  if (s < 0 || s > 0x7fffffff - DEC_MAX_TOK) { q.bad |= CMP_DEVERR_START_POS; return q; }
  q.s = s;
  q.n = n;
  q.row0 = c0;
  return q;
}
__device__ __forceinline__ DecReq dec_request(int b, int T, const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ seqused,
                                              const int32_t* __restrict__ start_pos) {
  int c0 = 0, c1 = 0, nu = 0, s = 0;
  if (cu) { c0 = cu[b]; c1 = cu[b + 1]; }
  if (seqused) nu = seqused[b];
  if (start_pos) s = start_pos[b];
  return dec_check(b, T, cu != nullptr, seqused != nullptr, c0, c1, nu, s);
}
// The same for a wave-uniform b: lanes 0-3 load the four fields with one
// vector load, so that they are in flight together (and beside the caller's
// other vector loads) instead of in dependent scalar-cache rounds.
__device__ __forceinline__ DecReq dec_request_wave(int b, int T, const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ seqused,
                                                   const int32_t* __restrict__ start_pos) {
  const int lane = threadIdx.x & 63;
  const int32_t* src = nullptr;
  if (lane == 0 && cu) src = cu + b;
  if (lane == 1 && cu) src = cu + b + 1;
  if (lane == 2 && seqused) src = seqused + b;
  if (lane == 3 && start_pos) src = start_pos + b;
  int v = 0;
  if (src) v = *src;
  return dec_check(b, T, cu != nullptr, seqused != nullptr, __builtin_amdgcn_readlane(v, 0),
                   __builtin_amdgcn_readlane(v, 1), __builtin_amdgcn_readlane(v, 2),
                   __builtin_amdgcn_readlane(v, 3));
}

// Ring pre-pooling: workgroups of the decode main kernel that pool, for each
// window a request completes in this call, the window's slots at positions
// before the call (from the state ring; [PyPTO] 压缩窗口与状态更新; [CANN]
// 计算公式 steps 3-5): per channel the softmax statistics (max m, sum l,
// weighted sum x) of those slots.  None of them depends on this call's
// projection, so they run while the GEMV streams the panel.  A window of
// more than 16 slots is split over workgroups of 16 slots (C128A: 8 of
// them); smaller windows take one.  Workgroup (b, k, sp) handles split sp of
// request b's k-th completed window.
constexpr int DEC_MAX_KSPLIT = 20;           // K ranges of the GEMV (H / 512 at most)
template <int R>
constexpr int dec_split() { return R <= 16 ? 1 : R / 16; }

template <int R, int COFF>
__device__ __forceinline__ void prepool_block(const Cfg& cf, int b, int k, int sp, int T,
                                              const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ seqused,
                                              const int32_t* __restrict__ start_pos,
                                              const float* __restrict__ kv_state,
                                              const float* __restrict__ score_state,
                                              const int32_t* __restrict__ kv_tab,
                                              const int32_t* __restrict__ st_tab,
                                              float* __restrict__ pp, int32_t* __restrict__ ppflag) {
  constexpr int NSPLIT = dec_split<R>();
  constexpr int NS = COFF * R / NSPLIT;          // slots per workgroup
  // one channel set: slot j of any window is ring slot j (the window starts
  // at a multiple of r), so the table entries of the workgroup's slots do
  // not depend on the position.  Lane t < NS loads slot t's entries with a
  // vector load while the request fields come through the scalar cache, so
  // the two are in flight together: one dependent round before the ring
  // reads instead of two (the empty asm keeps the loads ahead of the early
  // return).
  int32_t ekl = 0, esl = 0;
  if constexpr (COFF == 1) {
    const int tl = min((int)(threadIdx.x & 63), NS - 1);
    const long ti = (long)b * cf.stride + (sp * NS + tl) / cf.bs;
    ekl = kv_tab[ti];
    esl = st_tab[ti];
  }
  const DecReq q = dec_request_wave(b, T, cu, seqused, start_pos);
  if constexpr (COFF == 1) asm volatile("" ::"v"(ekl), "v"(esl));
  const int s = q.s, e = q.s + q.n;
  const int w = s / R + k;
  if (q.n == 0 || w >= e / R) return;            // no k-th window in this call
  const int D = cf.D, cD = COFF * D;
  // slot j of the window: C4A j < 4 -> first set of position (w-1)*4 + j,
  // j >= 4 -> second set of position w*4 + j - 4; coff 1 -> position w*R + j
  long rk[NS], rs[NS];
  bool use[NS];
  uint32_t bad = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int j = sp * NS + t;
    const int cs = COFF == 2 ? (j >= R) : 0;
    const int p = COFF == 2 ? (w - 1 + cs) * R + (j - cs * R) : w * R + j;
    use[t] = p >= 0 && p < s;                    // this call's tokens come later
    rk[t] = 0;
    rs[t] = 0;
    bool ok;
    if constexpr (COFF == 1) {
      const int32_t ek = __builtin_amdgcn_readlane(ekl, t), es = __builtin_amdgcn_readlane(esl, t);
      ok = ek >= 0 && ek < cf.nblocks && es >= 0 && es < cf.nblocks;
      rk[t] = (long)ek * cf.bs + j % cf.bs;
      rs[t] = (long)es * cf.bs + j % cf.bs;
    } else {
      ok = !use[t] || (state_row(cf, kv_tab, b, p, &rk[t]) && state_row(cf, st_tab, b, p, &rs[t]));
    }
    if (use[t] && !ok) {
      bad |= CMP_DEVERR_TABLE;
      use[t] = false;
    }
  }
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float kv[NS], z[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int j = sp * NS + t;
      const int cs = COFF == 2 ? (j >= R) : 0;
      kv[t] = use[t] ? kv_state[rk[t] * cD + cs * D + c] : 0.f;
      z[t] = use[t] ? score_state[rs[t] * cD + cs * D + c] : -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < NS; ++t) m = fmaxf(m, z[t]);
    float l = 0.f, x = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        const float ex = __expf(z[t] - m);       // exp(-inf) = 0 for empty slots
        l += ex;
        x = fmaf(ex, kv[t], x);
      }
    }
    float* o = pp + ((size_t)((b * DEC_MAX_WIN + k) * NSPLIT + sp) * 3) * D + c;
    o[0] = m;
    o[D] = l;
    o[2 * D] = x;
  }
  if (threadIdx.x == 0) ppflag[(b * DEC_MAX_WIN + k) * NSPLIT + sp] = (int32_t)bad;
}

// Request record of a single-token call (one row per request), written by
// the main kernel's first workgroup for the tail: start position, output
// row, flags and the ring rows of the token's state.  Record B holds the
// active-request count (s) and the argument-error bits (o).
enum DecRecFlag { DR_ACT = 1, DR_COMP = 2, DR_STORE = 4, DR_ROW_OK = 8 };
struct DecRec {
  int32_t s, o, flags, pad;
  long rk, rs;
};
template <int R, int COFF>
__device__ __forceinline__ void dec_records(const Cfg& cf, int B, const int32_t* __restrict__ seqused,
                                            const int32_t* __restrict__ start_pos,
                                            const int32_t* __restrict__ kv_tab,
                                            const int32_t* __restrict__ st_tab, DecRec* rec) {
  const int b = threadIdx.x;                       // one wave, B <= 64
  const bool in = b < B;
  const int n = in ? (seqused ? seqused[b] : 1) : 0;
  const int s = in && start_pos ? start_pos[b] : 0;
  const bool n_ok = n >= 0 && n <= 1;
  const bool s_ok = s >= 0 && s <= 0x7fffffff - DEC_MAX_TOK;
  const bool act = in && n_ok && s_ok && n == 1;
  const unsigned long long amask = __ballot(act);
  const uint32_t bad = (__ballot(in && !n_ok) ? CMP_DEVERR_SEQLEN : 0u) |
                       (__ballot(in && n_ok && !s_ok) ? CMP_DEVERR_START_POS : 0u);
  if (b == 0) {                                   // record B: count, error bits
    DecRec t;
    t.s = __popcll(amask);
    t.o = (int32_t)bad;
    t.flags = 0;
    t.pad = 0;
    t.rk = 0;
    t.rs = 0;
    rec[B] = t;
  }
  if (!in) return;
  const int e = s + 1;
  // the token's ring row stays live unless the window it closes is the
  // last one the ring needs (coff 1: a completed window is not kept)
  const int lo = max(s, R * (e / R) - (COFF - 1) * R);
  long rk = 0, rs = 0;
  const bool store = act && lo <= s;
  const bool row_ok = store && state_row(cf, kv_tab, b, s, &rk) && state_row(cf, st_tab, b, s, &rs);
  DecRec t;
  t.s = act ? s : 0;
  t.o = __popcll(amask & ((1ull << b) - 1ull));
  t.flags = (act ? DR_ACT : 0) | (act && e % R == 0 ? DR_COMP : 0) | (store ? DR_STORE : 0) |
            (row_ok ? DR_ROW_OK : 0);
  t.pad = 0;
  t.rk = rk;
  t.rs = rs;
  rec[b] = t;
}

// Decode main kernel.  Workgroups [0, B * nwin * split) pre-pool ring windows
// (prepool_block; nwin <= DEC_MAX_WIN is the most windows a request can
// complete in this call); with one row per request (cu NULL) workgroup 0
// also writes the request records.  The rest run the GEMV over the T packed
// rows: workgroup g owns the CBW column blocks from CBW * (g % (N / 32 /
// CBW)) and K range kr = g / (N / 32 / CBW); wave w covers wave range 8 kr + w
// (dec_wave_range) in runs of RUN k-steps, the x rows of a run staged once
// for the CBW blocks; the 8 waves reduce through LDS in a fixed order and
// the workgroup writes one fp32 partial per K range and column.
template <int NRB, int RUN, int R, int COFF, int CBW>
__global__ __launch_bounds__(GV_THREADS) void decode_main_kernel(
    Cfg cf, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
    float* __restrict__ partial, int B, int T, int nwin, int KS,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos,
    const float* __restrict__ kv_state, const float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    float* __restrict__ pp, int32_t* __restrict__ ppflag, DecRec* __restrict__ rec,
    uint32_t* __restrict__ err) {
  // per wave: the x rows of a run, then (after the runs) its accumulators
  static_assert(NRB * 32 * RUN * 32 >= CBW * NRB * 16 * 64 * 4, "the reduction fits the x region");
  __shared__ __attribute__((aligned(1024))) uint8_t xstage[GV_THREADS / 64][NRB * 32 * RUN * 32];
  constexpr int NSPLIT = dec_split<R>();
  const int npre = B * nwin * NSPLIT;
  if ((int)blockIdx.x < npre) {
    const int idx = blockIdx.x;
    if (idx == 0 && cu == nullptr && threadIdx.x < 64)
      dec_records<R, COFF>(cf, B, seqused, start_pos, kv_tab, st_tab, rec);
    prepool_block<R, COFF>(cf, idx / (nwin * NSPLIT), (idx / NSPLIT) % nwin,
                           idx % NSPLIT, T, cu, seqused, start_pos, kv_state, score_state, kv_tab,
                           st_tab, pp, ppflag);
    return;
  }
  const int g = blockIdx.x - npre;
  const int N = cf.N, K = cf.H, KT = K >> 4;
  const int ncg = N / 32 / CBW;                  // groups of CBW column blocks
  const int cb = g % ncg * CBW, kr = g / ncg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches
  if (g == 0 && tid == 0) *err = 0;   // this call's error word (only the tail sets bits)
  if (T == 0) return;
  int k0, k1;
  dec_wave_range(kr * (GV_THREADS / 64) + wave, KS, KT, &k0, &k1);
  const int n = k1 - k0;
  // fragment (column block cb, k-step k0 + u) is 1 KiB contiguous
  const uint16_t* wp = W + (((size_t)cb * KT + k0) * 64 + lane) * 8;
  const uint16_t* xk = X + (size_t)k0 * 16;
  uint8_t* xl = xstage[wave];

  f32x16 acc[CBW][NRB];
#pragma unroll
  for (int c = 0; c < CBW; ++c)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[c][rb][r] = 0.f;

  // the streaming hint on the panel loads: measured per ratio over graph
  // replays of 32-request steps, it saved 0.45-0.8 us per step with two
  // channel sets (ratio 4: one and two tokens per request, with and without
  // emitting requests) and cost 0.5 us at ratio 128 when few requests close
  // a window (the main kernel 6.2 -> 6.7 us in the trace)
  for (int s = 0; s < n; s += RUN)
    gemv_run<RUN, NRB, COFF == 2, CBW>(wp, (size_t)KT * 512, xk, K, T, s, n, xl, acc);
  float* red = reinterpret_cast<float*>(xl);            // [CBW * NRB * 16][64] of this wave
#pragma unroll
  for (int c = 0; c < CBW; ++c)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((c * NRB + rb) * 16 + r) * 64 + lane] = acc[c][rb][r];
  __syncthreads();
  // fixed-order sum of the 8 waves; element (reg, lane) -> (row, column)
  for (int e = tid; e < CBW * NRB * 16 * 64; e += GV_THREADS) {
    const int creg = e >> 6, ln = e & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < GV_THREADS / 64; ++w) v += reinterpret_cast<const float*>(xstage[w])[creg * 64 + ln];
    const int c = creg / (NRB * 16), reg = creg % (NRB * 16);
    const int rb = reg >> 4, r = reg & 15;
    const int row = rb * 32 + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
    const int col = (cb + c) * 32 + (ln & 31);
    if (row < T) partial[((size_t)kr * T + row) * N + col] = v;
  }
}

// ---------------------------------------------------------------------------
// Decode tail: one workgroup per request b, thread c owns channel c.
//  1. the kv and score of channel c of each of the request's n_b tokens in
//     every channel set: the K-range partials summed in a fixed order, Ape
//     added to the score of position p (row p mod r);
//  2. for each window the tokens complete ([PyPTO] 压缩窗口与状态更新; [CANN]
//     计算公式 steps 3-5): the pre-pooled statistics of its slots before the
//     call merged with its slots among this call's tokens, then RMSNorm, RoPE
//     on the last 64 channels and the optional Hadamard product, stored to
//     output row o_b + k; the request's other rows (up to o_b + ceil(n_b/r))
//     are +0 ([PyPTO] 返回值说明);
//  3. the tokens' state rows that stay live ([max(s, r*floor(e/r) -
//     (coff-1)*r), e)) into their ring slots.  The main kernel has finished
//     every read of the ring before this kernel starts.
// Output rows: o_b = sum over earlier requests of ceil(n/r) (one wave-wide
// scan, B <= 64).  Workgroup B zero-fills the rows after the last request's.
// ---------------------------------------------------------------------------
constexpr int TL_THREADS = 512;

// Error bits of the tails: into the call's error word, and into the caller's
// word err2 as well when one is given (the allocation-free entry point)
__device__ __forceinline__ void dec_report(uint32_t* err, uint32_t* err2, uint32_t bits) {
  set_error(err, bits);
  if (err2) set_error(err2, bits);
}

// kv and score (before Ape) of channel c of tokens t0 .. t0 + TC - 1 (packed
// rows row0 + t, t < n), in every channel set: the K-range partials of the
// TC tokens all in flight at once (KSB >= KS ranges each, unconditionally:
// indices past the last token or K range repeat it and are not summed),
// summed in K order.
template <int COFF, int KSB, int TC>
__device__ __forceinline__ void dec_token_values(const float* __restrict__ partial, int row0,
                                                 int t0, int n, int T, int N, int KS, int c,
                                                 float (&kv)[DEC_MAX_TOK][COFF],
                                                 float (&z)[DEC_MAX_TOK][COFF]) {
  const size_t kstride = (size_t)T * N;
  float pk[TC][COFF][KSB], pz[TC][COFF][KSB];
#pragma unroll
  for (int j = 0; j < TC; ++j) {
    const float* pb = partial + (size_t)(row0 + min(t0 + j, n - 1)) * N;
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) {
      const int ck = packed_col(0, cs, c, COFF), cz = packed_col(1, cs, c, COFF);
#pragma unroll
      for (int ks = 0; ks < KSB; ++ks) {
        const size_t kk = (size_t)min(ks, KS - 1) * kstride;
        pk[j][cs][ks] = pb[kk + ck];
        pz[j][cs][ks] = pb[kk + cz];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TC; ++j) {
    if (t0 + j >= DEC_MAX_TOK) break;
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSB; ++ks) {
        a += ks < KS ? pk[j][cs][ks] : 0.f;
        b += ks < KS ? pz[j][cs][ks] : 0.f;
      }
      kv[t0 + j][cs] = a;
      z[t0 + j][cs] = b;
    }
  }
}

template <int R, int COFF, int KSB>
__global__ __launch_bounds__(TL_THREADS) void decode_tail_kernel(
    Cfg cf, const float* __restrict__ partial, int KS, int B, int T,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seqused,
    const int32_t* __restrict__ start_pos, const float* __restrict__ ape,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    const float* __restrict__ pp, const int32_t* __restrict__ ppflag,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ had, uint16_t* __restrict__ out,
    int out_rows, uint32_t* __restrict__ err, uint32_t* __restrict__ err2) {
  constexpr int NSPLIT = dec_split<R>();
  __shared__ float red[TL_THREADS / 64];
  __shared__ float yv[512];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int D = cf.D, cD = COFF * D;
  const int b = blockIdx.x;
  const int c = tid;
  const bool own = c < D && b < B;
  const bool packed = cu != nullptr;

  // loads that need no request record, issued first: with one row per
  // request, token 0's partials (row b); the first window's pre-pooled
  // statistics; the norm weight
  float kvt[DEC_MAX_TOK][COFF], zt[DEC_MAX_TOK][COFF];
#pragma unroll
  for (int t = 0; t < DEC_MAX_TOK; ++t)
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) { kvt[t][cs] = 0.f; zt[t][cs] = 0.f; }
  // tokens whose partials are loaded in one round
  constexpr int TC = (128 / (KSB * 2 * COFF)) < 1 ? 1
                     : ((128 / (KSB * 2 * COFF)) > DEC_MAX_TOK ? DEC_MAX_TOK
                                                                : (128 / (KSB * 2 * COFF)));
  if (own && !packed) dec_token_values<COFF, KSB, 1>(partial, b, 0, 1, T, cf.N, KS, c, kvt, zt);
  float pm0[NSPLIT], pl0[NSPLIT], px0[NSPLIT];
#pragma unroll
  for (int sp = 0; sp < NSPLIT; ++sp) {
    pm0[sp] = -INFINITY;
    pl0[sp] = 0.f;
    px0[sp] = 0.f;
  }
  if (own) {
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp) {
      const float* st = pp + ((size_t)(b * DEC_MAX_WIN * NSPLIT + sp) * 3) * D + c;
      pm0[sp] = st[0];
      pl0[sp] = st[D];
      px0[sp] = st[2 * D];
    }
  }
  const float g = own ? bf2f(gamma[c]) : 0.f;

  // request records (lane j holds request j; B <= 64) and their output rows,
  // scanned across the wave
  DecReq qj{0, 0, 0, 0u};
  if (lane < B) qj = dec_request(lane, T, cu, seqused, start_pos);
  const int u = (qj.n + R - 1) / R;
  int incl = u;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  const int total = __shfl(incl, 63, 64);

  if ((int)blockIdx.x == B) {                    // rows after the last request's
    if (total > out_rows && tid == 0) dec_report(err, err2, CMP_DEVERR_OUT_ROWS);
    for (long i = (long)total * D + tid; i < (long)out_rows * D; i += TL_THREADS) out[i] = 0;
    return;
  }
  // request b's record from lane b
  const int o = __shfl(incl - u, b, 64);         // exclusive prefix of request b
  DecReq q;
  q.s = __shfl(qj.s, b, 64);
  q.n = __shfl(qj.n, b, 64);
  q.row0 = __shfl(qj.row0, b, 64);
  q.bad = (uint32_t)__shfl((int)qj.bad, b, 64);
  if (q.bad && tid == 0) dec_report(err, err2, q.bad);
  const int n = q.n, s = q.s, e = s + n;
  if (n == 0) return;
  const int ub = (n + R - 1) / R;
  if (o + ub > out_rows) {
    if (tid == 0) dec_report(err, err2, CMP_DEVERR_OUT_ROWS);
    return;
  }
  const int w0 = s / R, nwin = e / R - w0;       // windows completed here (<= 2)
  // the ring rows of the tokens whose state stays live, looked up now so the
  // stores at the end do not wait for the tables
  const int lo = max(s, R * (e / R) - (COFF - 1) * R);
  long srk[DEC_MAX_TOK], srs[DEC_MAX_TOK];
  bool sok[DEC_MAX_TOK];
  uint32_t tbad = 0;
#pragma unroll
  for (int t = 0; t < DEC_MAX_TOK; ++t) {
    const int p = s + t;
    srk[t] = 0;
    srs[t] = 0;
    sok[t] = t < n && p >= lo;
    if (sok[t] && !(state_row(cf, kv_tab, b, p, &srk[t]) && state_row(cf, st_tab, b, p, &srs[t]))) {
      tbad |= CMP_DEVERR_TABLE;
      sok[t] = false;
    }
  }

  const int rope0 = D - cf.rope;
  const bool rope_lane = own && c >= rope0;
  const int col = rope_lane ? ((c - rope0) >> 1) + ((c & 1) ? cf.rope / 2 : 0) : 0;
  // the first window's rotary values (a second window, possible only at
  // ratio 2, loads its own in the loop)
  float rc0 = 0.f, rs0 = 0.f;
  if (nwin > 0 && rope_lane) {
    rc0 = bf2f(cosv[(size_t)o * cf.rope + col]);
    rs0 = bf2f(sinv[(size_t)o * cf.rope + col]);
  }

  // 1. the tokens' projected values of channel c (packed rows: one token
  //    after the other), then Ape on the scores
  if (own) {
    if (packed) {
      // up to TC tokens per round, each round's loads for exactly its tokens
      // (one uniform branch per round: the round's loads still go out
      // together)
#pragma unroll
      for (int t0 = 0; t0 < DEC_MAX_TOK; t0 += TC) {
        if (t0 >= n) break;
        const int m = min(TC, n - t0);
        if (m >= TC)
          dec_token_values<COFF, KSB, TC>(partial, q.row0, t0, n, T, cf.N, KS, c, kvt, zt);
        else if constexpr (TC > 1) {
          if (m == 1)
            dec_token_values<COFF, KSB, 1>(partial, q.row0, t0, n, T, cf.N, KS, c, kvt, zt);
          else if constexpr (TC > 2) {
            if (m == 2)
              dec_token_values<COFF, KSB, 2>(partial, q.row0, t0, n, T, cf.N, KS, c, kvt, zt);
            else
              dec_token_values<COFF, KSB, 3>(partial, q.row0, t0, n, T, cf.N, KS, c, kvt, zt);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < DEC_MAX_TOK; ++t) {
      if (t >= n) break;
#pragma unroll
      for (int cs = 0; cs < COFF; ++cs) zt[t][cs] += ape[(long)((s + t) % R) * cD + cs * D + c];
    }
  }
  // 2. the completed windows
  for (int k = 0; k < nwin; ++k) {
    const int w = w0 + k;
    if (tid < NSPLIT) {
      const int32_t f = ppflag[(b * DEC_MAX_WIN + k) * NSPLIT + tid];
      if (f) dec_report(err, err2, (uint32_t)f);
    }
    float pooled = 0.f;
    if (own) {
      float pm[NSPLIT], pl[NSPLIT], px[NSPLIT];
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) {
        if (k == 0) {
          pm[sp] = pm0[sp];
          pl[sp] = pl0[sp];
          px[sp] = px0[sp];
        } else {
          const float* st = pp + ((size_t)((b * DEC_MAX_WIN + k) * NSPLIT + sp) * 3) * D + c;
          pm[sp] = st[0];
          pl[sp] = st[D];
          px[sp] = st[2 * D];
        }
      }
      // this call's tokens in the window and their channel set: C4A first
      // set for positions (w-1)*4 .. w*4-1, second set for w*4 .. w*4+3
      float zs[DEC_MAX_TOK], ks_[DEC_MAX_TOK];
      bool in[DEC_MAX_TOK];
#pragma unroll
      for (int t = 0; t < DEC_MAX_TOK; ++t) {
        const int p = s + t;
        const int lo = (w - (COFF - 1)) * R, hi = (w + 1) * R;
        in[t] = t < n && p >= lo && p < hi;
        const int cs = COFF == 2 ? (p >= w * R) : 0;
        zs[t] = cs ? zt[t][COFF - 1] : zt[t][0];
        ks_[t] = cs ? kvt[t][COFF - 1] : kvt[t][0];
        if (in[t] && zs[t] == -INFINITY) in[t] = false;
      }
      float m = -INFINITY;
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) if (pl[sp] > 0.f) m = fmaxf(m, pm[sp]);
#pragma unroll
      for (int t = 0; t < DEC_MAX_TOK; ++t) if (in[t]) m = fmaxf(m, zs[t]);
      float l = 0.f, x = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int t = 0; t < DEC_MAX_TOK; ++t) {
          if (!in[t]) continue;
          const float ex = __expf(zs[t] - m);
          l += ex;
          x = fmaf(ex, ks_[t], x);
        }
#pragma unroll
        for (int sp = 0; sp < NSPLIT; ++sp) {
          if (pl[sp] > 0.f) {
            const float sc = __expf(pm[sp] - m);
            l = fmaf(pl[sp], sc, l);
            x = fmaf(px[sp], sc, x);
          }
        }
      }
      pooled = l > 0.f ? x / l : 0.f;
    }
    // RMSNorm over the D channels (block-wide sum)
    float v = own ? pooled * pooled : 0.f;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float ss = 0.f;
#pragma unroll
    for (int qq = 0; qq < TL_THREADS / 64; ++qq) ss += red[qq];
    __syncthreads();                             // red is reused by the next window
    const float inv = rsqrtf(ss / float(D) + kRmsEps);
    float y = own ? pooled * inv * g : 0.f;
    // RoPE: pair (2i, 2i+1) of the trailing rope slice, partner via lane ^ 1;
    // the even element takes cos/sin column i, the odd one column 32 + i
    const float partner = __shfl_xor(y, 1, 64);
    const int orow = o + k;
    if (rope_lane) {
      const float rc = k == 0 ? rc0 : bf2f(cosv[(size_t)orow * cf.rope + col]);
      const float rsn = k == 0 ? rs0 : bf2f(sinv[(size_t)orow * cf.rope + col]);
      y = (c & 1) == 0 ? y * rc - partner * rsn : y * rc + partner * rsn;
    }
    uint16_t* op = out + (size_t)orow * D;
    if (!cf.rotate) {
      if (own) op[c] = f2bf(y);
    } else {
      if (own) yv[c] = y;
      __syncthreads();
      if (own) {
        float acc = 0.f;
#pragma unroll 8
        for (int i2 = 0; i2 < D; ++i2) acc += yv[i2] * bf2f(had[(size_t)i2 * D + c]);
        op[c] = f2bf(acc);
      }
      __syncthreads();                           // yv is reused by the next window
    }
  }
  // the request's rows without a window
  for (int k = nwin; k < ub; ++k)
    if (own) out[(size_t)(o + k) * D + c] = 0;

  // 3. the tokens' state rows that stay live
  if (own) {
#pragma unroll
    for (int t = 0; t < DEC_MAX_TOK; ++t) {
      if (!sok[t]) continue;
#pragma unroll
      for (int cs = 0; cs < COFF; ++cs) {
        kv_state[srk[t] * cD + cs * D + c] = kvt[t][cs];
        score_state[srs[t] * cD + cs * D + c] = zt[t][cs];
      }
    }
  }
  if (tbad && tid == 0) dec_report(err, err2, tbad);
}

// Decode tail for one row per request (no cu_seqlens): the general tail
// above specialised to a single token.  The main kernel has written the
// request records, so the workgroup's loads take two rounds: its record, the
// token's K-range partials (KSB >= KS of them, unconditionally: index KS - 1
// repeats and is not summed), the pre-pooled statistics and the norm weight
// at once; then Ape and the rotary values, which need the record's position
// and output row.
template <int R, int COFF, int KSB>
__global__ __launch_bounds__(TL_THREADS) void decode_tail1_kernel(
    Cfg cf, const float* __restrict__ partial, int KS, int B, const DecRec* __restrict__ rec,
    const float* __restrict__ ape, float* __restrict__ kv_state, float* __restrict__ score_state,
    const float* __restrict__ pp, const int32_t* __restrict__ ppflag,
    const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ cosv,
    const uint16_t* __restrict__ sinv, const uint16_t* __restrict__ had, uint16_t* __restrict__ out,
    int out_rows, uint32_t* __restrict__ err, uint32_t* __restrict__ err2) {
  constexpr int NSPLIT = dec_split<R>();
  __shared__ float red[TL_THREADS / 64];
  __shared__ float yv[512];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int D = cf.D, cD = COFF * D;

  if ((int)blockIdx.x == B) {                    // rows after the last request's
    const DecRec t = rec[B];
    const int total = t.s;
    if (tid == 0) dec_report(err, err2, (uint32_t)t.o | (total > out_rows ? CMP_DEVERR_OUT_ROWS : 0u));
    for (long i = (long)total * D + tid; i < (long)out_rows * D; i += TL_THREADS) out[i] = 0;
    return;
  }
  const int b = blockIdx.x;
  const int c = tid;
  const bool own = c < D;

  // 1. every load that does not depend on the record: the token's K-range
  //    partials (kv and score of channel c in every channel set), the
  //    pre-pooled statistics of the window it may close, the norm weight
  const DecRec rb = rec[b];
  float kvc[COFF], zc[COFF];
  float pm[NSPLIT], pl[NSPLIT], px[NSPLIT];
  const int cl = own ? c : 0;
  {
    const float* pb = partial + (size_t)b * cf.N;
    const size_t kstride = (size_t)B * cf.N;
    float pk[COFF][KSB], pz[COFF][KSB];
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) {
      const int ck = packed_col(0, cs, cl, COFF), cz = packed_col(1, cs, cl, COFF);
#pragma unroll
      for (int ks = 0; ks < KSB; ++ks) {
        const size_t kk = (size_t)min(ks, KS - 1) * kstride;
        pk[cs][ks] = pb[kk + ck];
        pz[cs][ks] = pb[kk + cz];
      }
    }
#pragma unroll
    for (int q = 0; q < NSPLIT; ++q) {
      const float* st = pp + ((size_t)(b * DEC_MAX_WIN * NSPLIT + q) * 3) * D + cl;
      pm[q] = st[0];
      pl[q] = st[D];
      px[q] = st[2 * D];
    }
#pragma unroll
    for (int cs = 0; cs < COFF; ++cs) {
      kvc[cs] = 0.f;
      zc[cs] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSB; ++ks) {
        kvc[cs] += ks < KS ? pk[cs][ks] : 0.f;
        zc[cs] += ks < KS ? pz[cs][ks] : 0.f;
      }
    }
  }
  const float g = bf2f(gamma[cl]);
  if (!(rb.flags & DR_ACT)) return;
  // 2nd round: Ape of the token's position (score of every channel set)
#pragma unroll
  for (int cs = 0; cs < COFF; ++cs) zc[cs] += ape[(long)(rb.s % R) * cD + cs * D + cl];
  const int o = rb.o;
  if (o >= out_rows) return;                     // reported by workgroup B
  const bool completing = (rb.flags & DR_COMP) != 0;
  if (completing && tid < NSPLIT) {
    const int32_t f = ppflag[b * DEC_MAX_WIN * NSPLIT + tid];
    if (f) dec_report(err, err2, (uint32_t)f);
  }
  // the rotary values of this channel for output row o
  const int rope0 = D - cf.rope;
  const bool rope_lane = own && c >= rope0;
  float rc = 0.f, rsn = 0.f;
  if (completing && rope_lane) {
    const int col = ((c - rope0) >> 1) + ((c & 1) ? cf.rope / 2 : 0);
    rc = bf2f(cosv[(size_t)o * cf.rope + col]);
    rsn = bf2f(sinv[(size_t)o * cf.rope + col]);
  }

  if (completing) {
    // 2. pooled value of channel c: the token is the window's last slot
    //    (second channel set for C4A)
    float pooled = 0.f;
    if (own) {
      const float zt = zc[COFF - 1], kt = kvc[COFF - 1];
      float m = zt;
#pragma unroll
      for (int q = 0; q < NSPLIT; ++q) m = fmaxf(m, pm[q]);
      float l = 0.f, x = 0.f;
      if (m != -INFINITY) {
        if (zt != -INFINITY) {
          const float et = __expf(zt - m);
          l = et;
          x = et * kt;
        }
#pragma unroll
        for (int q = 0; q < NSPLIT; ++q) {
          if (pl[q] > 0.f) {
            const float sc = __expf(pm[q] - m);
            l = fmaf(pl[q], sc, l);
            x = fmaf(px[q], sc, x);
          }
        }
      }
      pooled = l > 0.f ? x / l : 0.f;
    }
    // RMSNorm over the D channels (block-wide sum)
    float v = own ? pooled * pooled : 0.f;
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < TL_THREADS / 64; ++q) ss += red[q];
    const float inv = rsqrtf(ss / float(D) + kRmsEps);
    float y = own ? pooled * inv * g : 0.f;
    // RoPE: pair (2i, 2i+1) of the trailing rope slice, partner via lane ^ 1;
    // the even element takes cos/sin column i, the odd one column 32 + i
    const float partner = __shfl_xor(y, 1, 64);
    if (rope_lane) y = (c & 1) == 0 ? y * rc - partner * rsn : y * rc + partner * rsn;
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
  if (own && (rb.flags & DR_STORE)) {
    if (rb.flags & DR_ROW_OK) {
#pragma unroll
      for (int cs = 0; cs < COFF; ++cs) {
        kv_state[rb.rk * cD + cs * D + c] = kvc[cs];
        score_state[rb.rs * cD + cs * D + c] = zc[cs];
      }
    } else if (c == 0) {
      dec_report(err, err2, CMP_DEVERR_TABLE);
    }
  }
}

}  // namespace cmp
