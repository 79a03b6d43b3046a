// Prefill: projection GEMM with the window pooling fused into its epilogue.
//
// Tiles are window-aligned per request.  A tile covers BM (256, or 128 for
// short calls) consecutive positions P0 .. P0+BM-1 of one request (rows of x
// where the position is a token of this call; earlier positions come from
// the state ring, staged by the setup launch before the GEMM): 64 (32) windows
// for ratio 4, two (one) for ratio 128.
// For ratio 4 (coff = 2) window w pools the first channel set of window w-1
// and the second set of window w ([PyPTO] 压缩窗口与状态更新; [AscendC] C4A
// 计算公式).  The first window of a request's first tile takes window w-1 from
// the staged state rows (or padding); in later tiles that window is split:
// the tile stores the second-set statistics of its first window and the
// first-set statistics of its last window, and the post kernel merges the
// two halves of each split window (no halo recomputation, no tile waits).
//
// Epilogue: the accumulators of wave (wm, wn) hold 64 rows x 128 panel
// columns; the panel's column order puts every variant (kv / score, channel
// set) of a channel in one lane (packed_col), and a lane's rows come in runs
// of 4 consecutive rows.  So each lane forms, per channel, the softmax
// statistics (running max m, sum l, weighted sum x) of its window slots,
// merges them with the statistics its neighbour lane (or, at a row-wave
// boundary, the previous row-wave, through LDS) holds for the rest of the
// window, and writes the pooled value ([CANN] 计算公式 steps 3-5).  Scores get Ape first ([CANN] step 2).
// The same epilogue stores the state rows that stay live after the call
// (positions [max(s, r*floor(e/r) - (coff-1)*r), e)): the GEMM never reads
// the pool, so there is no read/write hazard inside the kernel.
#pragma once
#include "common.hpp"
#include "gemm.hpp"

namespace cmp {

// Stats (m, l, x) of softmax-weighted sums; m = -inf means empty.
struct Soft {
  float m, l, x;
};
__device__ __forceinline__ void soft_add(Soft& s, float z, float kv) {
  const float mn = fmaxf(s.m, z);
  const float sc = __expf(s.m - mn), pe = __expf(z - mn);
  s.l = s.l * sc + pe;
  s.x = s.x * sc + pe * kv;
  s.m = mn;
}
__device__ __forceinline__ Soft soft_merge(Soft a, Soft b) {
  if (a.l == 0.f) return b;
  if (b.l == 0.f) return a;
  const float mn = fmaxf(a.m, b.m);
  const float sa = __expf(a.m - mn), sb = __expf(b.m - mn);
  return Soft{mn, a.l * sa + b.l * sb, a.x * sa + b.x * sb};
}
__device__ __forceinline__ Soft soft_shfl_xor(Soft s, int mask) {
  return Soft{__shfl_xor(s.m, mask, 64), __shfl_xor(s.l, mask, 64), __shfl_xor(s.x, mask, 64)};
}

constexpr float kLog2e = 1.4426950408889634f;

// For a lane of the low half, `a` of the lane 32 above; for a lane of the
// high half, `b` of the lane 32 below (one v_permlane32_swap, no LDS).
__device__ __forceinline__ float cross_half(float a, float b, int hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(hi ? r[0] : r[1]);
}

// Softmax statistics of one run of 4 rows (scores z, values v): the max and
// the exp-weighted sums taken against it; an all -inf run is empty.
__device__ __forceinline__ Soft soft_group4(const float (&z)[4], const float (&v)[4]) {
  const float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  float l = 0.f, x = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float p = __builtin_amdgcn_exp2f((z[q] - mx) * kLog2e);
    l += p;
    x = fmaf(p, v[q], x);
  }
  return mx == -INFINITY ? Soft{-INFINITY, 0.f, 0.f} : Soft{mx, l, x};
}

// Pooled value of the union of two statistics (0 when both are empty).
__device__ __forceinline__ float soft_value2(Soft a, Soft b) {
  const float mn = fmaxf(a.m, b.m);
  const float sa = a.l > 0.f ? __builtin_amdgcn_exp2f((a.m - mn) * kLog2e) : 0.f;
  const float sb = b.l > 0.f ? __builtin_amdgcn_exp2f((b.m - mn) * kLog2e) : 0.f;
  const float den = a.l * sa + b.l * sb;
  return den > 0.f ? (a.x * sa + b.x * sb) / den : 0.f;
}

// Request whose tile range holds global M-tile `mt` (largest b with tile0 <= mt).
__device__ __forceinline__ int find_tile_request(const int32_t* __restrict__ plan, int B, int mt) {
  int lo = 0, hi = B - 1, ans = 0;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (plan[(long)mid * PL_WIDTH + PL_TILE0] <= mt) { ans = mid; lo = mid + 1; }
    else hi = mid - 1;
  }
  return ans;
}

// live-state store of one position's projected row (both channel sets)
template <int COFF>
__device__ __forceinline__ void store_state(const Cfg& cf, float* __restrict__ kv_state,
                                            float* __restrict__ score_state,
                                            const int32_t* __restrict__ kv_tab,
                                            const int32_t* __restrict__ st_tab, int b, int p,
                                            int c, const float (&kv)[COFF], const float (&z)[COFF],
                                            uint32_t& bad) {
  long rk, rs;
  if (!state_row(cf, kv_tab, b, p, &rk) || !state_row(cf, st_tab, b, p, &rs)) {
    bad |= CMP_DEVERR_TABLE;
    return;
  }
  const int cD = COFF * cf.D;
#pragma unroll
  for (int cs = 0; cs < COFF; ++cs) {
    kv_state[rk * cD + cs * cf.D + c] = kv[cs];
    score_state[rs * cD + cs * cf.D + c] = z[cs];
  }
}

// ---------------------------------------------------------------------------
// coff = 1 epilogue (ratios 2, 8, 16, ..., 128): the windows of a row-wave's
// 64 rows.  Register r of block i holds wave row 32 i + 8 (r / 4) + 4 h + r % 4
// (h = lane / 32), so a window of R <= 4 rows lies in one lane (R = 4: one
// run of 4 rows, R = 2: half a run), and a window of R >= 8 rows is split
// between the two lane halves: each half takes the statistics of its rows
// (max first, then the exponentials), one cross-half swap merges them, and
// the low half writes channel c0, the high half c1.  A window of 128 rows
// spans two row-waves: the odd one hands its statistics to the even one
// through LDS.  FAST: every row is a token of this call and every window
// complete (no per-row tests).
// ---------------------------------------------------------------------------
struct EpiCtx {
  const Cfg& cf;
  int base;            // position of wave row 0 (a multiple of R)
  int s, e, live_lo, first;
  const float* stg;    // staged ring rows of positions [first, s)
  const float* ape;
  const float* apet;   // Ape transposed, [channel][slot] (ratio >= 8)
  int c0, c1, h;
  int orow0;           // output row of the wave's first window, if complete
  int wfirst, wend, wg0;
  int out_rows;
  float* pooled;
  uint8_t* xch;        // LDS for the two row-waves of a 128-row window
  int wm, wn;
};

// slot of wave row jr in its window (the wave starts a window unless a
// window spans two row-waves)
template <int R>
__device__ __forceinline__ int epi_slot(const EpiCtx& t, int jr) {
  return (R > GM_WROWS ? t.base + jr : jr) & (R - 1);
}

// value of channel c of (kv or score) at wave row jr: the accumulator plus
// a_ape (the Ape of the row's slot), or the staged row for positions before
// the call; false if no token there
template <int R, bool FAST>
__device__ __forceinline__ bool epi_value(const EpiCtx& t, float a_kv, float a_z, float a_ape,
                                          int jr, int c, float& kv, float& z) {
  const int cD = t.cf.D;
  if (FAST) {
    kv = a_kv;
    z = a_z + a_ape;
    return true;
  }
  const int p = t.base + jr;
  if (p >= t.e) return false;
  if (p < t.s) {
    const float* row = t.stg + (size_t)(p - t.first) * 2 * cD;
    kv = row[c];
    z = row[cD + c];
  } else {
    kv = a_kv;
    z = a_z + a_ape;
  }
  return z != -INFINITY;
}

// pooled value of one window from its statistics, to its output row
__device__ __forceinline__ void epi_store(const EpiCtx& t, int wl, int c, const Soft& st) {
  const int wg = t.wg0 + wl;
  if (wg < t.wfirst || wg >= t.wend) return;
  const int row = t.orow0 + wl;
  if (row < t.out_rows) t.pooled[(size_t)row * t.cf.D + c] = st.l > 0.f ? st.x / st.l : 0.f;
}

template <int R, bool FAST>
__device__ __forceinline__ void epilogue_coff1(const EpiCtx& t, const f32x16 (&acc)[2][4]) {
  const int h = t.h;
  if constexpr (R <= 4) {
    // windows inside one lane: R = 4 -> (i, run), R = 2 -> (i, run, pair)
    constexpr int PER_RUN = 4 / R;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int pw = 0; pw < PER_RUN; ++pw) {
          float kv[2][R], z[2][R];
          bool ok[2][R];
#pragma unroll
          for (int q = 0; q < R; ++q) {
            const int r = 4 * rg + pw * R + q;
            const int jr = 32 * i + 8 * rg + 4 * h + pw * R + q;
            const int sl = epi_slot<R>(t, jr);
            ok[0][q] = epi_value<R, FAST>(t, acc[i][0][r], acc[i][1][r], t.ape[sl * t.cf.D + t.c0],
                                          jr, t.c0, kv[0][q], z[0][q]);
            ok[1][q] = epi_value<R, FAST>(t, acc[i][2][r], acc[i][3][r], t.ape[sl * t.cf.D + t.c1],
                                          jr, t.c1, kv[1][q], z[1][q]);
          }
          const int wl = (32 * i + 8 * rg + 4 * h + pw * R) / R;   // window in the wave
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
            float m = -INFINITY;
#pragma unroll
            for (int q = 0; q < R; ++q) if (ok[ch][q]) m = fmaxf(m, z[ch][q]);
            Soft st{m, 0.f, 0.f};
            if (m != -INFINITY) {
#pragma unroll
              for (int q = 0; q < R; ++q) {
                if (!ok[ch][q]) continue;
                const float pe = __builtin_amdgcn_exp2f((z[ch][q] - m) * kLog2e);
                st.l += pe;
                st.x = fmaf(pe, kv[ch][q], st.x);
              }
            }
            epi_store(t, wl, ch ? t.c1 : t.c0, st);
          }
        }
  } else {
    // R >= 8: wave window w holds blocks i and runs rg with
    // (32 i + 8 rg) / R == w, in both lane halves.  Statistics one 32-row
    // block and one channel at a time (max, then exponentials, of the
    // block's rows in this lane), merged into the window's.  Both passes
    // read the accumulators (or, for positions before the call, the staged
    // rows) again instead of copying the block's values: the accumulators
    // stay live anyway, and a copy of 32 values per channel beside them
    // spilled.
    constexpr int NW = R <= GM_WROWS ? GM_WROWS / R : 1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      Soft st[2] = {Soft{-INFINITY, 0.f, 0.f}, Soft{-INFINITY, 0.f, 0.f}};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if ((32 * i + 31) / R < w || (32 * i) / R > w) continue;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int c = ch ? t.c1 : t.c0;
          // the Ape of the block's rows: runs of 4 consecutive slots, one
          // 16-byte load each from the transposed table
          float4 ap[4];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            ap[g4] = *reinterpret_cast<const float4*>(
                t.apet + (size_t)c * R + epi_slot<R>(t, 32 * i + 8 * g4 + 4 * h));
          float m = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if ((32 * i + 8 * (r >> 2)) / R != w) continue;
            const float4 a4 = ap[r >> 2];
            const float av = (r & 3) == 0 ? a4.x : (r & 3) == 1 ? a4.y : (r & 3) == 2 ? a4.z : a4.w;
            float kv, z;
            if (epi_value<R, FAST>(t, acc[i][2 * ch][r], acc[i][2 * ch + 1][r], av,
                                   32 * i + 8 * (r >> 2) + 4 * h + (r & 3), c, kv, z))
              m = fmaxf(m, z);
          }
          Soft blk{m, 0.f, 0.f};
          if (m != -INFINITY) {
            // staged rows are loaded again rather than kept live
            if constexpr (!FAST) asm volatile("" ::: "memory");
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              if ((32 * i + 8 * (r >> 2)) / R != w) continue;
              const float4 a4 = ap[r >> 2];
              const float av = (r & 3) == 0 ? a4.x : (r & 3) == 1 ? a4.y : (r & 3) == 2 ? a4.z : a4.w;
              float kv, z;
              if (!epi_value<R, FAST>(t, acc[i][2 * ch][r], acc[i][2 * ch + 1][r], av,
                                      32 * i + 8 * (r >> 2) + 4 * h + (r & 3), c, kv, z))
                continue;
              const float pe = __builtin_amdgcn_exp2f((z - m) * kLog2e);
              blk.l += pe;
              blk.x = fmaf(pe, kv, blk.x);
            }
          }
          st[ch] = soft_merge(st[ch], blk);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the low half needs the high half's c0 rows, the high half the low
      // half's c1 rows
      const Soft mine = h ? st[1] : st[0];
      const Soft other{cross_half(st[0].m, st[1].m, h), cross_half(st[0].l, st[1].l, h),
                       cross_half(st[0].x, st[1].x, h)};
      const float mn = fmaxf(mine.m, other.m);
      Soft tot{mn, 0.f, 0.f};
      if (mine.l > 0.f) {
        const float sc = __builtin_amdgcn_exp2f((mine.m - mn) * kLog2e);
        tot.l += mine.l * sc;
        tot.x += mine.x * sc;
      }
      if (other.l > 0.f) {
        const float sc = __builtin_amdgcn_exp2f((other.m - mn) * kLog2e);
        tot.l += other.l * sc;
        tot.x += other.x * sc;
      }
      if constexpr (R > GM_WROWS) {
        // second half of the window in the odd row-wave of the pair
        Soft* xs = reinterpret_cast<Soft*>(t.xch) + ((t.wm >> 1) * 2 + t.wn) * 64 + (threadIdx.x & 63);
        if (t.wm & 1) *xs = tot;
        __syncthreads();
        if (!(t.wm & 1)) epi_store(t, w, h ? t.c1 : t.c0, soft_merge(tot, *xs));
      } else {
        epi_store(t, w, h ? t.c1 : t.c0, tot);
      }
    }
  }
}

// The copy ring takes all of the kernel's LDS; the epilogue's exchange (at
// most 3 KiB) sits in the panel stage that is idle between two tiles
// (GM_IDLE_OFF).
// ratio 4: [3 row-wave boundaries][2 column waves][32 lanes]; ratio 128:
// [2 row-wave pairs][2 column waves][64 lanes]
static_assert(3 * 2 * 32 * sizeof(Soft) <= GM_IDLE_BYTES && 2 * 2 * 64 * sizeof(Soft) <= GM_IDLE_BYTES,
              "the epilogue exchange fits the idle panel stage");

// One tile of a request: M-tile mt (its request b, the tile's first position
// P0 and its index tloc among the request's tiles) and N-tile nt.
struct PoolTile {
  int mt, nt, b, tloc, P0, n0;
  const int32_t* rec;
};

template <int R, int BM>
__device__ __forceinline__ PoolTile pool_tile(int tile, int tiles_n, const int32_t* __restrict__ plan,
                                              int B) {
  PoolTile t;
  // tiles_n = N / 256 = coff * D / 128 is a power of two (D is 128 or 512):
  // a shift keeps the tile walk in scalar registers, so the plan lookups
  // below are scalar loads that do not wait on the copies in flight
  t.mt = tile >> __builtin_ctz(tiles_n);
  t.nt = tile & (tiles_n - 1);
  t.b = find_tile_request(plan, B, t.mt);
  t.rec = plan + (long)t.b * PL_WIDTH;
  t.tloc = t.mt - t.rec[PL_TILE0];
  t.P0 = R * (t.rec[PL_START] / R) + t.tloc * BM;
  t.n0 = t.nt * GM_BN;
  return t;
}

// The tile's copy sources for copy role `role`: X rows of positions
// P0 + (tile row), clamped into x.
template <int WV>
__device__ __forceinline__ GmSrc pool_sources(const PoolTile& t, const Cfg& cf,
                                              const uint16_t* __restrict__ X,
                                              const uint16_t* __restrict__ W, int T, int role) {
  const int lane = threadIdx.x & 63;
  const int s = t.rec[PL_START], row0 = t.rec[PL_ROW0];
  int arow[GM_A_COPIES];
#pragma unroll
  for (int j = 0; j < GM_A_COPIES; ++j) {
    const int p = t.P0 + gm_copy_row(role, lane, j);
    arow[j] = min(max(row0 + (p - s), 0), T - 1);
  }
  return gm_sources<WV>(X, W, cf.H, t.n0, arow, min(max(row0 + (t.P0 - s), 0), T - 1), role);
}

// Workgroup barriers one pool_epilogue call passes, on every path: the
// exchange between row-waves (ratio 4, and windows that span two row-waves).
// The copy waves of the 4-wave shape pass the same number instead of running
// the epilogue.
template <int R, int COFF>
constexpr int epilogue_barriers() { return COFF == 2 || R > GM_WROWS ? 1 : 0; }

// Pooling epilogue of one tile (see the top of this file).  xch: LDS (at most
// 3 KiB used) that no copy fills and no K loop reads while the epilogue runs.
template <int R, int COFF, int WV>
__device__ __forceinline__ void pool_epilogue(
    const Cfg& cf, const f32x16 (&acc)[2][4], uint8_t* xch, const PoolTile& tl,
    const float* __restrict__ ape, const float* __restrict__ apet, const float* __restrict__ staging,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    float* __restrict__ pooled, int out_rows, float* __restrict__ split, uint32_t* __restrict__ err) {
  constexpr int BM = Gm<WV>::BM, LASTWM = Gm<WV>::NWM - 1;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, h = lane >> 5;
  const int b = tl.b, tloc = tl.tloc, P0 = tl.P0, n0 = tl.n0, mt = tl.mt;
  const int32_t* rec = tl.rec;
  const int s = rec[PL_START], e = rec[PL_END];
  uint8_t* smem = xch;
  const int D = cf.D, cD = COFF * D;
  const float* stg = staging + (size_t)b * COFF * R * 2 * cD;
  const int wfirst = s / R, wend = e / R;             // windows [wfirst, wend) complete
  const int o = rec[PL_OUT0];
  const int live_lo = max(s, R * (e / R) - (COFF - 1) * R);   // state rows to store
  uint32_t bad = 0;
  // the table entries of the staged rows (positions [max(first, 0), s)),
  // which the staging skipped if out of range: checked once per request
  if (tloc == 0 && tl.nt == 0 && wave == 0) {
    for (int p = max(rec[PL_FIRST], 0) + lane; p < s; p += 64) {
      long rk, rs;
      if (!state_row(cf, kv_tab, b, p, &rk) || !state_row(cf, st_tab, b, p, &rs))
        bad |= CMP_DEVERR_TABLE;
    }
  }

  if constexpr (COFF == 2) {
    // ---- ratio 4: lane (wn, lrow) owns channel c in all four variants ----
    const int c = ((n0 + wn * 128) >> 7) * 32 + lrow;
    float ape_a[4], ape_b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ape_a[q] = ape[q * cD + c];
      ape_b[q] = ape[q * cD + D + c];
    }
    if (tloc > 0 && P0 + BM <= live_lo) {   // (live_lo <= e)
      // Interior tile: every row is a token of this call, no state row is
      // stored, window 0 is split and every other window is complete.  Group
      // statistics in two passes (max, then exp) with no per-row tests.
      Soft sa[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = t >> 2, r0 = 4 * (t & 3);
        float z[4], v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[q] = acc[i][2][r0 + q] + ape_a[q];
          v[q] = acc[i][0][r0 + q];
        }
        sa[t] = soft_group4(z, v);
      }
      // the first window of row-wave wm > 0 needs the last window of wm - 1
      Soft* xch = reinterpret_cast<Soft*>(smem);   // [wm][wn][32 lanes]
      if (wm < LASTWM && h == 1) xch[(wm * 2 + wn) * 32 + lrow] = sa[7];
      __syncthreads();
      const Soft from_prev = xch[(max(wm - 1, 0) * 2 + wn) * 32 + lrow];
      float* sp = split + (size_t)mt * 6 * D;
      if (wm == LASTWM && h == 1) {
        sp[0 * D + c] = sa[7].m;
        sp[1 * D + c] = sa[7].l;
        sp[2 * D + c] = sa[7].x;
      }
      const int row_base = o + (P0 >> 2) + wm * 16 + h - wfirst;   // output row of slot 0
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int i = t >> 2, r0 = 4 * (t & 3);
        float z[4], v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[q] = acc[i][3][r0 + q] + ape_b[q];
          v[q] = acc[i][1][r0 + q];
        }
        const Soft sb = soft_group4(z, v);
        // first-set statistics of window w-1: window 2t-1 (low half) sits in
        // the high half at slot t-1, window 2t (high half) in the low half at
        // slot t
        const Soft& pa = sa[(t + 7) & 7];
        Soft prev{cross_half(pa.m, sa[t].m, h), cross_half(pa.l, sa[t].l, h),
                  cross_half(pa.x, sa[t].x, h)};
        if (t == 0 && h == 0 && wm == 0) {
          sp[3 * D + c] = sb.m;
          sp[4 * D + c] = sb.l;
          sp[5 * D + c] = sb.x;
        } else {
          if (t == 0 && h == 0) prev = from_prev;
          const int row = row_base + 2 * t;
          if (row < out_rows) pooled[(size_t)row * D + c] = soft_value2(prev, sb);
        }
      }
    } else {
    // value of (variant, block i, register r) with prefix substitution;
    // returns false for positions without a row (before 0, or not a token)
    auto fetch = [&](int i, int r, int p, float (&kv)[2], float (&z)[2]) -> bool {
      if (p >= e || p < 0) return false;
      if (p < s) {
        const float* row = stg + (size_t)(p - rec[PL_FIRST]) * 2 * cD;
        kv[0] = row[c];
        kv[1] = row[D + c];
        z[0] = row[cD + c];
        z[1] = row[cD + D + c];
      } else {
        kv[0] = acc[i][0][r];
        kv[1] = acc[i][1][r];
        z[0] = acc[i][2][r] + ape_a[r & 3];
        z[1] = acc[i][3][r] + ape_b[r & 3];
      }
      return true;
    };
    // statistics of the first channel set per window this lane holds:
    // window index in the tile w = wm*16 + 8 i + 2 i' + h, rows 4w .. 4w+3
    Soft sa[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) {
        Soft st{-INFINITY, 0.f, 0.f};
        const int w = wm * 16 + 8 * i + 2 * ip + h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float kv[2], z[2];
          if (fetch(i, 4 * ip + q, P0 + 4 * w + q, kv, z) && z[0] != -INFINITY) soft_add(st, z[0], kv[0]);
        }
        sa[i][ip] = st;
      }
    // the first window of row-wave wm > 0 needs the last window of wm - 1
    Soft* xch = reinterpret_cast<Soft*>(smem);       // [wm][wn][32 lanes]
    if (wm < LASTWM && h == 1) xch[(wm * 2 + wn) * 32 + lrow] = sa[1][3];
    __syncthreads();
    const Soft from_prev = xch[(max(wm - 1, 0) * 2 + wn) * 32 + lrow];
    // first-set statistics of the window before the tile: staged state rows
    // (or padding) in the request's first tile, else the previous tile's
    Soft before{-INFINITY, 0.f, 0.f};
    if (tloc == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = P0 - 4 + q;
        if (p >= 0) {
          const float* row = stg + (size_t)(p - rec[PL_FIRST]) * 2 * cD;
          const float z = row[cD + c];
          if (z != -INFINITY) soft_add(before, z, row[c]);
        }
      }
    }
    // split-window statistics of this tile: [mt][a = last window's first
    // set | b = first window's second set][m, l, x][D]
    float* sp = split + (size_t)mt * 6 * D;
    if (wm == LASTWM && h == 1) {
      sp[0 * D + c] = sa[1][3].m;
      sp[1 * D + c] = sa[1][3].l;
      sp[2 * D + c] = sa[1][3].x;
    }
    // the other lane half's statistics (every lane takes part in the shuffle)
    Soft other[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) other[i][ip] = soft_shfl_xor(sa[i][ip], 32);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) {
        const int w = wm * 16 + 8 * i + 2 * ip + h;
        // first-set statistics of window w-1: odd windows (h = 1) find it in
        // the partner lane at the same slot, even ones one slot earlier
        const Soft prev = h == 1 ? other[i][ip]
                                 : (ip > 0 ? other[i][ip - 1]
                                           : (i > 0 ? other[i - 1][3] : (wm > 0 ? from_prev : before)));
        // second set of window w, then the pooled value
        Soft sb{-INFINITY, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float kv[2], z[2];
          const int p = P0 + 4 * w + q;
          if (fetch(i, 4 * ip + q, p, kv, z)) {
            if (z[1] != -INFINITY) soft_add(sb, z[1], kv[1]);
            if (p >= live_lo)
              store_state<2>(cf, kv_state, score_state, kv_tab, st_tab, b, p, c, kv, z, bad);
          }
        }
        const int Wg = (P0 >> 2) + w;
        if (Wg >= wfirst && Wg < wend) {
          if (w == 0 && tloc > 0) {
            sp[3 * D + c] = sb.m;
            sp[4 * D + c] = sb.l;
            sp[5 * D + c] = sb.x;
          } else {
            const Soft t = soft_merge(prev, sb);
            const int row = o + (Wg - wfirst);
            if (row < out_rows) pooled[(size_t)row * D + c] = t.l > 0.f ? t.x / t.l : 0.f;
          }
        }
      }
    }
  } else {
    // ---- coff = 1: lane (wn, lrow) owns channels c0 (blocks 0: kv,
    // 1: score) and c1 (blocks 2, 3) ----
    const int g = (n0 + wn * 128) >> 7;
    const int c0 = g * 64 + lrow, c1 = c0 + 32;
    const int wbase = P0 + GM_WROWS * wm;   // position of the wave's first row
    EpiCtx ctx{cf, wbase, s, e, live_lo, rec[PL_FIRST], stg, ape, apet, c0, c1, h,
               o + wbase / R - wfirst, wfirst, wend, wbase / R,
               out_rows, pooled, smem, wm, wn};
    if (P0 >= s && P0 + BM <= live_lo) {
      epilogue_coff1<R, true>(ctx, acc);
    } else {
      epilogue_coff1<R, false>(ctx, acc);
      // state rows that stay live (only a request's last tile has any)
      if (wbase + GM_WROWS - 1 >= live_lo && wbase < e) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jr = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);   // row in the wave
            const int p = wbase + jr;
            if (p >= live_lo && p < e) {
              long rk, rs;
              if (state_row(cf, kv_tab, b, p, &rk) && state_row(cf, st_tab, b, p, &rs)) {
                const int q = p % R;
                kv_state[rk * cD + c0] = acc[i][0][r];
                kv_state[rk * cD + c1] = acc[i][2][r];
                score_state[rs * cD + c0] = acc[i][1][r] + ape[q * cD + c0];
                score_state[rs * cD + c1] = acc[i][3][r] + ape[q * cD + c1];
              } else {
                bad |= CMP_DEVERR_TABLE;
              }
            }
          }
        }
      }
    }
  }
  if (bad) set_error(err, bad);
}

// Persistent kernel: one workgroup per CU walks its tiles.  Workgroup i runs
// on XCD i % 8; each XCD owns a contiguous run of tiles (N fastest), so the
// XCD's co-running tiles share x rows and panel slices in its L2.  A
// workgroup's first two tiles are fixed (its slot in the XCD's first two
// rounds); the rest of the run is a queue: tiles[1 + xcd] counts the tiles
// taken from it, and a workgroup whose XCD queue is empty takes from the
// other XCDs' queues.  XCDs run at different clocks under this load (about
// 10% apart), and a static split left the fastest workgroups idle for the
// last ~6% of the call.  A workgroup takes the tile after its next one while
// the current epilogue runs (one lane's atomic, its result passed on through
// LDS), so the next tile's first three stages are copied while the current
// tile runs its last three K steps, as in a static walk.
struct TileQueue {
  int32_t* heads;   // per-XCD count of tiles taken
  int per_xcd, first_dyn, total;
};
// Tile range of XCD x's queue: [x*per_xcd + first_dyn, min((x+1)*per_xcd, total)).
__device__ __forceinline__ int queue_take(const TileQueue& q, int x) {
  const int lo = x * q.per_xcd + q.first_dyn, hi = min((x + 1) * q.per_xcd, q.total);
  if (lo >= hi) return -1;
  const int t = lo + atomicAdd(q.heads + x, 1);
  return t < hi ? t : -1;
}
// The other XCDs' queues, in turn, once the own one is empty.
__device__ __forceinline__ int queue_steal(const TileQueue& q, int xcd) {
  for (int d = 1; d < 8; ++d) {
    const int t = queue_take(q, (xcd + d) & 7);
    if (t >= 0) return t;
  }
  return -1;
}
// Byte offset in the idle panel stage of the word that passes a taken tile
// to every wave (past the epilogue's exchange).
constexpr int GM_QUEUE_SLOT = GM_IDLE_BYTES - 16;
static_assert(2 * 2 * 64 * sizeof(Soft) <= GM_QUEUE_SLOT && 3 * 2 * 32 * sizeof(Soft) <= GM_QUEUE_SLOT,
              "the queue word lies past the epilogue exchange");

// The tile walk of one wave in role MODE (GmMode); copy role `role`.  Every
// role passes the same barriers: the K loop's, the epilogue's (a copy wave
// passes epilogue_barriers() instead of running it) and the one that hands
// on each taken tile.  One instance per role keeps each role's registers
// apart (a single walk branching per tile spilled the MFMA loop's
// addresses).
template <int R, int COFF, int WV, int MODE>
__device__ __forceinline__ void pool_walk(
    const Cfg& cf, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, int T, int B,
    const int32_t* __restrict__ plan, const TileQueue& q, int xcd, int tile, int next,
    const float* __restrict__ ape, const float* __restrict__ apet, const float* __restrict__ staging,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    float* __restrict__ pooled, int out_rows, float* __restrict__ split,
    uint32_t* __restrict__ err, uint8_t* smem, int role) {
  constexpr bool COPY = MODE != GM_MFMA, MUL = MODE != GM_COPY;
  uint8_t* xch = smem + GM_IDLE_OFF;
  const int tiles_n = cf.N / GM_BN;
  const int KT = cf.H / GM_BK, ksteps = cf.H >> 4;
  PoolTile cur = pool_tile<R, Gm<WV>::BM>(tile, tiles_n, plan, B);
  GmSrc csrc{};
  if constexpr (COPY) {
    csrc = pool_sources<WV>(cur, cf, X, W, T, role);
    gm_prologue<WV>(smem, csrc, ksteps, role);
  }
  f32x16 acc[2][4];
  const int xstep = (KT >> 1) % 3;   // X buffer rotation per tile
  int xrot = 0;
  while (true) {
    const bool has_next = next >= 0;
    const PoolTile nxt = has_next ? pool_tile<R, Gm<WV>::BM>(next, tiles_n, plan, B) : cur;
    GmSrc nsrc{};
    if constexpr (COPY) nsrc = has_next ? pool_sources<WV>(nxt, cf, X, W, T, role) : csrc;
    gemm_tile_any<WV, MODE>(acc, smem, csrc, nsrc, has_next, KT, xrot, ksteps, role);
    // the tile after the next one: taken now, read after the epilogue
    int taken = -1;
    if constexpr (MUL) {
      if (has_next && threadIdx.x == 0) taken = queue_take(q, xcd);
      pool_epilogue<R, COFF, WV>(cf, acc, xch, cur, ape, apet, staging, kv_state, score_state,
                                 kv_tab, st_tab, pooled, out_rows, split, err);
    } else {
#pragma unroll
      for (int i = 0; i < epilogue_barriers<R, COFF>(); ++i) asm volatile("s_barrier" ::: "memory");
    }
    if (!has_next) break;
    if (MUL && threadIdx.x == 0) {
      if (taken < 0) taken = queue_steal(q, xcd);
      *reinterpret_cast<volatile int*>(xch + GM_QUEUE_SLOT) = taken;
    }
    // a bare barrier (a workgroup fence would also wait for the next tile's
    // copies in flight); the slot is read before the next K loop's copies
    // can reach the idle stage
    __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    next = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(xch + GM_QUEUE_SLOT));
    cur = nxt;
    if constexpr (COPY) {
      // rebuild the copy sources rather than carry them through the
      // epilogue, whose register demand would spill them (an opaque tile
      // field keeps the compiler from reusing the values computed before the
      // K loop)
      cur.P0 = __builtin_amdgcn_readfirstlane(cur.P0);
      asm volatile("" : "+s"(cur.P0));
      csrc = pool_sources<WV>(cur, cf, X, W, T, role);
    }
    xrot += xstep;
    if (xrot >= 3) xrot -= 3;
  }
}

template <int R, int COFF, int WV>
__global__ __launch_bounds__(Gm<WV>::THREADS, 1) void gemm_pool_kernel(
    Cfg cf, const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, int T, int B,
    const int32_t* __restrict__ plan, int32_t* __restrict__ tiles,
    const float* __restrict__ ape, const float* __restrict__ apet, const float* __restrict__ staging,
    float* __restrict__ kv_state, float* __restrict__ score_state,
    const int32_t* __restrict__ kv_tab, const int32_t* __restrict__ st_tab,
    float* __restrict__ pooled, int out_rows, float* __restrict__ split,
    uint32_t* __restrict__ err) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tiles_n = cf.N / GM_BN;
  const int total = tiles[0] * tiles_n;
  const int per_wg = gridDim.x >> 3;                // workgroups per XCD
  const int per_xcd = (total + 7) >> 3;             // tiles per XCD
  const int xcd = blockIdx.x & 7;
  const int lo = xcd * per_xcd;
  const int hi = min(lo + per_xcd, total);
  const TileQueue q{tiles + 1, per_xcd, 2 * per_wg, total};
  const int tile = lo + (blockIdx.x >> 3);
  if (tile >= hi) return;
  const int next = tile + per_wg < hi ? tile + per_wg : -1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (Gm<WV>::COPIERS == 0) {
    pool_walk<R, COFF, WV, GM_ALL>(cf, X, W, T, B, plan, q, xcd, tile, next, ape, apet, staging,
                                   kv_state, score_state, kv_tab, st_tab, pooled, out_rows, split,
                                   err, smem, wave);
  } else if (wave >= WV) {
    pool_walk<R, COFF, WV, GM_COPY>(cf, X, W, T, B, plan, q, xcd, tile, next, ape, apet, staging,
                                    kv_state, score_state, kv_tab, st_tab, pooled, out_rows, split,
                                    err, smem, wave - WV);
  } else {
    pool_walk<R, COFF, WV, GM_MFMA>(cf, X, W, T, B, plan, q, xcd, tile, next, ape, apet, staging,
                                    kv_state, score_state, kv_tab, st_tab, pooled, out_rows, split,
                                    err, smem, wave);
  }
  gm_drain();
}


}  // namespace cmp
