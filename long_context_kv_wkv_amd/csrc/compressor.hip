// Host side of the Compressor library: argument checks, workspace layout,
// kernel launches on the caller's stream, and the C ABI of compressor.h.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "compressor.h"
#include "nsa_compress.h"
#include "common.hpp"
#include "decode.hpp"
#include "gemm.hpp"
#include "pool.hpp"
#include "prefill.hpp"
#include "nsa.hpp"
#include "epilog.hpp"

using namespace cmp;

namespace {

// ---------------------------------------------------------------------------
// kernel timing (optional): an event pair around every launch
// ---------------------------------------------------------------------------
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
struct Timing {
  std::mutex mu;
  int on = 0;                       // 0 off, 1 every launch, 2 the projection GEMM only
  std::vector<TimedLaunch> recs;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> spare;
} g_timing;

template <typename F>
int launch(const char* name, hipStream_t stream, F&& fn) {
  hipEvent_t a = nullptr, b = nullptr;
  bool timed = false;
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.on == 1 || (g_timing.on == 2 && std::strcmp(name, "gemm") == 0)) {
      if (!g_timing.spare.empty()) {
        a = g_timing.spare.back().first;
        b = g_timing.spare.back().second;
        g_timing.spare.pop_back();
      } else {
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return CMP_ERR_HIP;
      }
      timed = true;
    }
  }
  if (timed && hipEventRecord(a, stream) != hipSuccess) return CMP_ERR_HIP;
  fn();
  if (hipGetLastError() != hipSuccess) return CMP_ERR_HIP;
  if (timed) {
    if (hipEventRecord(b, stream) != hipSuccess) return CMP_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.recs.push_back({name, a, b});
  }
  return CMP_OK;
}

#define CMP_TRY(x)                  \
  do {                              \
    int _rc = (x);                  \
    if (_rc != CMP_OK) return _rc;  \
  } while (0)

// ---------------------------------------------------------------------------
// shape checks
// ---------------------------------------------------------------------------
int check_shape(const compressor_shape* sh, Cfg* cf) {
  if (!sh) return CMP_ERR_NULLPTR;
  // cmp_ratio 2, 4, 8, 16, 32, 64 or 128 ([CANN] 约束说明)
  if (sh->ratio < 2 || sh->ratio > 128 || (sh->ratio & (sh->ratio - 1))) return CMP_ERR_UNSUPPORTED;
  if (sh->head_dim != 128 && sh->head_dim != 512) return CMP_ERR_UNSUPPORTED;
  if (sh->hidden < 1024 || sh->hidden > 10240 || sh->hidden % 512) return CMP_ERR_INVALID;
  if (sh->rope_head_dim != 64) return CMP_ERR_UNSUPPORTED;
  if (sh->block_size < 1 || sh->block_size > 1024) return CMP_ERR_INVALID;
  if (sh->num_blocks < 1) return CMP_ERR_INVALID;
  const int coff = sh->ratio == 4 ? 2 : 1;
  if (sh->table_stride < (coff * sh->ratio + sh->block_size - 1) / sh->block_size)
    return CMP_ERR_INVALID;
  cf->ratio = sh->ratio;
  cf->coff = coff;
  cf->bm = 256;
  cf->D = sh->head_dim;
  cf->H = sh->hidden;
  cf->N = 2 * coff * sh->head_dim;
  cf->rope = sh->rope_head_dim;
  cf->rotate = sh->rotate ? 1 : 0;
  cf->bs = sh->block_size;
  cf->nblocks = sh->num_blocks;
  cf->stride = sh->table_stride;
  return CMP_OK;
}

// The kernel of each ratio (coff = 2 only at ratio 4).
template <int R>
constexpr int coff_of() { return R == 4 ? 2 : 1; }
template <int R, int WV>
const void* gemm_kernel_of() {
  return reinterpret_cast<const void*>(gemm_pool_kernel<R, coff_of<R>(), WV>);
}
// Calls f.template operator()<R>() for the compile-time ratio equal to r.
template <typename F>
void with_ratio(int r, F&& f) {
  switch (r) {
    case 2: f.template operator()<2>(); break;
    case 4: f.template operator()<4>(); break;
    case 8: f.template operator()<8>(); break;
    case 16: f.template operator()<16>(); break;
    case 32: f.template operator()<32>(); break;
    case 64: f.template operator()<64>(); break;
    default: f.template operator()<128>(); break;
  }
}

// Prefill tile height set by compressor_set_prefill_tile_rows (0: automatic).
std::atomic<int> g_tile_rows{0};

// Compute units of the current device (cached per device).
int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cus.size() <= dev) cus.resize(dev + 1, 0);
  if (cus[dev] == 0) {
    hipDeviceProp_t prop;
    cus[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount >= 8
                   ? prop.multiProcessorCount
                   : 256;
  }
  return cus[dev];
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// workgroups that check and pack the D x D Hadamard matrix (256 lane pieces
// of 8 values each): 128 for D = 512, 8 for D = 128
inline int hadamard_pack_wgs(const Cfg& cf) { return cf.rotate ? cf.D * cf.D / 8 / 256 : 0; }

struct PrefillLayout {
  size_t err, tiles, hadflag, plan, pooled, hadF, apet, staging, split, total;
};
// Workgroups of the setup launch that copy Ape transposed: ratios >= 8
// (coff = 1), R/4 slots each.
int ape_transpose_wgs(const Cfg& cf) { return cf.ratio >= 8 ? cf.ratio / 4 : 0; }
int prefill_max_tiles(int T, int B, int bm);
PrefillLayout prefill_layout(const Cfg& cf, int T, int B, int out_rows) {
  PrefillLayout L;
  size_t o = 0;
  L.err = 0;
  L.tiles = 4;    o += 256;                // error word, GEMM tile count, tile queues
  // one "Had is not a scaled Sylvester matrix" flag per packing workgroup
  L.hadflag = o;  o = align256(o + (size_t)hadamard_pack_wgs(cf) * 4);
  L.plan = o;     o = align256(o + (size_t)B * PL_WIDTH * 4);
  L.pooled = o;   o = align256(o + (size_t)out_rows * cf.D * 4);
  L.hadF = o;     o = align256(o + (cf.rotate ? (size_t)cf.D * cf.D * 2 : 0));
  L.apet = o;     o = align256(o + (size_t)ape_transpose_wgs(cf) * 4 * cf.coff * cf.D * 4);
  L.staging = o;  o = align256(o + (size_t)B * cf.coff * cf.ratio * 2 * cf.coff * cf.D * 4);
  // sized for the shorter tiles, whichever the call runs
  L.split = o;    o = align256(o + (cf.coff == 2 ? (size_t)prefill_max_tiles(T, B, 128) * 6 * cf.D * 4 : 0));
  L.total = o;
  return L;
}

// Upper bound of the M-tiles of a call with bm-row tiles (each request adds
// at most two to its share of T / bm).
int prefill_max_tiles(int T, int B, int bm) {
  return (T + bm - 1) / bm + 2 * B;
}

// decode split: KS K ranges per 32-column block, for about 512 GEMV
// workgroups (two per CU) with 4 to 8 k-steps per wave (8 waves per range;
// dec_wave_range cuts the H / 16 k-steps into 8 * KS nearly equal parts, so
// no part of K is left out for any H).  KS <= H / 512 <= DEC_MAX_KSPLIT.
int decode_ksplit(const Cfg& cf, int side_wgs) {
  const int ncb = cf.N / 32, KT = cf.H / 16;
  // workgroups beside the GEMV (pre-pooling) hold CU slots too:
  // with 64 KiB of LDS two workgroups fit a CU, and a GEMV workgroup that
  // finds no slot runs as a second wave
  const int budget = std::max(ncb, 512 - side_wgs);
  int ks = std::max(1, budget / ncb);
  ks = std::max(ks, (KT + 63) / 64);        // at most 8 k-steps per wave
  ks = std::min(ks, KT / 32);               // at least 4 k-steps per wave
  return std::max(1, std::min(ks, DEC_MAX_KSPLIT));
}
// k-steps of the longest wave range, and the run length that covers it
int decode_run(const Cfg& cf, int ks, int nrb) {
  const int KT = cf.H / 16;
  const int steps = (KT + 8 * ks - 1) / (8 * ks);
  return nrb == 2 || steps <= 4 ? 4 : 8;
}

// Two column blocks per GEMV workgroup over the same K range (the x rows of
// the range staged once for both): single-row-block calls with two channel
// sets, K split so that the GEMV and side workgroups number one per CU (the
// pair kernel's registers allow one 8-wave workgroup per CU).  At the 32-request
// C4A step (H = 7168: 224 GEMV + 32 pre-pooling workgroups) it took 13.18 ->
// 12.86 us per graph-replayed step against single-block workgroups (448 + 32,
// two per CU).
int decode_ksplit_pairs(const Cfg& cf, int side_wgs) {
  const int ngrp = cf.N / 64, KT = cf.H / 16;
  int ks = std::max(1, (256 - side_wgs) / ngrp);
  ks = std::max(ks, (KT + 63) / 64);        // at most 8 k-steps per wave
  ks = std::min(ks, KT / 32);               // at least 4 k-steps per wave
  return std::max(1, std::min(ks, DEC_MAX_KSPLIT));
}
bool decode_pairs(const Cfg& cf, int nrb, int side_wgs) {
  if (nrb != 1 || cf.coff != 2 || side_wgs >= 256) return false;
  const int ks = decode_ksplit_pairs(cf, side_wgs);
  // only when every workgroup gets a CU in the first round (H up to 8192
  // with 32 side workgroups); otherwise single blocks, two per CU
  return side_wgs + cf.N / 64 * ks <= 256 && decode_run(cf, ks, 1) == 8;
}

constexpr int kDecodeMaxBatch = 64;
constexpr int kDecodeMaxRows = 64;       // packed x rows of a decode call

struct DecodeLayout {
  size_t err, partial, pp, ppflag, rec, total;
  int ks, split;
};
DecodeLayout decode_layout(const Cfg& cf, int B) {
  DecodeLayout L;
  L.ks = decode_ksplit(cf, 0);             // the most K ranges any call uses
  with_ratio(cf.ratio, [&]<int R>() { L.split = dec_split<R>(); });
  size_t o = 0;
  L.err = o;       o += 256;
  L.partial = o;   o = align256(o + (size_t)L.ks * kDecodeMaxRows * cf.N * 4);
  L.pp = o;        o = align256(o + (size_t)B * DEC_MAX_WIN * L.split * 3 * cf.D * 4);
  L.ppflag = o;    o = align256(o + (size_t)B * DEC_MAX_WIN * L.split * 4);
  L.rec = o;       o = align256(o + (size_t)(B + 1) * sizeof(DecRec));
  L.total = o;
  return L;
}

int check_args(const Cfg& cf, const compressor_args* a, bool decode, bool own_workspace = true) {
  if (!a) return CMP_ERR_NULLPTR;
  if (a->batch < 1 || a->T < 0) return CMP_ERR_INVALID;
  if (a->out_rows < 0) return CMP_ERR_OUT_ROWS;
  if (a->T > 0 && !a->x) return CMP_ERR_NULLPTR;
  if (!a->kv_state || !a->score_state || !a->state_block_table || !a->w_packed || !a->ape ||
      !a->norm_weight || (own_workspace && !a->workspace))
    return CMP_ERR_NULLPTR;
  // with no output rows nothing reads the rotary tables or writes out
  if (a->out_rows > 0 && (!a->out || !a->sin || !a->cos)) return CMP_ERR_NULLPTR;
  if (cf.rotate && !a->hadamard) return CMP_ERR_NULLPTR;
  if (decode) {
    if (!a->cu_seqlens && a->T != a->batch) return CMP_ERR_INVALID;
    if (a->batch > kDecodeMaxBatch || a->T > kDecodeMaxRows) return CMP_ERR_UNSUPPORTED;
  } else if (!a->cu_seqlens && a->T % a->batch) {
    return CMP_ERR_INVALID;
  }
  return CMP_OK;
}

// Kernels that use more than the default 64 KiB of dynamic LDS: the limit is
// raised once per device (the first call on each device, with it current).
static hipError_t set_lds_limits() {
  hipError_t e1 = hipSuccess;
  for (int r = 2; r <= 128; r *= 2)
    with_ratio(r, [&]<int R>() {
      const hipError_t e8 = hipFuncSetAttribute(gemm_kernel_of<R, 8>(),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                Gm<8>::LDS_BYTES);
      const hipError_t e4 = hipFuncSetAttribute(gemm_kernel_of<R, 4>(),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                Gm<4>::LDS_BYTES);
      if (e1 == hipSuccess) e1 = e8 != hipSuccess ? e8 : e4;
    });
  const void* posts[4] = {reinterpret_cast<const void*>(post_kernel<8, 32>),
                          reinterpret_cast<const void*>(post_kernel<8, 16>),
                          reinterpret_cast<const void*>(post_kernel<2, 32>),
                          reinterpret_cast<const void*>(post_kernel<2, 16>)};
  hipError_t e2 = hipSuccess;
  for (int i = 0; i < 4; ++i) {
    const hipError_t e = hipFuncSetAttribute(posts[i], hipFuncAttributeMaxDynamicSharedMemorySize,
                                             POST_ROWS * (i < 2 ? 512 : 128) * 2);
    if (e2 == hipSuccess) e2 = e;
  }
  return e1 != hipSuccess ? e1 : e2;
}
int ensure_lds_limits() {
  static std::mutex mu;
  static std::vector<char> done;                 // per device: 0 not yet, 1 set, 2 failed
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CMP_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)done.size() <= dev) done.resize(dev + 1, 0);
  if (done[dev] == 0) done[dev] = set_lds_limits() == hipSuccess ? 1 : 2;
  return done[dev] == 1 ? CMP_OK : CMP_ERR_HIP;
}

// One decode call on workspace ws (at least decode_layout(...).total bytes);
// err2, if not NULL, also receives the tails' error bits.
int decode_impl(Cfg cf, const DecodeLayout& L, const compressor_args* a, uint8_t* ws,
                uint32_t* err2, hipStream_t st) {
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + L.err);
  float* partial = reinterpret_cast<float*>(ws + L.partial);
  float* pp = reinterpret_cast<float*>(ws + L.pp);
  int32_t* ppflag = reinterpret_cast<int32_t*>(ws + L.ppflag);
  DecRec* rec = reinterpret_cast<DecRec*>(ws + L.rec);
  const int32_t* kvt = a->kv_block_table ? a->kv_block_table : a->state_block_table;
  const int B = a->batch;
  const int T = a->T;
  const uint16_t* cosv = static_cast<const uint16_t*>(a->cos);
  const uint16_t* sinv = static_cast<const uint16_t*>(a->sin);
  // the most windows a request can complete: its tokens (one without
  // cu_seqlens, else at most 4 and at most T) span ceil(tokens / ratio)
  const int max_tok = a->cu_seqlens ? std::min(T, DEC_MAX_TOK) : 1;
  const int nwin = std::max(1, std::min(DEC_MAX_WIN, (max_tok + cf.ratio - 1) / cf.ratio));
  const int side = B * nwin * L.split;
  const int nrb = T <= 32 ? 1 : 2;
  const bool pairs = decode_pairs(cf, nrb, side);
  const int ks = pairs ? decode_ksplit_pairs(cf, side) : decode_ksplit(cf, side);
  const dim3 gg(side + cf.N / 32 / (pairs ? 2 : 1) * ks);
  const int run = decode_run(cf, ks, nrb);
  CMP_TRY(launch("decode_main", st, [&] {
    const uint16_t* X = static_cast<const uint16_t*>(a->x);
    const uint16_t* W = static_cast<const uint16_t*>(a->w_packed);
    decltype(&decode_main_kernel<1, 8, 4, 2, 1>) kern = nullptr;
    with_ratio(cf.ratio, [&]<int R>() {
      constexpr int C = coff_of<R>();
      if constexpr (C == 2) {
        if (pairs) { kern = decode_main_kernel<1, 8, R, C, 2>; return; }
      }
      kern = nrb == 2 ? decode_main_kernel<2, 4, R, C, 1>
                      : (run == 8 ? decode_main_kernel<1, 8, R, C, 1>
                                  : decode_main_kernel<1, 4, R, C, 1>);
    });
    hipLaunchKernelGGL(kern, gg, dim3(GV_THREADS), 0, st, cf, X, W, partial, B, T, nwin, ks,
                       a->cu_seqlens, a->seqused, a->start_pos, a->kv_state, a->score_state, kvt,
                       a->state_block_table, pp, ppflag, rec, err);
  }));
  return launch("decode_tail", st, [&] {
    const uint16_t* gamma = static_cast<const uint16_t*>(a->norm_weight);
    const uint16_t* had = static_cast<const uint16_t*>(a->hadamard);
    uint16_t* out = static_cast<uint16_t*>(a->out);
    if (a->cu_seqlens) {
      decltype(&decode_tail_kernel<4, 2, 8>) tail = nullptr;
      with_ratio(cf.ratio, [&]<int R>() {
        constexpr int C = coff_of<R>();
        tail = ks == 7 ? decode_tail_kernel<R, C, 7>
               : ks <= 8 ? decode_tail_kernel<R, C, 8>
                         : (ks <= 16 ? decode_tail_kernel<R, C, 16>
                                     : decode_tail_kernel<R, C, DEC_MAX_KSPLIT>);
      });
      hipLaunchKernelGGL(tail, dim3(B + 1), dim3(TL_THREADS), 0, st, cf, partial, ks, B, T,
                         a->cu_seqlens, a->seqused, a->start_pos, a->ape, a->kv_state,
                         a->score_state, kvt, a->state_block_table, pp, ppflag, gamma, cosv,
                         sinv, had, out, a->out_rows, err, err2);
    } else {
      // the tail loads a fixed number of K ranges (>= ks, <= DEC_MAX_KSPLIT;
      // exactly 7, the split of the ratio-4 column-pair layout at H = 7168)
      decltype(&decode_tail1_kernel<4, 2, 8>) tail = nullptr;
      with_ratio(cf.ratio, [&]<int R>() {
        constexpr int C = coff_of<R>();
        tail = ks == 7 ? decode_tail1_kernel<R, C, 7>
               : ks <= 8 ? decode_tail1_kernel<R, C, 8>
                         : (ks <= 16 ? decode_tail1_kernel<R, C, 16>
                                     : decode_tail1_kernel<R, C, DEC_MAX_KSPLIT>);
      });
      hipLaunchKernelGGL(tail, dim3(B + 1), dim3(TL_THREADS), 0, st, cf, partial, ks, B, rec,
                         a->ape, a->kv_state, a->score_state, pp, ppflag, gamma, cosv, sinv, had,
                         out, a->out_rows, err, err2);
    }
  });
}

}  // namespace

// Scratch of compressor_decode_noalloc: a fixed per-device array in place of
// the caller's workspace.  Every decode workspace fits (decode calls are
// bounded: batch <= 64, T <= 64; the largest layout, D = 512 at ratio 128
// with H = 10240, needs under 12 MiB).  In host code the array's name is only
// a stand-in for the symbol: its device address, taken per device with
// hipGetSymbolAddress at the first call on that device, is what the kernels
// get.
static __device__ __align__(256) uint8_t scratch[CMP_DECODE_SCRATCH_BYTES];

static int scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return CMP_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)ptrs.size() <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CMP_ERR_HIP;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return CMP_OK;
}

extern "C" {

int compressor_set_prefill_tile_rows(int32_t rows) {
  if (rows != 0 && rows != 128 && rows != 256) return CMP_ERR_INVALID;
  g_tile_rows.store(rows, std::memory_order_relaxed);
  return CMP_OK;
}

const char* compressor_status_str(int status) {
  switch (status) {
    case CMP_OK: return "ok";
    case CMP_ERR_NULLPTR: return "a required pointer is NULL";
    case CMP_ERR_INVALID: return "shape or range violation";
    case CMP_ERR_UNSUPPORTED: return "unsupported configuration";
    case CMP_ERR_WORKSPACE: return "workspace too small";
    case CMP_ERR_OUT_ROWS: return "out_rows too small";
    case CMP_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int compressor_prefill_workspace_size(const compressor_shape* shape, int32_t T, int32_t batch,
                                      int32_t out_rows, size_t* bytes) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  if (!bytes) return CMP_ERR_NULLPTR;
  if (T < 0 || batch < 1 || out_rows < 0) return CMP_ERR_INVALID;
  *bytes = prefill_layout(cf, T, batch, out_rows).total;
  return CMP_OK;
}

int compressor_decode_workspace_size(const compressor_shape* shape, int32_t batch,
                                     int32_t out_rows, size_t* bytes) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  if (!bytes) return CMP_ERR_NULLPTR;
  if (batch < 1 || out_rows < 0) return CMP_ERR_INVALID;
  if (batch > kDecodeMaxBatch) return CMP_ERR_UNSUPPORTED;
  *bytes = decode_layout(cf, batch).total;
  return CMP_OK;
}

int compressor_pack_weights(const compressor_shape* shape, const void* wkv, const void* wgate,
                            void* w_packed, void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  if (!wkv || !wgate || !w_packed) return CMP_ERR_NULLPTR;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launch("pack", st, [&] {
    hipLaunchKernelGGL(pack_weights_kernel, dim3(cf.N), dim3(256), 0, st, cf,
                       static_cast<const uint16_t*>(wkv), static_cast<const uint16_t*>(wgate),
                       static_cast<uint16_t*>(w_packed));
  });
}

int compressor_state_init(const compressor_shape* shape, float* kv_state, float* score_state,
                          void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  if (!kv_state || !score_state) return CMP_ERR_NULLPTR;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long n = (long)cf.nblocks * cf.bs * cf.coff * cf.D;
  CMP_TRY(launch("state_fill", st, [&] {
    hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, st, kv_state, n, 0.f);
  }));
  return launch("state_fill", st, [&] {
    hipLaunchKernelGGL(fill_kernel, dim3(1024), dim3(256), 0, st, score_state, n, -INFINITY);
  });
}

int compressor_state_reset(const compressor_shape* shape, float* kv_state, float* score_state,
                           const int32_t* kv_block_table, const int32_t* state_block_table,
                           const int32_t* rows, int32_t n, int32_t table_rows,
                           uint32_t* device_error, void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  if (n < 0) return CMP_ERR_INVALID;
  if (n == 0) return CMP_OK;
  if (table_rows < 1) return CMP_ERR_INVALID;
  if (!kv_state || !score_state || !state_block_table || !rows) return CMP_ERR_NULLPTR;
  const int32_t* kvt = kv_block_table ? kv_block_table : state_block_table;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int used = (cf.coff * cf.ratio + cf.bs - 1) / cf.bs;
  return launch("state_fill", st, [&] {
    hipLaunchKernelGGL(reset_rows_kernel, dim3(used, n), dim3(256), 0, st, cf, kv_state,
                       score_state, kvt, state_block_table, rows, table_rows, device_error);
  });
}

int compressor_prefill(const compressor_shape* shape, const compressor_args* a, void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  CMP_TRY(check_args(cf, a, false));
  const PrefillLayout L = prefill_layout(cf, a->T, a->batch, a->out_rows);
  if (a->workspace_bytes < L.total) return CMP_ERR_WORKSPACE;
  CMP_TRY(ensure_lds_limits());
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  uint32_t* err = reinterpret_cast<uint32_t*>(ws + L.err);
  int32_t* tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  uint32_t* had_flags = reinterpret_cast<uint32_t*>(ws + L.hadflag);
  int32_t* plan = reinterpret_cast<int32_t*>(ws + L.plan);
  float* pooled = reinterpret_cast<float*>(ws + L.pooled);
  uint16_t* hadF = reinterpret_cast<uint16_t*>(ws + L.hadF);
  float* staging = reinterpret_cast<float*>(ws + L.staging);
  float* apet = reinterpret_cast<float*>(ws + L.apet);
  float* split = reinterpret_cast<float*>(ws + L.split);
  const int32_t* kvt = a->kv_block_table ? a->kv_block_table : a->state_block_table;
  const int B = a->batch, T = a->T;
  // GEMM tile height: 256 rows (8 waves), or 128 (4 waves) when the call is
  // too short to give every CU a 256-row tile
  const int tiles_n = cf.N / GM_BN;
  const int cus = device_cu_count() / 8 * 8;
  const int forced = g_tile_rows.load(std::memory_order_relaxed);
  cf.bm = forced ? forced : (long)((T + 255) / 256) * tiles_n < cus ? 128 : 256;

  const int nhad = hadamard_pack_wgs(cf);
  const int napet = T > 0 ? ape_transpose_wgs(cf) : 0;
  const int nstage = T > 0 ? B * cf.coff * cf.ratio : 0;
  CMP_TRY(launch("setup", st, [&] {
    hipLaunchKernelGGL(setup_kernel, dim3(1 + nhad + napet + nstage), dim3(SETUP_THREADS), 0, st,
                       cf, a->cu_seqlens, a->seqused, a->start_pos, B, T, a->out_rows, plan, tiles,
                       err, static_cast<const uint16_t*>(a->hadamard), hadF, had_flags, nhad,
                       a->ape, apet, napet, a->kv_state, a->score_state, kvt,
                       a->state_block_table, staging);
  }));
  if (T > 0) {
    // persistent: one workgroup per CU (a multiple of 8, one run of tiles
    // per XCD), never more than there are tiles
    const long nwg = (long)prefill_max_tiles(T, B, cf.bm) * tiles_n;
    const int grid = int(std::min<long>(cus, (nwg + 7) / 8 * 8));
    CMP_TRY(launch("gemm", st, [&] {
      decltype(&gemm_pool_kernel<4, 2, 8>) kern = nullptr;
      with_ratio(cf.ratio, [&]<int R>() {
        kern = cf.bm == 128 ? gemm_pool_kernel<R, coff_of<R>(), 4>
                            : gemm_pool_kernel<R, coff_of<R>(), 8>;
      });
      const int threads = cf.bm == 128 ? Gm<4>::THREADS : Gm<8>::THREADS;
      const int lds = cf.bm == 128 ? Gm<4>::LDS_BYTES : Gm<8>::LDS_BYTES;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, cf,
                         static_cast<const uint16_t*>(a->x),
                         static_cast<const uint16_t*>(a->w_packed), T, B, plan, tiles, a->ape,
                         apet, staging, a->kv_state, a->score_state, kvt, a->state_block_table,
                         pooled, a->out_rows, split, err);
    }));
  }
  if (a->out_rows > 0) {
    // 16-row workgroups when 32-row ones would not give every CU one
    const bool short_call = (a->out_rows + POST_ROWS - 1) / POST_ROWS <= device_cu_count();
    const int pr = short_call ? 16 : POST_ROWS;
    const dim3 qg((a->out_rows + pr - 1) / pr);
    const int lds = cf.rotate ? POST_ROWS * cf.D * 2 : 0;
    CMP_TRY(launch("post", st, [&] {
      decltype(&post_kernel<8, 32>) kern =
          cf.D == 512 ? (short_call ? post_kernel<8, 16> : post_kernel<8, 32>)
                      : (short_call ? post_kernel<2, 16> : post_kernel<2, 32>);
      hipLaunchKernelGGL(kern, qg, dim3(256), lds, st, cf, pooled, split, plan, B, a->out_rows,
                         static_cast<const uint16_t*>(a->norm_weight),
                         static_cast<const uint16_t*>(a->cos),
                         static_cast<const uint16_t*>(a->sin), hadF, had_flags, nhad,
                         static_cast<uint16_t*>(a->out));
    }));
  }
  return CMP_OK;
}

int compressor_decode(const compressor_shape* shape, const compressor_args* a, void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  CMP_TRY(check_args(cf, a, true));
  const DecodeLayout L = decode_layout(cf, a->batch);
  if (a->workspace_bytes < L.total) return CMP_ERR_WORKSPACE;
  return decode_impl(cf, L, a, static_cast<uint8_t*>(a->workspace), nullptr,
                     static_cast<hipStream_t>(stream));
}

int compressor_decode_noalloc(const compressor_shape* shape, const compressor_args* a,
                              uint32_t* device_error, void* stream) {
  Cfg cf;
  CMP_TRY(check_shape(shape, &cf));
  CMP_TRY(check_args(cf, a, true, false));
  const DecodeLayout L = decode_layout(cf, a->batch);
  if (L.total > CMP_DECODE_SCRATCH_BYTES) return CMP_ERR_WORKSPACE;
  void* ws = nullptr;
  CMP_TRY(scratch_address(&ws));
  return decode_impl(cf, L, a, static_cast<uint8_t*>(ws), device_error,
                     static_cast<hipStream_t>(stream));
}

int compressor_last_device_error(const void* workspace, void* stream, int32_t* code) {
  if (!workspace || !code) return CMP_ERR_NULLPTR;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return CMP_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return CMP_ERR_HIP;
  *code = int32_t(v);
  return CMP_OK;
}

int compressor_timing_enable(int32_t on) {
  if (on < 0 || on > 2) return CMP_ERR_INVALID;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& r : g_timing.recs) g_timing.spare.push_back({r.start, r.stop});
  g_timing.recs.clear();
  g_timing.on = on;
  return CMP_OK;
}

int compressor_timing_query(const char* kernel, int32_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return CMP_ERR_NULLPTR;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  int n = 0;
  double tot = 0.0;
  for (auto& r : g_timing.recs) {
    if (r.name != kernel) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return CMP_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return CMP_ERR_HIP;
    tot += ms;
    ++n;
  }
  *launches = n;
  *total_ms = tot;
  return CMP_OK;
}


int compressor_epilog(const void* rows, int32_t n_rows, int32_t head_dim,
                      const int32_t* slot_mapping, void* cache, float* cache_scale,
                      int64_t num_slots, uint32_t* device_error, void* stream) {
  if (n_rows < 0 || num_slots < 0 || head_dim <= 0 || head_dim % EPL_BLOCK || head_dim > 8192)
    return CMP_ERR_INVALID;
  const int nblk_row = head_dim / EPL_BLOCK;
  const long n_blocks = (long)n_rows * nblk_row;
  if (n_blocks > 0x7fffffffL - EPL_THREADS * EPL_GROUP_BLOCKS) return CMP_ERR_INVALID;
  if (n_rows == 0) return CMP_OK;
  if (!rows || !slot_mapping || !cache || !cache_scale) return CMP_ERR_NULLPTR;
  const long groups = (n_blocks + EPL_GROUP_BLOCKS - 1) / EPL_GROUP_BLOCKS;
  const long grid = (groups + EPL_THREADS / 16 - 1) / (EPL_THREADS / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch("epilog", s, [&] {
    hipLaunchKernelGGL(epilog_kernel, dim3((unsigned)grid), dim3(EPL_THREADS), 0, s,
                       static_cast<const uint16_t*>(rows), (int)n_blocks, nblk_row, slot_mapping,
                       static_cast<uint8_t*>(cache), cache_scale, (long)num_slots, device_error);
  });
}

int nsa_compress_with_cache(const nsa_shape* sh, const nsa_args* a, void* stream) {
  if (!sh || !a) return CMP_ERR_NULLPTR;
  // [NSA] 约束说明
  if (sh->head_num < 1 || sh->head_num > 64 || (sh->head_num > 50 && sh->head_num % 2))
    return CMP_ERR_UNSUPPORTED;
  if (sh->head_dim < 16 || sh->head_dim > 256 || sh->head_dim % 16) return CMP_ERR_UNSUPPORTED;
  const int st = sh->compress_stride, cb = sh->compress_block_size;
  if (st != 16 && st != 32 && st != 48 && st != 64) return CMP_ERR_UNSUPPORTED;
  if (cb % 16 || cb < st || cb > 64) return CMP_ERR_UNSUPPORTED;
  if (sh->page_block_size != 64 && sh->page_block_size != 128) return CMP_ERR_UNSUPPORTED;
  if (sh->dtype != NSA_BF16 && sh->dtype != NSA_F16) return CMP_ERR_UNSUPPORTED;
  if (sh->layout != NSA_LAYOUT_PAGED && sh->layout != NSA_LAYOUT_TND) return CMP_ERR_UNSUPPORTED;
  if (!a->input || !a->weight || !a->slot_mapping || !a->act_seq_len || !a->output_cache)
    return CMP_ERR_NULLPTR;
  if (a->batch < 1 || a->result_len < 1) return CMP_ERR_INVALID;
  const bool paged = sh->layout == NSA_LAYOUT_PAGED;
  if (paged) {
    if (!a->block_table) return CMP_ERR_NULLPTR;
    if (a->table_stride < 1 || a->num_blocks < 1) return CMP_ERR_INVALID;
  } else if (a->T < 0) {
    return CMP_ERR_INVALID;
  }
  NsaCfg cf{sh->head_num, sh->head_dim, cb, st, sh->page_block_size, sh->dtype == NSA_F16,
            paged ? 1 : 0};
  const long E = (long)sh->head_num * sh->head_dim;
  const dim3 grid(a->batch, (unsigned)((E + NSA_CHUNK - 1) / NSA_CHUNK));
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch("nsa", s, [&] {
    auto kern = cb == 16 ? nsa_compress_kernel<16>
                : cb == 32 ? nsa_compress_kernel<32>
                : cb == 48 ? nsa_compress_kernel<48> : nsa_compress_kernel<64>;
    hipLaunchKernelGGL(kern, grid, dim3(NSA_THREADS), 0, s, cf,
                       static_cast<const uint16_t*>(a->input),
                       static_cast<const uint16_t*>(a->weight), a->slot_mapping, a->act_seq_len,
                       a->block_table, a->batch, a->table_stride, a->num_blocks, (long)a->T,
                       static_cast<uint16_t*>(a->output_cache), (long)a->result_len,
                       a->device_error);
  });
}

}  // extern "C"
