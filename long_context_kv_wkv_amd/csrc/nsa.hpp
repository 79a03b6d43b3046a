// NSA KV compression (NsaCompressWithCache, [NSA] 计算公式): for every batch
// whose length s triggers (s >= cbs, (s - cbs) % stride == 0), the
// head-weighted sum of its last cbs tokens, written to its output slot.
//
// HBM-bound gather and reduce: each workgroup takes one batch and 2048
// consecutive elements of the N x D token row (8 per thread, one head per
// thread since D % 16 == 0); a thread issues its loads 32 tokens at a time
// (16-byte loads, coalesced along D), accumulates in fp32 in token order and
// stores 16 bytes rounded nearest-even.  The window spans at most two pages
// (cbs <= 64 <= page size), so the block table is read once per page.
#pragma once
#include "common.hpp"

namespace cmp {

struct NsaCfg {
  int N, D, cbs, stride, page, f16, paged;
};

constexpr int NSA_THREADS = 256;
constexpr int NSA_PER_THREAD = 8;
constexpr int NSA_CHUNK = NSA_THREADS * NSA_PER_THREAD;   // elements per workgroup

__device__ __forceinline__ float nsa_to_f32(uint16_t v, int f16) {
  if (f16) {
    _Float16 h;
    __builtin_memcpy(&h, &v, 2);
    return (float)h;
  }
  return bf2f(v);
}
__device__ __forceinline__ uint16_t nsa_from_f32(float x, int f16) {
  if (f16) {
    const _Float16 h = (_Float16)x;            // nearest-even
    uint16_t v;
    __builtin_memcpy(&v, &h, 2);
    return v;
  }
  return f2bf(x);
}

template <int CBS>
__global__ __launch_bounds__(NSA_THREADS) void nsa_compress_kernel(
    NsaCfg cf, const uint16_t* __restrict__ in, const uint16_t* __restrict__ w,
    const int32_t* __restrict__ slot_mapping, const int64_t* __restrict__ act,
    const int32_t* __restrict__ table, int /*batch: the grid's x*/, int table_stride, int num_blocks, long T,
    uint16_t* __restrict__ out, long result_len, uint32_t* __restrict__ err) {
  __shared__ long s_cu;
  __shared__ int32_t s_tab[NSA_THREADS];
  const int b = blockIdx.x;
  const long E = (long)cf.N * cf.D;
  // a table row of at most NSA_THREADS entries is read whole, together with
  // the batch's length and slot, so that the page lookup below is no second
  // dependent round trip
  const bool tab_lds = cf.paged && table_stride <= NSA_THREADS;
  if (tab_lds && (int)threadIdx.x < table_stride)
    s_tab[threadIdx.x] = table[(long)b * table_stride + threadIdx.x];
  const int slot = slot_mapping[b];
  const long s = act[b];
  uint32_t bad = 0;
  if (s < 0) bad |= NSA_DEVERR_SEQLEN;
  const bool fires = s >= CBS && (s - CBS) % cf.stride == 0;
  // packed layout: the batch's first row is the sum of the earlier lengths
  long cu = 0;
  if (!cf.paged) {
    if (threadIdx.x == 0) s_cu = 0;
    __syncthreads();
    long part = 0;
    for (int j = threadIdx.x; j < b; j += NSA_THREADS) part += act[j] > 0 ? act[j] : 0;
    if (part) atomicAdd(reinterpret_cast<unsigned long long*>(&s_cu), (unsigned long long)part);
    __syncthreads();
    cu = s_cu;
  } else if (tab_lds) {
    __syncthreads();
  }
  const long e0 = ((long)blockIdx.y * NSA_THREADS + threadIdx.x) * NSA_PER_THREAD;
  if (!fires || bad) {
    if (bad && threadIdx.x == 0 && blockIdx.y == 0 && err) atomicOr(err, bad);
    return;
  }
  if (slot < 0 || slot >= result_len) bad |= NSA_DEVERR_SLOT;
  const long first = s - CBS;                    // compressIdx * stride
  long base0 = 0, base1 = 0;                     // element offsets of the window's pages
  long page0 = 0;
  if (cf.paged) {
    page0 = first / cf.page;
    const long page1 = (s - 1) / cf.page;
    if (page1 >= table_stride) {
      bad |= NSA_DEVERR_TABLE;
    } else {
      const int b0 = tab_lds ? s_tab[page0] : table[(long)b * table_stride + page0];
      const int b1 = tab_lds ? s_tab[page1] : table[(long)b * table_stride + page1];
      if (b0 < 0 || b0 >= num_blocks || b1 < 0 || b1 >= num_blocks) bad |= NSA_DEVERR_TABLE;
      base0 = (long)b0 * cf.page * E;
      base1 = (long)b1 * cf.page * E;
    }
  } else if (cu + s > T) {
    bad |= NSA_DEVERR_SEQLEN;
  }
  if (bad) {
    if (threadIdx.x == 0 && blockIdx.y == 0 && err) atomicOr(err, bad);
    return;
  }
  if (e0 >= E) return;
  const int n = (int)(e0 / cf.D);
  float acc[NSA_PER_THREAD];
#pragma unroll
  for (int i = 0; i < NSA_PER_THREAD; ++i) acc[i] = 0.f;
  // the window in batches of up to 32 tokens, every load of a batch in
  // flight before its first use (CBS is a compile-time constant)
#pragma unroll
  for (int j0 = 0; j0 < CBS; j0 += 32) {
    constexpr int NB0 = CBS < 32 ? CBS : 32;
    const int nb = CBS - j0 < NB0 ? CBS - j0 : NB0;   // 32, or the last 16
    uint4 v[NB0];
    float wj[NB0];
#pragma unroll
    for (int u = 0; u < NB0; ++u) {
      if (u >= nb) break;
      const long t = first + j0 + u;
      long off;
      if (cf.paged) {
        const long pg = t / cf.page;
        off = (pg == page0 ? base0 : base1) + (t - pg * cf.page) * E + e0;
      } else {
        off = (cu + t) * E + e0;
      }
      v[u] = *reinterpret_cast<const uint4*>(in + off);
      wj[u] = nsa_to_f32(w[(long)(j0 + u) * cf.N + n], cf.f16);
    }
#pragma unroll
    for (int u = 0; u < NB0; ++u) {
      if (u >= nb) break;
      const uint32_t q[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(nsa_to_f32(uint16_t(q[i] & 0xFFFFu), cf.f16), wj[u], acc[2 * i]);
        acc[2 * i + 1] = fmaf(nsa_to_f32(uint16_t(q[i] >> 16), cf.f16), wj[u], acc[2 * i + 1]);
      }
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = uint32_t(nsa_from_f32(acc[2 * i], cf.f16)) |
           (uint32_t(nsa_from_f32(acc[2 * i + 1], cf.f16)) << 16);
  *reinterpret_cast<uint4*>(out + (long)slot * E + e0) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace cmp
