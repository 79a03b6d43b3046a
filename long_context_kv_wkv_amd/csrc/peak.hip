// Measured ceilings on the GPU the library runs on, for the roofline context
// of the benchmark (not part of the operator): a plain bf16 MFMA loop and a
// read-only HBM stream.  Both launch on the caller's stream and do no timing
// of their own; the caller brackets them with events.
//
//  * peak_mfma_bf16: every wave keeps four independent 32x32 fp32
//    accumulators and issues back-to-back v_mfma_f32_32x32x16_bf16 on
//    operands loaded once from `seed` (so the matrix cores see the bit
//    patterns of the caller's data, e.g. N(0, 1) bf16, not constants:
//    operand values change the chip's power draw and with it its clock).
//    Work: blocks * 4 waves * iters * 4 MFMAs * 2*32*32*16 flops.  One
//    4-wave workgroup per CU (one wave per SIMD) measured highest: on
//    MI355X with N(0, 1) operands 1.63 PFLOP/s, against 1.32-1.37 with two
//    workgroups per CU and 1.44-1.47 with three (constant operands: 2.45,
//    1.63 and 1.75-1.83).
//  * peak_stream_read: reads `bytes` (a multiple of 16 KiB) once with
//    16-byte loads, four in flight per thread, and folds them into one word
//    that is stored only if it matches a constant (so no load is dropped).
#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pk_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // 4 waves

__global__ __launch_bounds__(kThreads) void mfma_loop(const pk_bf16x8* __restrict__ seed,
                                                      float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  pk_bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = seed[(wave * 8 + i) * 64 + lane];
    b[i] = seed[(wave * 8 + 4 + i) * 64 + lane];
  }
  pk_f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; it += 2) {       // iters even: 8 MFMAs per trip
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 1) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void stream_read(const uint4* __restrict__ p, size_t n16,
                                                        uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t step = (size_t)gridDim.x * kThreads * 4;
  for (size_t i = (size_t)blockIdx.x * kThreads * 4 + threadIdx.x; i < n16; i += step) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + (size_t)u * kThreads];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

// seed: at least 2048 bf16x8 values (32 KiB) in device memory; sink: blocks *
// 256 floats; iters even.  Returns 0, or a HIP error code.
extern "C" int peak_mfma_bf16(const void* seed, float* sink, int blocks, int iters, void* stream) {
  if (!seed || !sink || blocks < 1 || iters < 2 || iters % 2) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const pk_bf16x8*>(seed), sink, iters);
  return (int)hipGetLastError();
}

// buf: `bytes` of device memory, bytes a multiple of 16 KiB (each block
// iteration reads 4 x 256 x 16 bytes); sink: one word.
extern "C" int peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % (kThreads * 4 * 16) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}
