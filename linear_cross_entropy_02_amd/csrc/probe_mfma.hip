// Throughput probe of the bf16 matrix instructions alone, for the roofline
// of the fused cross-entropy kernels: a grid of 4-wave blocks in which every
// wave streams v_mfma_f32_16x16x32_bf16 (16 independent 4-float fragments) or
// v_mfma_f32_32x32x16_bf16 (8 independent 16-float fragments) over operands
// held in registers, with no memory traffic in the loop.
// The operands are either pseudo-random bf16 values (full mantissas, both
// signs, varying per lane and per fragment) or zeros, since the MFMA units'
// power -- and hence the clock the chip sustains -- depends on the operand
// bits.  The rate it reaches is what the GEMM kernels' MFMA-busy fraction
// is measured against.  Built as its own library (libflce_probe.so); the
// fused path does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flce_probe.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef int i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Random bf16 pair with a normal exponent range (|x| in [2^-8, 2^8)): no
// NaN, infinity or denormal, so every product is an ordinary one.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t h) {
  const uint32_t lo = ((h & 0x807fu) | ((119u + ((h >> 8) & 15u)) << 7)) & 0xffffu;
  const uint32_t g = mix(h);
  const uint32_t hi = ((g & 0x807fu) | ((119u + ((g >> 8) & 15u)) << 7)) & 0xffffu;
  return lo | (hi << 16);
}

// Random operand registers of one lane: 4 A and 4 B fragments of 8 bf16 each.
__device__ __forceinline__ __attribute__((unused)) void make_operands(int random_operands, i4 (&a)[4], i4 (&b)[4]) {
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 0x9e3779b9u;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[f][r] = random_operands ? (int)bf16_pair(mix(seed + 8u * f + r)) : 0;
      b[f][r] = random_operands ? (int)bf16_pair(mix(seed + 8u * f + r + 4u)) : 0;
    }
}

// 16 x 16 x 32: 16 accumulators, so each one is reused every 16 issues (far
// beyond the instruction's latency); A changes every issue, B every fourth.
__global__ void __launch_bounds__(256) mfma16_stream_kernel(int iters, int random_operands,
                                                            float* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  i4 a[4], b[4];
  make_operands(random_operands, a, b);
  f4 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = (f4){0.f, 0.f, 0.f, 0.f};
  // the VALU writes of the operands must be two wait states from the asm
  // MFMAs that read them (the hazard recognizer does not see inside asm)
  asm volatile("s_nop 4" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                   : "+a"(acc[k])
                   : "v"(a[k & 3]), "v"(b[(k >> 2) & 3]));
  }
  // drain the MFMA pipe before the accumulators are read
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int k = 0; k < 16; ++k) asm volatile("" : "+a"(acc[k]));
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
#endif
}

// 32 x 32 x 16: 8 accumulators of 16 floats (128 AGPRs), reused every 8
// issues; A changes every issue, B every second.
__global__ void __launch_bounds__(256) mfma32_stream_kernel(int iters, int random_operands,
                                                            float* __restrict__ sink) {
#if defined(__HIP_DEVICE_COMPILE__)
  i4 a[4], b[4];
  make_operands(random_operands, a, b);
  f16v acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  asm volatile("s_nop 4" ::: "memory");
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(acc[k])
                   : "v"(a[k & 3]), "v"(b[(k >> 1) & 3]));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int k = 0; k < 8; ++k) asm volatile("" : "+a"(acc[k]));
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
#endif
}

}  // namespace

extern "C" {

int32_t flce_probe_mfma_stream(int32_t shape, int32_t blocks, int32_t iters,
                               int32_t random_operands, float* sink, void* stream) {
  if ((shape != 16 && shape != 32) || blocks <= 0 || iters <= 0 || !sink) return 1;
  if (shape == 16)
    hipLaunchKernelGGL(mfma16_stream_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       iters, random_operands, sink);
  else
    hipLaunchKernelGGL(mfma32_stream_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       iters, random_operands, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double flce_probe_mfma_flops(int32_t shape, int32_t blocks, int32_t iters) {
  // per wave and iteration: 16 issues of 16x16x32 or 8 of 32x32x16, i.e.
  // 2 * 16 * 16 * 32 * 16 = 2 * 32 * 32 * 16 * 8 flops either way
  if (shape != 16 && shape != 32) return 0.0;
  return 4.0 * blocks * (double)iters * 2.0 * 16 * 16 * 32 * 16;
}

}  // extern "C"
