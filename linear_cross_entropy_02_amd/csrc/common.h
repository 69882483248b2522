// Device-side helpers shared by the fused linear cross-entropy kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 values are carried as their 16-bit patterns.
struct bf16 {
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// e^x through the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

template <typename T> struct Elem;
template <> struct Elem<bf16> {
  static constexpr int kVec = 8;  // elements per 16-byte vector
  __device__ __forceinline__ static float to_f32(bf16 v) {
    return __builtin_bit_cast(float, (uint32_t)v.bits << 16);
  }
  __device__ __forceinline__ static bf16 from_f32(float x) {
    // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(bf16, (__bf16)x);
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};

// Pack 8 floats into one 16-byte vector of bf16 (4 x v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint4 pack8_bf16(const float* v) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[0], v[1], 0, 0}.xy, bf16x2));
  r.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[2], v[3], 0, 0}.xy, bf16x2));
  r.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[4], v[5], 0, 0}.xy, bf16x2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f4){v[6], v[7], 0, 0}.xy, bf16x2));
  return r;
}
__device__ __forceinline__ void unpack8_bf16(uint4 p, float* v) {
  v[0] = __builtin_bit_cast(float, p.x << 16);
  v[1] = __builtin_bit_cast(float, p.x & 0xffff0000u);
  v[2] = __builtin_bit_cast(float, p.y << 16);
  v[3] = __builtin_bit_cast(float, p.y & 0xffff0000u);
  v[4] = __builtin_bit_cast(float, p.z << 16);
  v[5] = __builtin_bit_cast(float, p.z & 0xffff0000u);
  v[6] = __builtin_bit_cast(float, p.w << 16);
  v[7] = __builtin_bit_cast(float, p.w & 0xffff0000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// Block id -> logical block index such that consecutive logical blocks run
// on one XCD.  The hardware hands consecutive block ids to the 8 XCDs in
// turn, each with its own L2; blocks whose rows share cache lines should sit
// on the same one.  A bijection on [0, gridDim.x).
__device__ __forceinline__ int xcd_local_block() {
  const int nblk = (int)gridDim.x, bid = (int)blockIdx.x;
  const int q = nblk >> 3, r = nblk & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd * q + min(xcd, r) + slot;
}

// Valid target: not the ignore index and inside [0, V).  The equality test
// comes first, so the ignore index may be a real vocabulary id.
__device__ __forceinline__ bool target_valid(int64_t y, int64_t ignore_index, int64_t V) {
  return y != ignore_index && y >= 0 && y < V;
}

}  // namespace flce
