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
// ln x through the hardware base-2 logarithm (v_log_f32).
__device__ __forceinline__ float log_fast(float x) {
  return __builtin_amdgcn_logf(x) * kLn2;
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

// DPP lane moves inside one 16-lane row.  The four steps below visit every
// lane of the row once, so folding a commutative, associative combine over
// them leaves the row's reduction in all 16 lanes:
//   xor 1 and xor 2 inside each quad (quad_perm), then rotate the row by 4
//   and by 8 lanes (row_ror).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowRor4>(v);
  v += dpp_f<kDppRowRor8>(v);
  return v;
}
// (max, index of the max) with the lowest index winning ties.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& m, int& a) {
  const float om = dpp_f<CTRL>(m);
  const int oa = dpp_i<CTRL>(a);
  const bool take = om > m || (om == m && oa < a);
  m = take ? om : m;
  a = take ? oa : a;
}
__device__ __forceinline__ void row16_argmax(float& m, int& a) {
  argmax_step<kDppQuadXor1>(m, a);
  argmax_step<kDppQuadXor2>(m, a);
  argmax_step<kDppRowRor4>(m, a);
  argmax_step<kDppRowRor8>(m, a);
}

// Orders this wave's LDS traffic: everything issued before completes before
// anything after it is issued or scheduled.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

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
