// Device-side helpers shared by the Parallax HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family parts.
constexpr int kBufferRsrcWord3 = 0x00020000;
// s_waitcnt immediate for "vmcnt(0)" with expcnt and lgkmcnt left unconstrained
// (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8,
// vmcnt[5:4] bits 15:14).
constexpr int kWaitVmcnt0 = 0x0F70;
// Running-max sentinel: finite, so that exp2(sentinel - m) is 0 and
// exp2(sentinel - sentinel) is 1 without NaN from -inf - -inf.
constexpr float kMinit = -1.0e30f;

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane moves inside a row of 16 lanes (CDNA DPP control codes).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;    // lane i <-> 15-i inside each 16 lanes

// Sum over aligned groups of N consecutive lanes (N in {4,8,16,32});
// every lane of a group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// 16 bytes per lane from base + voff into LDS at lds + 16 * lane (lds must be
// wave-uniform), through a raw buffer descriptor of `bytes` bytes: lanes whose
// offset is at or past `bytes` write zeros.  (buffer_load_dwordx4 ... lds)
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, void* lds,
                                                  uint32_t voff) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 0);
}

struct Max {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// op(x[lane], x[lane ^ 16]) and op(x[lane], x[lane ^ 32]) for a commutative op.
// With PLX_PERMLANE_SWAP the exchange uses gfx950's v_permlane{16,32}_swap (a
// VALU operation: each lane ends up holding both values of its pair across the
// two results); otherwise a cross-lane shuffle through the LDS crossbar.
#ifndef PLX_PERMLANE_SWAP
#define PLX_PERMLANE_SWAP 1
#endif
template <class Op>
__device__ __forceinline__ float lane_xor16(float x, Op op) {
#if PLX_PERMLANE_SWAP
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
  return op(x, __shfl_xor(x, 16));
#endif
}
template <class Op>
__device__ __forceinline__ float lane_xor32(float x, Op op) {
#if PLX_PERMLANE_SWAP
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
  return op(x, __shfl_xor(x, 32));
#endif
}

}  // namespace plx
