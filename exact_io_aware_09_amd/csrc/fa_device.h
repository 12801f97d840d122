// fa_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Matrix-core operand layout used throughout (v_mfma_f32_32x32x16_bf16,
// one 64-lane wavefront; lane = l, half h = l >> 5, column c = l & 31):
//   A (32 x 16, row-major M x K): lane l supplies row c, k-slots 8h .. 8h+7
//   B (16 x 32, K x N)          : lane l supplies column c, k-slots 8h .. 8h+7
//   D (32 x 32)                 : lane l holds column c; register r holds
//                                 row 8*(r>>2) + 4*h + (r&3)
// A and B use the same k-slot assignment, so any consistent relabelling of
// the contraction index across the two operands leaves D unchanged; the
// kernels use that freedom to feed a D fragment (scores) straight back in as
// the B operand of the next contraction without a trip through LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of bfloat16 tensors

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ float bf16_to_f32(bf16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// Workgroup -> logical tile index such that consecutive logical tiles land on
// the same XCD.  Hardware hands workgroup w to XCD (w mod 8); a bijection
// maps it to a contiguous run of logical indices per XCD, so all Q blocks of
// one (batch, head) share one L2 while that head's K/V are being re-read.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total / kNumXcd, r = total % kNumXcd;
  const int x = w % kNumXcd, idx = w / kNumXcd;
  return x * q + (x < r ? x : r) + idx;
}

// 16-byte global load returning zeros when `ok` is false.
__device__ __forceinline__ uint4 load16_or_zero(const bf16_t* p, bool ok) {
  if (ok) return *reinterpret_cast<const uint4*>(p);
  return make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace fa
