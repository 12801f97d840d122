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

// ---------------------------------------------------------------------------
// LDS tiles.  A tile holds R rows of D bf16 (row-major, no padding); the
// 16-byte chunk c of row r is stored at chunk position c ^ swz(r).  The XOR
// pattern is chosen so that both access patterns used by the kernels are free
// of bank conflicts on gfx950's 64-bank LDS:
//   * 16-byte row reads by 16 consecutive lanes (16 rows, one chunk), and
//   * transpose reads (ds_read_b64_tr_b16) by a half-wave: 4 consecutive rows
//     times 4 consecutive chunks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) {
    return ((row >> 2) & 3) | (((row >> 1) & 1) << 2);  // 8 chunks per row
  } else {
    return ((row & 3) << 2) | ((row >> 2) & 3);          // >= 16 chunks per row
  }
}

// Element offset of (row, col) in a swizzled tile; col may be any element
// index (the low 3 bits select inside the 16-byte chunk).
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// ds_read_b64_tr_b16: within each 16-lane group, output lane i receives
// element (i & 3) of the 8-byte words addressed by lanes 4k + (i >> 2),
// k = 0..3 of its group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// A operand (32 x 16) whose rows are 32 consecutive tile rows r0.. and whose
// k-slots are 16 consecutive columns k0..: one 16-byte read per lane.
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const bf16_t* tile, int r0, int k0, int c32, int h) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D>(r0 + c32, k0 + 8 * h));
}

// A operand (32 x 16) that is the TRANSPOSE of a tile block: its rows are 32
// consecutive tile columns c0.. and its k-slots are 16 tile rows r0..r0+15,
// slot e of half h being row r0 + 8*(e>>2) + 4*h + (e&3).  Two transpose
// reads (rows r0+4h.. and r0+8+4h..), each a 4-row x 16-column block per
// 16-lane group.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const bf16_t* tile, int r0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = r0 + 4 * (g >> 1) + (s >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (s & 3);
  const bf16x4 lo = lds_read_tr16(tile + tile_off<D>(row, col));
  const bf16x4 hi = lds_read_tr16(tile + tile_off<D>(row + 8, col));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Buffer loads: a resource covering one head's [N, D] tensor; reads at byte
// offsets at or beyond `bytes` return zeros (hardware range check), so tails
// need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Sum of the two bf16 products a.x*b.x + a.y*b.y accumulated into c (fp32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

}  // namespace fa
