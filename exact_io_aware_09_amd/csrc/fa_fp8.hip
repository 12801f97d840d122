// fa_fp8.hip -- attention forward in 8-bit floating point with block
// quantisation, for gfx950.
//
// The third version of the kernel described in "Lecture 8 . GPU Performance
// & FlashAttention" (CS324 notes, section 8.1) and "FlashAttention and GPU
// memory" (section 11) runs attention in FP8 with block quantisation.  Here:
//
//  * Format: OCP E4M3 (v_cvt_pk_fp8_f32 on gfx950, round to nearest even).
//  * Blocks of 32 elements along the axis a product contracts over share one
//    power-of-two scale held as an 8-bit biased exponent (E8M0): 32
//    consecutive head dims of a Q or K row, 32 consecutive keys of one head
//    dim of V.  The exponent e is the smallest with amax <= 448 * 2^e, so no
//    element overflows.  These are exactly the blocks the scaled matrix
//    instruction v_mfma_scale_f32_32x32x64_f8f6f4 applies its per-lane scales
//    to, so dequantisation costs nothing.
//  * V is stored transposed (head dim major, keys contiguous, padded with
//    zeros to a multiple of 64 keys): the A operand of O^T += V^T P^T is then
//    two 16-byte reads per lane.
//
// Matrix instruction layout (32 x 32 x 64, measured): lane (c, h) supplies row
// (or column) c and the 32 contraction slots 16h .. 16h+15 and 32+16h ..
// 32+16h+15 (bytes 0-15 and 16-31 of its operand); the scale of the 32-slot
// block kb of row c is the one lane c + 32 kb holds.  The D fragment has the
// layout of every 32 x 32 instruction.
//
// Forward kernel: the second version's loop order (one block of 128 query
// rows per workgroup, loop over blocks of 64 keys, O divided once at the
// end), with the online softmax of the pages (a block's maximum raises the
// running maximum, O and l are rescaled), except that the running maximum
// is raised only when a block's maximum exceeds it by more than FA_FP8_LAG.
// The weights enter P V as E4M3 after scaling by 2^8 (e^(s - m) * 256 lies
// in (0, 2^8.75], so small weights keep 2^-17 of resolution relative to the
// row sum); the row sum is taken in fp32 before rounding.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kScaleOne = 127;  // E8M0 encoding of 2^0

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Smallest e with amax <= 448 * 2^e (0 for amax = 0), clamped to [-127, 127]:
// with amax = f 2^E, f in [0.5, 1), and 448 = 0.875 * 2^9, e = E - 9 + [f > 0.875].
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = E - 9 + (f > 0.875f ? 1 : 0);
  return min(127, max(-127, e));
}

// Four floats to four E4M3 bytes (RNE), the first in the lowest byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// 32 values -> 32 E4M3 bytes with a shared power-of-two scale; returns the
// biased exponent byte.
__device__ __forceinline__ uint32_t quantize32(const float (&v)[32], uint32_t (&out)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = block_exponent(amax);
  const float inv = ldexpf(1.f, -e);  // exact: e in [-127, 120] for bf16 inputs
#pragma unroll
  for (int j = 0; j < 8; ++j)
    out[j] = pack_fp8x4(v[4 * j] * inv, v[4 * j + 1] * inv, v[4 * j + 2] * inv, v[4 * j + 3] * inv);
  return (uint32_t)(e + 127);
}

// Q or K: one thread per block of 32 consecutive elements of a row; the
// scales of rows N .. Np-1 (padding, so that every head's scales are whole
// dwords) hold the exponent of an all-zero block.
template <int D>
__global__ __launch_bounds__(256)
void quant_rows_kernel(const bf16_t* __restrict__ X, uint8_t* __restrict__ X8,
                       uint8_t* __restrict__ Xs, long long nblocks, int N, int Np) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  constexpr int BPR = D / 32;  // blocks per row
  const int blk = (int)(b % BPR);
  const long long r = b / BPR;
  const int row = (int)(r % Np);
  const long long bh = r / Np;
  if (row >= N) {
    Xs[b] = (uint8_t)127;
    return;
  }
  const size_t e0 = ((size_t)bh * N + row) * D + blk * 32;  // first element of the block
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = *reinterpret_cast<const uint4*>(X + e0 + 8 * i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  uint32_t q[8];
  const uint32_t eb = quantize32(v, q);
  uint4* dst = reinterpret_cast<uint4*>(X8 + e0);
  dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
  dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
  Xs[b] = (uint8_t)eb;
}

// V: one workgroup per (head, 64 keys), staged through LDS so that both the
// bfloat16 rows read and the transposed E4M3 rows written are coalesced.
// Each thread quantises (head dim, 32-key block) items from the LDS copy;
// the codes go to an LDS tile [D][64] that is then written out as whole
// 64-byte rows of V^T [D, Np], the scale of block kb to
// Vs[(head * Np/32 + kb) * D + dim].  Keys >= N are 0.
template <int D>
__global__ __launch_bounds__(256)
void quant_keys_kernel(const bf16_t* __restrict__ V, uint8_t* __restrict__ V8,
                       uint8_t* __restrict__ Vs, int N, int Np) {
  __shared__ __attribute__((aligned(16))) bf16_t vin[64 * D];
  __shared__ __attribute__((aligned(16))) uint8_t vout[D * 64];
  const int tid = threadIdx.x;
  const int tiles = Np / 64;
  const long long bh = blockIdx.x / tiles;
  const int j0 = (blockIdx.x % tiles) * 64;
  const bf16_t* src = V + (size_t)bh * N * D;
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
#pragma unroll
  for (int i = tid; i < 64 * CPR; i += 256) {
    const int r = i / CPR, cc = i % CPR;
    const uint4 u = j0 + r < N ? *reinterpret_cast<const uint4*>(src + (size_t)(j0 + r) * D + cc * 8)
                               : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(vin + r * D + cc * 8) = u;
  }
  __syncthreads();
  for (int it = tid; it < 2 * D; it += 256) {
    const int d = it % D, kb = it / D;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(vin[(32 * kb + i) * D + d]);
    uint32_t q[8];
    const uint32_t eb = quantize32(v, q);
    uint4* dst = reinterpret_cast<uint4*>(vout + d * 64 + 32 * kb);
    dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
    dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
    Vs[((size_t)bh * (Np / 32) + j0 / 32 + kb) * D + d] = (uint8_t)eb;
  }
  __syncthreads();
  uint8_t* out = V8 + (size_t)bh * D * Np + j0;
  for (int i = tid; i < D * 4; i += 256) {
    const int d = i / 4, cc = i % 4;
    *reinterpret_cast<uint4*>(out + (size_t)d * Np + cc * 16) =
        *reinterpret_cast<const uint4*>(vout + d * 64 + cc * 16);
  }
}

// ---------------------------------------------------------------------------
// Byte tiles in LDS: rows of RB bytes in 16-byte chunks; chunk k of row r sits
// at slot k ^ swz8<RB>(r), so that 16 lanes reading one chunk of 16
// consecutive rows hit 16 different bank groups.
template <int RB>
__device__ __forceinline__ int swz8(int row) {
  constexpr int CPR = RB / 16, RPG = 256 / RB;  // chunks per row, rows per 256 bytes
  return (row / RPG) & (CPR - 1);
}
template <int RB>
__device__ __forceinline__ int off8(int row, int chunk) {
  return row * RB + ((chunk ^ swz8<RB>(row)) << 4);
}

// Active forward steps at head dim 256 spread their K/V copies between the
// score section's matrix instructions instead of issuing them at the start of
// the step (at head dim 64 the burst measured faster)
#ifndef FA_FP8_SPREAD
#define FA_FP8_SPREAD 1
#endif

// The running maximum is raised only when a block's maximum exceeds it by
// more than FA_FP8_LAG (log2 units).  Weights are scaled so that the running
// maximum maps to 2^8 and E4M3 holds up to 448 = 2^8.807, so a base that
// lags a row's largest score by at most 0.75 keeps every weight below
// 2^8.75 < 448; the base never exceeds the row's largest score, so the row
// sum stays >= 2^8 and a subnormal weight's rounding stays within 2^-18 of
// the row's total.  Rows then rescale O and l far less often.
#ifndef FA_FP8_LAG
#define FA_FP8_LAG 0.75f
#endif

// lds_copy4 without the compiler memory clobber (see lds_copy16_free).
__device__ __forceinline__ void lds_copy4_free(copy_rsrc r, uint32_t voff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r));
}

// Copy number i of dma_tile8 on its own, issued without the compiler memory
// clobber (lds_copy16_free): for a stage nothing reads before the next ring
// barrier.
template <int RB, int ROWS, int NT>
__device__ __forceinline__ void dma_tile8_part(copy_rsrc r, int r0, uint32_t gstride, uint32_t col0,
                                               uint8_t* tile, int tid, int i) {
  constexpr int CPR = RB / 16;
  constexpr int NWAVE = NT / kWave;
  const int w = tid >> 6, lane = tid & 63;
  const int blk = w + i * NWAVE;
  const int pos = blk * 64 + lane;
  const int row = pos / CPR, k = (pos % CPR) ^ swz8<RB>(row);
  lds_copy16_free(r, (uint32_t)(r0 + row) * gstride + col0 + (uint32_t)k * 16u,
                  lds_address(tile + blk * 1024));
}

// Copy of ROWS rows of RB bytes -- global row r at byte (r0 + r) * gstride +
// col0 -- into a swizzled tile, without VGPRs (lane L of an instruction fills
// LDS slot 64 i + L, so it fetches the chunk the swizzle puts there).
template <int RB, int ROWS, int NT>
__device__ __forceinline__ void dma_tile8(copy_rsrc r, int r0, uint32_t gstride, uint32_t col0,
                                          uint8_t* tile, int tid) {
  constexpr int CPR = RB / 16;
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int NWAVE = NT / kWave;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the threads");
  const int w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < CHUNKS / NT; ++i) {
    const int blk = w + i * NWAVE;
    const int pos = blk * 64 + lane;
    const int row = pos / CPR, k = (pos % CPR) ^ swz8<RB>(row);
    lds_copy16(r, (uint32_t)(r0 + row) * gstride + col0 + (uint32_t)k * 16u,
               lds_address(tile + blk * 1024));
  }
}

template <int D>
__device__ __forceinline__ i32x8 frag8(const uint8_t* tile, int row, int c0, int c1) {
  constexpr int RB = D;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + off8<RB>(row, c0));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + off8<RB>(row, c1));
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// One workgroup: NW wavefronts x 32 query rows; blocks of 64 keys in an
// ST-stage LDS ring (K tile [64][D], V^T tile [D][64], then the two scale
// blocks: K's [64][D/32] at byte 0, V's [2][D] at byte 512).
// NOMASK (chosen by the launcher at head dim 256): no causal mask and N a
// multiple of the 64-key block, so no block needs masking and the loop
// carries no mask code, which frees the registers the compiler otherwise
// parks in AGPRs (5.36 -> 5.16 ms at 2·16·16384·256).
template <int D, int NW, int ST, int OCC, bool CAUSAL, bool NOMASK = false>
__global__ __launch_bounds__(NW * 64, OCC)
void fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ Qs,
                    const uint8_t* __restrict__ K8, const uint8_t* __restrict__ Ks,
                    const uint8_t* __restrict__ V8, const uint8_t* __restrict__ Vs,
                    bf16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, int Np,
                    int nqb, int G, float c) {
  constexpr int NT = NW * kWave, BR = NW * 32, BC = 64;
  constexpr int KS = D / 64;  // contraction steps of S^T = K Q^T
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int TILE = 64 * D;
  constexpr int PER = 2 * (TILE / 16 / NT) + 1;  // copies per lane per block
  constexpr int NKV = TILE / 16 / NT;             // copies per tile per lane
  constexpr bool SPREAD = FA_FP8_SPREAD && D >= 256 && NKV == KS;  // one copy per S instruction
  static_assert(NW == 4, "the scale copies take one wavefront per 256 bytes");
  static_assert(!(NOMASK && CAUSAL), "the causal mask needs the mask code");
  static_assert(ST == 2 || ST == 3, "two or three stages");
  __shared__ __attribute__((aligned(16))) uint8_t k0s[TILE], v0s[TILE], s0s[1024];
  __shared__ __attribute__((aligned(16))) uint8_t k1s[TILE], v1s[TILE], s1s[1024];
  __shared__ __attribute__((aligned(16))) uint8_t k2s[ST > 2 ? TILE : 16], v2s[ST > 2 ? TILE : 16],
      s2s[ST > 2 ? 1024 : 16];
  auto kst = [&](auto S) -> uint8_t* {
    if constexpr (decltype(S)::value == 0) return k0s;
    else if constexpr (decltype(S)::value == 1) return k1s;
    else return k2s;
  };
  auto vst = [&](auto S) -> uint8_t* {
    if constexpr (decltype(S)::value == 0) return v0s;
    else if constexpr (decltype(S)::value == 1) return v1s;
    else return v2s;
  };
  auto sst = [&](auto S) -> uint8_t* {
    if constexpr (decltype(S)::value == 0) return s0s;
    else if constexpr (decltype(S)::value == 1) return s1s;
    else return s2s;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int bh, rank;
  grouped_order(xcd_remap(blockIdx.x, BH * nqb), nqb, BH, G, bh, rank);
  const int qb = CAUSAL ? (nqb - 1 - rank) : rank;  // longest causal blocks first
  const int q0 = qb * BR, q0w = q0 + w * 32;
  const int query = q0w + c32;

  const auto rk = make_copy_rsrc(K8 + (size_t)bh * N * D, (uint32_t)N * D);
  const auto rv = make_copy_rsrc(V8 + (size_t)bh * D * Np, (uint32_t)D * Np);
  const auto rks = make_copy_rsrc(Ks + (size_t)bh * Np * (D / 32), (uint32_t)Np * (D / 32));
  const auto rvs = make_copy_rsrc(Vs + (size_t)bh * Np / 32 * D, (uint32_t)(Np / 32) * D);

  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  auto fetch = [&](int t, auto S) {
    const int j0 = t * BC;
    dma_tile8<D, 64, NT>(rk, j0, (uint32_t)D, 0u, kst(S), tid);
    dma_tile8<64, D, NT>(rv, 0, (uint32_t)Np, (uint32_t)j0, vst(S), tid);
    // 256 bytes per wavefront: K's scales (two halves), then V's (wu is the
    // wavefront index made uniform, so the descriptor stays in SGPRs)
    const uint32_t off = wu < 2 ? (uint32_t)j0 * (D / 32) + 256u * wu
                                : (uint32_t)(j0 / 32) * D + 256u * (wu - 2);
    lds_copy4(wu < 2 ? rks : rvs, off + 4u * lane, lds_address(sst(S) + 256 * wu));
  };

  fetch(0, std::integral_constant<int, 0>{});
  // Q fragments (B operands of S^T = K Q^T) and their scales, straight from HBM
  i32x8 qf[KS];
  int qsc[KS];
  {
    const auto rq = make_rsrc(Q8 + (size_t)bh * N * D, (uint32_t)N * D);
    const auto rqs = make_rsrc(Qs + (size_t)bh * Np * (D / 32), (uint32_t)Np * (D / 32));
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 lo = buf_load16(rq, (uint32_t)query * D + 64 * s + 16 * h);
      const uint4 hi = buf_load16(rq, (uint32_t)query * D + 64 * s + 32 + 16 * h);
      qf[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      qsc[s] = (int)__builtin_amdgcn_raw_buffer_load_b8(rqs, (uint32_t)query * (D / 32) + 2 * s + h, 0, 0);
    }
  }
  if constexpr (ST > 2) {
    if (1 < ntiles) fetch(1, std::integral_constant<int, 1>{});
  }
  wait_vmem_tiles<PER, ST - 2>(min(ST - 2, ntiles - 1));
  ring_barrier();
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) pin_ready((int)qf[s][i]);
    pin_ready(qsc[s]);
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  auto step = [&](int t, auto S) {
    constexpr int SN = (decltype(S)::value + ST - 1) % ST;  // stage of step t+ST-1
    const int j0 = t * BC;
    const bool active = !CAUSAL || j0 <= q0w + 31;
    // Active steps spread their copies over the score section, one after
    // each matrix instruction (a copy holds up its wavefront's issue until
    // the texture unit takes it; a burst at the start of the step stalls all
    // four wavefronts).  There they are issued unconditionally: past the last
    // block they fetch zeros or unneeded rows into a stage not read again.
    if (!SPREAD || !active) {
      if (t + ST - 1 < ntiles) fetch(t + ST - 1, std::integral_constant<int, SN>{});
    }
    auto copy_part = [&](int i) {
      const int j1 = (t + ST - 1) * BC;
      __builtin_amdgcn_sched_barrier(0x406);
      if (i < NKV) {
        dma_tile8_part<D, 64, NT>(rk, j1, (uint32_t)D, 0u, kst(std::integral_constant<int, SN>{}), tid, i);
      } else if (i < 2 * NKV) {
        dma_tile8_part<64, D, NT>(rv, 0, (uint32_t)Np, (uint32_t)j1, vst(std::integral_constant<int, SN>{}), tid,
                                  i - NKV);
      } else {
        const uint32_t off = wu < 2 ? (uint32_t)j1 * (D / 32) + 256u * wu
                                    : (uint32_t)(j1 / 32) * D + 256u * (wu - 2);
        lds_copy4_free(wu < 2 ? rks : rvs, off + 4u * lane,
                       lds_address(sst(std::integral_constant<int, SN>{}) + 256 * wu));
      }
      __builtin_amdgcn_sched_barrier(0x406);
    };
    if (active) {
      const uint8_t* Kt = kst(S);
      const uint8_t* Vt = vst(S);
      const uint8_t* Sc = sst(S);
      // S^T = K Q^T (lane: query; registers: keys j0 + 32kb + 8g + 4h + e)
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int row = 32 * kb + c32;
          const i32x8 kf = frag8<D>(Kt, row, 4 * s + h, 4 * s + 2 + h);
          const int ksc = Sc[row * (D / 32) + 2 * s + h];
          const f32x16 z = {};
          sacc[kb] = mfma_fp8(kf, qf[s], s == 0 ? z : sacc[kb], ksc, qsc[s]);
          if constexpr (SPREAD) copy_part(kb * KS + s);
        }
      if constexpr (SPREAD) copy_part(2 * NKV);  // the scale blocks
      const bool need_mask = !NOMASK && ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w));
      if (need_mask) {
        keep_branch();
        const int nk = N - j0 - 4 * h;  // key >= N  <=>  key offset >= nk
        const int kq = j0 + 4 * h - query;
        const int lim = CAUSAL ? min(-kq, nk - 1) : nk - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = kb * 32 + 8 * (r >> 2) + (r & 3);
            if (koff > lim) sacc[kb][r] = -INFINITY;
          }
      }
      // online softmax: a block's maximum (log2 units) more than FA_FP8_LAG
      // above m raises m
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx) * c;
      if (wave_any(mx > m + FA_FP8_LAG)) {
        keep_branch();
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);  // 0 on the first block (m = -inf)
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m = mn;
      }
      // weights * 2^8 = exp2(c s + 8 - m), in (0, 2^8.75]; row sum in fp32
      const float bias = 8.f - m;
      float part[16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c, bias));
          sacc[kb][r + 1] = fast_exp2(fmaf(sacc[kb][r + 1], c, bias));
          part[kb * 8 + r / 2] = sacc[kb][r] + sacc[kb][r + 1];
        }
#pragma unroll
      for (int n = 16; n > 1; n /= 2)
#pragma unroll
        for (int i = 0; i < n / 2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
      l += part[0];
      // P^T as the B operand: E4M3 bytes, rearranged across the two halves
      // of the wave so that half h holds keys j0 + 32kb + 16h .. +15
      // (bytes 16kb ..) in order.  Before: dword g of block kb holds keys
      // 32kb + 8g + 4h + 0..3; swapping the high half of dword g with the
      // low half of dword g+2 (g = 0, 1) gives both halves their 16 keys.
      uint32_t pw[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        uint32_t dw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          dw[g] = pack_fp8x4(sacc[kb][4 * g], sacc[kb][4 * g + 1], sacc[kb][4 * g + 2], sacc[kb][4 * g + 3]);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const auto r = __builtin_amdgcn_permlane32_swap(dw[g], dw[g + 2], false, false);
          pw[4 * kb + 2 * g] = r[0];
          pw[4 * kb + 2 * g + 1] = r[1];
        }
      }
      const i32x8 pf = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                        (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
      // O^T += V^T P^T (lane: query; registers: head dims 32db + 8g + 4h + e)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 32 * db + c32;
        const i32x8 vf = frag8<64>(Vt, row, h, 2 + h);
        const int vsc = Sc[512 + h * D + row];
        oacc[db] = mfma_fp8(vf, pf, oacc[db], vsc, kScaleOne);
      }
    }
    if (t + 1 < ntiles) {
      wait_vmem_tiles<PER, ST - 2>(min(ST - 2, ntiles - t - 2));
      ring_barrier();
    }
  };
  for (int t0 = 0; t0 < ntiles; t0 += ST) {
    step(t0, std::integral_constant<int, 0>{});
    if (t0 + 1 < ntiles) step(t0 + 1, std::integral_constant<int, 1>{});
    if constexpr (ST > 2) {
      if (t0 + 2 < ntiles) step(t0 + 2, std::integral_constant<int, 2>{});
    }
  }
  // the last step's copies (issued unconditionally) land before the
  // workgroup ends
  if constexpr (SPREAD) wait_vmem_le<0>();

  // O = acc / l (bf16); LSE = (m + log2 l - 8) ln 2 (l counts weights * 2^8)
  const float lt = sum_halves(l);
  const float inv = __builtin_amdgcn_rcpf(lt);
  if (query < N) {
    bf16_t* Or = O + ((size_t)bh * N + query) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        const uint32_t hi = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(Or + db * 32 + 8 * g + 4 * h) = make_uint2(lo, hi);
      }
    if (h == 0) LSE[(size_t)bh * N + query] = (m + __builtin_amdgcn_logf(lt) - 8.f) * kLn2;
  }
}

template <int D, int NW, int ST, int OCC, bool CAUSAL>
hipError_t run_fwd_fp8(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                       const void* V8, const void* Vs, void* O, float* LSE, const Problem& p,
                       hipStream_t stream) {
  const int BH = p.B * p.H;
  const int nqb = (p.N + NW * 32 - 1) / (NW * 32);
  const long long grid = (long long)BH * nqb;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int G = head_group(OCC * 4 / NW, nqb);
  if constexpr (!CAUSAL && D >= 256) {  // at head dim 64 it measured 1% slower
    if (p.N % 64 == 0) {
      hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, ST, OCC, false, true>), dim3((unsigned)grid),
                         dim3(NW * 64), 0, stream, (const uint8_t*)Q8, (const uint8_t*)Qs,
                         (const uint8_t*)K8, (const uint8_t*)Ks, (const uint8_t*)V8, (const uint8_t*)Vs,
                         (bf16_t*)O, LSE, BH, p.N, fp8_keys_padded(p.N), nqb, G, p.scale * kLog2e);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_fp8_kernel<D, NW, ST, OCC, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0,
                     stream, (const uint8_t*)Q8, (const uint8_t*)Qs, (const uint8_t*)K8,
                     (const uint8_t*)Ks, (const uint8_t*)V8, (const uint8_t*)Vs, (bf16_t*)O, LSE, BH,
                     p.N, fp8_keys_padded(p.N), nqb, G, p.scale * kLog2e);
  return hipGetLastError();
}

template <int D, int NW, int ST, int OCC>
hipError_t run_fwd_fp8_c(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                         const void* V8, const void* Vs, void* O, float* LSE, const Problem& p,
                         hipStream_t stream) {
  return p.causal ? run_fwd_fp8<D, NW, ST, OCC, true>(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream)
                  : run_fwd_fp8<D, NW, ST, OCC, false>(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream);
}

// Launch configurations per head dim: wavefronts per workgroup, stages,
// minimum wavefronts per SIMD.
#ifndef FA_FP8_CFG_D64
#define FA_FP8_CFG_D64 4, 2, 3
#endif
#ifndef FA_FP8_CFG_D128
#define FA_FP8_CFG_D128 4, 2, 2
#endif
#ifndef FA_FP8_CFG_D256
#define FA_FP8_CFG_D256 4, 2, 1
#endif

}  // namespace

#ifndef FA_D256_UNIT
hipError_t launch_quantize_fp8(const void* X, void* X8, void* Xs, const Problem& p, bool keys,
                               hipStream_t stream) {
  const long long BH = (long long)p.B * p.H;
  const int Np = fp8_keys_padded(p.N);
  if (!keys) {
    const long long nblocks = BH * Np * (p.d / 32);
    const long long grid = (nblocks + 255) / 256;
    if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (p.d) {
      case 64:
        hipLaunchKernelGGL(quant_rows_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, nblocks, p.N, Np);
        break;
      case 128:
        hipLaunchKernelGGL(quant_rows_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, nblocks, p.N, Np);
        break;
      case 256:
        hipLaunchKernelGGL(quant_rows_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, nblocks, p.N, Np);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const long long grid = BH * (Np / 64);
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  switch (p.d) {
    case 64:
      hipLaunchKernelGGL(quant_keys_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                         (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, p.N, Np);
      break;
    case 128:
      hipLaunchKernelGGL(quant_keys_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                         (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, p.N, Np);
      break;
    case 256:
      hipLaunchKernelGGL(quant_keys_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream,
                         (const bf16_t*)X, (uint8_t*)X8, (uint8_t*)Xs, p.N, Np);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_forward_fp8(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                              const void* V8, const void* Vs, void* O, float* LSE,
                              const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return run_fwd_fp8_c<64, FA_FP8_CFG_D64>(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream);
    case 128: return run_fwd_fp8_c<128, FA_FP8_CFG_D128>(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream);
    case 256: return launch_forward_fp8_d256(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream);
    default: return hipErrorInvalidValue;
  }
}
#else
// Head dim 256 (this source compiled a second time as fa_fp8_d256.hip)
hipError_t launch_forward_fp8_d256(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                                   const void* V8, const void* Vs, void* O, float* LSE,
                                   const Problem& p, hipStream_t stream) {
  return run_fwd_fp8_c<256, FA_FP8_CFG_D256>(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p, stream);
}
#endif

}  // namespace fa
