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
constexpr int kCusPerXcd = 32;

// Heads per group for grouped_order: about one XCD's worth of resident
// workgroups (wgs_per_cu of them on each of its CUs) per group.
constexpr int head_group(int wgs_per_cu, int nblk) {
  const int slots = kCusPerXcd * (wgs_per_cu > 0 ? wgs_per_cu : 1);
  return slots / nblk > 0 ? slots / nblk : 1;
}

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

// Combine a value with the one held by the lane 32 positions away (the other
// half of the wave) using v_permlane32_swap (a VALU op; no LDS round trip).
// After swapping a register with a copy of itself, r[0] holds the low-half
// value and r[1] the high-half value in every lane, so both halves compute
// the same result from operands in the same order.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0): every outstanding vector-memory load has landed.  Used
// once before a main loop so that loads issued in the prologue (register
// fragments) are not tracked into the loop, where the compiler would
// otherwise wait on the in-order counter -- i.e. on the next block's
// prefetch -- before each use.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int PER, int MAXT>
__device__ __forceinline__ void wait_vmem_tiles(int tiles);

// s_waitcnt vmcnt(N): at most N vector-memory loads of this wavefront still
// outstanding (they complete in issue order).  N < 64.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most `tiles` * PER loads are outstanding (tiles <= MAXT,
// uniform across the wavefront); the immediate is selected by a switch.
template <int PER, int MAXT>
__device__ __forceinline__ void wait_vmem_tiles(int tiles) {
  static_assert(MAXT <= 6, "extend the switch");
  switch (tiles) {
    case 0: wait_vmem_le<0>(); break;
    case 1: wait_vmem_le<(1 <= MAXT ? PER : 0)>(); break;
    case 2: wait_vmem_le<(2 <= MAXT ? 2 * PER : 0)>(); break;
    case 3: wait_vmem_le<(3 <= MAXT ? 3 * PER : 0)>(); break;
    case 4: wait_vmem_le<(4 <= MAXT ? 4 * PER : 0)>(); break;
    case 5: wait_vmem_le<(5 <= MAXT ? 5 * PER : 0)>(); break;
    default: wait_vmem_le<(6 <= MAXT ? 6 * PER : 0)>(); break;
  }
}

// Workgroup -> logical tile index such that consecutive logical tiles land on
// the same XCD.  Hardware hands workgroup w to XCD (w mod 8); a bijection
// maps it to a contiguous run of logical indices per XCD, so all Q blocks of
// one (batch, head) share one L2 while that head's K/V are being re-read.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total / kNumXcd, r = total % kNumXcd;
  const int x = w % kNumXcd, idx = w / kNumXcd;
  return x * q + (x < r ? x : r) + idx;
}

// Logical tile index -> (head, rank) for launches of nblk blocks per head
// whose lengths differ (causal): heads are taken in groups of G, and inside a
// group every head's rank-0 block comes first, then every rank-1 block, and
// so on.  Rank 0 is the longest block.  With G * nblk close to the number of
// workgroups one XCD holds at once, each XCD starts its long blocks first
// (short tail at the end of the launch) while the K/V (or Q/dO) of only G
// heads are live in its L2.  The last group may hold fewer than G heads.
__device__ __forceinline__ void grouped_order(int L, int nblk, int BH, int G, int& bh, int& rank) {
  const int per = G * nblk;
  const int g = L / per, r = L - g * per;
  const int gh = min(G, BH - g * G);
  bh = g * G + r % gh;
  rank = r / gh;
}

// Offsets of the blocks (BSZ rows or keys each, BSZ dividing 128) that a
// workgroup visits in its main loop.  Dense: every block from `start` below
// `end`.  Block-sparse, mask form (n < 0): only the blocks inside the set
// 128 x 128 tiles of the workgroup's row (or column) of the tile mask:
// tiles u <= hi, entry m[u * stride] (int32; the index is uniform, so the
// entries are read through the scalar cache).  Block-sparse, list form
// (n >= 0): the blocks of the n tiles whose indices m[0..n) lists in
// increasing order (a balanced schedule's run of tiles); an index outside
// [0, end / 128] ends the walk.  Offsets are returned in increasing order,
// -1 after the last; next() must be given the offset returned last.
// The mask is read-only for the whole launch: entries are loaded through
// the constant address space, i.e. with scalar loads, which are waited on
// with lgkmcnt and so never wait for the vector-memory copies in flight.
typedef const __attribute__((address_space(4))) int* const_int_ptr;

template <int BSZ, bool SPARSE>
struct BlockWalk {
  static_assert(128 % BSZ == 0, "blocks must tile the 128-wide mask tiles");
  int end;
  const_int_ptr m;
  int stride, hi;
  int n = -1;  // list form: number of listed tiles
  int p = 0;   // list form: position of the current tile
  // first set tile at or after tile u, as an offset, or -1
  __device__ __forceinline__ int tile_from(int u) const {
    while (u <= hi && m[u * stride] == 0) ++u;
    return (u <= hi && u * 128 < end) ? u * 128 : -1;
  }
  // tile at list position q, as an offset, or -1
  __device__ __forceinline__ int listed(int q) const {
    if (q >= n) return -1;
    const int u = m[q];
    return (u >= 0 && u < (end + 127) / 128) ? u * 128 : -1;
  }
  // `start` is a multiple of 128 when SPARSE (unused in the list form)
  __device__ __forceinline__ int first(int start) {
    if constexpr (SPARSE) {
      if (n >= 0) {
        p = 0;
        return listed(0);
      }
      return tile_from(start >> 7);
    } else {
      return start < end ? start : -1;
    }
  }
  __device__ __forceinline__ int next(int off) {
    const int o = off + BSZ;
    if constexpr (SPARSE) {
      if ((o & 127) != 0 && o < end) return o;
      if (n >= 0) return listed(++p);
      return tile_from((off >> 7) + 1);
    } else {
      return o < end ? o : -1;
    }
  }
};

// Reads item `k` of a balanced schedule (4 ints, see SparseArgs) and checks
// it against the schedule's sizes; false for an item that would leave them.
__device__ __forceinline__ bool sched_item(const int* items, int k, int nb, int list_len,
                                           int slots, int& t, int& off, int& cnt, int& slotw) {
  const const_int_ptr it = (const_int_ptr)items + 4 * k;
  t = it[0];
  off = it[1];
  cnt = it[2];
  slotw = it[3];
  return t >= 0 && t < nb && off >= 0 && cnt >= 0 && off <= list_len - cnt &&
         (slotw == -1 || (slotw >= 0 && (slotw >> 1) < slots));
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
  if constexpr (D > 128) {
    // the swizzle (< 16) changes only the low 4 bits of the chunk index, so
    // the chunks of columns 128 apart differ by a constant: written so, the
    // offsets of a row's reads share 8 lane-dependent terms plus immediates
    const int c = col >> 3;
    return row * D + ((c & ~15) << 3) + (((c & 15) ^ swz<D>(row)) << 3) + (col & 7);
  } else {
    return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
  }
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

// Two fp32 values rounded (RNE) to bf16 and packed into one dword with a
// single v_cvt_pk_bf16_f32; `a` lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x8 bf16x8_from(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

// Workgroup barrier for the LDS rings.  Every wavefront first waits for its
// own LDS reads (lgkmcnt 0) and, before calling this, for its own copies of
// the next block (explicit vmcnt wait); after the barrier the block is
// complete and no wavefront still reads the stage that the next copies
// overwrite.  Unlike __syncthreads() this does not also drain the copies of
// later blocks still in flight (a workgroup-scope release fence would wait
// for every outstanding load).  The asm statement is also a compiler barrier
// for memory accesses.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies (buffer_load ... lds).  They are issued from
// inline assembly so that the compiler does not track them: otherwise it
// waits for every copy in flight before any later LDS read it cannot prove
// disjoint, which would serialise the ring of stages.  Completion is
// awaited explicitly (s_waitcnt vmcnt, then ring_barrier) before a block is
// read.  M0 (the LDS base of the wavefront) is saved and restored around
// each copy, and the copy waits one cycle after M0 is written.
typedef int copy_rsrc __attribute__((ext_vector_type(4)));  // buffer descriptor words

// Descriptor over `bytes` bytes at `base` (stride 0, raw buffer); reads at
// or beyond `bytes` return zeros.  Same fields as make_rsrc.
__device__ __forceinline__ copy_rsrc make_copy_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  copy_rsrc r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p));
}

// Lane L copies 16 bytes at byte offset voff to LDS address lds + 16 L.
__device__ __forceinline__ void lds_copy16(copy_rsrc r, uint32_t voff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r)
      : "memory");
}

// Lane L copies 4 bytes at byte offset voff to LDS address lds + 4 L.
__device__ __forceinline__ void lds_copy4(copy_rsrc r, uint32_t voff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r)
      : "memory");
}

// Copy of one [ROWS x D] bf16 block (rows r0.. of the descriptor's tensor)
// into a swizzled LDS tile, without VGPRs.  Each wavefront instruction
// writes 64 x 16 bytes to consecutive LDS addresses, so lane L fetches the
// global chunk that the swizzle places at that position.  Rows past the end
// of the descriptor read as zeros.  CHUNKS / NT copies per lane.
template <int D, int ROWS, int NT>
__device__ __forceinline__ void dma_tile(copy_rsrc r, int r0, bf16_t* tile, int tid) {
  constexpr int CPR = D / 8;               // chunks per row
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int NWAVE = NT / kWave;
  static_assert(CHUNKS % NT == 0, "block must split evenly over the threads");
  const int w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < CHUNKS / NT; ++i) {
    const int blk = w + i * NWAVE;           // 1 KB block of the tile written by this instruction
    const int pos = blk * 64 + lane;         // chunk position in LDS
    const int row = pos / CPR, c = (pos % CPR) ^ swz<D>(row);
    const uint32_t goff = ((uint32_t)(r0 + row) * D + c * 8) * 2u;
    lds_copy16(r, goff, lds_address(tile + blk * 512));
  }
}

// The same copy, without the compiler memory clobber: for copies into a
// stage that nothing reads until the next ring barrier (whose asm statement
// does clobber memory), so that the compiler may keep scheduling LDS reads
// of other stages around it.
__device__ __forceinline__ void lds_copy16_free(copy_rsrc r, uint32_t voff, uint32_t lds) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r));
}

// Copy of `ROWS` (<= 64) consecutive floats starting at row r0 of a float
// vector into LDS (lane L -> dst[L]; lanes past ROWS repeat rows, so dst
// must hold 64 floats; rows past the descriptor's end read as 0).  One copy
// per lane.
template <int ROWS>
__device__ __forceinline__ void dma_rows_f32(copy_rsrc r, int r0, float* dst, int lane) {
  static_assert(ROWS <= kWave, "one lane per row");
  lds_copy4(r, (uint32_t)(r0 + (lane % ROWS)) * 4u, lds_address(dst));
}

// Scheduling hints: ask the compiler's scheduler to interleave instruction
// classes in the enclosing region (MFMA, transcendental, other VALU, LDS read).
#define FA_SCHED_MFMA(n) __builtin_amdgcn_sched_group_barrier(0x008, (n), 0)
#define FA_SCHED_VALU(n) __builtin_amdgcn_sched_group_barrier(0x002, (n), 0)
#define FA_SCHED_TRANS(n) __builtin_amdgcn_sched_group_barrier(0x400, (n), 0)
#define FA_SCHED_DSREAD(n) __builtin_amdgcn_sched_group_barrier(0x100, (n), 0)

// Sum of the two bf16 products a.x*b.x + a.y*b.y accumulated into c (fp32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Keeps a rarely taken, wave-uniform block as a real branch: the compiler may
// not execute an asm statement speculatively, so it cannot if-convert the
// block into selects evaluated on every iteration.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// Makes the value's registers an input of an empty volatile asm statement:
// the loads producing it complete (the compiler waits for them) before this
// point, and volatile asm statements keep their order, so those loads are
// not scheduled after the untracked LDS copies issued later.
template <typename T>
__device__ __forceinline__ void pin_ready(const T& x) { asm volatile("" ::"v"(x)); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

}  // namespace fa
