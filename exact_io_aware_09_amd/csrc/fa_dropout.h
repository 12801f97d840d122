// fa_dropout.h -- dropout draws for the fused attention kernels (gfx950).
//
// Dropout on the attention weights is applied inside the fused kernel, after
// the softmax and before the product with V ("FlashAttention and GPU
// memory", section 07); the forward keeps no mask, only the generator's key,
// and the backward regenerates the same draws ("FlashAttention and GPU
// memory", section 09; "Lecture 8 . GPU Performance & FlashAttention",
// section 5.4).
//
// Draws: one Philox4x32-10 block (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011) per 4 x 4 tile of (query,
// key) pairs of a head: counter (key / 4, query / 4, head, 0), key = the
// 64-bit seed; the pair's 8-bit draw is byte (key mod 4) of word (query mod 4).
// A pair is kept iff its draw is below the threshold t (keep probability
// t / 256); kept weights are scaled by 256 / t.
//
// Each kernel holds a 32 x 32 block of scores as an MFMA D fragment: lane
// (c, h) and register 4g + e hold the pair (column c, row 8g + 4h + e).  The
// 16 pairs of a lane fall in four tiles, and the four lanes of a quad
// (columns 4a .. 4a+3) need the same four tiles: each lane of the quad
// generates one tile's block and a 4 x 4 transpose across the quad hands
// every lane its share -- one generator call per lane per block, whichever
// of query or key is the column.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Philox4x32-10: ten rounds of two 32 x 32 -> 64-bit products; the high
// halves are mixed into the other two words with the round key, and the key
// advances by the two Weyl increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
    const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    x1 = (uint32_t)p1;
    x3 = (uint32_t)p0;
    x0 = y0;
    x2 = y2;
  }
  return make_uint4(x0, x1, x2, x3);
}

// 4 x 4 transpose across the lanes of a quad: on return x[g] of lane l is
// what x[l & 3] was in lane (l & ~3) + g.  Two exchange steps with DPP quad
// permutations: swap within the 2 x 2 sub-blocks (lanes l ^ 1, words w ^ 1),
// then swap the off-diagonal sub-blocks (lanes l ^ 2, words w ^ 2).
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2;
#pragma unroll
  for (int a = 0; a < 4; a += 2) {
    const uint32_t send = b0 ? x[a] : x[a + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    if (b0) x[a] = recv;
    else x[a + 1] = recv;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const uint32_t send = b1 ? x[a] : x[a + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    if (b1) x[a] = recv;
    else x[a + 2] = recv;
  }
}

// Draws of a lane's 16 pairs in a 32 x 32 block whose columns are queries
// (forward and dQ kernels): queries q0 + c, keys j0 + 8g + 4h + e; q0 and
// j0 multiples of 4.  Byte e of w[g] is the draw of register 4g + e.
__device__ __forceinline__ void draws_query_cols(int q0, int j0, int head, int lane, uint32_t k0,
                                                 uint32_t k1, uint32_t (&w)[4]) {
  const int c = lane & 31, h = lane >> 5;
  // this lane generates the tile of key group g = c & 3 for its quad's queries
  const uint4 b = philox4x32_10((uint32_t)((j0 >> 2) + 2 * (c & 3) + h), (uint32_t)((q0 + c) >> 2),
                                (uint32_t)head, 0u, k0, k1);
  w[0] = b.x;  // word = query within the tile, byte = key within the tile
  w[1] = b.y;
  w[2] = b.z;
  w[3] = b.w;
  quad_transpose(w, lane);
}

// Draws of a lane's 16 pairs in a 32 x 32 block whose columns are keys (dK/dV
// kernel): keys j0 + c, queries i0 + 8g + 4h + e; i0 and j0 multiples of 4.
// Byte e of w[g] is the draw of register 4g + e.
__device__ __forceinline__ void draws_key_cols(int i0, int j0, int head, int lane, uint32_t k0,
                                               uint32_t k1, uint32_t (&w)[4]) {
  const int c = lane & 31, h = lane >> 5;
  // this lane generates the tile of query group g = c & 3 for its quad's keys
  const uint4 b = philox4x32_10((uint32_t)((j0 + c) >> 2), (uint32_t)((i0 >> 2) + 2 * (c & 3) + h),
                                (uint32_t)head, 0u, k0, k1);
  // 4 x 4 byte transpose: word k gathers byte k (key k of the tile) of the
  // four query words, so that a word holds one key's four queries
  const uint32_t x[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = ((x[0] >> (8 * k)) & 0xFFu) | (((x[1] >> (8 * k)) & 0xFFu) << 8) |
           (((x[2] >> (8 * k)) & 0xFFu) << 16) | (((x[3] >> (8 * k)) & 0xFFu) << 24);
  quad_transpose(w, lane);
}

// Keep test of register r (draw byte r & 3 of word r >> 2).
__device__ __forceinline__ bool kept(const uint32_t (&w)[4], int r, int thresh) {
  return (int)((w[r >> 2] >> (8 * (r & 3))) & 0xFFu) < thresh;
}

}  // namespace fa
