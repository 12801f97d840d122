// fa_fwd.hip -- attention forward for gfx950, bfloat16 in, fp32 accumulate.
//
// Algorithm: the tiled forward with an online softmax ("Lecture 8 . GPU
// Performance & FlashAttention", CS324 notes, sections 5.2-5.3), in the loop
// order of the second version described in section 8.1 of those notes and in
// "FlashAttention and GPU memory" section 07: one block of query rows per
// workgroup, an inner loop over K/V blocks, an unnormalised output
// accumulator divided by the row sum once at the end, and only O and the
// per-row log-sum-exp written to device memory.
//
// Mapping to CDNA4:
//  * NW wavefronts per workgroup, 32 query rows each; the Q fragments stay in
//    VGPRs for the whole kernel.
//  * K/V blocks of BC keys are copied HBM -> LDS by direct buffer->LDS loads
//    (no VGPRs), into XOR-swizzled unpadded tiles: K is read back by rows
//    (16-byte reads) and V through the LDS transpose unit
//    (ds_read_b64_tr_b16), so neither needs a transposed copy.  Rows past
//    the end of the head arrive as zeros (hardware range check).
//  * ST-stage ring of K/V blocks in LDS, one barrier per block: the loads of
//    block t+ST-1 are issued before block t is computed, so the copy engine
//    runs ST-1 blocks ahead.  Several workgroups share a CU, and their
//    wavefronts overlap each other's matrix, vector and memory phases.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane holds scores of ONE
//    query row, so the row maximum is an in-lane reduction plus one
//    v_permlane32_swap.  The exponentiated scores, rounded to bf16, are
//    directly the B operand of O^T += V^T P^T; the row sum is taken from the
//    fp32 values.
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA.  The
//    running maximum of a row is taken from its first block only and then
//    kept as the base of the exponent for as long as the block row sums stay
//    below a bound (2^16 per lane's half of a 32-key block), which the sum
//    that the online softmax needs anyway checks for free: no per-block
//    maximum, and O = acc / l and the log-sum-exp are unchanged because
//    numerator and denominator share the base.  A block that breaks the
//    bound (rare: the scores of a row must grow by more than about 2^12 in
//    weight) is redone with its own maximum and O, l rescaled, as in the
//    pages' update.  Rows decide individually, so each row's arithmetic
//    depends on its own scores alone.
//  * Software-pipelined loop (head dim 256; head dim 64 without the causal
//    mask, and, for causal rows of 2048 keys or more, over the blocks left of
//    each query block's diagonal): the P.V product of block t-1 runs
//    interleaved with the softmax of block t, K copied one block ahead of V.
//  * Workgroups are remapped so that all query blocks of a head run on one
//    XCD (shared L2 for the re-read K/V); within a group of heads that fills
//    an XCD, the longest causal blocks of every head start first.
#include <type_traits>

#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kMaxWeight = 65536.0f;  // bound on one lane's share of a block's row sum

// Head dim 256 (one wavefront per SIMD, so the order of a wavefront's own
// instructions decides how much overlaps):
//  * FA_FWD_IGLP_D256: K fragment reads issued that many matrix instructions
//    ahead of their use (V fragments: FA_FWD_PIPE_VA);
//  * FA_FWD_PIPE_D256: software-pipelined loop (the P.V product of block t-1
//    runs on the matrix cores while the softmax of block t runs on the
//    vector ALU);
//  * FA_FWD_DMA_GAP: matrix instructions between two of a step's K/V copies.
// Head dim 64 without the causal mask (four wavefronts per SIMD):
//  * FA_FWD_PIPE_D64: the same pipelined loop, four exponentials per P.V
//    matrix instruction; K fragment reads FA_FWD_PIPE_D64_KA, V fragment
//    reads FA_FWD_PIPE_D64_VA matrix instructions ahead (longer read-ahead
//    spills at 128 VGPRs).  The causal kernel keeps the plain loop: with
//    the pipeline it needs more registers than four wavefronts leave.
#ifndef FA_FWD_IGLP_D256
#define FA_FWD_IGLP_D256 5
#endif
#ifndef FA_FWD_PIPE_D256
#define FA_FWD_PIPE_D256 1
#endif
#ifndef FA_FWD_PIPE_D64
#define FA_FWD_PIPE_D64 1
#endif
#ifndef FA_FWD_PIPE_D64_KA
#define FA_FWD_PIPE_D64_KA 2
#endif
#ifndef FA_FWD_PIPE_D64_VA
#define FA_FWD_PIPE_D64_VA 1
#endif
// Causal head-dim-64 forwards with N >= FA_FWD_LONG_N run the two-loop
// kernel (NOMASK): measured 1.5% faster at N = 2048, 6-8% at 8192-65536, and
// 5% slower at N = 1024, where few blocks lie left of the diagonal.  The
// split-KV and dropout forwards follow the same rule (at N = 65536: 7% and
// 2.4% faster).
#ifndef FA_FWD_LONG_N
#define FA_FWD_LONG_N 2048
#endif
#ifndef FA_FWD_PIPE_VA
#define FA_FWD_PIPE_VA 5
#endif
#ifndef FA_FWD_DMA_GAP
#define FA_FWD_DMA_GAP 2
#endif

// Output accumulator rescaled in place in AGPRs (units compiled with the
// matrix instructions in their AGPR form): keeps the accumulator's registers
// AGPRs across the loop, instead of a VGPR copy that the compiler would
// otherwise make at every step to share one register class with the rare
// rescale.
#ifndef FA_FWD_ACC_AGPR
#define FA_FWD_ACC_AGPR 0
#endif

// acc *= s on an accumulator held in AGPRs.  The first statement waits out
// the matrix-instruction result latency itself (the compiler does not track
// hazards inside asm), the last one gives the writes time to settle before a
// matrix instruction reads them.
__device__ __forceinline__ void scale_acc_agpr(f32x16& acc, float s) {
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = acc[r];
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "s_nop 0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x[r]), "=&v"(t)
        : "v"(s));
  }
  asm volatile("s_nop 4" ::: "memory");
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = x[r];
}

template <int D, int NW, int RB, int BC, int ST>
struct FwdCfg {
  static constexpr int NT = NW * kWave;        // threads per workgroup
  static constexpr int RW = 32 * RB;           // query rows per wavefront
  static constexpr int BR = NW * RW;           // query rows per workgroup
  static constexpr int TILE = BC * D;          // elements of one K or V tile
  static constexpr int KSTEPS = D / 16;        // k-steps of K Q^T
  static constexpr int DB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int KB = BC / 32;           // 32-key blocks per tile
  static constexpr int PU = BC / 16;           // k-steps of V^T P^T
  static constexpr int DMA_PER_TILE = TILE / 8 / NT;  // loads per tile per lane
  // Q block staged through LDS (coalesced copy in, O out through the same
  // rows) when it fits in 16 KB; otherwise Q fragments load straight from HBM
  // (the Q fragments stay in VGPRs either way)
  static constexpr bool QL = BR * D * 2 <= 16384;
  static constexpr bool QST = QL;
  // software-pipelined loop (head dim 256 at one wavefront per SIMD, where no
  // other wavefront fills the matrix cores during a softmax; head dim 64,
  // where a wavefront's own P.V then overlaps its softmax)
  static constexpr bool PIPE = ((D >= 256 && FA_FWD_PIPE_D256 && KSTEPS == 16) ||
                                (D == 64 && FA_FWD_PIPE_D64)) &&
                               RB == 1 && (KB == 1 || KB == 2) && PU == 2 * KB;
  static_assert(ST >= 2 && ST <= 3, "two or three K/V stages");
};

// Per block t: S^T = K Q^T, mask, online softmax, O^T += V^T P^T, with the
// K/V blocks of the next ST-1 steps in flight (direct buffer->LDS loads).
// A wavefront owns RB blocks of 32 query rows: every K and V fragment read
// from LDS feeds RB matrix instructions, which divides LDS reads and
// HBM->LDS copies per FLOP by RB.
//
// SPLIT: the keys are cut into ranges of sa.span keys (a multiple of 64);
// workgroup (tile, range) runs the loop over its range only and writes the
// range's partial result -- O normalised over the range (float32) and the
// range's log-sum-exp, -inf for rows that see no key of the range -- to
// sa.Opart / sa.Lpart, for merge_kernel to combine.
//
// SPARSE: block-sparse attention; the loop visits only the K/V blocks of
// the 128 x 128 tiles set in row qb of the tile mask (the query block is one
// tile row: BR = 128).  A query block with no set tile (in reach of the
// causal mask) writes O = 0 and LSE = -inf.
//
// DROP: dropout on the weights.  The row sums (and so the LSE) are taken
// before it; the dropped weights are zeroed before P V, and the kept ones
// are scaled by 256 / t in the final division.
template <int D, int NW, int RB, int BC, int ST, int OCC, bool CAUSAL, bool SPLIT = false,
          bool SPARSE = false, bool DROP = false, bool NOMASK = false>
__global__ __launch_bounds__(NW * 64, OCC)
void fwd_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                     const bf16_t* __restrict__ V, bf16_t* __restrict__ O,
                     float* __restrict__ LSE, int BH, int N, int nqb, int G, float c,
                     SplitArgs sa = {}, SparseArgs sp = {}, DropArgs dr = {}) {
  using C = FwdCfg<D, NW, RB, BC, ST>;
  static_assert((int)SPLIT + (int)SPARSE + (int)DROP <= 1, "one variant at a time");
  // NOMASK (chosen by the launcher): the pipelined loop carries no mask.
  // Causal head dim 64 with long rows: it runs over the blocks left of the
  // workgroup's diagonal only (every wavefront active, nothing masked), the
  // plain loop over the rest; a pipelined loop that also handled waves past
  // their diagonal would need more registers than four wavefronts leave, so
  // short causal rows keep the plain loop alone.  Without the causal mask
  // (head dim 256): N is a multiple of the block size, so no block has a
  // tail.
  constexpr bool PIPE = C::PIPE && !SPARSE && (D != 64 || !CAUSAL || NOMASK);
  constexpr bool TWO = PIPE && CAUSAL && D == 64;
  static_assert(!NOMASK || !CAUSAL || TWO, "no mask: causal only for the two-loop kernel");
  static_assert(!TWO || ST == 2, "two-loop causal forward: two stages");
  static_assert(!SPARSE || (ST == 2 && C::BR == 128), "sparse walk: two stages, 128-row query blocks");
  // One LDS variable per stage and operand: with the stage a compile-time
  // constant at every access, the compiler can tell the block being read
  // from the blocks still being copied in, and inserts no wait for them.
  __shared__ __attribute__((aligned(16))) bf16_t k0s[C::TILE], v0s[C::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t k1s[ST > 1 ? C::TILE : 8], v1s[ST > 1 ? C::TILE : 8];
  __shared__ __attribute__((aligned(16))) bf16_t k2s[ST > 2 ? C::TILE : 8], v2s[ST > 2 ? C::TILE : 8];
  __shared__ __attribute__((aligned(16))) bf16_t qs[C::QST ? C::BR * D : 8];
  auto kst = [&](auto S) -> bf16_t* {
    if constexpr (decltype(S)::value == 0) return k0s;
    else if constexpr (decltype(S)::value == 1) return k1s;
    else return k2s;
  };
  auto vst = [&](auto S) -> bf16_t* {
    if constexpr (decltype(S)::value == 0) return v0s;
    else if constexpr (decltype(S)::value == 1) return v1s;
    else return v2s;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  int bh, rank, split = 0;
  if constexpr (SPLIT) {
    // the ranges of one tile are adjacent in the order
    const int L = xcd_remap(blockIdx.x, BH * nqb * sa.splits);
    split = L % sa.splits;
    grouped_order(L / sa.splits, nqb, BH, G, bh, rank);
  } else {
    grouped_order(xcd_remap(blockIdx.x, BH * nqb), nqb, BH, G, bh, rank);
  }
  int qb = CAUSAL ? (nqb - 1 - rank) : rank;  // longest causal blocks first
  // balanced schedule: item `rank` names the tile row and its run of tiles
  int list_off = 0, list_cnt = -1, slotw = -1;
  if constexpr (SPARSE) {
    if (sp.rows != nullptr &&
        !sched_item(sp.rows, rank, sp.nb, sp.list_len, sp.row_slots, qb, list_off, list_cnt, slotw))
      return;
  }
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rk = make_copy_rsrc(K + hoff, head_bytes);
  const auto rv = make_copy_rsrc(V + hoff, head_bytes);

  const int q0 = qb * C::BR;
  const int q0w = q0 + w * C::RW;  // first query row of this wavefront
  // this lane's query row in row block rb is q0w + 32 * rb + c32

  // keys [kbase, kend) of this workgroup: blocks kbase + t*BC, t < ntiles
  const int kbase = SPLIT ? split * sa.span : 0;
  const int kend0 = CAUSAL ? min(N, q0 + C::BR) : N;
  const int kend = SPLIT ? min(kend0, kbase + sa.span) : kend0;
  const int ntiles = kend > kbase ? (kend - kbase + BC - 1) / BC : 0;
  if constexpr (SPLIT) {
    if (ntiles == 0) {
      // no key of the range is visible to any row of the tile
      const size_t rows = (size_t)BH * N;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int query = q0w + 32 * rb + c32;
        if (query < N) {
          if (h == 0) sa.Lpart[split * rows + (size_t)bh * N + query] = -INFINITY;
          float* Op = sa.Opart + (split * rows + (size_t)bh * N + query) * D;
#pragma unroll
          for (int cc = 0; cc < D / 2; cc += 4)
            *reinterpret_cast<float4*>(Op + h * (D / 2) + cc) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      return;
    }
  }

  // keys visited: dense blocks kbase + t*BC, or the blocks of the set tiles
  BlockWalk<BC, SPARSE> walk{kend,
                             list_cnt >= 0 ? (const_int_ptr)sp.lists + list_off
                                           : (const_int_ptr)(sp.mask + (size_t)qb * sp.nb),
                             1, CAUSAL ? qb : sp.nb - 1, list_cnt};
  const int jfirst = SPARSE ? walk.first(0) : kbase;
  if constexpr (SPARSE) {
    if (jfirst < 0) {
      // no set tile: every row of the block sees no key
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int query = q0w + 32 * rb + c32;
        if (query < N) {
          if (h == 0) LSE[(size_t)bh * N + query] = -INFINITY;
          bf16_t* Or = O + hoff + (size_t)query * D + h * (D / 2);
#pragma unroll
          for (int cc = 0; cc < D / 2; cc += 8)
            *reinterpret_cast<uint4*>(Or + cc) = make_uint4(0u, 0u, 0u, 0u);
        }
      }
      return;
    }
  }

  auto fetch_at = [&](int j0, auto S) {
    dma_tile<D, BC, C::NT>(rk, j0, kst(S), tid);
    dma_tile<D, BC, C::NT>(rv, j0, vst(S), tid);
  };
  auto fetch = [&](int t, auto S) { fetch_at(kbase + t * BC, S); };
  // The first K/V copies go out before Q is read, so that the latencies
  // overlap.
  if constexpr (PIPE) dma_tile<D, BC, C::NT>(rk, jfirst, k0s, tid);
  else fetch_at(jfirst, std::integral_constant<int, 0>{});
  bf16x8 qf[RB][C::KSTEPS];  // B operands of S^T = K Q^T (lane = query row)
  if constexpr (C::QST) {
    // Q block copied row-major (coalesced) into LDS, rows past N as zeros
    dma_tile<D, C::BR, C::NT>(make_copy_rsrc(Q + hoff, head_bytes), q0, qs, tid);
  } else {
    const auto rq = make_rsrc(Q + hoff, head_bytes);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qf[rb][s] = as_bf16x8(
            buf_load16(rq, ((uint32_t)(q0w + 32 * rb + c32) * D + 16 * s + 8 * h) * 2u));
    // Q resident here: the compiler does not count the copies, so its own
    // waits for Q must not fall inside the loop (where they would also
    // drain the copies in flight).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) pin_ready(qf[rb][s]);
  }
  if constexpr (PIPE) {
    // pipelined loop: K of blocks 0..ST-2 and V of blocks 0..ST-3 before
    // step 0; K of block 0 (and Q) resident, the rest may stay in flight
    if constexpr (ST > 2) {
      const bool k1 = 1 < ntiles;
      if (k1) dma_tile<D, BC, C::NT>(rk, jfirst + BC, k1s, tid);
      dma_tile<D, BC, C::NT>(rv, jfirst, v0s, tid);
      wait_vmem_tiles<C::DMA_PER_TILE, 2>((int)k1 + 1);
    } else {
      wait_vmem_le<0>();
    }
  } else {
    if constexpr (ST > 2) {
      if (1 < ntiles) fetch(1, std::integral_constant<int, 1>{});
    }
    wait_vmem_tiles<2 * C::DMA_PER_TILE, ST - 2>(min(ST - 2, ntiles - 1));
  }
  ring_barrier();
  if constexpr (C::QL) {
    // each wavefront reads (and later overwrites with O) only its own rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
        qf[rb][s] = frag_rows<D>(qs, w * C::RW + 32 * rb, 16 * s, c32, h);
  }

  f32x16 oacc[RB][C::DB];
  float m[RB], l[RB];
  // Base of the exponent.  Every row sees key 0 of its first block, so m is
  // finite -- except for a key range that starts after a causal row, which
  // sees nothing of the range: its weights are then exp2(-inf) = 0.
  auto base = [](float mrow) { return (SPLIT && CAUSAL && mrow == -INFINITY) ? 0.f : mrow; };
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[rb][db][r] = 0.f;
    m[rb] = -INFINITY;
    l[rb] = 0.f;
  }

  // S^T = K Q^T for the block at key j0 (lane: query; registers: keys), each
  // K fragment feeding the RB row blocks; causal-future keys and keys past
  // the end become -inf, on the blocks that need it only.
  auto scores = [&](const bf16_t* Ks, int j0, f32x16 (&sacc)[RB][C::KB]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      bf16x8 kfr[C::KSTEPS];
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) kfr[s] = frag_rows<D>(Ks, kb * 32, 16 * s, c32, h);
      const f32x16 z = {};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma32x32x16(kfr[0], qf[rb][0], z);
#pragma unroll
      for (int s = 1; s < C::KSTEPS; ++s)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma32x32x16(kfr[s], qf[rb][s], sacc[rb][kb]);
      if constexpr (D >= 256 && FA_FWD_IGLP_D256 > 0) {
        // scheduling groups: the first A K reads, then one matrix
        // instruction and one read alternate, so that A reads stay ahead
        constexpr int A = FA_FWD_IGLP_D256;
        __builtin_amdgcn_sched_group_barrier(0x100, A, 0);
#pragma unroll
        for (int i = 0; i < C::KSTEPS - A; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
      }
    }
    const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w);
    if (need_mask) {
      keep_branch();
      const int nk = N - j0 - 4 * h;  // key >= N  <=>  key offset >= nk
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // key - query = kq + key offset; future keys and keys past the end
        // both have key offset > lim
        const int kq = j0 + 4 * h - (q0w + 32 * rb + c32);
        const int lim = CAUSAL ? min(-kq, nk - 1) : nk - 1;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = kb * 32 + 8 * (r >> 2) + (r & 3);
            if (koff > lim) sacc[rb][kb][r] = -INFINITY;
          }
      }
    }
  };
  // Row maximum of a block, scaled to log2 units (both halves of the row).
  auto block_max = [&](const f32x16 (&sacc)[C::KB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    return max_halves(mx) * c;
  };
  // P^T = exp2(c S^T - m) in place; returns this lane's share of the row sum.
  auto exponentiate = [&](f32x16 (&sacc)[C::KB], float mrow) {
    float part[C::KB * 8];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c, -mrow));
        sacc[kb][r + 1] = fast_exp2(fmaf(sacc[kb][r + 1], c, -mrow));
        part[kb * 8 + r / 2] = sacc[kb][r] + sacc[kb][r + 1];
      }
#pragma unroll
    for (int n = C::KB * 8; n > 1; n /= 2)
#pragma unroll
      for (int i = 0; i < n / 2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
    return part[0];
  };

  // Step t on the block at key j0; jn is the next block's key (SPARSE: it
  // is copied in during this step; -1 when this is the last).
  auto step = [&](int t, int j0, int jn, auto S) {
    constexpr int SN = (decltype(S)::value + ST - 1) % ST;  // stage of step t+ST-1
    // the stage of step t-1 is free (barrier at the end of the last step)
    if constexpr (SPARSE) {
      if (jn >= 0) fetch_at(jn, std::integral_constant<int, SN>{});
    } else {
      if (t + ST - 1 < ntiles) fetch(t + ST - 1, std::integral_constant<int, SN>{});
    }
    const bool active = !CAUSAL || j0 <= q0w + C::RW - 1;
    if (active) {
      const bf16_t* Ks = kst(S);
      const bf16_t* Vs = vst(S);
      f32x16 sacc[RB][C::KB];
      scores(Ks, j0, sacc);
      // Running maximum m (log2 units): taken from a row's first block
      // (which always holds key 0, so it is finite) and afterwards kept
      // while every exponentiated score of the row stays below kMaxWeight;
      // numerator and denominator share the base, so O and the
      // log-sum-exp do not depend on when m is raised.
      if (t == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) m[rb] = block_max(sacc[rb]);
      }
      float rs[RB];
      bool over = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        rs[rb] = exponentiate(sacc[rb], base(m[rb]));
        over |= !(rs[rb] <= kMaxWeight);
      }
      if (wave_any(over)) {
        // Some row overflowed the bound: rows whose own share (either half)
        // did so take the block's maximum, rescale O and l, and are
        // exponentiated again; the other rows recompute the same values.
        keep_branch();
        f32x16 s2[RB][C::KB];
        scores(Ks, j0, s2);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bool own = !(rs[rb] <= kMaxWeight);
          const bool row = max_halves(own ? 1.f : 0.f) > 0.f;
          const float mx = block_max(s2[rb]);
          if (row) {
            const float alpha = fast_exp2(m[rb] - mx);
            m[rb] = mx;
            l[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                if constexpr (FA_FWD_ACC_AGPR && D >= 256) {
                  if (r == 0) scale_acc_agpr(oacc[rb][db], alpha);
                } else {
                  oacc[rb][db][r] *= alpha;
                }
              }
          }
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) sacc[rb][kb] = s2[rb][kb];
          rs[rb] = exponentiate(sacc[rb], base(m[rb]));
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l[rb] += rs[rb];
      if constexpr (DROP) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            uint32_t dw[4];
            draws_query_cols(q0w + 32 * rb, j0 + 32 * kb, bh, lane, dr.k0, dr.k1, dw);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!kept(dw, r, dr.thresh)) sacc[rb][kb][r] = 0.f;
          }
      }

      // P^T as B operand (k-step u: registers 8*(u&1).. of key block u>>1,
      // i.e. keys 16u + 8*(e>>2) + 4h + (e&3)), rounded to bf16, then
      // O^T += V^T P^T with each V fragment feeding the RB row blocks.
      {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          bf16x8 pf[RB];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const f32x16& pv = sacc[rb][u >> 1];
            const int r0 = 8 * (u & 1);
            pf[rb] = bf16x8_from(pack_bf16x2(pv[r0], pv[r0 + 1]), pack_bf16x2(pv[r0 + 2], pv[r0 + 3]),
                                 pack_bf16x2(pv[r0 + 4], pv[r0 + 5]), pack_bf16x2(pv[r0 + 6], pv[r0 + 7]));
          }
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 vfr = frag_tr<D>(Vs, 16 * u, db * 32, lane);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32x32x16(vfr, pf[rb], oacc[rb][db]);
          }
        }
        if constexpr (D >= 256 && FA_FWD_IGLP_D256 > 0) {
          // two transpose reads per V fragment
          constexpr int A = FA_FWD_IGLP_D256, NV = C::PU * C::DB;
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * A, 0);
#pragma unroll
          for (int i = 0; i < NV - A; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, A, 0);
        }
      }
    }
    // step t+1 must be resident; later steps may still be in flight
    if (SPARSE ? jn >= 0 : t + 1 < ntiles) {
      wait_vmem_tiles<2 * C::DMA_PER_TILE, ST - 2>(SPARSE ? 0 : min(ST - 2, ntiles - t - 2));
      ring_barrier();
    }
  };
  if constexpr (PIPE) {
    // Software pipeline.  Step t computes the scores of block t, then its
    // softmax on the vector ALU interleaved with O^T += V^T P^T of block t-1
    // on the matrix cores (at head dim 256, one wavefront per SIMD: nothing
    // else would fill the matrix cores during the softmax; at head dim 64 the
    // wavefront's own P.V overlaps its softmax besides what the SIMD's other
    // three wavefronts overlap).  Step t copies in K of block
    // t+ST-1 and V of block t+ST-2: the K ring holds blocks t..t+ST-1 and
    // the V ring blocks t-1..t+ST-2, each block in stage (block mod ST).
    // Causal steps are active up to the wavefront's diagonal and inactive
    // after it, so an active step always has the previous block's P.V
    // pending.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2 % ST>;
    bf16x8 pp[C::PU];  // P^T of the previous block, B operands of V^T P^T
    bool pend = false;
    auto pv = [&](const bf16_t* Vs) {
#pragma unroll
      for (int u = 0; u < C::PU; ++u)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          oacc[0][db] = mfma32x32x16(frag_tr<D>(Vs, 16 * u, db * 32, lane), pp[u], oacc[0][db]);
    };
    // Copy plan of the ring: copy i of a [BC x D] tile takes LDS block
    // w + i*NWAVE of the stage (1 KB, lane L its 16 bytes at 16 L) from the
    // global chunk the swizzle places there; its per-lane byte offset for
    // row 0 and its LDS offset are fixed for the whole kernel.
    constexpr int NWAVE = NW;
    uint32_t cvo[C::DMA_PER_TILE], clo[C::DMA_PER_TILE];
#pragma unroll
    for (int i = 0; i < C::DMA_PER_TILE; ++i) {
      const int blk = w + i * NWAVE;
      const int pos = blk * 64 + lane;
      const int row = pos / (D / 8), cc = (pos % (D / 8)) ^ swz<D>(row);
      cvo[i] = ((uint32_t)row * D + cc * 8) * 2u;
      clo[i] = __builtin_amdgcn_readfirstlane((uint32_t)blk * 1024u);
    }
    const uint32_t lk[3] = {lds_address(k0s), lds_address(k1s), lds_address(k2s)};
    const uint32_t lv[3] = {lds_address(v0s), lds_address(v1s), lds_address(v2s)};
    // copy i of block r0's K (V) tile into stage st
    auto copy_k = [&](int r0, int st, int i) {
      lds_copy16_free(rk, cvo[i] + (uint32_t)r0 * (uint32_t)(D * 2), lk[st] + clo[i]);
    };
    auto copy_v = [&](int r0, int st, int i) {
      lds_copy16_free(rv, cvo[i] + (uint32_t)r0 * (uint32_t)(D * 2), lv[st] + clo[i]);
    };
    // keeps the matrix instructions and the copies in program order (vector
    // and scalar ALU instructions may still move across)
    auto pin = [] { __builtin_amdgcn_sched_barrier(0x406); };
    auto pstep = [&](int t, auto S, auto FIRST, auto OFFD) {
      constexpr int s = decltype(S)::value;
      constexpr bool first = decltype(FIRST)::value;
      constexpr bool offd = decltype(OFFD)::value;  // a block left of the diagonal
      constexpr int sk = (s + ST - 1) % ST;  // stage of K(t+ST-1), and of V(t-1)
      constexpr int sv = (s + ST - 2) % ST;  // stage of V(t+ST-2)
      const int j0 = kbase + t * BC;
      const bool kf = t + ST - 1 < ntiles, vf = t + ST - 2 < ntiles;
      const bf16_t* Ks = kst(S);
      const bf16_t* Vp = vst(std::integral_constant<int, sk>{});  // V of block t-1
      const bool active = offd || !CAUSAL || j0 <= q0w + C::RW - 1;
      // Main path (active steps after the first): the copies are spread
      // over the score section, one after every FA_FWD_DMA_GAP-th matrix
      // instruction.  Each copy holds up the wavefront's issue until the
      // texture unit takes it, which a burst at the start of the step turns
      // into a stall of all four wavefronts.  There they are issued
      // unconditionally: a copy past the last block reads rows past the
      // range (zeros) or rows it does not need, into a stage that is not
      // read again.
      constexpr bool spread = !first;
      auto copy_part = [&](int i) {  // copies of K of block t+ST-1, then of V of block t+ST-2
        if (i < C::DMA_PER_TILE) copy_k(j0 + (ST - 1) * BC, sk, i);
        else copy_v(j0 + (ST - 2) * BC, sv, i - C::DMA_PER_TILE);
      };
      if (!spread || !active) {
        if (kf) dma_tile<D, BC, C::NT>(rk, j0 + (ST - 1) * BC, kst(std::integral_constant<int, sk>{}), tid);
        if (vf) dma_tile<D, BC, C::NT>(rv, j0 + (ST - 2) * BC, vst(std::integral_constant<int, sv>{}), tid);
      }
      if (active) {
        f32x16 sacc[RB][C::KB];
        if constexpr (spread) {
          // S^T = K Q^T written in issue order (the KB 32-key blocks one
          // after the other): K fragment reads A ahead, copies between the
          // matrix instructions
          constexpr int A = D == 64 ? FA_FWD_PIPE_D64_KA : FA_FWD_IGLP_D256 > 0 ? FA_FWD_IGLP_D256 : 3;
          constexpr int W = A + 1, NS = C::KB * C::KSTEPS;
          auto kread = [&](int n) { return frag_rows<D>(Ks, 32 * (n / C::KSTEPS), 16 * (n % C::KSTEPS), c32, h); };
          bf16x8 kw[W];
#pragma unroll
          for (int i = 0; i < A; ++i) kw[i] = kread(i);
          const f32x16 z = {};
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            if (i + A < NS) kw[(i + A) % W] = kread(i + A);
            const int kb = i / C::KSTEPS, ks = i % C::KSTEPS;
            sacc[0][kb] = mfma32x32x16(kw[i % W], qf[0][ks], ks == 0 ? z : sacc[0][kb]);
            if (i % FA_FWD_DMA_GAP == 0 && i / FA_FWD_DMA_GAP < 2 * C::DMA_PER_TILE) {
              pin();
              copy_part(i / FA_FWD_DMA_GAP);
              pin();
            }
          }
          const bool need_mask = !offd && ((j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w));
          if (need_mask) {
            keep_branch();
            const int nk = N - j0 - 4 * h;
            const int kq = j0 + 4 * h - (q0w + c32);
            const int lim = CAUSAL ? min(-kq, nk - 1) : nk - 1;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[0][kb][r] = -INFINITY;
          }
        } else {
          scores(Ks, j0, sacc);
        }
        float rs[RB];
        if constexpr (first) {
          m[0] = block_max(sacc[0]);
          rs[0] = exponentiate(sacc[0], base(m[0]));
        } else {
          {
            // written in issue order: V fragment reads A ahead, then each
            // matrix instruction followed by its share of the exponentials
            constexpr int A = D == 64 ? FA_FWD_PIPE_D64_VA : FA_FWD_PIPE_VA, NV = C::PU * C::DB, W = A + 1;
            const float mb = base(m[0]);
            bf16x8 vw[W];
#pragma unroll
            for (int i = 0; i < A; ++i) vw[i] = frag_tr<D>(Vp, 16 * (i / C::DB), (i % C::DB) * 32, lane);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
              if (i + A < NV) {
                const int n = i + A;
                vw[n % W] = frag_tr<D>(Vp, 16 * (n / C::DB), (n % C::DB) * 32, lane);
              }
              oacc[0][i % C::DB] = mfma32x32x16(vw[i % W], pp[i / C::DB], oacc[0][i % C::DB]);
              // the block's 16 KB exponentials spread evenly over the NV
              // matrix instructions (one each at head dim 256)
              constexpr int EPM = 16 * C::KB / NV;
              static_assert(EPM * NV == 16 * C::KB, "exponentials per matrix instruction");
#pragma unroll
              for (int e = 0; e < EPM; ++e) {
                const int n = i * EPM + e;
                sacc[0][n / 16][n % 16] = fast_exp2(fmaf(sacc[0][n / 16][n % 16], c, -mb));
              }
              if constexpr (spread) {
                // the copies that did not fit in the score section
                constexpr int NS = (C::KB * C::KSTEPS + FA_FWD_DMA_GAP - 1) / FA_FWD_DMA_GAP;
                if (NS + (i - 2) / 3 < 2 * C::DMA_PER_TILE && i >= 2 && (i - 2) % 3 == 0) {
                  pin();
                  copy_part(NS + (i - 2) / 3);
                  pin();
                }
              }
            }
            // row sum in the order exponentiate() takes it
            float part[C::KB * 8];
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
              for (int r = 0; r < 8; ++r) part[kb * 8 + r] = sacc[0][kb][2 * r] + sacc[0][kb][2 * r + 1];
#pragma unroll
            for (int n = C::KB * 8; n > 1; n /= 2)
#pragma unroll
              for (int i = 0; i < n / 2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
            rs[0] = part[0];
          }
        }
        if (wave_any(!(rs[0] <= kMaxWeight))) {
          // a row broke the bound: as in the plain loop (O already holds
          // block t-1, so the rescale covers it)
          keep_branch();
          f32x16 s2[RB][C::KB];
          scores(Ks, j0, s2);
          const bool own = !(rs[0] <= kMaxWeight);
          const bool row = max_halves(own ? 1.f : 0.f) > 0.f;
          const float mx = block_max(s2[0]);
          if (row) {
            const float alpha = fast_exp2(m[0] - mx);
            m[0] = mx;
            l[0] *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                if constexpr (FA_FWD_ACC_AGPR) {
                  if (r == 0) scale_acc_agpr(oacc[0][db], alpha);
                } else {
                  oacc[0][db][r] *= alpha;
                }
              }
          }
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) sacc[0][kb] = s2[0][kb];
          rs[0] = exponentiate(sacc[0], base(m[0]));
        }
        l[0] += rs[0];
        if constexpr (DROP) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            uint32_t dw[4];
            draws_query_cols(q0w, j0 + 32 * kb, bh, lane, dr.k0, dr.k1, dw);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!kept(dw, r, dr.thresh)) sacc[0][kb][r] = 0.f;
          }
        }
        // k-step u of V^T P^T: registers 8*(u&1).. of key block u>>1 (keys
        // 16u + 8*(e>>2) + 4h + (e&3))
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const f32x16& pv_ = sacc[0][u >> 1];
          const int r0 = 8 * (u & 1);
          pp[u] = bf16x8_from(pack_bf16x2(pv_[r0], pv_[r0 + 1]), pack_bf16x2(pv_[r0 + 2], pv_[r0 + 3]),
                              pack_bf16x2(pv_[r0 + 4], pv_[r0 + 5]), pack_bf16x2(pv_[r0 + 6], pv_[r0 + 7]));
        }
        pend = true;
      } else if (pend) {
        pv(Vp);
        pend = false;
      }
      // K of block t+1 and V of block t resident (this step's copies may
      // stay in flight); the stages read in this step are free
      if constexpr (ST == 2) wait_vmem_le<0>();
      else wait_vmem_tiles<C::DMA_PER_TILE, 2>((int)kf + (int)vf);
      ring_barrier();
    };
    using OFF = std::integral_constant<bool, TWO || (NOMASK && !CAUSAL)>;
    // blocks run by the pipelined loop: all, or those left of the diagonal
    const int ntp = TWO ? min(ntiles, max(0, (q0 - kbase) / BC)) : ntiles;
    if (ntp > 0) pstep(0, S0{}, std::true_type{}, OFF{});
    for (int t = 1; t < ntp; t += ST) {
      pstep(t, S1{}, std::false_type{}, OFF{});
      if (t + 1 < ntp) pstep(t + 1, S2{}, std::false_type{}, OFF{});
      if constexpr (ST > 2) {
        if (t + 2 < ntp) pstep(t + 2, S0{}, std::false_type{}, OFF{});
      }
    }
    if (TWO && ntp < ntiles) {
      // Hand over to the plain loop at block ntp: its K came in during the
      // last pipelined step (or before the loop); copy its V into the stage
      // of its parity (which held block ntp-2's), add block ntp-1's pending
      // product, and let the plain loop go on from there.
      const int jn = kbase + ntp * BC;
      if ((ntp & 1) == 0) dma_tile<D, BC, C::NT>(rv, jn, v0s, tid);
      else dma_tile<D, BC, C::NT>(rv, jn, v1s, tid);
      if (pend) {
        if ((ntp & 1) == 0) pv(v1s);
        else pv(v0s);
        pend = false;
      }
      wait_vmem_le<0>();
      ring_barrier();
      int t = ntp;
      if (t & 1) {
        step(t, jn, -1, std::integral_constant<int, 1>{});
        ++t;
      }
      for (; t < ntiles; t += 2) {
        step(t, kbase + t * BC, -1, std::integral_constant<int, 0>{});
        if (t + 1 < ntiles) step(t + 1, kbase + (t + 1) * BC, -1, std::integral_constant<int, 1>{});
      }
    } else if (pend) {
      // P.V of the last block
      const int sl = (ntiles - 1) % ST;
      if (sl == 0) {
        pv(v0s);
      } else {
        if constexpr (ST > 2) {
          if (sl == 2) pv(v2s);
          else pv(v1s);
        } else {
          pv(v1s);
        }
      }
    }
  } else if constexpr (SPARSE) {
    int j0 = jfirst, jn = walk.next(j0);
    for (int t = 0;; t += 2) {
      step(t, j0, jn, std::integral_constant<int, 0>{});
      if (jn < 0) break;
      j0 = jn;
      jn = walk.next(j0);
      step(t + 1, j0, jn, std::integral_constant<int, 1>{});
      if (jn < 0) break;
      j0 = jn;
      jn = walk.next(j0);
    }
  } else {
    for (int t0 = 0; t0 < ntiles; t0 += ST) {
      step(t0, kbase + t0 * BC, -1, std::integral_constant<int, 0>{});
      if (t0 + 1 < ntiles) step(t0 + 1, kbase + (t0 + 1) * BC, -1, std::integral_constant<int, 1>{});
      if constexpr (ST > 2) {
        if (t0 + 2 < ntiles) step(t0 + 2, kbase + (t0 + 2) * BC, -1, std::integral_constant<int, 2>{});
      }
    }
  }

  if constexpr (SPARSE) {
    if (slotw >= 0) {
      // segment of a split tile row: O normalised over the segment (float32)
      // and the segment's log-sum-exp, for the merge kernel; every row sees
      // the first key of the segment's first tile, so l > 0
      const size_t prow = ((size_t)(slotw >> 1) * BH + bh) * C::BR;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int query = q0w + 32 * rb + c32;
        const float lt = sum_halves(l[rb]);
        const float inv = __builtin_amdgcn_rcpf(lt);
        if (query < N) {
          float* Op = sp.part_o + (prow + (query - q0)) * D;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<float4*>(Op + db * 32 + 8 * g + 4 * h) =
                  make_float4(oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv,
                              oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
          if (h == 0) sp.part_l[prow + (query - q0)] = (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2;
        }
      }
      return;
    }
  }

  if constexpr (SPLIT) {
    // Partial result of the range: O normalised over it (float32, each lane
    // its 4-value groups db*32 + 8g + 4h + 0..3) and its log-sum-exp; a row
    // that saw no key of the range has l = 0 and gets O = 0, LSE = -inf.
    const size_t rows = (size_t)BH * N;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int query = q0w + 32 * rb + c32;
      const float lt = sum_halves(l[rb]);
      const float inv = lt > 0.f ? __builtin_amdgcn_rcpf(lt) : 0.f;
      if (query < N) {
        const size_t r = split * rows + (size_t)bh * N + query;
        float* Op = sa.Opart + r * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(Op + db * 32 + 8 * g + 4 * h) =
                make_float4(oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv,
                            oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
        if (h == 0) sa.Lpart[r] = lt > 0.f ? (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
      }
    }
    return;
  }

  // Epilogue: O = acc / l (bf16), LSE = m ln2 + ln l (fp32, natural log).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int query = q0w + 32 * rb + c32;
    const float lt = sum_halves(l[rb]);  // >= 1: the row maximum has weight >= 1
    const float inv = DROP ? __builtin_amdgcn_rcpf(lt) * dr.scale : __builtin_amdgcn_rcpf(lt);
    if constexpr (C::QST) {
      // O fragment (dims db*32 + 8g + 4h + 0..3 of this lane's row) into
      // this wavefront's rows of the Q staging tile
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = pack_bf16x2(oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv);
          const uint32_t hi = pack_bf16x2(oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(qs + tile_off<D>(w * C::RW + 32 * rb + c32, db * 32 + 8 * g + 4 * h)) =
              make_uint2(lo, hi);
        }
    } else if (query < N) {
      bf16_t* Or = O + hoff + (size_t)query * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = pack_bf16x2(oacc[rb][db][4 * g] * inv, oacc[rb][db][4 * g + 1] * inv);
          const uint32_t hi = pack_bf16x2(oacc[rb][db][4 * g + 2] * inv, oacc[rb][db][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(Or + db * 32 + 8 * g + 4 * h) = make_uint2(lo, hi);
        }
    }
    if (h == 0 && query < N) LSE[(size_t)bh * N + query] = (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2;
  }
  if constexpr (C::QST) {
    // rows back out of LDS as whole 16-byte chunks: 8 lanes per row, so each
    // store instruction writes 8 complete rows
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::RW * CPR / kWave; ++i) {
      const int chunk = i * kWave + lane;
      const int r = chunk / CPR, cc = chunk % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(qs + tile_off<D>(w * C::RW + r, cc * 8));
      if (q0w + r < N) *reinterpret_cast<uint4*>(O + hoff + (size_t)(q0w + r) * D + cc * 8) = v;
    }
  }
}

template <int D, int NW, int RB, int BC, int ST, int OCC, bool CAUSAL>
hipError_t run_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   const Problem& p, hipStream_t stream, SparseArgs sp) {
  using C = FwdCfg<D, NW, RB, BC, ST>;
  const int BH = p.B * p.H;
  // workgroups per head: query blocks, or the balanced schedule's row items
  const int nqb = sp.rows != nullptr ? sp.n_rows : (p.N + C::BR - 1) / C::BR;
  const long long grid = (long long)BH * nqb;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = p.scale * kLog2e;
  const int G = head_group(OCC * 4 / NW, nqb);
  if (sp.on()) {
    // the sparse walk takes 128-row query blocks in two stages
    if constexpr (C::BR == 128)
      hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, 2, OCC, CAUSAL, false, true>), dim3((unsigned)grid),
                         dim3(C::NT), 0, stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                         (bf16_t*)O, LSE, BH, p.N, nqb, G, c, SplitArgs{}, sp);
    else
      return hipErrorNotSupported;
  } else {
    // the unmasked pipelined loop: causal head dim 64 with long rows, or head
    // dim 256 without the causal mask and without a partial block (0.8%
    // faster at 2·16·16384·256; neutral at head dim 64, which keeps one kernel)
    constexpr bool can = C::PIPE && (CAUSAL ? D == 64 : D >= 256);
    if constexpr (can) {
      if (CAUSAL ? p.N >= FA_FWD_LONG_N : p.N % BC == 0) {
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL, false, false, false, true>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (bf16_t*)O, LSE, BH, p.N, nqb, G, c,
                           SplitArgs{}, SparseArgs{});
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL>), dim3((unsigned)grid),
                       dim3(C::NT), 0, stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (bf16_t*)O, LSE, BH, p.N, nqb, G, c, SplitArgs{}, SparseArgs{});
  }
  return hipGetLastError();
}

template <int D, int NW, int RB, int BC, int ST, int OCC, bool CAUSAL>
hipError_t run_fwd_drop(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        const Problem& p, const DropArgs& dr, hipStream_t stream) {
  using C = FwdCfg<D, NW, RB, BC, ST>;
  const int BH = p.B * p.H;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  const long long grid = (long long)BH * nqb;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = p.scale * kLog2e;
  const int G = head_group(OCC * 4 / NW, nqb);
  if constexpr (CAUSAL && D == 64 && C::PIPE) {
    if (p.N >= FA_FWD_LONG_N) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL, false, false, true, true>),
                         dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q,
                         (const bf16_t*)K, (const bf16_t*)V, (bf16_t*)O, LSE, BH, p.N, nqb, G, c,
                         SplitArgs{}, SparseArgs{}, dr);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL, false, false, true>),
                     dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q, (const bf16_t*)K,
                     (const bf16_t*)V, (bf16_t*)O, LSE, BH, p.N, nqb, G, c, SplitArgs{}, SparseArgs{},
                     dr);
  return hipGetLastError();
}

template <int D, int NW, int RB, int BC, int ST, int OCC>
hipError_t run_fwd_drop_c(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          const Problem& p, const DropArgs& dr, hipStream_t stream) {
  return p.causal ? run_fwd_drop<D, NW, RB, BC, ST, OCC, true>(Q, K, V, O, LSE, p, dr, stream)
                  : run_fwd_drop<D, NW, RB, BC, ST, OCC, false>(Q, K, V, O, LSE, p, dr, stream);
}

template <int D, int NW, int RB, int BC, int ST, int OCC>
hipError_t run_fwd_c(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     const Problem& p, hipStream_t stream, SparseArgs sp) {
  return p.causal ? run_fwd<D, NW, RB, BC, ST, OCC, true>(Q, K, V, O, LSE, p, stream, sp)
                  : run_fwd<D, NW, RB, BC, ST, OCC, false>(Q, K, V, O, LSE, p, stream, sp);
}

// Merge of partial results (CS324 notes, exercises 3 and 7, and the
// Flash-Decoding scheme of section 8.2): for each row, with L_s the parts'
// log-sum-exps and M = max_s L_s,
//   LSE = M + ln sum_s e^{L_s - M},   O = sum_s e^{L_s - LSE} O_s,
// which is the pairwise merge of (m, l, O) states applied to all parts at
// once (a part's state is (L_s, 1) up to the common factor).  Parts with
// L_s = -inf carry no weight and their O_s is not read.  D/4 lanes per row,
// four consecutive values each; memory-bound.
template <int D, typename OutT>
__global__ __launch_bounds__(256)
void merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart, int splits,
                  long long rows, OutT* __restrict__ O, float* __restrict__ LSE) {
  constexpr int TPR = D / 4;       // lanes per row
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  if (row >= rows) return;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, Lpart[s * rows + row]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float sum = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float Ls = Lpart[s * rows + row];
      if (Ls == -INFINITY) continue;
      const float wgt = expf(Ls - M);
      const float4 v = *reinterpret_cast<const float4*>(Opart + ((size_t)s * rows + row) * D + 4 * part);
      sum += wgt;
      acc.x = fmaf(wgt, v.x, acc.x);
      acc.y = fmaf(wgt, v.y, acc.y);
      acc.z = fmaf(wgt, v.z, acc.z);
      acc.w = fmaf(wgt, v.w, acc.w);
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if constexpr (sizeof(OutT) == 2) {
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(O) + row * D + 4 * part) =
        make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(O) + row * D + 4 * part) = o;
  }
  if (part == 0) LSE[row] = sum > 0.f ? M + logf(sum) : -INFINITY;
}

template <int D, int NW, int RB, int BC, int ST, int OCC, bool CAUSAL>
hipError_t run_fwd_split(const void* Q, const void* K, const void* V, const Problem& p,
                         int splits, float* Opart, float* Lpart, hipStream_t stream) {
  using C = FwdCfg<D, NW, RB, BC, ST>;
  const int BH = p.B * p.H;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  const long long grid = (long long)BH * nqb * splits;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = p.scale * kLog2e;
  const int G = head_group(OCC * 4 / NW, nqb);
  SplitArgs sa;
  sa.span = split_span(p.N, splits);
  sa.splits = splits;
  sa.Opart = Opart;
  sa.Lpart = Lpart;
  if constexpr (CAUSAL && D == 64 && C::PIPE) {
    if (p.N >= FA_FWD_LONG_N) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL, true, false, false, true>),
                         dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q,
                         (const bf16_t*)K, (const bf16_t*)V, (bf16_t*)nullptr, (float*)nullptr, BH,
                         p.N, nqb, G, c, sa);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, RB, BC, ST, OCC, CAUSAL, true>), dim3((unsigned)grid),
                     dim3(C::NT), 0, stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                     (bf16_t*)nullptr, (float*)nullptr, BH, p.N, nqb, G, c, sa);
  return hipGetLastError();
}

template <int D, int NW, int RB, int BC, int ST, int OCC>
hipError_t run_fwd_split_c(const void* Q, const void* K, const void* V, const Problem& p,
                           int splits, float* Opart, float* Lpart, hipStream_t stream) {
  return p.causal
             ? run_fwd_split<D, NW, RB, BC, ST, OCC, true>(Q, K, V, p, splits, Opart, Lpart, stream)
             : run_fwd_split<D, NW, RB, BC, ST, OCC, false>(Q, K, V, p, splits, Opart, Lpart, stream);
}

template <int D>
hipError_t run_merge(const float* Opart, const float* Lpart, int splits, void* O, float* LSE,
                     long long rows, bool bf16, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 4);
  const long long grid = (rows + RPB - 1) / RPB;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16)
    hipLaunchKernelGGL((merge_kernel<D, bf16_t>), dim3((unsigned)grid), dim3(256), 0, stream, Opart,
                       Lpart, splits, rows, (bf16_t*)O, LSE);
  else
    hipLaunchKernelGGL((merge_kernel<D, float>), dim3((unsigned)grid), dim3(256), 0, stream, Opart,
                       Lpart, splits, rows, (float*)O, LSE);
  return hipGetLastError();
}

// Launch configurations per head dim: wavefronts per workgroup, 32-row
// query blocks per wavefront, keys per K/V block, pipeline stages, minimum
// wavefronts per SIMD.
#ifndef FA_FWD_CFG_D64
#define FA_FWD_CFG_D64 4, 1, 32, 2, 4
#endif
#ifndef FA_FWD_CFG_D128
#define FA_FWD_CFG_D128 4, 1, 64, 2, 2
#endif
#ifndef FA_FWD_CFG_D256
#define FA_FWD_CFG_D256 4, 1, 32, 2, 1
#endif
// plain non-causal head-dim-256 forward: 64-key blocks (half the steps,
// barriers and row-sum checks per key).  The causal, sparse, key-split and
// dropout kernels keep 32-key blocks: compiled with 64, the causal kernel
// needs 704 bytes of scratch per lane (the registers run out) and ran 15x
// slower.
#ifndef FA_FWD_CFG_D256_NC
#define FA_FWD_CFG_D256_NC 4, 1, 64, 2, 1
#endif

}  // namespace

#ifndef FA_D256_UNIT
hipError_t launch_forward_split_bf16(const void* Q, const void* K, const void* V, const Problem& p,
                                     int splits, float* Opart, float* Lpart, hipStream_t stream) {
  switch (p.d) {
    case 64: return run_fwd_split_c<64, FA_FWD_CFG_D64>(Q, K, V, p, splits, Opart, Lpart, stream);
    case 128: return run_fwd_split_c<128, FA_FWD_CFG_D128>(Q, K, V, p, splits, Opart, Lpart, stream);
    case 256: return launch_forward_split_bf16_d256(Q, K, V, p, splits, Opart, Lpart, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge(const float* Opart, const float* Lpart, int splits, void* O, float* LSE,
                        const Problem& p, bool bf16, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.N;
  switch (p.d) {
    case 64: return run_merge<64>(Opart, Lpart, splits, O, LSE, rows, bf16, stream);
    case 128: return run_merge<128>(Opart, Lpart, splits, O, LSE, rows, bf16, stream);
    case 256: return run_merge<256>(Opart, Lpart, splits, O, LSE, rows, bf16, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_dropout_bf16(const void* Q, const void* K, const void* V, void* O,
                                       float* LSE, const Problem& p, const DropArgs& dr,
                                       hipStream_t stream) {
  switch (p.d) {
    case 64: return run_fwd_drop_c<64, FA_FWD_CFG_D64>(Q, K, V, O, LSE, p, dr, stream);
    case 128: return run_fwd_drop_c<128, FA_FWD_CFG_D128>(Q, K, V, O, LSE, p, dr, stream);
    case 256: return launch_forward_dropout_bf16_d256(Q, K, V, O, LSE, p, dr, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const Problem& p, hipStream_t stream, SparseArgs sp) {
  switch (p.d) {
    case 64: return run_fwd_c<64, FA_FWD_CFG_D64>(Q, K, V, O, LSE, p, stream, sp);
    case 128: return run_fwd_c<128, FA_FWD_CFG_D128>(Q, K, V, O, LSE, p, stream, sp);
    case 256: return launch_forward_bf16_d256(Q, K, V, O, LSE, p, stream, sp);
    default: return hipErrorInvalidValue;
  }
}
#else
// Head dim 256 (this source compiled a second time as fa_fwd_d256.hip)
hipError_t launch_forward_split_bf16_d256(const void* Q, const void* K, const void* V,
                                          const Problem& p, int splits, float* Opart, float* Lpart,
                                          hipStream_t stream) {
  return run_fwd_split_c<256, FA_FWD_CFG_D256>(Q, K, V, p, splits, Opart, Lpart, stream);
}

hipError_t launch_forward_dropout_bf16_d256(const void* Q, const void* K, const void* V, void* O,
                                            float* LSE, const Problem& p, const DropArgs& dr,
                                            hipStream_t stream) {
  return run_fwd_drop_c<256, FA_FWD_CFG_D256>(Q, K, V, O, LSE, p, dr, stream);
}

hipError_t launch_forward_bf16_d256(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, const Problem& p, hipStream_t stream,
                                    SparseArgs sp) {
  if (!p.causal && !sp.on()) return run_fwd<256, FA_FWD_CFG_D256_NC, false>(Q, K, V, O, LSE, p, stream, sp);
  return run_fwd_c<256, FA_FWD_CFG_D256>(Q, K, V, O, LSE, p, stream, sp);
}
#endif

}  // namespace fa
