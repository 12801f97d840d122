// fa_bwd.hip -- attention backward for gfx950, bfloat16 in, fp32 accumulate.
//
// Algorithm: the recomputing backward ("Lecture 8 . GPU Performance &
// FlashAttention", CS324 notes, section 5.4; "FlashAttention and GPU memory"
// section 09).  Only O and the per-row log-sum-exp were saved by the
// forward; every block of S and P is rebuilt on chip from Q, K and LSE and
// used at once, so no N x N matrix reaches device memory.  The chain rule
// through softmax gives, per block,
//     P = exp(scale Q K^T - LSE),  dV += P^T dO,  dP = dO V^T,
//     dS = P * (dP - D),  dQ += scale dS K,  dK += scale dS^T Q,
// with D_i = sum_k dO_ik O_ik (the identity stated in section 5.4), which
// needs only N x d data.
//
// Three kernels, no atomics (results are bitwise reproducible):
//   dq    one block of 128 query rows per workgroup (32 per wavefront),
//         loop over K/V blocks staged in LDS; dQ written once.  It also
//         forms D for its rows from the O and dO fragments it holds and
//         stores D for the next kernel.
//   dkdv  one block of 128 keys per workgroup (32 per wavefront, K and V
//         fragments held in VGPRs), loop over query chunks staged in LDS;
//         dK and dV accumulate in registers and are written once.
//   pre   D = rowsum(dO * O) alone, fp32, bandwidth-bound; only for callers
//         that run the dK/dV stage without the dQ stage.
// Matrix-core orientation is chosen per kernel so that the operand that is
// reused stays in registers, softmax statistics are per-lane where possible,
// and the P / dS fragments produced by one v_mfma_f32_32x32x16_bf16 are fed
// straight back as the B operand of the next one.
#include <type_traits>

#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// -D_i = -sum_k dO_ik O_ik  (fp32), one row per D/8 lanes (16-byte loads),
// and LSE_i * log2(e) beside it.
template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_bf16_kernel(const bf16_t* __restrict__ O, const bf16_t* __restrict__ dO,
                         const float* __restrict__ LSE, float* __restrict__ Dws,
                         float* __restrict__ Lws, long long rows) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + part * 8;
    const uint4 a = *reinterpret_cast<const uint4*>(O + off);
    const uint4 b = *reinterpret_cast<const uint4*>(dO + off);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w};
    const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_to_f32((bf16_t)(av[e] & 0xffffu)), bf16_to_f32((bf16_t)(bv[e] & 0xffffu)), acc);
      acc = fmaf(bf16_to_f32((bf16_t)(av[e] >> 16)), bf16_to_f32((bf16_t)(bv[e] >> 16)), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) {
    Dws[row] = -acc;
    Lws[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  Per wavefront: KB blocks of 32 keys whose K and V fragments stay
// in VGPRs; every Q, dO, LSE and D fragment read from LDS feeds the KB
// blocks' matrix instructions.  Per
// step: a chunk of BQ = 32*QB query rows of Q and dO, with that chunk's
// LSE*log2(e) and -D, copied HBM -> LDS by direct buffer->LDS loads into an
// ST-stage ring (one LDS variable per stage and operand).  Q and dO are read
// by rows for S = Q K^T and dP = dO V^T, and through the LDS transpose unit
// for dK^T += Q^T dS and dV^T += dO^T P.
template <int D, int NW, int KB, int QB, int ST>
struct DkdvCfg {
  static constexpr int NT = NW * kWave;
  static constexpr int KW = KB * 32;          // keys per wavefront
  static constexpr int BK = NW * KW;          // keys per workgroup
  static constexpr int BQ = 32 * QB;          // query rows per chunk
  static constexpr int TILE = BQ * D;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int PU = BQ / 16;
  // per stage and wavefront: Q and dO tiles, then one 4-byte copy each of
  // the chunk's LSE*log2e and D
  static constexpr int DMA_PER_TILE = 2 * (TILE / 8 / NT) + 2;
  // K and V blocks staged through LDS (coalesced copies in, dK and dV out
  // through the same rows) when both fit in 32 KB; otherwise their
  // fragments load straight from HBM
  static constexpr bool KL = 2 * BK * D * 2 <= 32768;
  static_assert(BQ <= kWave, "one lane per chunk row copies LSE and D");
  static_assert(ST >= 2 && ST <= 3, "two or three Q/dO stages");
};

// SPARSE: block-sparse attention; the loop visits only the query chunks of
// the 128 x 128 tiles set in column kb of the tile mask (the key block is
// one tile column: BK = 128); with none, dK and dV are 0.
//
// DROP: dropout on the weights, the draws regenerated as in the forward,
// with Z the keep mask: dV = (256/t) sum (Z P)^T dO, and dS = P (Z dP' 256/t
// - D) computed as (256/t) P (Z ? dP' - D t/256 : -D t/256) by starting the
// dP' accumulation from -D t/256; the factor 256/t of dK is part of `scale`
// (the host passes scale * 256/t).
//
// PARTS: bit 0 = dV, bit 1 = dK.  A launch with one part recomputes S (and,
// for dK, dP) and accumulates only that gradient: two launches instead of
// one when the two accumulators would not fit the registers (head dim 256:
// 2 x 128 registers of accumulators beside 128 of K and V fragments).
template <int D, int NW, int KB, int QB, int ST, int OCC, bool CAUSAL, bool SPARSE = false,
          bool DROP = false, int PARTS = 3>
__global__ __launch_bounds__(NW * 64, OCC)
void bwd_dkdv_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                          const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                          const float* __restrict__ Lws, const float* __restrict__ Dws,
                          bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int BH, int N,
                          int nkb, int G, float c, float scale, SparseArgs sp = {},
                          DropArgs dr = {}) {
  using C = DkdvCfg<D, NW, KB, QB, ST>;
  static_assert(!(SPARSE && DROP), "one variant at a time");
  static_assert(!SPARSE || (ST == 2 && C::BK == 128), "sparse walk: two stages, 128-key blocks");
  static_assert(PARTS >= 1 && PARTS <= 3, "dV, dK or both");
  constexpr bool DVP = PARTS & 1, DKP = PARTS & 2;
  // per stage: Q tile, dO tile, and 64 floats each of LSE*log2e and D
  __shared__ __attribute__((aligned(16))) bf16_t q0s[C::TILE], o0s[C::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t q1s[C::TILE], o1s[C::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t q2s[ST > 2 ? C::TILE : 8], o2s[ST > 2 ? C::TILE : 8];
  __shared__ __attribute__((aligned(16))) float l0s[kWave], d0s[kWave], l1s[kWave], d1s[kWave];
  __shared__ __attribute__((aligned(16))) float l2s[ST > 2 ? kWave : 4], d2s[ST > 2 ? kWave : 4];
  __shared__ __attribute__((aligned(16))) bf16_t ksg[C::KL ? C::BK * D : 8], vsg[C::KL ? C::BK * D : 8];
  auto qst = [&](auto S) -> bf16_t* {
    if constexpr (decltype(S)::value == 0) return q0s;
    else if constexpr (decltype(S)::value == 1) return q1s;
    else return q2s;
  };
  auto ost = [&](auto S) -> bf16_t* {
    if constexpr (decltype(S)::value == 0) return o0s;
    else if constexpr (decltype(S)::value == 1) return o1s;
    else return o2s;
  };
  auto lst = [&](auto S) -> float* {
    if constexpr (decltype(S)::value == 0) return l0s;
    else if constexpr (decltype(S)::value == 1) return l1s;
    else return l2s;
  };
  auto dst_ = [&](auto S) -> float* {
    if constexpr (decltype(S)::value == 0) return d0s;
    else if constexpr (decltype(S)::value == 1) return d1s;
    else return d2s;
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  int bh, kb;  // causal: low key blocks see the most queries, run them first
  grouped_order(xcd_remap(blockIdx.x, BH * nkb), nkb, BH, G, bh, kb);
  // balanced schedule: item kb names the tile column and its run of tiles
  int list_off = 0, list_cnt = -1, slotw = -1;
  if constexpr (SPARSE) {
    if (sp.cols != nullptr &&
        !sched_item(sp.cols, kb, sp.nb, sp.list_len, sp.col_slots, kb, list_off, list_cnt, slotw))
      return;
  }
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_copy_rsrc(Q + hoff, head_bytes);
  const auto ro = make_copy_rsrc(dO + hoff, head_bytes);
  const auto rl = make_copy_rsrc(Lws + (size_t)bh * N, (uint32_t)N * 4u);
  const auto rd = make_copy_rsrc(Dws + (size_t)bh * N, (uint32_t)N * 4u);

  const int k0 = kb * C::BK;
  const int k0w = k0 + w * C::KW;  // this lane's key rows: k0w + 32 kk + c32 (MFMA column)

  f32x16 dkacc[KB][C::DB], dvacc[KB][C::DB];
#pragma unroll
  for (int kk = 0; kk < KB; ++kk)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[kk][db][r] = 0.f;
        dvacc[kk][db][r] = 0.f;
      }

  const int qstart = CAUSAL ? (k0 / C::BQ) * C::BQ : 0;
  const int nchunks = (N - qstart + C::BQ - 1) / C::BQ;
  // query chunks visited: dense from qstart, or those of the set tiles
  BlockWalk<C::BQ, SPARSE> walk{N,
                                list_cnt >= 0 ? (const_int_ptr)sp.lists + list_off
                                              : (const_int_ptr)(sp.mask + kb),
                                sp.nb, sp.nb - 1, list_cnt};
  const int ifirst = SPARSE ? walk.first(qstart) : qstart;

  auto fetch_at = [&](int i0, auto S) {
    dma_tile<D, C::BQ, C::NT>(rq, i0, qst(S), tid);
    dma_tile<D, C::BQ, C::NT>(ro, i0, ost(S), tid);
    dma_rows_f32<C::BQ>(rl, i0, lst(S), lane);
    dma_rows_f32<C::BQ>(rd, i0, dst_(S), lane);
  };
  auto fetch = [&](int t, auto S) { fetch_at(qstart + t * C::BQ, S); };
  // The first Q/dO copies go out before K and V are read, so that the
  // latencies overlap.
  if (ifirst >= 0) fetch_at(ifirst, std::integral_constant<int, 0>{});
  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (lane = key).
  bf16x8 kf[KB][C::KSTEPS], vf[KB][C::KSTEPS];
  if constexpr (C::KL) {
    // K and V blocks copied row-major (coalesced) into LDS, rows past N as 0
    dma_tile<D, C::BK, C::NT>(make_copy_rsrc(K + hoff, head_bytes), k0, ksg, tid);
    dma_tile<D, C::BK, C::NT>(make_copy_rsrc(V + hoff, head_bytes), k0, vsg, tid);
  } else {
    const auto rk = make_rsrc(K + hoff, head_bytes);
    const auto rv = make_rsrc(V + hoff, head_bytes);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const uint32_t off = ((uint32_t)(k0w + 32 * kk + c32) * D + 16 * s + 8 * h) * 2u;
        kf[kk][s] = as_bf16x8(buf_load16(rk, off));
        if constexpr (DKP) vf[kk][s] = as_bf16x8(buf_load16(rv, off));
      }
    // K and V resident here: the compiler does not count the copies, so its
    // own waits for K and V must not fall inside the loop (where they would
    // also drain the copies in flight).
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        pin_ready(kf[kk][s]);
        if constexpr (DKP) pin_ready(vf[kk][s]);
      }
  }
  if constexpr (ST > 2) {
    if (1 < nchunks) fetch(1, std::integral_constant<int, 1>{});
  }
  wait_vmem_tiles<C::DMA_PER_TILE, ST - 2>(min(ST - 2, nchunks - 1));
  ring_barrier();
  if constexpr (C::KL) {
    // each wavefront reads (and later overwrites with dK, dV) only its rows
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        kf[kk][s] = frag_rows<D>(ksg, w * C::KW + 32 * kk, 16 * s, c32, h);
        if constexpr (DKP) vf[kk][s] = frag_rows<D>(vsg, w * C::KW + 32 * kk, 16 * s, c32, h);
      }
  }

  // Step t on the chunk at query i0; in is the next chunk's query (SPARSE:
  // it is copied in during this step; -1 when this is the last).
  auto step = [&](int t, int i0, int in, auto S) {
    constexpr int SN = (decltype(S)::value + ST - 1) % ST;  // stage of step t+ST-1
    if constexpr (SPARSE) {
      if (in >= 0) fetch_at(in, std::integral_constant<int, SN>{});
    } else {
      if (t + ST - 1 < nchunks) fetch(t + ST - 1, std::integral_constant<int, SN>{});
    }
    // some query of the chunk sees some key of this wavefront
    const bool active = !CAUSAL || i0 + C::BQ - 1 >= k0w;
    if (active) {
      const bf16_t* Qs = qst(S);
      const bf16_t* Os = ost(S);
      const float* ls = lst(S);
      const float* ds = dst_(S);

      // S = Q K^T and dP - D = dO V^T - D (lane: key; registers: query
      // rows); the dP accumulator starts from the workspace's -D, register
      // 4g + e holding row 8g + 4h + e of the block (16-byte LDS reads).
      f32x16 sacc[QB][KB], pacc[QB][KB];
      f32x16 ndq[DROP ? QB : 1];  // DROP: -D t/256, the dS factor of dropped pairs
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 nd = {};
        if constexpr (DKP) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(ds + qb * 32 + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) nd[4 * g + e] = DROP ? v[e] * dr.keep : v[e];
          }
        }
        if constexpr (DROP) ndq[qb] = nd;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 aq = frag_rows<D>(Qs, qb * 32, 16 * s, c32, h);
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const f32x16 z = {};
            sacc[qb][kk] = mfma32x32x16(aq, kf[kk][s], s == 0 ? z : sacc[qb][kk]);
          }
          if constexpr (DKP) {
            const bf16x8 ao = frag_rows<D>(Os, qb * 32, 16 * s, c32, h);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
              pacc[qb][kk] = mfma32x32x16(ao, vf[kk][s], s == 0 ? nd : pacc[qb][kk]);
          }
        }
      }

      // P = exp2(S c - LSE2), in place; masked entries (causal future, query
      // tail) are zeroed on the blocks that need it only (a real branch).
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // rows 8g + 4h + 0..3 of this 32-row block: one 16-byte LDS read
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(ls + qb * 32 + 8 * g + 4 * h);
#pragma unroll
          for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sacc[qb][kk][4 * g + e] = fast_exp2(fmaf(sacc[qb][kk][4 * g + e], c, -lse4[e]));
        }
      const bool tail = i0 + C::BQ > N;
      if (tail || (CAUSAL && i0 < k0w + C::KW - 1)) {
        keep_branch();
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          // key > query  <=>  kqh > query offset
          const int kqh = k0w + 32 * kk + c32 - i0 - 4 * h;
          if (!tail) {
            // causal diagonal only: one compare per entry
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int qoff = qb * 32 + 8 * (r >> 2) + (r & 3);
                if (qoff < kqh) sacc[qb][kk][r] = 0.f;
              }
          } else {
            const int nq = N - i0 - 4 * h;  // query >= N  <=>  query offset >= nq
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int qoff = qb * 32 + 8 * (r >> 2) + (r & 3);
                if ((CAUSAL && kqh > qoff) || qoff >= nq) sacc[qb][kk][r] = 0.f;
              }
          }
        }
      }
      // dS = P (dP - D); P and dS packed to bf16 as B operands (k-step
      // u = 2*qb + (g>>1) holds registers 8*(g&1) .. of block qb).
      if constexpr (DROP) {
        // pacc becomes dS (up to 256/t): P (dP' - D t/256) for kept pairs,
        // P (-D t/256) for dropped ones; sacc becomes Z P, the weights of dV
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            uint32_t dw[4];
            draws_key_cols(i0 + 32 * qb, k0w + 32 * kk, bh, lane, dr.k0, dr.k1, dw);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const bool k = kept(dw, r, dr.thresh);
              const float pv = sacc[qb][kk][r];
              if constexpr (DKP) pacc[qb][kk][r] = pv * (k ? pacc[qb][kk][r] : ndq[qb][r]);
              sacc[qb][kk][r] = k ? pv : 0.f;
            }
          }
      }
      uint32_t pw[KB][C::PU][4], sw[KB][C::PU][4];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& pr = sacc[qb][kk];
            const int u = 2 * qb + (g >> 1), w0 = 2 * (g & 1);
            if constexpr (DVP) {
              pw[kk][u][w0] = pack_bf16x2(pr[4 * g], pr[4 * g + 1]);
              pw[kk][u][w0 + 1] = pack_bf16x2(pr[4 * g + 2], pr[4 * g + 3]);
            }
            if constexpr (DKP) {
              float dsv[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                dsv[e] = DROP ? pacc[qb][kk][4 * g + e] : pr[4 * g + e] * pacc[qb][kk][4 * g + e];
              sw[kk][u][w0] = pack_bf16x2(dsv[0], dsv[1]);
              sw[kk][u][w0 + 1] = pack_bf16x2(dsv[2], dsv[3]);
            }
          }

      // dV^T += dO^T P,  dK^T += Q^T dS  (lane: key; registers: head dims);
      // each transposed Q / dO fragment feeds the KB key blocks.
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          if constexpr (DVP) {
            const bf16x8 ao = frag_tr<D>(Os, 16 * u, db * 32, lane);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
              dvacc[kk][db] = mfma32x32x16(
                  ao, bf16x8_from(pw[kk][u][0], pw[kk][u][1], pw[kk][u][2], pw[kk][u][3]), dvacc[kk][db]);
          }
          if constexpr (DKP) {
            const bf16x8 aq = frag_tr<D>(Qs, 16 * u, db * 32, lane);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
              dkacc[kk][db] = mfma32x32x16(
                  aq, bf16x8_from(sw[kk][u][0], sw[kk][u][1], sw[kk][u][2], sw[kk][u][3]), dkacc[kk][db]);
          }
        }
      }
    }
    // step t+1 must be resident; later steps may still be in flight
    if (SPARSE ? in >= 0 : t + 1 < nchunks) {
      wait_vmem_tiles<C::DMA_PER_TILE, ST - 2>(SPARSE ? 0 : min(ST - 2, nchunks - t - 2));
      ring_barrier();
    }
  };
  if constexpr (SPARSE) {
    int i0 = ifirst, in = i0 >= 0 ? walk.next(i0) : -1;
    for (int t = 0; i0 >= 0; t += 2) {
      step(t, i0, in, std::integral_constant<int, 0>{});
      if (in < 0) break;
      i0 = in;
      in = walk.next(i0);
      step(t + 1, i0, in, std::integral_constant<int, 1>{});
      i0 = in;
      in = i0 >= 0 ? walk.next(i0) : -1;
    }
  } else {
    for (int t0 = 0; t0 < nchunks; t0 += ST) {
      step(t0, qstart + t0 * C::BQ, -1, std::integral_constant<int, 0>{});
      if (t0 + 1 < nchunks) step(t0 + 1, qstart + (t0 + 1) * C::BQ, -1, std::integral_constant<int, 1>{});
      if constexpr (ST > 2) {
        if (t0 + 2 < nchunks) step(t0 + 2, qstart + (t0 + 2) * C::BQ, -1, std::integral_constant<int, 2>{});
      }
    }
  }

  if constexpr (DROP && DVP) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dvacc[kk][db][r] *= dr.scale;
  }
  if constexpr (SPARSE) {
    if (slotw >= 0) {
      // segment of a split tile column: its shares of dK and dV (float32)
      const size_t prow = ((size_t)(slotw >> 1) * BH + bh) * C::BK;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int key = k0w + 32 * kk + c32;
        if (key < N) {
          float* Pk = sp.part_dk + (prow + (key - k0)) * D;
          float* Pv = sp.part_dv + (prow + (key - k0)) * D;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = db * 32 + 8 * g + 4 * h;
              if constexpr (DKP)
                *reinterpret_cast<float4*>(Pk + col) =
                    make_float4(dkacc[kk][db][4 * g] * scale, dkacc[kk][db][4 * g + 1] * scale,
                                dkacc[kk][db][4 * g + 2] * scale, dkacc[kk][db][4 * g + 3] * scale);
              if constexpr (DVP)
                *reinterpret_cast<float4*>(Pv + col) =
                    make_float4(dvacc[kk][db][4 * g], dvacc[kk][db][4 * g + 1],
                                dvacc[kk][db][4 * g + 2], dvacc[kk][db][4 * g + 3]);
            }
        }
      }
      return;
    }
  }
  if constexpr (C::KL) {
    // fragments (dims db*32 + 8g + 4h + 0..3 of this lane's key rows) into
    // this wavefront's rows of the staging tiles, then out as whole rows:
    // 8 lanes per row, each store instruction writes 8 complete rows
    constexpr int CPR = D / 8;
    static_assert(PARTS == 3, "LDS-staged K/V: both gradients in one launch");
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(ksg + tile_off<D>(w * C::KW + 32 * kk + c32, db * 32 + 8 * g + 4 * h)) =
              make_uint2(pack_bf16x2(dkacc[kk][db][4 * g] * scale, dkacc[kk][db][4 * g + 1] * scale),
                         pack_bf16x2(dkacc[kk][db][4 * g + 2] * scale, dkacc[kk][db][4 * g + 3] * scale));
#pragma unroll
    for (int i = 0; i < C::KW * CPR / kWave; ++i) {
      const int chunk = i * kWave + lane;
      const int r = chunk / CPR, cc = chunk % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(ksg + tile_off<D>(w * C::KW + r, cc * 8));
      if (k0w + r < N) *reinterpret_cast<uint4*>(dK + hoff + (size_t)(k0w + r) * D + cc * 8) = v;
    }
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(vsg + tile_off<D>(w * C::KW + 32 * kk + c32, db * 32 + 8 * g + 4 * h)) =
              make_uint2(pack_bf16x2(dvacc[kk][db][4 * g], dvacc[kk][db][4 * g + 1]),
                         pack_bf16x2(dvacc[kk][db][4 * g + 2], dvacc[kk][db][4 * g + 3]));
#pragma unroll
    for (int i = 0; i < C::KW * CPR / kWave; ++i) {
      const int chunk = i * kWave + lane;
      const int r = chunk / CPR, cc = chunk % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(vsg + tile_off<D>(w * C::KW + r, cc * 8));
      if (k0w + r < N) *reinterpret_cast<uint4*>(dV + hoff + (size_t)(k0w + r) * D + cc * 8) = v;
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int key = k0w + 32 * kk + c32;
      if (key < N) {
        bf16_t* dKr = dK + hoff + (size_t)key * D;
        bf16_t* dVr = dV + hoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 vk, vv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              vk[e] = to_bf16(dkacc[kk][db][4 * g + e] * scale);
              vv[e] = to_bf16(dvacc[kk][db][4 * g + e]);
            }
            const int col = db * 32 + 8 * g + 4 * h;
            if constexpr (DKP) *reinterpret_cast<bf16x4*>(dKr + col) = vk;
            if constexpr (DVP) *reinterpret_cast<bf16x4*>(dVr + col) = vv;
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ.  Per wavefront: RB blocks of 32 query rows (Q and dO fragments in
// VGPRs, LSE and D per lane; D is formed here and stored for the dK/dV
// kernel, beside LSE*log2(e)).  Per step: a block of BC keys of K and V, copied HBM -> LDS by
// direct buffer->LDS loads into an ST-stage ring (one LDS variable per
// stage, so reads of the current block never wait for the copies in
// flight): K and V read by rows for S^T = K Q^T and dP^T = V dO^T, K
// through the transpose unit for dQ^T += K^T dS^T.  Each fragment read
// from LDS feeds the RB row blocks.
template <int D, int NW, int RB, int BC, int ST>
struct DqCfg {
  static constexpr int NT = NW * kWave;
  static constexpr int RW = 32 * RB;          // query rows per wavefront
  static constexpr int BR = NW * RW;          // query rows per workgroup
  static constexpr int TILE = BC * D;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KB = BC / 32;
  static constexpr int PU = BC / 16;
  static constexpr int DMA_PER_TILE = TILE / 8 / NT;
  // Q and dO blocks staged through LDS (coalesced copies in, dQ out through
  // the Q rows) when both fit in 32 KB; otherwise their fragments load
  // straight from HBM
  static constexpr bool QL = 2 * BR * D * 2 <= 32768;
  static_assert(ST >= 2 && ST <= 3, "two or three K/V stages");
};

// SPARSE: block-sparse attention; the loop visits only the K/V blocks of
// the 128 x 128 tiles set in row qb of the tile mask (the query block is one
// tile row: BR = 128); with none, dQ is 0.
//
// DROP: dropout on the weights, the draws regenerated as in the forward.
// dS = P (Z dP' 256/t - D) with dP' = dO V^T and Z the keep mask, computed
// as (256/t) P (Z ? dP' - D t/256 : -D t/256); the factor 256/t is part of
// `scale` (the host passes scale * 256/t).
template <int D, int NW, int RB, int BC, int ST, int OCC, bool CAUSAL, bool SPARSE = false,
          bool DROP = false>
__global__ __launch_bounds__(NW * 64, OCC)
void bwd_dq_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                        const bf16_t* __restrict__ V, const bf16_t* __restrict__ O,
                        const bf16_t* __restrict__ dO, const float* __restrict__ LSE,
                        float* __restrict__ Dws, float* __restrict__ Lws, bf16_t* __restrict__ dQ,
                        int BH, int N, int nqb, int G, float c, float scale, SparseArgs sp = {},
                        DropArgs dr = {}) {
  using C = DqCfg<D, NW, RB, BC, ST>;
  static_assert(!(SPARSE && DROP), "one variant at a time");
  static_assert(!SPARSE || (ST == 2 && C::BR == 128), "sparse walk: two stages, 128-row query blocks");
  __shared__ __attribute__((aligned(16))) bf16_t k0s[C::TILE], v0s[C::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t k1s[C::TILE], v1s[C::TILE];
  __shared__ __attribute__((aligned(16))) bf16_t k2s[ST > 2 ? C::TILE : 8], v2s[ST > 2 ? C::TILE : 8];
  __shared__ __attribute__((aligned(16))) bf16_t qsg[C::QL ? C::BR * D : 8], osg[C::QL ? C::BR * D : 8];
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
  int bh, rank;
  grouped_order(xcd_remap(blockIdx.x, BH * nqb), nqb, BH, G, bh, rank);
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
  const int q0w = q0 + w * C::RW;  // row block rb of this lane: query q0w + 32 rb + c32

  f32x16 dqacc[RB][C::DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqacc[rb][db][r] = 0.f;

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  // keys visited: dense from 0, or the blocks of the set tiles
  BlockWalk<BC, SPARSE> walk{kend,
                             list_cnt >= 0 ? (const_int_ptr)sp.lists + list_off
                                           : (const_int_ptr)(sp.mask + (size_t)qb * sp.nb),
                             1, CAUSAL ? qb : sp.nb - 1, list_cnt};
  const int jfirst = SPARSE ? walk.first(0) : 0;

  auto fetch_at = [&](int j0, auto S) {
    dma_tile<D, BC, C::NT>(rk, j0, kst(S), tid);
    dma_tile<D, BC, C::NT>(rv, j0, vst(S), tid);
  };
  auto fetch = [&](int t, auto S) { fetch_at(t * BC, S); };
  // The first K/V copies go out before Q, dO and O are read, so that the
  // latencies overlap.
  if (jfirst >= 0) fetch_at(jfirst, std::integral_constant<int, 0>{});
  if constexpr (C::QL) {
    // Q and dO blocks copied row-major (coalesced) into LDS, rows past N as 0
    dma_tile<D, C::BR, C::NT>(make_copy_rsrc(Q + hoff, head_bytes), q0, qsg, tid);
    dma_tile<D, C::BR, C::NT>(make_copy_rsrc(dO + hoff, head_bytes), q0, osg, tid);
  }
  if constexpr (ST > 2) {
    if (1 < ntiles) fetch(1, std::integral_constant<int, 1>{});
  }

  // Q and dO fragments (B operands, lane = query row: half h holds head dims
  // 16s + 8h .. +7), LSE in log2 units, and D_i = sum_k dO_ik O_ik formed
  // here from the matching O fragment (read once, straight from HBM) and
  // stored for the dK/dV kernel.
  bf16x8 qf[RB][C::KSTEPS], of[RB][C::KSTEPS], ov[RB][C::KSTEPS];
  float lse2[RB], dd[RB];
  {
    const auto rq = make_rsrc(Q + hoff, head_bytes);
    const auto ro = make_rsrc(dO + hoff, head_bytes);
    const auto rO = make_rsrc(O + hoff, head_bytes);
    const auto rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int query = q0w + 32 * rb + c32;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const uint32_t off = ((uint32_t)query * D + 16 * s + 8 * h) * 2u;
        if constexpr (!C::QL) {
          qf[rb][s] = as_bf16x8(buf_load16(rq, off));
          of[rb][s] = as_bf16x8(buf_load16(ro, off));
        }
        ov[rb][s] = as_bf16x8(buf_load16(rO, off));
      }
      lse2[rb] = buf_load_f32(rl, (uint32_t)query * 4u) * kLog2e;
    }
  }
  wait_vmem_tiles<2 * C::DMA_PER_TILE, ST - 2>(min(ST - 2, ntiles - 1));
  ring_barrier();
  if constexpr (C::QL) {
    // each wavefront reads (and later overwrites with dQ) only its own rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        qf[rb][s] = frag_rows<D>(qsg, w * C::RW + 32 * rb, 16 * s, c32, h);
        of[rb][s] = frag_rows<D>(osg, w * C::RW + 32 * rb, 16 * s, c32, h);
      }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int query = q0w + 32 * rb + c32;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)of[rb][s][e], (float)ov[rb][s][e], part);
    dd[rb] = sum_halves(part);
    // (of a split tile row, the first segment stores the row vectors)
    if (h == 0 && query < N && (slotw < 0 || (slotw & 1))) {
      Dws[(size_t)bh * N + query] = -dd[rb];
      Lws[(size_t)bh * N + query] = lse2[rb];
    }
  }
  // Q and dO resident here: the compiler does not count the copies, so its
  // own waits for them must not fall inside the loop (where they would also
  // drain the copies in flight).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      pin_ready(qf[rb][s]);
      pin_ready(of[rb][s]);
    }

  // Step t on the block at key j0; jn is the next block's key (SPARSE: it
  // is copied in during this step; -1 when this is the last).
  auto step = [&](int t, int j0, int jn, auto S) {
    constexpr int SN = (decltype(S)::value + ST - 1) % ST;  // stage of step t+ST-1
    if constexpr (SPARSE) {
      if (jn >= 0) fetch_at(jn, std::integral_constant<int, SN>{});
    } else {
      if (t + ST - 1 < ntiles) fetch(t + ST - 1, std::integral_constant<int, SN>{});
    }
    const bool active = !CAUSAL || j0 <= q0w + C::RW - 1;
    if (active) {
      const bf16_t* Ks = kst(S);
      const bf16_t* Vs = vst(S);

      // S^T = K Q^T, dP^T = V dO^T (lane: query; registers: keys).
      f32x16 sacc[RB][C::KB], pacc[RB][C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 ak = frag_rows<D>(Ks, kb * 32, 16 * s, c32, h);
          const bf16x8 av = frag_rows<D>(Vs, kb * 32, 16 * s, c32, h);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if (s == 0) {
              const f32x16 z = {};
              sacc[rb][kb] = mfma32x32x16(ak, qf[rb][s], z);
              pacc[rb][kb] = mfma32x32x16(av, of[rb][s], z);
            } else {
              sacc[rb][kb] = mfma32x32x16(ak, qf[rb][s], sacc[rb][kb]);
              pacc[rb][kb] = mfma32x32x16(av, of[rb][s], pacc[rb][kb]);
            }
          }
        }
      }

      // P^T = exp2(S^T c - LSE2), in place; masked entries (causal future,
      // key tail) are zeroed on the blocks that need it only (a real branch).
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[rb][kb][r] = fast_exp2(fmaf(sacc[rb][kb][r], c, -lse2[rb]));
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
              if (koff > lim) sacc[rb][kb][r] = 0.f;
            }
        }
      }
      if constexpr (DROP) {
        // dropped pairs: dP' -> 0, and D scaled by t/256 (see above)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            uint32_t dw[4];
            draws_query_cols(q0w + 32 * rb, j0 + 32 * kb, bh, lane, dr.k0, dr.k1, dw);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!kept(dw, r, dr.thresh)) pacc[rb][kb][r] = 0.f;
          }
      }
      // dS^T = P^T (dP^T - D), packed to bf16: register r of block kb is
      // k-step 2*kb + (r>>3), element r & 7; then dQ^T += K^T dS^T (lane:
      // query; registers: head dims), each K^T fragment feeding RB blocks.
#pragma unroll
      for (int u = 0; u < C::PU; ++u) {
        bf16x8 sf[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          uint32_t sw[4];
          const int kb = u >> 1, r0 = 8 * (u & 1);
          const float dsub = DROP ? dd[rb] * dr.keep : dd[rb];
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            sw[e >> 1] = pack_bf16x2(sacc[rb][kb][r0 + e] * (pacc[rb][kb][r0 + e] - dsub),
                                     sacc[rb][kb][r0 + e + 1] * (pacc[rb][kb][r0 + e + 1] - dsub));
          sf[rb] = bf16x8_from(sw[0], sw[1], sw[2], sw[3]);
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 a = frag_tr<D>(Ks, 16 * u, db * 32, lane);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) dqacc[rb][db] = mfma32x32x16(a, sf[rb], dqacc[rb][db]);
        }
      }
    }
    // step t+1 must be resident; later steps may still be in flight
    if (SPARSE ? jn >= 0 : t + 1 < ntiles) {
      wait_vmem_tiles<2 * C::DMA_PER_TILE, ST - 2>(SPARSE ? 0 : min(ST - 2, ntiles - t - 2));
      ring_barrier();
    }
  };
  if constexpr (SPARSE) {
    int j0 = jfirst, jn = j0 >= 0 ? walk.next(j0) : -1;
    for (int t = 0; j0 >= 0; t += 2) {
      step(t, j0, jn, std::integral_constant<int, 0>{});
      if (jn < 0) break;
      j0 = jn;
      jn = walk.next(j0);
      step(t + 1, j0, jn, std::integral_constant<int, 1>{});
      j0 = jn;
      jn = j0 >= 0 ? walk.next(j0) : -1;
    }
  } else {
    for (int t0 = 0; t0 < ntiles; t0 += ST) {
      step(t0, t0 * BC, -1, std::integral_constant<int, 0>{});
      if (t0 + 1 < ntiles) step(t0 + 1, (t0 + 1) * BC, -1, std::integral_constant<int, 1>{});
      if constexpr (ST > 2) {
        if (t0 + 2 < ntiles) step(t0 + 2, (t0 + 2) * BC, -1, std::integral_constant<int, 2>{});
      }
    }
  }

  if constexpr (SPARSE) {
    if (slotw >= 0) {
      // segment of a split tile row: its share of dQ (float32) for the sum
      const size_t prow = ((size_t)(slotw >> 1) * BH + bh) * C::BR;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int query = q0w + 32 * rb + c32;
        if (query < N) {
          float* Pr = sp.part_dq + (prow + (query - q0)) * D;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
              *reinterpret_cast<float4*>(Pr + db * 32 + 8 * g + 4 * h) =
                  make_float4(dqacc[rb][db][4 * g] * scale, dqacc[rb][db][4 * g + 1] * scale,
                              dqacc[rb][db][4 * g + 2] * scale, dqacc[rb][db][4 * g + 3] * scale);
        }
      }
      return;
    }
  }

  if constexpr (C::QL) {
    // fragments (dims db*32 + 8g + 4h + 0..3 of this lane's row) into this
    // wavefront's rows of the Q staging tile, then out as whole rows: 8 lanes
    // per row, each store instruction writes 8 complete rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(qsg + tile_off<D>(w * C::RW + 32 * rb + c32, db * 32 + 8 * g + 4 * h)) =
              make_uint2(pack_bf16x2(dqacc[rb][db][4 * g] * scale, dqacc[rb][db][4 * g + 1] * scale),
                         pack_bf16x2(dqacc[rb][db][4 * g + 2] * scale, dqacc[rb][db][4 * g + 3] * scale));
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < C::RW * CPR / kWave; ++i) {
      const int chunk = i * kWave + lane;
      const int r = chunk / CPR, cc = chunk % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(qsg + tile_off<D>(w * C::RW + r, cc * 8));
      if (q0w + r < N) *reinterpret_cast<uint4*>(dQ + hoff + (size_t)(q0w + r) * D + cc * 8) = v;
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int query = q0w + 32 * rb + c32;
      if (query < N) {
        bf16_t* dQr = dQ + hoff + (size_t)query * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_bf16(dqacc[rb][db][4 * g + e] * scale);
            *reinterpret_cast<bf16x4*>(dQr + db * 32 + 8 * g + 4 * h) = v;
          }
      }
    }
  }
}

// Head dims whose dK and dV are accumulated by two launches (dV, then dK).
#ifndef FA_DKDV_SPLIT_D256
#define FA_DKDV_SPLIT_D256 true
#endif
template <int D>
constexpr bool kDkdvSplit = D == 256 ? FA_DKDV_SPLIT_D256 : false;

template <int D, int NWK, int KBK, int QB, int STK, int OCCK, int NWQ, int RBQ, int BC, int STQ,
          int OCCQ, bool CAUSAL, bool SPARSE, bool DROP = false>
hipError_t run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV, float* ws, const Problem& p,
                   unsigned stages, SparseArgs sp, hipStream_t stream, DropArgs dr = {}) {
  const int BH = p.B * p.H;
  const long long rows = (long long)BH * p.N;
  const float c = p.scale * kLog2e;
  const float gscale = DROP ? p.scale * dr.scale : p.scale;  // of dQ and dK
  float* Dws = ws;         // -D, one float per row
  float* Lws = ws + ws_lse_offset(rows);  // LSE * log2(e), one float per row
  if (stages & kStagePre) {
    constexpr int RPB = 256 / (D / 8);
    const long long grid = (rows + RPB - 1) / RPB;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)O, (const bf16_t*)dO, LSE, Dws, Lws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDq) {
    using C = DqCfg<D, NWQ, RBQ, BC, STQ>;
    // workgroups per head: query blocks, or the balanced schedule's row items
    const int nqb = SPARSE && sp.rows != nullptr ? sp.n_rows : (p.N + C::BR - 1) / C::BR;
    const long long grid = (long long)BH * nqb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int G = head_group(OCCQ * 4 / NWQ, nqb);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, NWQ, RBQ, BC, STQ, OCCQ, CAUSAL, SPARSE, DROP>),
                       dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q, (const bf16_t*)K,
                       (const bf16_t*)V, (const bf16_t*)O, (const bf16_t*)dO, LSE, Dws, Lws,
                       (bf16_t*)dQ, BH, p.N, nqb, G, c, gscale, sp, dr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDkDv) {
    using C = DkdvCfg<D, NWK, KBK, QB, STK>;
    // workgroups per head: key blocks, or the balanced schedule's column items
    const int nkb = SPARSE && sp.cols != nullptr ? sp.n_cols : (p.N + C::BK - 1) / C::BK;
    const long long grid = (long long)BH * nkb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int G = head_group(OCCK * 4 / NWK, nkb);
    auto launch = [&](auto parts) {
      hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, NWK, KBK, QB, STK, OCCK, CAUSAL, SPARSE, DROP,
                                               decltype(parts)::value>),
                         dim3((unsigned)grid), dim3(C::NT), 0, stream, (const bf16_t*)Q,
                         (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, (const float*)Lws,
                         (const float*)Dws, (bf16_t*)dK, (bf16_t*)dV, BH, p.N, nkb, G, c, gscale,
                         sp, dr);
      return hipGetLastError();
    };
    if constexpr (kDkdvSplit<D>) {
      hipError_t e = launch(std::integral_constant<int, 1>{});  // dV
      if (e != hipSuccess) return e;
      e = launch(std::integral_constant<int, 2>{});             // dK
      if (e != hipSuccess) return e;
    } else {
      hipError_t e = launch(std::integral_constant<int, 3>{});
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Launch configurations per head dim: dK/dV (wavefronts per workgroup,
// 32-key blocks per wavefront, 32-row query blocks per chunk, Q/dO stages,
// minimum wavefronts per SIMD), then dQ (wavefronts per workgroup, 32-row
// query blocks per wavefront, keys per K/V block, K/V stages, minimum
// wavefronts per SIMD).
#ifndef FA_BWD_CFG_D64
#define FA_BWD_CFG_D64 4, 1, 1, 2, 2, 4, 1, 32, 2, 3
#endif
#ifndef FA_BWD_CFG_D128
#define FA_BWD_CFG_D128 4, 1, 1, 2, 1, 4, 1, 32, 2, 2
#endif
#ifndef FA_BWD_CFG_D256
#define FA_BWD_CFG_D256 4, 1, 1, 2, 1, 4, 1, 32, 2, 1
#endif

// All variants (dropout, block-sparse, plain) for one value of the causal
// flag.
template <int D, int NWK, int KBK, int QB, int STK, int OCCK, int NWQ, int RBQ, int BC, int STQ,
          int OCCQ, bool CAUSAL>
hipError_t run_bwd_cz(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, float* ws, const Problem& p,
                      unsigned stages, SparseArgs sp, hipStream_t stream, const DropArgs* dr) {
  if (dr != nullptr) {
    if (sp.on()) return hipErrorNotSupported;
    return run_bwd<D, NWK, KBK, QB, STK, OCCK, NWQ, RBQ, BC, STQ, OCCQ, CAUSAL, false, true>(
        Q, K, V, O, dO, LSE, dQ, dK, dV, ws, p, stages, sp, stream, *dr);
  }
  if (sp.on()) {
    // the sparse walk takes 128-key and 128-row blocks in two stages
    if constexpr (NWK * KBK * 32 == 128 && STK == 2 && NWQ * RBQ * 32 == 128 && STQ == 2)
      return run_bwd<D, NWK, KBK, QB, STK, OCCK, NWQ, RBQ, BC, STQ, OCCQ, CAUSAL, true>(
          Q, K, V, O, dO, LSE, dQ, dK, dV, ws, p, stages, sp, stream);
    else
      return hipErrorNotSupported;
  }
  return run_bwd<D, NWK, KBK, QB, STK, OCCK, NWQ, RBQ, BC, STQ, OCCQ, CAUSAL, false>(
      Q, K, V, O, dO, LSE, dQ, dK, dV, ws, p, stages, sp, stream);
}

template <int D, int NWK, int KBK, int QB, int STK, int OCCK, int NWQ, int RBQ, int BC, int STQ,
          int OCCQ>
hipError_t run_bwd_c(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, float* ws, const Problem& p,
                     unsigned stages, SparseArgs sp, hipStream_t stream, const DropArgs* dr) {
  return p.causal
             ? run_bwd_cz<D, NWK, KBK, QB, STK, OCCK, NWQ, RBQ, BC, STQ, OCCQ, true>(
                   Q, K, V, O, dO, LSE, dQ, dK, dV, ws, p, stages, sp, stream, dr)
             : run_bwd_cz<D, NWK, KBK, QB, STK, OCCK, NWQ, RBQ, BC, STQ, OCCQ, false>(
                   Q, K, V, O, dO, LSE, dQ, dK, dV, ws, p, stages, sp, stream, dr);
}

}  // namespace

#if !defined(FA_D256_UNIT) && !defined(FA_D128NC_UNIT)
hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                float* Dws, const Problem& p, unsigned stages,
                                hipStream_t stream, SparseArgs sp, const DropArgs* dr) {
  switch (p.d) {
    case 64:
      return run_bwd_c<64, FA_BWD_CFG_D64>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, sp, stream, dr);
    case 128:
      if (!p.causal)
        return launch_backward_bf16_d128nc(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream, sp, dr);
      return run_bwd_c<128, FA_BWD_CFG_D128>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, sp, stream, dr);
    case 256:
      return launch_backward_bf16_d256(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream, sp, dr);
    default:
      return hipErrorInvalidValue;
  }
}
#elif defined(FA_D128NC_UNIT)
// Head dim 128 without the causal mask (this source compiled a second time
// as fa_bwd_d128nc.hip)
hipError_t launch_backward_bf16_d128nc(const void* Q, const void* K, const void* V, const void* O,
                                       const void* dO, const float* LSE, void* dQ, void* dK,
                                       void* dV, float* Dws, const Problem& p, unsigned stages,
                                       hipStream_t stream, SparseArgs sp, const DropArgs* dr) {
  if (p.causal) return hipErrorInvalidValue;
  return run_bwd_cz<128, FA_BWD_CFG_D128, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, sp,
                                                 stream, dr);
}
#else
// Head dim 256 (this source compiled a second time as fa_bwd_d256.hip)
hipError_t launch_backward_bf16_d256(const void* Q, const void* K, const void* V, const void* O,
                                     const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                     float* Dws, const Problem& p, unsigned stages,
                                     hipStream_t stream, SparseArgs sp, const DropArgs* dr) {
  return run_bwd_c<256, FA_BWD_CFG_D256>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, sp, stream, dr);
}
#endif

}  // namespace fa
