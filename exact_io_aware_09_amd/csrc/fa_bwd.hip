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
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik  (fp32), one row per D/8 lanes (16-byte loads).
template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_bf16_kernel(const bf16_t* __restrict__ O, const bf16_t* __restrict__ dO,
                         float* __restrict__ Dws, long long rows) {
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
  if (row < rows && part == 0) Dws[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV.  Per wavefront: 32 keys whose K and V fragments stay in VGPRs.  Per
// iteration: a chunk of BQ = 32*QB query rows of Q and dO staged in LDS
// (swizzled, double-buffered), plus that chunk's LSE*log2(e) and D.  Q and
// dO are read by rows for S = Q K^T and dP = dO V^T, and through the LDS
// transpose unit for dK^T += Q^T dS and dV^T += dO^T P.
template <int D, int NW, int QB>
struct DkdvCfg {
  static constexpr int NT = NW * kWave;
  static constexpr int BK = NW * 32;          // keys per workgroup
  static constexpr int BQ = 32 * QB;          // query rows per chunk
  static constexpr int TILE = BQ * D;
  // one buffer: Q tile, dO tile, then LSE*log2e and D (2*BQ floats)
  static constexpr int BUF_ELEMS = 2 * TILE + 4 * BQ;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BQ * CPR / NT;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int PU = BQ / 16;
  static_assert(BQ * CPR % NT == 0, "chunk must split evenly over threads");
  static_assert(BQ <= NT, "one thread per query row loads LSE and D");
};

template <int D, int NW, int QB, int OCC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, OCC)
void bwd_dkdv_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                          const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dws,
                          bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int BH, int N,
                          int nkb, int G, float c, float scale) {
  using C = DkdvCfg<D, NW, QB>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  int bh, kb;  // causal: low key blocks see the most queries, run them first
  grouped_order(xcd_remap(blockIdx.x, BH * nkb), nkb, BH, G, bh, kb);
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + hoff, head_bytes);
  const auto ro = make_rsrc(dO + hoff, head_bytes);
  const auto rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  const auto rd = make_rsrc(Dws + (size_t)bh * N, (uint32_t)N * 4u);

  const int k0 = kb * C::BK;
  const int k0w = k0 + w * 32;
  const int key = k0w + c32;  // this lane's key row (MFMA column)

  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (lane = key).
  bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
  {
    const auto rk = make_rsrc(K + hoff, head_bytes);
    const auto rv = make_rsrc(V + hoff, head_bytes);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      const uint32_t off = ((uint32_t)key * D + 16 * s + 8 * h) * 2u;
      kf[s] = as_bf16x8(buf_load16(rk, off));
      vf[s] = as_bf16x8(buf_load16(rv, off));
    }
  }

  f32x16 dkacc[C::DB], dvacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[db][r] = 0.f;
      dvacc[db][r] = 0.f;
    }

  const int qstart = CAUSAL ? (k0 / C::BQ) * C::BQ : 0;
  const int nchunks = (N - qstart + C::BQ - 1) / C::BQ;

  uint4 qreg[C::CPT], oreg[C::CPT];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int t) {
    const int i0 = qstart + t * C::BQ;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const uint32_t off = ((uint32_t)(i0 + chunk / C::CPR) * D + (chunk % C::CPR) * 8) * 2u;
      qreg[i] = buf_load16(rq, off);
      oreg[i] = buf_load16(ro, off);
    }
    if (tid < C::BQ) {
      lreg = buf_load_f32(rl, (uint32_t)(i0 + tid) * 4u) * kLog2e;
      dreg = buf_load_f32(rd, (uint32_t)(i0 + tid) * 4u);
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* Qs = lds + buf * C::BUF_ELEMS;
    bf16_t* Os = Qs + C::TILE;
    float* fl = reinterpret_cast<float*>(Qs + 2 * C::TILE);
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int off = tile_off<D>(chunk / C::CPR, (chunk % C::CPR) * 8);
      *reinterpret_cast<uint4*>(Qs + off) = qreg[i];
      *reinterpret_cast<uint4*>(Os + off) = oreg[i];
    }
    if (tid < C::BQ) {
      fl[tid] = lreg;
      fl[C::BQ + tid] = dreg;
    }
  };

  gload(0);
  lstore(0);
  wait_vmem_all();
  __syncthreads();

  for (int t = 0; t < nchunks; ++t) {
    const int buf = t & 1;
    if (t + 1 < nchunks) gload(t + 1);
    const int i0 = qstart + t * C::BQ;
    // some query of the chunk sees some key of this wavefront
    const bool active = !CAUSAL || i0 + C::BQ - 1 >= k0w;
    if (active) {
      const bf16_t* Qs = lds + buf * C::BUF_ELEMS;
      const bf16_t* Os = Qs + C::TILE;
      const float* fl = reinterpret_cast<const float*>(Qs + 2 * C::TILE);

      // S = Q K^T and dP = dO V^T (lane: key; registers: query rows).
      f32x16 sacc[QB], pacc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 aq = frag_rows<D>(Qs, qb * 32, 16 * s, c32, h);
          const bf16x8 ao = frag_rows<D>(Os, qb * 32, 16 * s, c32, h);
          if (s == 0) {
            const f32x16 z = {};
            sacc[qb] = mfma32x32x16(aq, kf[s], z);
            pacc[qb] = mfma32x32x16(ao, vf[s], z);
          } else {
            sacc[qb] = mfma32x32x16(aq, kf[s], sacc[qb]);
            pacc[qb] = mfma32x32x16(ao, vf[s], pacc[qb]);
          }
        }
      }

      // P = exp2(S c - LSE2); masked entries (causal future, query tail) are
      // zeroed on the blocks that need it only (a real branch).
      float pv[QB][16];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // rows 8g + 4h + 0..3 of this 32-row block: one 16-byte LDS read
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(fl + qb * 32 + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[qb][4 * g + e] = fast_exp2(fmaf(sacc[qb][4 * g + e], c, -lse4[e]));
        }
      const bool need_mask = (i0 + C::BQ > N) || (CAUSAL && i0 < k0w + 31);
      if (need_mask) {
        keep_branch();
        const int kqh = key - i0 - 4 * h;  // key > query  <=>  kqh > query offset
        const int nq = N - i0 - 4 * h;     // query >= N  <=>  query offset >= nq
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qoff = qb * 32 + 8 * (r >> 2) + (r & 3);
            if ((CAUSAL && kqh > qoff) || qoff >= nq) pv[qb][r] = 0.f;
          }
      }
      // dS = P (dP - D); P and dS packed to bf16 as B operands (k-step
      // u = 2*qb + (g>>1) holds registers 8*(g&1) .. of block qb).
      uint32_t pw[C::PU][4], sw[C::PU][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 dd4 = *reinterpret_cast<const f32x4*>(fl + C::BQ + qb * 32 + 8 * g + 4 * h);
          float ds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[e] = pv[qb][4 * g + e] * (pacc[qb][4 * g + e] - dd4[e]);
          const int u = 2 * qb + (g >> 1), w0 = 2 * (g & 1);
          pw[u][w0] = pack_bf16x2(pv[qb][4 * g], pv[qb][4 * g + 1]);
          pw[u][w0 + 1] = pack_bf16x2(pv[qb][4 * g + 2], pv[qb][4 * g + 3]);
          sw[u][w0] = pack_bf16x2(ds[0], ds[1]);
          sw[u][w0 + 1] = pack_bf16x2(ds[2], ds[3]);
        }

      // dV^T += dO^T P,  dK^T += Q^T dS  (lane: key; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const bf16x8 ao = frag_tr<D>(Os, 16 * u, db * 32, lane);
          const bf16x8 aq = frag_tr<D>(Qs, 16 * u, db * 32, lane);
          dvacc[db] = mfma32x32x16(ao, bf16x8_from(pw[u][0], pw[u][1], pw[u][2], pw[u][3]), dvacc[db]);
          dkacc[db] = mfma32x32x16(aq, bf16x8_from(sw[u][0], sw[u][1], sw[u][2], sw[u][3]), dkacc[db]);
        }
      }
    }
    if (t + 1 < nchunks) lstore(buf ^ 1);
    __syncthreads();
  }

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
          vk[e] = to_bf16(dkacc[db][4 * g + e] * scale);
          vv[e] = to_bf16(dvacc[db][4 * g + e]);
        }
        const int col = db * 32 + 8 * g + 4 * h;
        *reinterpret_cast<bf16x4*>(dKr + col) = vk;
        *reinterpret_cast<bf16x4*>(dVr + col) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ.  Per wavefront: 32 query rows (Q and dO fragments in VGPRs, LSE and D
// per lane; D is formed here and stored for the dK/dV kernel).  Per iteration: a block of BC keys of K and V in LDS (swizzled,
// double-buffered): K and V read by rows for S^T = K Q^T and dP^T = V dO^T,
// K through the transpose unit for dQ^T += K^T dS^T.
template <int D, int NW, int BC>
struct DqCfg {
  static constexpr int NT = NW * kWave;
  static constexpr int BR = NW * 32;
  static constexpr int TILE = BC * D;
  static constexpr int BUF_ELEMS = 2 * TILE;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BC * CPR / NT;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KB = BC / 32;
  static constexpr int PU = BC / 16;
  static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
};

template <int D, int NW, int BC, int OCC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, OCC)
void bwd_dq_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                        const bf16_t* __restrict__ V, const bf16_t* __restrict__ O,
                        const bf16_t* __restrict__ dO, const float* __restrict__ LSE,
                        float* __restrict__ Dws, bf16_t* __restrict__ dQ, int BH, int N, int nqb,
                        int G, float c, float scale) {
  using C = DqCfg<D, NW, BC>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  int bh, rank;
  grouped_order(xcd_remap(blockIdx.x, BH * nqb), nqb, BH, G, bh, rank);
  const int qb = CAUSAL ? (nqb - 1 - rank) : rank;  // longest causal blocks first
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rk = make_rsrc(K + hoff, head_bytes);
  const auto rv = make_rsrc(V + hoff, head_bytes);

  const int q0 = qb * C::BR;
  const int q0w = q0 + w * 32;
  const int query = q0w + c32;

  // Q and dO fragments (B operands, lane = query row: half h holds head dims
  // 16s + 8h .. +7), LSE in log2 units, and D_i = sum_k dO_ik O_ik formed
  // here from the matching O fragment and stored for the dK/dV kernel.
  bf16x8 qf[C::KSTEPS], of[C::KSTEPS];
  float lse2, dd;
  {
    const auto rq = make_rsrc(Q + hoff, head_bytes);
    const auto ro = make_rsrc(dO + hoff, head_bytes);
    const auto rO = make_rsrc(O + hoff, head_bytes);
    bf16x8 ov[C::KSTEPS];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      const uint32_t off = ((uint32_t)query * D + 16 * s + 8 * h) * 2u;
      qf[s] = as_bf16x8(buf_load16(rq, off));
      of[s] = as_bf16x8(buf_load16(ro, off));
      ov[s] = as_bf16x8(buf_load16(rO, off));
    }
    const auto rl = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
    lse2 = buf_load_f32(rl, (uint32_t)query * 4u) * kLog2e;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)of[s][e], (float)ov[s][e], part);
    dd = sum_halves(part);
    if (h == 0 && query < N) Dws[(size_t)bh * N + query] = dd;
  }

  f32x16 dqacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  uint4 kreg[C::CPT], vreg[C::CPT];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const uint32_t off = ((uint32_t)(t * BC + chunk / C::CPR) * D + (chunk % C::CPR) * 8) * 2u;
      kreg[i] = buf_load16(rk, off);
      vreg[i] = buf_load16(rv, off);
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* Ks = lds + buf * C::BUF_ELEMS;
    bf16_t* Vs = Ks + C::TILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int off = tile_off<D>(chunk / C::CPR, (chunk % C::CPR) * 8);
      *reinterpret_cast<uint4*>(Ks + off) = kreg[i];
      *reinterpret_cast<uint4*>(Vs + off) = vreg[i];
    }
  };

  gload(0);
  lstore(0);
  wait_vmem_all();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int j0 = t * BC;
    const bool active = !CAUSAL || j0 <= q0w + 31;
    if (active) {
      const bf16_t* Ks = lds + buf * C::BUF_ELEMS;
      const bf16_t* Vs = Ks + C::TILE;

      // S^T = K Q^T, dP^T = V dO^T (lane: query; registers: keys).
      f32x16 sacc[C::KB], pacc[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 ak = frag_rows<D>(Ks, kb * 32, 16 * s, c32, h);
          const bf16x8 av = frag_rows<D>(Vs, kb * 32, 16 * s, c32, h);
          if (s == 0) {
            const f32x16 z = {};
            sacc[kb] = mfma32x32x16(ak, qf[s], z);
            pacc[kb] = mfma32x32x16(av, of[s], z);
          } else {
            sacc[kb] = mfma32x32x16(ak, qf[s], sacc[kb]);
            pacc[kb] = mfma32x32x16(av, of[s], pacc[kb]);
          }
        }
      }

      // P^T = exp2(S^T c - LSE2); masked entries (causal future, key tail) are
      // zeroed on the blocks that need it only (a real branch).
      float pv[C::KB][16];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[kb][r] = fast_exp2(fmaf(sacc[kb][r], c, -lse2));
      const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w);
      if (need_mask) {
        keep_branch();
        const int kq = j0 + 4 * h - query;  // key - query = kq + key offset
        const int nk = N - j0 - 4 * h;      // key >= N  <=>  key offset >= nk
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = kb * 32 + 8 * (r >> 2) + (r & 3);
            if ((CAUSAL && kq + koff > 0) || koff >= nk) pv[kb][r] = 0.f;
          }
      }
      // dS^T = P^T (dP^T - D), packed to bf16: register r of block kb is
      // k-step 2*kb + (r>>3), element r & 7.
      uint32_t sw[C::PU][4];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          sw[2 * kb + (r >> 3)][(r & 7) >> 1] =
              pack_bf16x2(pv[kb][r] * (pacc[kb][r] - dd), pv[kb][r + 1] * (pacc[kb][r + 1] - dd));

      // dQ^T += K^T dS^T (lane: query; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const bf16x8 a = frag_tr<D>(Ks, 16 * u, db * 32, lane);
          dqacc[db] = mfma32x32x16(a, bf16x8_from(sw[u][0], sw[u][1], sw[u][2], sw[u][3]), dqacc[db]);
        }
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  if (query < N) {
    bf16_t* dQr = dQ + hoff + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(dqacc[db][4 * g + e] * scale);
        *reinterpret_cast<bf16x4*>(dQr + db * 32 + 8 * g + 4 * h) = v;
      }
  }
}

template <int D, int NWK, int QB, int OCCK, int NWQ, int BC, int OCCQ, bool CAUSAL>
hipError_t run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV, float* Dws, const Problem& p,
                   unsigned stages, hipStream_t stream) {
  const int BH = p.B * p.H;
  const long long rows = (long long)BH * p.N;
  const float c = p.scale * kLog2e;
  if (stages & kStagePre) {
    constexpr int RPB = 256 / (D / 8);
    const long long grid = (rows + RPB - 1) / RPB;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)O, (const bf16_t*)dO, Dws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDq) {
    using C = DqCfg<D, NWQ, BC>;
    const int nqb = (p.N + C::BR - 1) / C::BR;
    const long long grid = (long long)BH * nqb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int G = head_group(OCCQ * 4 / NWQ, nqb);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, NWQ, BC, OCCQ, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (const bf16_t*)O, (const bf16_t*)dO, LSE, Dws, (bf16_t*)dQ, BH, p.N, nqb, G,
                       c, p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDkDv) {
    using C = DkdvCfg<D, NWK, QB>;
    const int nkb = (p.N + C::BK - 1) / C::BK;
    const long long grid = (long long)BH * nkb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    const int G = head_group(OCCK * 4 / NWK, nkb);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, NWK, QB, OCCK, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (const bf16_t*)dO, LSE, Dws, (bf16_t*)dK, (bf16_t*)dV, BH, p.N, nkb, G, c,
                       p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Launch configurations per head dim: dK/dV (wavefronts per workgroup,
// 32-row query blocks per chunk, minimum wavefronts per SIMD), then dQ
// (wavefronts per workgroup, keys per K/V block, minimum wavefronts per SIMD).
#ifndef FA_BWD_CFG_D64
#define FA_BWD_CFG_D64 4, 2, 2, 4, 64, 2
#endif
#ifndef FA_BWD_CFG_D128
#define FA_BWD_CFG_D128 4, 1, 1, 4, 64, 1
#endif
#ifndef FA_BWD_CFG_D256
#define FA_BWD_CFG_D256 4, 1, 1, 4, 32, 1
#endif

template <int D, int NWK, int QB, int OCCK, int NWQ, int BC, int OCCQ>
hipError_t run_bwd_c(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* LSE, void* dQ, void* dK, void* dV, float* Dws, const Problem& p,
                     unsigned stages, hipStream_t stream) {
  return p.causal ? run_bwd<D, NWK, QB, OCCK, NWQ, BC, OCCQ, true>(Q, K, V, O, dO, LSE, dQ, dK, dV,
                                                                  Dws, p, stages, stream)
                  : run_bwd<D, NWK, QB, OCCK, NWQ, BC, OCCQ, false>(Q, K, V, O, dO, LSE, dQ, dK,
                                                                   dV, Dws, p, stages, stream);
}

}  // namespace

hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                float* Dws, const Problem& p, unsigned stages,
                                hipStream_t stream) {
  switch (p.d) {
    case 64:
      return run_bwd_c<64, FA_BWD_CFG_D64>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    case 128:
      return run_bwd_c<128, FA_BWD_CFG_D128>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    case 256:
      return run_bwd_c<256, FA_BWD_CFG_D256>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
