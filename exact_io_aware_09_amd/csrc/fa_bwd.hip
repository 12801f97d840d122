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
//   pre   D = rowsum(dO * O), fp32, bandwidth-bound.
//   dkdv  one block of 128 keys per workgroup (32 per wavefront, K and V
//         fragments held in VGPRs), loop over query chunks staged in LDS;
//         dK and dV accumulate in registers and are written once.
//   dq    one block of 128 query rows per workgroup (32 per wavefront),
//         loop over K/V blocks staged in LDS; dQ written once.
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
// dK, dV.  Per wavefront: 32 keys.  Per iteration: a chunk of BQ = 32*QB
// query rows in LDS, stored row-major (A operand of S = Q K^T and of
// dP = dO V^T) and transposed (A operand of dK^T += Q^T dS, dV^T += dO^T P).
template <int D, int QB>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * kWave;
  static constexpr int BK = NW * 32;          // keys per workgroup
  static constexpr int BQ = 32 * QB;          // query rows per chunk
  static constexpr int RS = D + 8;            // row-major stride (elements)
  static constexpr int TS = BQ + 8;           // transposed stride (elements)
  static constexpr int ROWT = BQ * RS;
  static constexpr int TRT = D * TS;
  // one buffer: Q, dO row-major; Q^T, dO^T; then LSE*log2e and D (floats)
  static constexpr int BUF_ELEMS = 2 * ROWT + 2 * TRT + 2 * BQ * 2;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BQ * CPR / NT;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int PU = BQ / 16;
  static_assert(BQ * CPR % NT == 0, "chunk must split evenly over threads");
};

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2))
void bwd_dkdv_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                          const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                          const float* __restrict__ LSE, const float* __restrict__ Dws,
                          bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int BH, int N,
                          int nkb, float c, float scale) {
  using C = DkdvCfg<D, QB>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, BH * nkb);
  const int bh = L / nkb;
  const int kb = L % nkb;  // causal: low key blocks see the most queries, run them first
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* Qh = Q + hoff;
  const bf16_t* dOh = dO + hoff;
  const float* Lh = LSE + (size_t)bh * N;
  const float* Dh = Dws + (size_t)bh * N;

  const int k0 = kb * C::BK;
  const int k0w = k0 + w * 32;
  const int key = k0w + c32;  // this lane's key row (MFMA column)

  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (lane = key).
  bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
  {
    const bool ok = key < N;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      const size_t off = hoff + (size_t)key * D + 16 * s + 8 * h;
      kf[s] = as_bf16x8(load16_or_zero(K + off, ok));
      vf[s] = as_bf16x8(load16_or_zero(V + off, ok));
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
      const int row = chunk / C::CPR, col = (chunk % C::CPR) * 8;
      const bool ok = i0 + row < N;
      const size_t off = (size_t)(i0 + row) * D + col;
      qreg[i] = load16_or_zero(Qh + off, ok);
      oreg[i] = load16_or_zero(dOh + off, ok);
    }
    if (tid < C::BQ) {
      const bool ok = i0 + tid < N;
      lreg = ok ? Lh[i0 + tid] * kLog2e : 0.f;
      dreg = ok ? Dh[i0 + tid] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* base = lds + buf * C::BUF_ELEMS;
    bf16_t* Qs = base;
    bf16_t* dOs = base + C::ROWT;
    bf16_t* Qt = base + 2 * C::ROWT;
    bf16_t* dOt = base + 2 * C::ROWT + C::TRT;
    float* fl = reinterpret_cast<float*>(base + 2 * C::ROWT + 2 * C::TRT);
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int row = chunk / C::CPR, col = (chunk % C::CPR) * 8;
      *reinterpret_cast<uint4*>(Qs + row * C::RS + col) = qreg[i];
      *reinterpret_cast<uint4*>(dOs + row * C::RS + col) = oreg[i];
      const uint32_t qv[4] = {qreg[i].x, qreg[i].y, qreg[i].z, qreg[i].w};
      const uint32_t ov[4] = {oreg[i].x, oreg[i].y, oreg[i].z, oreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Qt[(col + 2 * e) * C::TS + row] = (bf16_t)(qv[e] & 0xffffu);
        Qt[(col + 2 * e + 1) * C::TS + row] = (bf16_t)(qv[e] >> 16);
        dOt[(col + 2 * e) * C::TS + row] = (bf16_t)(ov[e] & 0xffffu);
        dOt[(col + 2 * e + 1) * C::TS + row] = (bf16_t)(ov[e] >> 16);
      }
    }
    if (tid < C::BQ) {
      fl[tid] = lreg;
      fl[C::BQ + tid] = dreg;
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < nchunks; ++t) {
    const int buf = t & 1;
    if (t + 1 < nchunks) gload(t + 1);
    const int i0 = qstart + t * C::BQ;
    // some query of the chunk sees some key of this wavefront
    const bool active = !CAUSAL || i0 + C::BQ - 1 >= k0w;
    if (active) {
      const bf16_t* base = lds + buf * C::BUF_ELEMS;
      const bf16_t* Qs = base;
      const bf16_t* dOs = base + C::ROWT;
      const bf16_t* Qt = base + 2 * C::ROWT;
      const bf16_t* dOt = base + 2 * C::ROWT + C::TRT;
      const float* fl = reinterpret_cast<const float*>(base + 2 * C::ROWT + 2 * C::TRT);

      // S = Q K^T and dP = dO V^T (lane: key; registers: query rows).
      f32x16 sacc[QB], pacc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[qb][r] = 0.f;
          pacc[qb][r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const int off = (qb * 32 + c32) * C::RS + 16 * s + 8 * h;
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + off);
          const bf16x8 ao = *reinterpret_cast<const bf16x8*>(dOs + off);
          sacc[qb] = mfma32x32x16(aq, kf[s], sacc[qb]);
          pacc[qb] = mfma32x32x16(ao, vf[s], pacc[qb]);
        }
      }

      const bool need_mask = (i0 + C::BQ > N) || (CAUSAL && i0 < k0w + 31);
      bf16x8 pb[C::PU], sb[C::PU];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // rows 8g + 4h + 0..3 of this 32-row block: one 16-byte LDS read each
          const int qi = qb * 32 + 8 * g + 4 * h;
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(fl + qi);
          const f32x4 dd4 = *reinterpret_cast<const f32x4*>(fl + C::BQ + qi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = fast_exp2(fmaf(sacc[qb][r], c, -lse4[e]));
            if (need_mask) {
              const int query = i0 + qi + e;
              if (query >= N || (CAUSAL && key > query)) p = 0.f;
            }
            const float ds = p * (pacc[qb][r] - dd4[e]);
            // k-step u = 2*qb + (g>>1), element 4*(g&1) + e
            pb[2 * qb + (g >> 1)][4 * (g & 1) + e] = to_bf16(p);
            sb[2 * qb + (g >> 1)][4 * (g & 1) + e] = to_bf16(ds);
          }
        }
      }

      // dV^T += dO^T P,  dK^T += Q^T dS  (lane: key; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const int off = (db * 32 + c32) * C::TS + 16 * u + 4 * h;
          const bf16x4 olo = *reinterpret_cast<const bf16x4*>(dOt + off);
          const bf16x4 ohi = *reinterpret_cast<const bf16x4*>(dOt + off + 8);
          const bf16x4 qlo = *reinterpret_cast<const bf16x4*>(Qt + off);
          const bf16x4 qhi = *reinterpret_cast<const bf16x4*>(Qt + off + 8);
          const bf16x8 ao = __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 aq = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
          dvacc[db] = mfma32x32x16(ao, pb[u], dvacc[db]);
          dkacc[db] = mfma32x32x16(aq, sb[u], dkacc[db]);
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
// dQ.  Per wavefront: 32 query rows (Q and dO fragments in VGPRs).  Per
// iteration: a block of BC keys in LDS: K and V row-major (A operands of
// S^T = K Q^T and dP^T = V dO^T) and K transposed (A operand of
// dQ^T += K^T dS^T).
template <int D, int BC>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * kWave;
  static constexpr int BR = NW * 32;
  static constexpr int RS = D + 8;
  static constexpr int TS = BC + 8;
  static constexpr int ROWT = BC * RS;
  static constexpr int TRT = D * TS;
  static constexpr int BUF_ELEMS = 2 * ROWT + TRT;
  static constexpr int CPR = D / 8;
  static constexpr int CPT = BC * CPR / NT;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KB = BC / 32;
  static constexpr int PU = BC / 16;
  static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
};

template <int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2))
void bwd_dq_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                        const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ Dws,
                        bf16_t* __restrict__ dQ, int BH, int N, int nqb, float c, float scale) {
  using C = DqCfg<D, BC>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * C::BUF_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, BH * nqb);
  const int bh = L / nqb;
  const int qb = CAUSAL ? (nqb - 1 - L % nqb) : (L % nqb);
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* Kh = K + hoff;
  const bf16_t* Vh = V + hoff;

  const int q0 = qb * C::BR;
  const int q0w = q0 + w * 32;
  const int query = q0w + c32;
  const bool qok = query < N;

  bf16x8 qf[C::KSTEPS], of[C::KSTEPS];
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s) {
    const size_t off = hoff + (size_t)query * D + 16 * s + 8 * h;
    qf[s] = as_bf16x8(load16_or_zero(Q + off, qok));
    of[s] = as_bf16x8(load16_or_zero(dO + off, qok));
  }
  const float lse2 = qok ? LSE[(size_t)bh * N + query] * kLog2e : 0.f;
  const float dd = qok ? Dws[(size_t)bh * N + query] : 0.f;

  f32x16 dqacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  uint4 kreg[C::CPT], vreg[C::CPT];
  auto gload = [&](int t) {
    const int j0 = t * BC;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int row = chunk / C::CPR, col = (chunk % C::CPR) * 8;
      const bool ok = j0 + row < N;
      const size_t off = (size_t)(j0 + row) * D + col;
      kreg[i] = load16_or_zero(Kh + off, ok);
      vreg[i] = load16_or_zero(Vh + off, ok);
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* Ks = lds + buf * C::BUF_ELEMS;
    bf16_t* Vs = Ks + C::ROWT;
    bf16_t* Kt = Ks + 2 * C::ROWT;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int row = chunk / C::CPR, col = (chunk % C::CPR) * 8;
      *reinterpret_cast<uint4*>(Ks + row * C::RS + col) = kreg[i];
      *reinterpret_cast<uint4*>(Vs + row * C::RS + col) = vreg[i];
      const uint32_t kv[4] = {kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Kt[(col + 2 * e) * C::TS + row] = (bf16_t)(kv[e] & 0xffffu);
        Kt[(col + 2 * e + 1) * C::TS + row] = (bf16_t)(kv[e] >> 16);
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int j0 = t * BC;
    const bool active = !CAUSAL || j0 <= q0w + 31;
    if (active) {
      const bf16_t* Ks = lds + buf * C::BUF_ELEMS;
      const bf16_t* Vs = Ks + C::ROWT;
      const bf16_t* Kt = Ks + 2 * C::ROWT;

      // S^T = K Q^T, dP^T = V dO^T (lane: query; registers: keys).
      f32x16 sacc[C::KB], pacc[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[kb][r] = 0.f;
          pacc[kb][r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const int off = (kb * 32 + c32) * C::RS + 16 * s + 8 * h;
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + off);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vs + off);
          sacc[kb] = mfma32x32x16(ak, qf[s], sacc[kb]);
          pacc[kb] = mfma32x32x16(av, of[s], pacc[kb]);
        }
      }

      const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w);
      bf16x8 sb[C::PU];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sacc[kb][r], c, -lse2));
          if (need_mask) {
            const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key >= N || (CAUSAL && key > query)) p = 0.f;
          }
          const float ds = p * (pacc[kb][r] - dd);
          sb[2 * kb + (r >> 3)][r & 7] = to_bf16(ds);
        }

      // dQ^T += K^T dS^T (lane: query; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const bf16_t* kp = Kt + (db * 32 + c32) * C::TS + 16 * u + 4 * h;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(kp);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(kp + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[db] = mfma32x32x16(a, sb[u], dqacc[db]);
        }
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  if (qok) {
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

template <int D, int QB, int BC, bool CAUSAL>
hipError_t run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV, float* Dws, const Problem& p,
                   hipStream_t stream) {
  const int BH = p.B * p.H;
  const long long rows = (long long)BH * p.N;
  const float c = p.scale * kLog2e;
  {
    constexpr int RPB = 256 / (D / 8);
    const long long grid = (rows + RPB - 1) / RPB;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_pre_bf16_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)O, (const bf16_t*)dO, Dws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using C = DkdvCfg<D, QB>;
    const int nkb = (p.N + C::BK - 1) / C::BK;
    const long long grid = (long long)BH * nkb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, QB, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (const bf16_t*)dO, LSE, Dws, (bf16_t*)dK, (bf16_t*)dV, BH, p.N, nkb, c,
                       p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    using C = DqCfg<D, BC>;
    const int nqb = (p.N + C::BR - 1) / C::BR;
    const long long grid = (long long)BH * nqb;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, BC, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V,
                       (const bf16_t*)dO, LSE, Dws, (bf16_t*)dQ, BH, p.N, nqb, c, p.scale);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                float* Dws, const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64:
      return p.causal ? run_bwd<64, 2, 64, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream)
                      : run_bwd<64, 2, 64, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream);
    case 128:
      return p.causal ? run_bwd<128, 1, 64, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream)
                      : run_bwd<128, 1, 64, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream);
    case 256:
      return p.causal ? run_bwd<256, 1, 32, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream)
                      : run_bwd<256, 1, 32, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
