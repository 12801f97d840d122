// fa_fwd.hip -- attention forward for gfx950, bfloat16 in, fp32 accumulate.
//
// Algorithm: the tiled forward with an online softmax ("Lecture 8 . GPU
// Performance & FlashAttention", CS324 notes, sections 5.2-5.3), in the loop
// order of the second version described in section 8.1 of those notes and in
// "FlashAttention and GPU memory" section 07: one block of query rows per
// workgroup, an inner loop over K/V blocks, an unnormalised output
// accumulator that is divided by the row sum once at the end, and only O and
// the per-row log-sum-exp written to device memory.
//
// Mapping to CDNA4:
//  * 4 wavefronts per workgroup, each owning 32*QSUB query rows; the query
//    fragments stay in VGPRs for the whole kernel.
//  * K/V blocks of BC keys are staged in LDS (double-buffered, one barrier
//    per block).  K is stored row-major and V transposed, so that both
//    contractions read 16- or 8-byte operand fragments.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane then holds 16 scores
//    of ONE query row, so the row maximum is an in-lane reduction plus one
//    exchange with the other half-wave, and the row sum needs no exchange
//    until the end.  The scores, exponentiated and rounded to bf16, are
//    directly the B operand of O^T += V^T P^T (no LDS round trip for P).
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA.
//  * Workgroups are remapped so that all query blocks of a head run on one
//    XCD (shared L2 for the re-read K/V), longest causal blocks first.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, int QSUB, int BC>
struct FwdCfg {
  static constexpr int NW = 4;                 // wavefronts per workgroup
  static constexpr int NT = NW * kWave;        // threads per workgroup
  static constexpr int BR = NW * 32 * QSUB;    // query rows per workgroup
  static constexpr int KS = D + 8;             // LDS row stride of K (elements)
  static constexpr int VS = BC + 8;            // LDS row stride of V^T (elements)
  static constexpr int KTILE = BC * KS;
  static constexpr int VTILE = D * VS;
  static constexpr int LDS_ELEMS = 2 * (KTILE + VTILE);
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / NT;    // chunks per thread per tile
  static constexpr int KSTEPS = D / 16;        // k-steps of Q K^T
  static constexpr int DB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int KB = BC / 32;           // 32-key blocks per tile
  static constexpr int PU = BC / 16;           // k-steps of P V
  static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
};

template <int D, int QSUB, int BC, bool CAUSAL>
__global__ __launch_bounds__(256, (D >= 256 ? 1 : 2))
void fwd_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                     const bf16_t* __restrict__ V, bf16_t* __restrict__ O,
                     float* __restrict__ LSE, int BH, int N, int nqb, float c) {
  using C = FwdCfg<D, QSUB, BC>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, BH * nqb);
  const int bh = L / nqb;
  const int qb = CAUSAL ? (nqb - 1 - L % nqb) : (L % nqb);
  const size_t hoff = (size_t)bh * N * D;
  const bf16_t* Qh = Q + hoff;
  const bf16_t* Kh = K + hoff;
  const bf16_t* Vh = V + hoff;
  bf16_t* Oh = O + hoff;
  float* Lh = LSE + (size_t)bh * N;

  const int q0 = qb * C::BR;
  const int q0w = q0 + w * 32 * QSUB;

  // Query fragments: B operand of S^T = K Q^T (lane = query row).
  bf16x8 qf[QSUB][C::KSTEPS];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const int row = q0w + qs * 32 + c32;
    const bool ok = row < N;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      qf[qs][s] = as_bf16x8(load16_or_zero(Qh + (size_t)row * D + 16 * s + 8 * h, ok));
  }

  const int kend = CAUSAL ? min(N, q0 + C::BR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  f32x16 oacc[QSUB][C::DB];
  float m[QSUB], l[QSUB];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    m[qs] = -INFINITY;
    l[qs] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qs][db][r] = 0.f;
  }

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
    bf16_t* Ks = lds + buf * C::KTILE;
    bf16_t* Vt = lds + 2 * C::KTILE + buf * C::VTILE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const int row = chunk / C::CPR, col = (chunk % C::CPR) * 8;
      *reinterpret_cast<uint4*>(Ks + row * C::KS + col) = kreg[i];
      const uint32_t wv[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(col + 2 * e) * C::VS + row] = (bf16_t)(wv[e] & 0xffffu);
        Vt[(col + 2 * e + 1) * C::VS + row] = (bf16_t)(wv[e] >> 16);
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
    const bool active = !CAUSAL || j0 <= q0w + 32 * QSUB - 1;
    if (active) {
      const bf16_t* Ks = lds + buf * C::KTILE;
      const bf16_t* Vt = lds + 2 * C::KTILE + buf * C::VTILE;

      // S^T = K Q^T for this tile (lane: query; registers: keys).
      f32x16 sacc[QSUB][C::KB];
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs)
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qs][kb][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + c32) * C::KS + 16 * s + 8 * h);
#pragma unroll
          for (int qs = 0; qs < QSUB; ++qs) sacc[qs][kb] = mfma32x32x16(a, qf[qs][s], sacc[qs][kb]);
        }
      }

      // Causal diagonal and key tail: masked scores become -inf.
      const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int qs = 0; qs < QSUB; ++qs) {
          const int query = q0w + qs * 32 + c32;
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              if (key >= N || (CAUSAL && key > query)) sacc[qs][kb][r] = -INFINITY;
            }
        }
      }

      // Online softmax in base 2 (c = scale * log2 e > 0).
      bf16x8 pf[QSUB][C::PU];
#pragma unroll
      for (int qs = 0; qs < QSUB; ++qs) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qs][kb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float mnew = fmaxf(m[qs], mx * c);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(m[qs] - muse);
        m[qs] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[qs][kb][r], c, -muse));
            rs += p;
            sacc[qs][kb][r] = p;
          }
        l[qs] = fmaf(l[qs], alpha, rs);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qs][db][r] *= alpha;
        // P^T as the B operand of O^T += V^T P^T: k-step u takes registers
        // 8*(u&1) .. +7 of key block u>>1, i.e. keys 16u + 8*(e>>2) + 4h + (e&3).
#pragma unroll
        for (int u = 0; u < C::PU; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[qs][u][e] = to_bf16(sacc[qs][u >> 1][8 * (u & 1) + e]);
      }

      // O^T += V^T P^T (lane: query; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const bf16_t* vp = Vt + (db * 32 + c32) * C::VS + 16 * u + 4 * h;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vp);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vp + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qs = 0; qs < QSUB; ++qs) oacc[qs][db] = mfma32x32x16(a, pf[qs][u], oacc[qs][db]);
        }
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l (bf16), LSE = m ln2 + ln l (fp32, natural log).
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const float lt = l[qs] + xor32(l[qs]);
    const float inv = 1.f / lt;
    const int query = q0w + qs * 32 + c32;
    if (query < N) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = to_bf16(oacc[qs][db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(Oh + (size_t)query * D + db * 32 + 8 * g + 4 * h) = v;
        }
      if (h == 0) Lh[query] = fmaf(m[qs], kLn2, logf(lt));
    }
  }
}

template <int D, int QSUB, int BC, bool CAUSAL>
hipError_t run_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   const Problem& p, hipStream_t stream) {
  using C = FwdCfg<D, QSUB, BC>;
  const int BH = p.B * p.H;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  const long long grid = (long long)BH * nqb;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QSUB, BC, CAUSAL>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, (bf16_t*)O, LSE, BH,
                     p.N, nqb, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64:
      return p.causal ? run_fwd<64, 2, 64, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd<64, 2, 64, false>(Q, K, V, O, LSE, p, stream);
    case 128:
      return p.causal ? run_fwd<128, 1, 64, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd<128, 1, 64, false>(Q, K, V, O, LSE, p, stream);
    case 256:
      return p.causal ? run_fwd<256, 1, 32, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd<256, 1, 32, false>(Q, K, V, O, LSE, p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
