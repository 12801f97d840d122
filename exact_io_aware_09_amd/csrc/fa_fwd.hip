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
//  * NW wavefronts per workgroup, each owning 32*QSUB query rows whose Q
//    fragments stay in VGPRs for the whole kernel.
//  * K/V blocks of BC keys are staged in LDS, double-buffered with one
//    barrier per block.  Tiles are unpadded and XOR-swizzled at 16-byte
//    granularity; K is read by rows (16-byte reads) and V through the LDS
//    transpose unit (ds_read_b64_tr_b16), so neither needs a transposed copy.
//  * Global reads are buffer loads whose hardware range check returns zeros
//    past the end of the head, so tail blocks need no branches.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: each lane holds scores of ONE
//    query row, so the row maximum is an in-lane reduction plus one exchange
//    with the other half-wave.  The exponentiated scores, rounded to bf16,
//    are directly the B operand of O^T += V^T P^T; the row sum is taken from
//    the fp32 values (summing the rounded ones would cost ~2^-9 relative in
//    l, too much for the log-sum-exp at short rows).
//  * exp is evaluated as exp2 with scale*log2(e) folded into one FMA.  The
//    running maximum of a row is only raised (and that row's O, l rescaled)
//    when a block's maximum exceeds it by more than 2^8 in the exponent;
//    otherwise the stale maximum is kept, which leaves every weight at most
//    2^8 and the final O = acc / l unchanged (numerator and denominator share
//    the same base).
//  * Workgroups are remapped so that all query blocks of a head run on one
//    XCD (shared L2 for the re-read K/V), longest causal blocks first.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units: defer rescaling up to a factor 256

template <int D, int NW, int QSUB, int BC>
struct FwdCfg {
  static constexpr int NT = NW * kWave;        // threads per workgroup
  static constexpr int BR = NW * 32 * QSUB;    // query rows per workgroup
  static constexpr int TILE = BC * D;          // elements of one K or V tile
  static constexpr int LDS_ELEMS = 4 * TILE;   // K, V x double buffer
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int CPT = BC * CPR / NT;    // chunks per thread per tile
  static constexpr int KSTEPS = D / 16;        // k-steps of K Q^T
  static constexpr int DB = D / 32;            // 32-wide blocks of the head dim
  static constexpr int KB = BC / 32;           // 32-key blocks per tile
  static constexpr int PU = BC / 16;           // k-steps of V^T P^T
  static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
};

template <int D, int NW, int QSUB, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (D >= 256 ? 1 : 2))
void fwd_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                     const bf16_t* __restrict__ V, bf16_t* __restrict__ O,
                     float* __restrict__ LSE, int BH, int N, int nqb, float c) {
  using C = FwdCfg<D, NW, QSUB, BC>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, BH * nqb);
  const int bh = L / nqb;
  const int qb = CAUSAL ? (nqb - 1 - L % nqb) : (L % nqb);
  const size_t hoff = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rq = make_rsrc(Q + hoff, head_bytes);
  const auto rk = make_rsrc(K + hoff, head_bytes);
  const auto rv = make_rsrc(V + hoff, head_bytes);
  bf16_t* Oh = O + hoff;
  float* Lh = LSE + (size_t)bh * N;

  const int q0 = qb * C::BR;
  const int q0w = q0 + w * 32 * QSUB;

  // Query fragments: B operand of S^T = K Q^T (lane = query row).
  bf16x8 qf[QSUB][C::KSTEPS];
#pragma unroll
  for (int qs = 0; qs < QSUB; ++qs) {
    const uint32_t row = (uint32_t)(q0w + qs * 32 + c32);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      qf[qs][s] = as_bf16x8(buf_load16(rq, (row * D + 16 * s + 8 * h) * 2u));
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
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int chunk = tid + i * C::NT;
      const uint32_t row = (uint32_t)(t * BC + chunk / C::CPR);
      const uint32_t off = (row * D + (chunk % C::CPR) * 8) * 2u;
      kreg[i] = buf_load16(rk, off);
      vreg[i] = buf_load16(rv, off);
    }
  };
  auto lstore = [&](int buf) {
    bf16_t* Ks = lds + buf * C::TILE;
    bf16_t* Vs = lds + (2 + buf) * C::TILE;
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
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int j0 = t * BC;
    const bool active = !CAUSAL || j0 <= q0w + 32 * QSUB - 1;
    if (active) {
      const bf16_t* Ks = lds + buf * C::TILE;
      const bf16_t* Vs = lds + (2 + buf) * C::TILE;

      // S^T = K Q^T for this tile (lane: query; registers: keys).
      f32x16 sacc[QSUB][C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 a = frag_rows<D>(Ks, kb * 32, 16 * s, c32, h);
#pragma unroll
          for (int qs = 0; qs < QSUB; ++qs) {
            if (s == 0) {
              const f32x16 z = {};
              sacc[qs][kb] = mfma32x32x16(a, qf[qs][s], z);
            } else {
              sacc[qs][kb] = mfma32x32x16(a, qf[qs][s], sacc[qs][kb]);
            }
          }
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
        mx = fmaxf(mx, xor32(mx)) * c;
        // Only rows whose own maximum moved past the slack are rescaled (the
        // others multiply by exactly 1), so each row's arithmetic depends on
        // its own scores alone.
        const bool need = mx > m[qs] + kRescaleSlack;
        if (wave_any(need)) {
          const float mnew = need ? mx : m[qs];
          const float alpha = !need ? 1.f : (m[qs] == -INFINITY) ? 0.f : fast_exp2(m[qs] - mnew);
          m[qs] = mnew;
          l[qs] *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qs][db][r] *= alpha;
        }
        const float muse = (m[qs] == -INFINITY) ? 0.f : m[qs];
        // P^T as the B operand of O^T += V^T P^T: k-step u takes registers
        // 8*(u&1) .. +7 of key block u>>1, i.e. keys 16u + 8*(e>>2) + 4h + (e&3).
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = fast_exp2(fmaf(sacc[qs][u >> 1][8 * (u & 1) + e], c, -muse));
            const float p1 = fast_exp2(fmaf(sacc[qs][u >> 1][8 * (u & 1) + e + 1], c, -muse));
            pf[qs][u][e] = to_bf16(p0);
            pf[qs][u][e + 1] = to_bf16(p1);
            rs += p0 + p1;
          }
        }
        l[qs] += rs;
      }

      // O^T += V^T P^T (lane: query; registers: head dims).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int u = 0; u < C::PU; ++u) {
          const bf16x8 a = frag_tr<D>(Vs, 16 * u, db * 32, lane);
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

template <int D, int NW, int QSUB, int BC, bool CAUSAL>
hipError_t run_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   const Problem& p, hipStream_t stream) {
  using C = FwdCfg<D, NW, QSUB, BC>;
  const int BH = p.B * p.H;
  const int nqb = (p.N + C::BR - 1) / C::BR;
  const long long grid = (long long)BH * nqb;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QSUB, BC, CAUSAL>), dim3((unsigned)grid), dim3(C::NT),
                     0, stream, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, (bf16_t*)O,
                     LSE, BH, p.N, nqb, c);
  return hipGetLastError();
}

template <int D, int NW, int QSUB, int BC>
hipError_t run_fwd_c(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     const Problem& p, hipStream_t stream) {
  return p.causal ? run_fwd<D, NW, QSUB, BC, true>(Q, K, V, O, LSE, p, stream)
                  : run_fwd<D, NW, QSUB, BC, false>(Q, K, V, O, LSE, p, stream);
}

}  // namespace

hipError_t launch_forward_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return run_fwd_c<64, 4, 2, 64>(Q, K, V, O, LSE, p, stream);
    case 128: return run_fwd_c<128, 4, 1, 64>(Q, K, V, O, LSE, p, stream);
    case 256: return run_fwd_c<256, 4, 1, 32>(Q, K, V, O, LSE, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
