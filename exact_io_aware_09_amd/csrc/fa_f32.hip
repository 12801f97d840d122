// fa_f32.hip -- float32 attention forward and backward on the vector ALUs.
//
// The same tiled algorithm as the bfloat16 matrix-core kernels (online
// softmax forward, CS324 "Lecture 8 . GPU Performance & FlashAttention"
// sections 5.2-5.3; recomputing backward, section 5.4), kept in float32 end
// to end so that it meets float32 tolerances.  It is the correctness path
// for float32 callers, not a throughput path.
//
// Each row (a query row in the forward and dQ kernels, a key row in the
// dK/dV kernel) is owned by TPR = d/16 consecutive lanes, each holding 16 of
// the d columns; dot products are reduced across those lanes with a xor
// butterfly (every lane ends with the bitwise-identical sum).  The streamed
// operand (K/V blocks, or Q/dO blocks) is staged in LDS 32 rows at a time.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kTile = 32;  // rows of the streamed operand per LDS stage

template <int TPR>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void load16f(float* dst, const float* src, bool ok) {
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 v = ok ? *reinterpret_cast<const float4*>(src + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[e] = v.x;
    dst[e + 1] = v.y;
    dst[e + 2] = v.z;
    dst[e + 3] = v.w;
  }
}

// Cooperative copy of `rows` x D floats (rows starting at r0, zero beyond N)
// into an LDS tile of kTile x D.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int r0, int N) {
  constexpr int CPR = D / 4;
  for (int chunk = threadIdx.x; chunk < kTile * CPR; chunk += blockDim.x) {
    const int row = chunk / CPR, col = (chunk % CPR) * 4;
    const bool ok = r0 + row < N;
    const float4 v = ok ? *reinterpret_cast<const float4*>(src + (size_t)(r0 + row) * D + col)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dst + row * D + col) = v;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256)
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                    int N, int nqb, float scale) {
  constexpr int TPR = D / 16, RPB = 256 / TPR;
  __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * D];
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * RPB;
  const int row = q0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const bool ok = row < N;
  float q[16], acc[16];
  load16f(q, Q + hoff + (size_t)row * D + part * 16, ok);
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? min(N, q0 + RPB) : N;
  for (int j0 = 0; j0 < kend; j0 += kTile) {
    __syncthreads();
    stage_rows<D>(Ks, K + hoff, j0, N);
    stage_rows<D>(Vs, V + hoff, j0, N);
    __syncthreads();
    float s[kTile];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) dot = fmaf(q[e], Ks[j * D + part * 16 + e], dot);
      dot = group_sum<TPR>(dot) * scale;
      const int key = j0 + j;
      s[j] = (key >= N || (CAUSAL && key > row)) ? -INFINITY : dot;
      mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = expf(m - muse);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = expf(s[j] - muse);
      l += p;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = fmaf(p, Vs[j * D + part * 16 + e], acc[e]);
    }
    m = mnew;
  }
  if (ok) {
    float* o = O + hoff + (size_t)row * D + part * 16;
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<float4*>(o + e) =
          make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    if (part == 0) LSE[(size_t)bh * N + row] = m + logf(l);
  }
}

template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                        const float* __restrict__ LSE, float* __restrict__ Dws,
                        float* __restrict__ Lws, long long rows) {
  constexpr int TPR = D / 16, RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float a[16], b[16];
  const bool ok = row < rows;
  load16f(a, O + (size_t)row * D + part * 16, ok);
  load16f(b, dO + (size_t)row * D + part * 16, ok);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc = fmaf(a[e], b[e], acc);
  acc = group_sum<TPR>(acc);
  if (ok && part == 0) {
    Dws[row] = -acc;
    Lws[row] = LSE[row] * kLog2e;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256)
void bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, const float* __restrict__ dO,
                         const float* __restrict__ Lws, const float* __restrict__ Dws,
                         float* __restrict__ dK, float* __restrict__ dV, int N, int nkb,
                         float scale) {
  constexpr int TPR = D / 16, RPB = 256 / TPR;
  __shared__ __attribute__((aligned(16))) float Qs[kTile * D];
  __shared__ __attribute__((aligned(16))) float Os[kTile * D];
  __shared__ float Ls[kTile], Ds[kTile];
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const size_t hoff = (size_t)bh * N * D;
  const int k0 = kb * RPB;
  const int key = k0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const bool ok = key < N;
  float kk[16], vv[16], dk[16], dv[16];
  load16f(kk, K + hoff + (size_t)key * D + part * 16, ok);
  load16f(vv, V + hoff + (size_t)key * D + part * 16, ok);
#pragma unroll
  for (int e = 0; e < 16; ++e) dk[e] = dv[e] = 0.f;
  const int istart = CAUSAL ? (k0 / kTile) * kTile : 0;
  for (int i0 = istart; i0 < N; i0 += kTile) {
    __syncthreads();
    stage_rows<D>(Qs, Q + hoff, i0, N);
    stage_rows<D>(Os, dO + hoff, i0, N);
    if (threadIdx.x < kTile) {
      const int r = i0 + threadIdx.x;
      Ls[threadIdx.x] = r < N ? Lws[(size_t)bh * N + r] : 0.f;  // LSE * log2(e)
      Ds[threadIdx.x] = r < N ? -Dws[(size_t)bh * N + r] : 0.f;  // the workspace holds -D
    }
    __syncthreads();
    for (int i = 0; i < kTile; ++i) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s = fmaf(Qs[i * D + part * 16 + e], kk[e], s);
        dp = fmaf(Os[i * D + part * 16 + e], vv[e], dp);
      }
      s = group_sum<TPR>(s) * scale;
      dp = group_sum<TPR>(dp);
      const int query = i0 + i;
      const bool vis = query < N && (!CAUSAL || key <= query);
      const float p = vis ? exp2f(fmaf(s, kLog2e, -Ls[i])) : 0.f;
      const float ds = p * (dp - Ds[i]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        dv[e] = fmaf(p, Os[i * D + part * 16 + e], dv[e]);
        dk[e] = fmaf(ds, Qs[i * D + part * 16 + e], dk[e]);
      }
    }
  }
  if (ok) {
    float* pk = dK + hoff + (size_t)key * D + part * 16;
    float* pv = dV + hoff + (size_t)key * D + part * 16;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      *reinterpret_cast<float4*>(pk + e) =
          make_float4(dk[e] * scale, dk[e + 1] * scale, dk[e + 2] * scale, dk[e + 3] * scale);
      *reinterpret_cast<float4*>(pv + e) = make_float4(dv[e], dv[e + 1], dv[e + 2], dv[e + 3]);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256)
void bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const float* __restrict__ dO,
                       const float* __restrict__ LSE, const float* __restrict__ Dws,
                       float* __restrict__ dQ, int N, int nqb, float scale) {
  constexpr int TPR = D / 16, RPB = 256 / TPR;
  __shared__ __attribute__((aligned(16))) float Ks[kTile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * D];
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const size_t hoff = (size_t)bh * N * D;
  const int q0 = qb * RPB;
  const int row = q0 + threadIdx.x / TPR, part = threadIdx.x % TPR;
  const bool ok = row < N;
  float q[16], o[16], dq[16];
  load16f(q, Q + hoff + (size_t)row * D + part * 16, ok);
  load16f(o, dO + hoff + (size_t)row * D + part * 16, ok);
#pragma unroll
  for (int e = 0; e < 16; ++e) dq[e] = 0.f;
  const float lse = ok ? LSE[(size_t)bh * N + row] : 0.f;
  const float dd = ok ? -Dws[(size_t)bh * N + row] : 0.f;  // the workspace holds -D
  const int kend = CAUSAL ? min(N, q0 + RPB) : N;
  for (int j0 = 0; j0 < kend; j0 += kTile) {
    __syncthreads();
    stage_rows<D>(Ks, K + hoff, j0, N);
    stage_rows<D>(Vs, V + hoff, j0, N);
    __syncthreads();
    for (int j = 0; j < kTile; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s = fmaf(q[e], Ks[j * D + part * 16 + e], s);
        dp = fmaf(o[e], Vs[j * D + part * 16 + e], dp);
      }
      s = group_sum<TPR>(s) * scale;
      dp = group_sum<TPR>(dp);
      const int key = j0 + j;
      const bool vis = ok && key < N && (!CAUSAL || key <= row);
      const float p = vis ? expf(s - lse) : 0.f;
      const float ds = p * (dp - dd);
#pragma unroll
      for (int e = 0; e < 16; ++e) dq[e] = fmaf(ds, Ks[j * D + part * 16 + e], dq[e]);
    }
  }
  if (ok) {
    float* pq = dQ + hoff + (size_t)row * D + part * 16;
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      *reinterpret_cast<float4*>(pq + e) =
          make_float4(dq[e] * scale, dq[e + 1] * scale, dq[e + 2] * scale, dq[e + 3] * scale);
  }
}

template <int D, bool CAUSAL>
hipError_t run_fwd_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                       const Problem& p, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 16);
  const int nqb = (p.N + RPB - 1) / RPB;
  const long long grid = (long long)p.B * p.H * nqb;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream, Q, K,
                     V, O, LSE, p.N, nqb, p.scale);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t run_bwd_f32(const float* Q, const float* K, const float* V, const float* O,
                       const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                       float* ws, const Problem& p, unsigned stages, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 16);
  const long long rows = (long long)p.B * p.H * p.N;
  float* Dws = ws;         // -D, one float per row
  float* Lws = ws + ws_lse_offset(rows);  // LSE * log2(e), one float per row
  const long long gpre = (rows + RPB - 1) / RPB;
  const int nb = (p.N + RPB - 1) / RPB;
  const long long grid = (long long)p.B * p.H * nb;
  if (gpre > 0x7fffffffLL || grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // the dQ stage forms D and LSE*log2(e) itself (here with the standalone
  // kernel) and leaves them in the workspace for the dK/dV stage
  if (stages & (kStagePre | kStageDq)) {
    hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)gpre), dim3(256), 0, stream, O, dO,
                       LSE, Dws, Lws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDq) {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, stream,
                       Q, K, V, dO, LSE, Dws, dQ, p.N, nb, p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageDkDv) {
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0,
                       stream, Q, K, V, dO, (const float*)Lws, (const float*)Dws, dK, dV, p.N, nb,
                       p.scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_forward_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                              const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 64:
      return p.causal ? run_fwd_f32<64, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd_f32<64, false>(Q, K, V, O, LSE, p, stream);
    case 128:
      return p.causal ? run_fwd_f32<128, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd_f32<128, false>(Q, K, V, O, LSE, p, stream);
    case 256:
      return p.causal ? run_fwd_f32<256, true>(Q, K, V, O, LSE, p, stream)
                      : run_fwd_f32<256, false>(Q, K, V, O, LSE, p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_f32(const float* Q, const float* K, const float* V, const float* O,
                               const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                               float* Dws, const Problem& p, unsigned stages,
                               hipStream_t stream) {
  switch (p.d) {
    case 64:
      return p.causal ? run_bwd_f32<64, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream)
                      : run_bwd_f32<64, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    case 128:
      return p.causal ? run_bwd_f32<128, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream)
                      : run_bwd_f32<128, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    case 256:
      return p.causal ? run_bwd_f32<256, true>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream)
                      : run_bwd_f32<256, false>(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, stages, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fa
