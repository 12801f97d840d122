// fa_api.hip -- the C ABI declared in include/fa.h: argument validation,
// dispatch on (dtype, d, causal) and kernel launches.  Nothing here
// allocates, frees or synchronises; everything is enqueued on the caller's
// stream.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

// Device scratch of fa_backward_noalloc: the backward workspace (-D and
// LSE * log2(e)) for callers that cannot allocate.  Each GPU the library
// runs on holds its own copy from module load until the process ends.  In
// host code the name `scratch` is only a stand-in for the symbol: kernels
// receive the device address that hipGetSymbolAddress returns for the
// current device (scratch_address below), never the name itself.
__device__ __attribute__((aligned(256))) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

// Per-device address of `scratch`, looked up once per device (with that
// device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Address of this device's scratch for work enqueued on `stream`: the
// stream must belong to the current device (the symbol is looked up for the
// current device).
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_HIP;
  if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if ((int)sdev != dev) return FA_ERR_INVALID_ARG;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return FA_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FA_OK;
}

constexpr int kVersion = 400;  // 0.4.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int B, int H, int N, int d, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  // Per-head byte offsets are 32-bit inside the kernels (with room for one
  // tail tile past the end); the B*H*N row count and every grid stay below
  // 2^31.
  if ((long long)N * d > 0x7fff0000LL) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * N > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_common(int B, int H, int N, int d, float scale, int causal, int dtype) {
  const int rc = check_sizes(B, H, N, d, dtype);
  if (rc != FA_OK) return rc;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Dropout: keep threshold t = round((1 - p) * 256) on the 8-bit draws,
// 1 <= t <= 256 (p in [0, 1) and not so close to 1 that nothing is kept).
int make_drop(float p_drop, unsigned long long seed, fa::DropArgs& dr) {
  if (!isfinite(p_drop) || p_drop < 0.f || p_drop >= 1.f) return FA_ERR_INVALID_ARG;
  const int t = (int)floor((1.0 - (double)p_drop) * 256.0 + 0.5);
  if (t < 1 || t > 256) return FA_ERR_INVALID_ARG;
  dr.k0 = (uint32_t)seed;
  dr.k1 = (uint32_t)(seed >> 32);
  dr.thresh = t;
  dr.scale = (float)(256.0 / t);
  dr.keep = (float)(t / 256.0);
  return FA_OK;
}
constexpr int kMaxSplits = 256;

// Split-forward workspace: the partial outputs [splits, rows, d], then the
// partial log-sum-exps [splits, rows] from a 256-byte aligned offset.
size_t split_lse_offset(size_t rows, int d, int splits) {
  return ((size_t)splits * rows * d * sizeof(float) + 255) & ~(size_t)255;
}

// Balanced schedule: launch sizes from the host copy, item pointers into the
// device copy, partial buffers carved out of the workspace.
int sched_args(const int* schedule, const int* schedule_dev, int N, int causal,
                      fa::SchedView& v, fa::SparseArgs& sp) {
  if (!fa::read_schedule(schedule, v) || schedule_dev == nullptr) return FA_ERR_INVALID_ARG;
  if (v.nb != (N + 127) / 128 || v.causal != causal) return FA_ERR_INVALID_ARG;
  if (!aligned16(schedule_dev)) return FA_ERR_MISALIGNED;
  sp.nb = v.nb;
  sp.rows = schedule_dev + v.off_rows;
  sp.cols = schedule_dev + v.off_cols;
  sp.n_rows = v.n_rows;
  sp.n_cols = v.n_cols;
  sp.lists = schedule_dev + v.off_lists;
  sp.list_len = v.list_len;
  sp.row_slots = v.row_slots;
  sp.col_slots = v.col_slots;
  return FA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size, scale not finite and > 0, causal not 0/1)";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (d must be 64, 128 or 256; dtype FA_BF16 or FA_F32; sizes below 2^31)";
    case FA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case FA_ERR_NO_WORKSPACE: return "workspace missing or smaller than the *_workspace_bytes() size";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
               int N, int d, float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = (dtype == FA_BF16)
                     ? fa::launch_forward_bf16(Q, K, V, O, LSE, p, s)
                     : fa::launch_forward_f32((const float*)Q, (const float*)K, (const float*)V,
                                              (float*)O, LSE, p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_forward_split_workspace_bytes(int B, int H, int N, int d, int splits, int dtype) {
  if (check_sizes(B, H, N, d, dtype) != FA_OK || splits < 1 || splits > kMaxSplits) return 0;
  if (splits == 1) return 0;
  const size_t rows = (size_t)B * H * N;
  return split_lse_offset(rows, d, splits) + (size_t)splits * rows * sizeof(float);
}

int fa_forward_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     float scale, int causal, int splits, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  if (splits == 1) return fa_forward(Q, K, V, O, LSE, B, H, N, d, scale, causal, dtype, stream);
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_forward_split_workspace_bytes(B, H, N, d, splits, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
      !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t rows = (size_t)B * H * N;
  float* Opart = static_cast<float*>(workspace);
  float* Lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_lse_offset(rows, d, splits));
  hipError_t e = fa::launch_forward_split_bf16(Q, K, V, p, splits, Opart, Lpart, s);
  if (e == hipSuccess) e = fa::launch_merge(Opart, Lpart, splits, O, LSE, p, true, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_merge_partials(const float* O_parts, const float* LSE_parts, int splits, void* O, float* LSE,
                      int B, int H, int N, int d, int dtype, void* stream) {
  int rc = check_sizes(B, H, N, d, dtype);
  if (rc != FA_OK) return rc;
  if (splits < 1 || splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  if (!O_parts || !LSE_parts || !O || !LSE) return FA_ERR_INVALID_ARG;
  if (!aligned16(O_parts) || !aligned16(LSE_parts) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, 1.0f, false};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = fa::launch_merge(O_parts, LSE_parts, splits, O, LSE, p, dtype == FA_BF16, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      const int* block_mask, int B, int H, int N, int d, float scale, int causal,
                      int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !LSE || !block_mask) return FA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
      !aligned16(block_mask))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  const fa::SparseArgs sp{block_mask, (N + 127) / 128};
  hipError_t e = fa::launch_forward_bf16(Q, K, V, O, LSE, p, reinterpret_cast<hipStream_t>(stream), sp);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_sparse(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, const int* block_mask, void* dQ, void* dK, void* dV,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !dO || !LSE || !block_mask || !dQ || !dK || !dV)
    return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(block_mask) || !aligned16(dQ) || !aligned16(dK) ||
      !aligned16(dV) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  const fa::SparseArgs sp{block_mask, (N + 127) / 128};
  hipError_t e = fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV,
                                          static_cast<float*>(workspace), p, fa::kStagesGrad,
                                          reinterpret_cast<hipStream_t>(stream), sp);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_sparse_balanced(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const int* schedule, const int* schedule_dev, void* workspace,
                               size_t workspace_bytes, int B, int H, int N, int d, float scale,
                               int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !LSE || !schedule) return FA_ERR_INVALID_ARG;
  fa::SchedView v;
  fa::SparseArgs sp;
  rc = sched_args(schedule, schedule_dev, N, causal, v, sp);
  if (rc != FA_OK) return rc;
  const size_t need = fa_sparse_workspace_bytes(schedule, B, H, N, d, 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
      (need > 0 && !aligned16(workspace)))
    return FA_ERR_MISALIGNED;
  const size_t tile = (size_t)B * H * 128;
  char* ws = static_cast<char*>(workspace);
  if (need > 0) {
    sp.part_o = reinterpret_cast<float*>(ws);
    sp.part_l = reinterpret_cast<float*>(ws + align256((size_t)v.row_slots * tile * d * 4));
  }
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = fa::launch_forward_bf16(Q, K, V, O, LSE, p, s, sp);
  if (e == hipSuccess)
    e = fa::launch_merge_rows(sp.part_o, sp.part_l, v.row_slots, schedule_dev + v.off_long_rows,
                              v.n_long_rows, O, LSE, p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_sparse_balanced(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, const int* schedule,
                                const int* schedule_dev, void* dQ, void* dK, void* dV,
                                void* workspace, size_t workspace_bytes, int B, int H, int N,
                                int d, float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !schedule)
    return FA_ERR_INVALID_ARG;
  fa::SchedView v;
  fa::SparseArgs sp;
  rc = sched_args(schedule, schedule_dev, N, causal, v, sp);
  if (rc != FA_OK) return rc;
  const size_t need = fa_sparse_workspace_bytes(schedule, B, H, N, d, 1);
  if (need == 0 || !workspace || workspace_bytes < need) return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) ||
      !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const size_t tile = (size_t)B * H * 128;
  char* ws = static_cast<char*>(workspace);
  size_t at = align256(fa_backward_workspace_bytes(B, H, N, d, dtype));
  sp.part_dq = reinterpret_cast<float*>(ws + at);
  at += align256((size_t)v.row_slots * tile * d * 4);
  sp.part_dk = reinterpret_cast<float*>(ws + at);
  at += align256((size_t)v.col_slots * tile * d * 4);
  sp.part_dv = reinterpret_cast<float*>(ws + at);
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV,
                                          reinterpret_cast<float*>(ws), p, fa::kStagesGrad, s, sp);
  if (e == hipSuccess)
    e = fa::launch_sum_parts(sp.part_dq, v.row_slots, schedule_dev + v.off_long_rows,
                             v.n_long_rows, dQ, p, s);
  if (e == hipSuccess)
    e = fa::launch_sum_parts(sp.part_dk, v.col_slots, schedule_dev + v.off_long_cols,
                             v.n_long_cols, dK, p, s);
  if (e == hipSuccess)
    e = fa::launch_sum_parts(sp.part_dv, v.col_slots, schedule_dev + v.off_long_cols,
                             v.n_long_cols, dV, p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int H, int N, int d, float scale, int causal, float p_drop,
                       unsigned long long seed, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  fa::DropArgs dr;
  rc = make_drop(p_drop, seed, dr);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipError_t e = fa::launch_forward_dropout_bf16(Q, K, V, O, LSE, p, dr, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
int fa_backward_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, int B, int H, int N, int d, float scale,
                        int causal, float p_drop, unsigned long long seed, int dtype,
                        void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  fa::DropArgs dr;
  rc = make_drop(p_drop, seed, dr);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) ||
      !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipError_t e = fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV,
                                          static_cast<float*>(workspace), p, fa::kStagesGrad,
                                          reinterpret_cast<hipStream_t>(stream), fa::SparseArgs{}, &dr);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
size_t fa_fp8_bytes(int B, int H, int N, int d, int layout) {
  if (check_sizes(B, H, N, d, FA_BF16) != FA_OK) return 0;
  if (layout == FA_FP8_ROWS) return (size_t)B * H * N * d;
  if (layout == FA_FP8_KEYS) return (size_t)B * H * d * fa::fp8_keys_padded(N);
  return 0;
}
size_t fa_fp8_scale_bytes(int B, int H, int N, int d, int layout) {
  if (check_sizes(B, H, N, d, FA_BF16) != FA_OK) return 0;
  if (layout == FA_FP8_ROWS) return (size_t)B * H * fa::fp8_keys_padded(N) * (d / 32);
  if (layout == FA_FP8_KEYS) return (size_t)B * H * (fa::fp8_keys_padded(N) / 32) * d;
  return 0;
}
int fa_quantize_fp8(const void* X, void* X8, void* Xs, int B, int H, int N, int d, int layout,
                    void* stream) {
  int rc = check_sizes(B, H, N, d, FA_BF16);
  if (rc != FA_OK) return rc;
  if (layout != FA_FP8_ROWS && layout != FA_FP8_KEYS) return FA_ERR_INVALID_ARG;
  if (!X || !X8 || !Xs) return FA_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(X8) || !aligned16(Xs)) return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, 1.0f, false};
  hipError_t e = fa::launch_quantize_fp8(X, X8, Xs, p, layout == FA_FP8_KEYS,
                                         reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
int fa_forward_fp8(const void* Q8, const void* Qs, const void* K8, const void* Ks, const void* V8,
                   const void* Vs, void* O, float* LSE, int B, int H, int N, int d, float scale,
                   int causal, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, FA_BF16);
  if (rc != FA_OK) return rc;
  if (!Q8 || !Qs || !K8 || !Ks || !V8 || !Vs || !O || !LSE) return FA_ERR_INVALID_ARG;
  if (!aligned16(Q8) || !aligned16(Qs) || !aligned16(K8) || !aligned16(Ks) || !aligned16(V8) ||
      !aligned16(Vs) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipError_t e = fa::launch_forward_fp8(Q8, Qs, K8, Ks, V8, Vs, O, LSE, p,
                                        reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
size_t fa_backward_workspace_bytes(int B, int H, int N, int d, int dtype) {
  if (check_sizes(B, H, N, d, dtype) != FA_OK) return 0;
  // D, then LSE * log2(e) from a 256-byte aligned offset
  const long long rows = (long long)B * H * N;
  return (size_t)(fa::ws_lse_offset(rows) + fa::ws_lse_offset(rows)) * sizeof(float);
}

int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) ||
      !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* Dws = static_cast<float*>(workspace);
  hipError_t e =
      (dtype == FA_BF16)
          ? fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, fa::kStagesGrad, s)
          : fa::launch_backward_f32((const float*)Q, (const float*)K, (const float*)V,
                                    (const float*)O, (const float*)dO, LSE, (float*)dQ,
                                    (float*)dK, (float*)dV, Dws, p, fa::kStagesGrad, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int N, int d,
                        float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_INVALID_ARG;
  const size_t need = fa_backward_workspace_bytes(B, H, N, d, dtype);
  if (need == 0 || need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return FA_ERR_MISALIGNED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = scratch_address(s, &ws);
  if (rc != FA_OK) return rc;
  // the same kernels as fa_backward, with the workspace in the scratch
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  float* Dws = static_cast<float*>(ws);
  hipError_t e =
      (dtype == FA_BF16)
          ? fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, Dws, p, fa::kStagesGrad, s)
          : fa::launch_backward_f32((const float*)Q, (const float*)K, (const float*)V,
                                    (const float*)O, (const float*)dO, LSE, (float*)dQ,
                                    (float*)dK, (float*)dV, Dws, p, fa::kStagesGrad, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_preprocess(const void* O, const void* dO, const float* LSE, void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d, int dtype,
                           void* stream) {
  int rc = check_sizes(B, H, N, d, dtype);
  if (rc != FA_OK) return rc;
  if (!O || !dO || !LSE) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(O) || !aligned16(dO) || !aligned16(LSE) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, 1.0f, false};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* Dws = static_cast<float*>(workspace);
  hipError_t e = (dtype == FA_BF16)
                     ? fa::launch_backward_bf16(nullptr, nullptr, nullptr, O, dO, LSE, nullptr,
                                                nullptr, nullptr, Dws, p, fa::kStagePre, s)
                     : fa::launch_backward_f32(nullptr, nullptr, nullptr, (const float*)O,
                                               (const float*)dO, LSE, nullptr, nullptr,
                                               nullptr, Dws, p, fa::kStagePre, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                     const void* workspace, size_t workspace_bytes, void* dK, void* dV, int B,
                     int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !dO || !dK || !dV) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dK) ||
      !aligned16(dV) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* Dws = const_cast<float*>(static_cast<const float*>(workspace));
  hipError_t e =
      (dtype == FA_BF16)
          ? fa::launch_backward_bf16(Q, K, V, nullptr, dO, nullptr, nullptr, dK, dV, Dws, p,
                                     fa::kStageDkDv, s)
          : fa::launch_backward_f32((const float*)Q, (const float*)K, (const float*)V, nullptr,
                                    (const float*)dO, nullptr, nullptr, (float*)dK, (float*)dV,
                                    Dws, p, fa::kStageDkDv, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_dq(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* workspace, size_t workspace_bytes, void* dQ, int B,
                   int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  int rc = check_common(B, H, N, d, scale, causal, dtype);
  if (rc != FA_OK) return rc;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_backward_workspace_bytes(B, H, N, d, dtype))
    return FA_ERR_NO_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  const fa::Problem p{B, H, N, d, scale, causal != 0};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* Dws = static_cast<float*>(workspace);
  hipError_t e =
      (dtype == FA_BF16)
          ? fa::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, nullptr, nullptr, Dws, p,
                                     fa::kStageDq, s)
          : fa::launch_backward_f32((const float*)Q, (const float*)K, (const float*)V,
                                    (const float*)O, (const float*)dO, LSE, (float*)dQ, nullptr,
                                    nullptr, Dws, p, fa::kStageDq, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
