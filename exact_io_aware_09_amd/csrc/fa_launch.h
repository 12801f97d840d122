// fa_launch.h -- host-side launchers behind the C ABI (internal, C++ linkage).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct Problem {
  int B, H, N, d;
  float scale;
  bool causal;
};

// Key ranges of the split forward: `span` keys each (a multiple of 64, so
// of every K/V block size), the last ranges possibly short or empty.
inline int split_span(int N, int splits) {
  const int per = (N + splits - 1) / splits;
  return (per + 63) / 64 * 64;
}

struct SplitArgs {
  int span = 0, splits = 1;
  float* Opart = nullptr;  // [splits, B*H*N, d] float32
  float* Lpart = nullptr;  // [splits, B*H*N] float32
};

// Block-sparse attention: int32 tile mask [nb, nb] over 128 x 128 tiles of
// (query rows, keys), shared by every head; nonzero = the tile is computed.
//
// Balanced schedule (rows != nullptr; the mask is then not read): the
// forward and dQ kernels take work item `rank` of `rows`, the dK/dV kernel
// item `rank` of `cols`, instead of tile row / column `rank`.  An item is 4
// ints: tile index t, offset and count of its run of tile indices in
// `lists` (increasing; the tiles of row t, or the query tiles of column t,
// that the item visits), and the slot word: -1 when the item is the whole
// row (column) and writes the final result, else 2 * slot + (1 for the
// first segment of its row), and the item writes float32 partial results
// to that slot of the part_* buffers ([slot][B*H][128][d], LSE parts
// [slot][B*H][128]) for the merge kernels.
struct SparseArgs {
  const int* mask = nullptr;
  int nb = 0;
  const int* rows = nullptr;
  const int* cols = nullptr;
  int n_rows = 0, n_cols = 0;  // items in rows, cols
  const int* lists = nullptr;
  int list_len = 0;
  int row_slots = 0, col_slots = 0;
  float* part_o = nullptr;   // forward: O of a segment, normalised over it
  float* part_l = nullptr;   // forward: the segment's log-sum-exp
  float* part_dq = nullptr;  // dQ of a segment (scale applied)
  float* part_dk = nullptr;  // dK of a segment (scale applied)
  float* part_dv = nullptr;  // dV of a segment
  bool on() const { return mask != nullptr || rows != nullptr; }
};

// Header of a balanced schedule (host copy), read and checked for internal
// consistency by read_schedule.
struct SchedView {
  int nb, causal, n_rows, n_cols, row_slots, col_slots, n_long_rows, n_long_cols;
  int off_rows, off_cols, off_long_rows, off_long_cols, off_lists, list_len, total;
};
bool read_schedule(const int* schedule, SchedView& v);

// Rows of the merge kernels: for entry e of `longs` (4 ints: tile t, first
// slot, number of slots, unused) and head bh, rows t*128 .. t*128+127 (< N).
hipError_t launch_merge_rows(const float* part_o, const float* part_l, int slots, const int* longs,
                             int n_longs, void* O, float* LSE, const Problem& p,
                             hipStream_t stream);
// Sum of the float32 partial gradients of every entry of `longs`, in slot
// order, into the bf16 gradient rows.
hipError_t launch_sum_parts(const float* part, int slots, const int* longs, int n_longs, void* out,
                            const Problem& p, hipStream_t stream);

// Dropout on the attention weights: 64-bit generator key (k0 low word), keep
// threshold t in 1..256 on the 8-bit draws, kept weights scaled by 256 / t.
struct DropArgs {
  uint32_t k0 = 0, k1 = 0;
  int thresh = 256;
  float scale = 1.f;  // 256 / t
  float keep = 1.f;   // t / 256
};

// bfloat16 inputs, fp32 accumulation on the matrix cores.
hipError_t launch_forward_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const Problem& p, hipStream_t stream, SparseArgs sp = {});
// With dropout (dense, not split, not sparse).
hipError_t launch_forward_dropout_bf16(const void* Q, const void* K, const void* V, void* O,
                                       float* LSE, const Problem& p, const DropArgs& dr,
                                       hipStream_t stream);
// Split forward: partial results of every key range into Opart / Lpart;
// then the merge of `splits` partial results into O (bf16 or float32) and
// LSE.
hipError_t launch_forward_split_bf16(const void* Q, const void* K, const void* V, const Problem& p,
                                     int splits, float* Opart, float* Lpart, hipStream_t stream);
hipError_t launch_merge(const float* Opart, const float* Lpart, int splits, void* O, float* LSE,
                        const Problem& p, bool bf16, hipStream_t stream);

// Backward workspace: -D (one float per query row), then, starting at float
// index ws_lse_offset(rows), LSE * log2(e) (one float per row).
inline long long ws_lse_offset(long long rows) { return (rows + 63) & ~63LL; }

// Backward stages, enqueued in this order when several bits are set:
//   kStagePre   D = rowsum(dO * O) and LSE * log2(e) into the workspace;
//   kStageDq    dQ; also forms both workspace vectors and stores them;
//   kStageDkDv  dK, dV; reads both vectors from the workspace.
enum : unsigned { kStagePre = 1u, kStageDq = 2u, kStageDkDv = 4u, kStagesGrad = 6u };

// A non-null sp.mask selects the block-sparse instantiations, a non-null dr
// the dropout ones (not both).
hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                float* Dws, const Problem& p, unsigned stages, hipStream_t stream,
                                SparseArgs sp = {}, const DropArgs* dr = nullptr);

// FP8 (E4M3) with power-of-two block scales.  Q and K: [B,H,N,d] bytes and
// [B,H,Np,d/32] scale bytes (blocks of 32 head dims; rows padded to
// Np = fp8_keys_padded(N)).  V: transposed [B,H,d,Np] bytes, keys padded
// with zeros, and [B,H,Np/32,d] scale bytes (blocks of 32 keys).
inline int fp8_keys_padded(int N) { return (N + 63) / 64 * 64; }
hipError_t launch_quantize_fp8(const void* X, void* X8, void* Xs, const Problem& p, bool keys,
                               hipStream_t stream);
hipError_t launch_forward_fp8(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                              const void* V8, const void* Vs, void* O, float* LSE,
                              const Problem& p, hipStream_t stream);

// Head dim 256: the same kernels, built in their own units (fa_*_d256.hip)
// with the matrix instructions' accumulators kept in VGPRs; the launchers
// above forward d = 256 to these.
hipError_t launch_forward_bf16_d256(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, const Problem& p, hipStream_t stream,
                                    SparseArgs sp);
hipError_t launch_forward_dropout_bf16_d256(const void* Q, const void* K, const void* V, void* O,
                                            float* LSE, const Problem& p, const DropArgs& dr,
                                            hipStream_t stream);
hipError_t launch_forward_split_bf16_d256(const void* Q, const void* K, const void* V,
                                          const Problem& p, int splits, float* Opart, float* Lpart,
                                          hipStream_t stream);
hipError_t launch_backward_bf16_d256(const void* Q, const void* K, const void* V, const void* O,
                                     const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                     float* Dws, const Problem& p, unsigned stages,
                                     hipStream_t stream, SparseArgs sp, const DropArgs* dr);
// Head dim 128 without the causal mask: the backward built with the same
// VGPR-form matrix instructions (its dK/dV runs one wavefront per SIMD).
hipError_t launch_backward_bf16_d128nc(const void* Q, const void* K, const void* V, const void* O,
                                       const void* dO, const float* LSE, void* dQ, void* dK,
                                       void* dV, float* Dws, const Problem& p, unsigned stages,
                                       hipStream_t stream, SparseArgs sp, const DropArgs* dr);
hipError_t launch_forward_fp8_d256(const void* Q8, const void* Qs, const void* K8, const void* Ks,
                                   const void* V8, const void* Vs, void* O, float* LSE,
                                   const Problem& p, hipStream_t stream);

// float32 throughout (vector ALU).
hipError_t launch_forward_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                              const Problem& p, hipStream_t stream);
hipError_t launch_backward_f32(const float* Q, const float* K, const float* V, const float* O,
                               const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                               float* Dws, const Problem& p, unsigned stages, hipStream_t stream);

}  // namespace fa
