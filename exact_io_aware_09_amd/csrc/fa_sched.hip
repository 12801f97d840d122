// fa_sched.hip -- balanced work schedules for block-sparse attention.
//
// Block-sparse attention ("FlashAttention and GPU memory", section 10; CS324
// notes, section 5.7) visits only the set 128 x 128 tiles of the mask, so its
// IO and FLOPs scale with the number of set tiles.  With one workgroup per
// tile row (forward, dQ) or tile column (dK/dV), a mask whose rows or
// columns hold very different numbers of set tiles -- a sliding window with a
// few global tokens, say -- leaves the whole work of a long row on one
// workgroup while the others have long finished.  The schedule cuts every row
// (column) longer than `seg` tiles into segments of at most `seg` tiles, one
// workgroup each, and lists the items longest first; a split row's segments
// write float32 partial results which the kernels below combine in a fixed
// order, so the results do not depend on timing.
//
// Host side: fa_sparse_schedule builds the schedule from a host copy of the
// mask; fa_sparse_workspace_bytes sizes the partial buffers.  Device side:
// merge_rows_kernel combines the forward's segment results (the merge of
// partial softmax states, CS324 notes exercises 3 and 7), sum_parts_kernel
// adds the segments' gradient shares.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "fa.h"
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kTile = 128;

// Entry e of a `longs` list: tile t, first slot s0, slot count ns; false if
// it would leave the schedule's sizes.
__device__ __forceinline__ bool long_entry(const int* longs, int e, int nb, int slots, int& t,
                                           int& s0, int& ns) {
  const const_int_ptr it = (const_int_ptr)longs + 4 * e;
  t = it[0];
  s0 = it[1];
  ns = it[2];
  return t >= 0 && t < nb && s0 >= 0 && ns >= 1 && s0 <= slots - ns;
}

// One row per D/4 lanes (a float4 each), 256 / (D/4) rows per workgroup;
// row index R = ((e * BH) + bh) * 128 + i.
//   LSE = M + ln sum_s e^{L_s - M},  O = sum_s e^{L_s - M} O_s / sum_s e^{L_s - M}
// with M = max_s L_s over the segments' log-sum-exps L_s; segments with
// L_s = -inf carry no weight.
template <int D>
__global__ __launch_bounds__(256)
void merge_rows_kernel(const float* __restrict__ part_o, const float* __restrict__ part_l,
                       const int* __restrict__ longs, int n_longs, int nb, int slots, int BH,
                       int N, bf16_t* __restrict__ O, float* __restrict__ LSE) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long long R = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  if (R >= (long long)n_longs * BH * kTile) return;
  const int e = (int)(R / ((long long)BH * kTile));
  const int bh = (int)((R / kTile) % BH), i = (int)(R % kTile);
  int t, s0, ns;
  if (!long_entry(longs, e, nb, slots, t, s0, ns)) return;
  const int query = t * kTile + i;
  if (query >= N) return;
  auto prow = [&](int s) { return ((size_t)(s0 + s) * BH + bh) * kTile + i; };
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_l[prow(s)]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float sum = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float Ls = part_l[prow(s)];
      if (Ls == -INFINITY) continue;
      const float wgt = expf(Ls - M);
      const float4 v = *reinterpret_cast<const float4*>(part_o + prow(s) * D + 4 * part);
      sum += wgt;
      acc.x = fmaf(wgt, v.x, acc.x);
      acc.y = fmaf(wgt, v.y, acc.y);
      acc.z = fmaf(wgt, v.z, acc.z);
      acc.w = fmaf(wgt, v.w, acc.w);
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const size_t orow = (size_t)bh * N + query;
  *reinterpret_cast<uint2*>(O + orow * D + 4 * part) =
      make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  if (part == 0) LSE[orow] = sum > 0.f ? M + logf(sum) : -INFINITY;
}

// Same rows: out = sum over the entry's slots, in slot order, rounded once.
template <int D>
__global__ __launch_bounds__(256)
void sum_parts_kernel(const float* __restrict__ part, const int* __restrict__ longs, int n_longs,
                      int nb, int slots, int BH, int N, bf16_t* __restrict__ out) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long long R = (long long)blockIdx.x * RPB + tid / TPR;
  const int lane4 = tid % TPR;
  if (R >= (long long)n_longs * BH * kTile) return;
  const int e = (int)(R / ((long long)BH * kTile));
  const int bh = (int)((R / kTile) % BH), i = (int)(R % kTile);
  int t, s0, ns;
  if (!long_entry(longs, e, nb, slots, t, s0, ns)) return;
  const int row = t * kTile + i;
  if (row >= N) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // (unrolled so that several loads are in flight; the sum stays in slot order)
#pragma unroll 8
  for (int s = 0; s < ns; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(
        part + (((size_t)(s0 + s) * BH + bh) * kTile + i) * D + 4 * lane4);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<uint2*>(out + ((size_t)bh * N + row) * D + 4 * lane4) =
      make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

template <int D>
long long combine_grid(int n_longs, int BH) {
  constexpr int RPB = 256 / (D / 4);
  const long long rows = (long long)n_longs * BH * kTile;
  return (rows + RPB - 1) / RPB;
}

}  // namespace

hipError_t launch_merge_rows(const float* part_o, const float* part_l, int slots, const int* longs,
                             int n_longs, void* O, float* LSE, const Problem& p,
                             hipStream_t stream) {
  if (n_longs <= 0) return hipSuccess;
  const int BH = p.B * p.H, nb = (p.N + kTile - 1) / kTile;
  auto run = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    const long long grid = combine_grid<D>(n_longs, BH);
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((merge_rows_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream, part_o,
                       part_l, longs, n_longs, nb, slots, BH, p.N, (bf16_t*)O, LSE);
    return hipGetLastError();
  };
  switch (p.d) {
    case 64: return run(std::integral_constant<int, 64>{});
    case 128: return run(std::integral_constant<int, 128>{});
    case 256: return run(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sum_parts(const float* part, int slots, const int* longs, int n_longs, void* out,
                            const Problem& p, hipStream_t stream) {
  if (n_longs <= 0) return hipSuccess;
  const int BH = p.B * p.H, nb = (p.N + kTile - 1) / kTile;
  auto run = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    const long long grid = combine_grid<D>(n_longs, BH);
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((sum_parts_kernel<D>), dim3((unsigned)grid), dim3(256), 0, stream, part,
                       longs, n_longs, nb, slots, BH, p.N, (bf16_t*)out);
    return hipGetLastError();
  };
  switch (p.d) {
    case 64: return run(std::integral_constant<int, 64>{});
    case 128: return run(std::integral_constant<int, 128>{});
    case 256: return run(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
}

bool read_schedule(const int* s, SchedView& v) {
  if (s == nullptr || s[FA_SCHED_MAGIC] != FA_SCHED_MAGIC_VALUE ||
      s[FA_SCHED_HEADER_INTS] != FA_SCHED_HEADER)
    return false;
  v.nb = s[FA_SCHED_NB];
  v.causal = s[FA_SCHED_CAUSAL];
  v.n_rows = s[FA_SCHED_N_ROWS];
  v.n_cols = s[FA_SCHED_N_COLS];
  v.row_slots = s[FA_SCHED_ROW_SLOTS];
  v.col_slots = s[FA_SCHED_COL_SLOTS];
  v.n_long_rows = s[FA_SCHED_N_LONG_ROWS];
  v.n_long_cols = s[FA_SCHED_N_LONG_COLS];
  v.off_rows = s[FA_SCHED_OFF_ROWS];
  v.off_cols = s[FA_SCHED_OFF_COLS];
  v.off_long_rows = s[FA_SCHED_OFF_LONG_ROWS];
  v.off_long_cols = s[FA_SCHED_OFF_LONG_COLS];
  v.off_lists = s[FA_SCHED_OFF_LISTS];
  v.list_len = s[FA_SCHED_LIST_LEN];
  v.total = s[FA_SCHED_TOTAL];
  if (v.nb < 1 || (v.causal != 0 && v.causal != 1)) return false;
  // every row and column has at least one item; a split one has >= 2 slots
  if (v.n_rows < v.nb || v.n_cols < v.nb || v.n_long_rows < 0 || v.n_long_rows > v.nb ||
      v.n_long_cols < 0 || v.n_long_cols > v.nb || v.row_slots < 2 * v.n_long_rows ||
      v.col_slots < 2 * v.n_long_cols || v.list_len < 0)
    return false;
  // the sections in order, each at a 4-int boundary, within the total
  const long long secs[5][2] = {{v.off_rows, 4LL * v.n_rows},
                                {v.off_cols, 4LL * v.n_cols},
                                {v.off_long_rows, 4LL * v.n_long_rows},
                                {v.off_long_cols, 4LL * v.n_long_cols},
                                {v.off_lists, (long long)v.list_len}};
  long long at = FA_SCHED_HEADER;
  for (const auto& sec : secs) {
    if (sec[0] < at || (sec[0] & 3) != 0) return false;
    at = sec[0] + sec[1];
  }
  return at <= v.total;
}

}  // namespace fa

namespace {

struct Item {
  int t, off, cnt, slotw;
};

// Items of one direction (rows or columns): lists[off[t] .. off[t+1]) holds
// the tiles of tile t; a list longer than `seg` is cut into the fewest
// segments of at most `seg` tiles, their lengths differing by at most one.
void cut(const std::vector<int>& off, int seg, std::vector<Item>& items,
         std::vector<int>& longs, int& slots) {
  const int nb = (int)off.size() - 1;
  for (int t = 0; t < nb; ++t) {
    const int T = off[t + 1] - off[t];
    if (T <= seg) {
      items.push_back({t, off[t], T, -1});
      continue;
    }
    const int ns = (T + seg - 1) / seg, q = T / ns, rem = T % ns;
    longs.insert(longs.end(), {t, slots, ns, 0});
    int at = off[t];
    for (int s = 0; s < ns; ++s) {
      const int cnt = q + (s < rem ? 1 : 0);
      items.push_back({t, at, cnt, 2 * (slots + s) + (s == 0 ? 1 : 0)});
      at += cnt;
    }
    slots += ns;
  }
  // longest first (ties in tile order): the long items start while the
  // short ones fill in behind them
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& b) { return a.cnt > b.cnt; });
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int fa_sparse_schedule(const int* block_mask, int N, int causal, int B, int H, int seg_tiles,
                       int* schedule, size_t schedule_ints, size_t* needed_ints) {
  if (block_mask == nullptr || needed_ints == nullptr || N < 1 || B < 1 || H < 1 ||
      (causal != 0 && causal != 1) || seg_tiles < 0)
    return FA_ERR_INVALID_ARG;
  const int nb = (N + 127) / 128;
  if ((long long)nb * nb > (1LL << 28)) return FA_ERR_UNSUPPORTED;  // offsets stay in int32
  std::vector<int> lists, roff(nb + 1), coff(nb + 1);
  for (int r = 0; r < nb; ++r) {
    roff[r] = (int)lists.size();
    const int hi = causal ? r : nb - 1;
    for (int u = 0; u <= hi; ++u)
      if (block_mask[(size_t)r * nb + u] != 0) lists.push_back(u);
  }
  roff[nb] = (int)lists.size();
  const long long nnz = roff[nb];
  for (int c = 0; c < nb; ++c) {
    coff[c] = (int)lists.size();
    for (int u = causal ? c : 0; u < nb; ++u)
      if (block_mask[(size_t)u * nb + c] != 0) lists.push_back(u);
  }
  coff[nb] = (int)lists.size();
  // default segment: the set tiles of all heads shared out over about 1024
  // workgroups at once (4 on each of the 256 CUs), at least 8 tiles
  long long seg = seg_tiles;
  if (seg == 0) {
    const long long work = (long long)B * H * nnz;
    seg = std::max(8LL, (work + 1023) / 1024);
  }
  if (seg > nb) seg = nb;
  std::vector<Item> rows, cols;
  std::vector<int> long_rows, long_cols;
  int row_slots = 0, col_slots = 0;
  cut(roff, (int)seg, rows, long_rows, row_slots);
  cut(coff, (int)seg, cols, long_cols, col_slots);
  const long long off_rows = FA_SCHED_HEADER;
  const long long off_cols = off_rows + 4LL * (long long)rows.size();
  const long long off_long_rows = off_cols + 4LL * (long long)cols.size();
  const long long off_long_cols = off_long_rows + (long long)long_rows.size();
  const long long off_lists = off_long_cols + (long long)long_cols.size();
  const long long total = off_lists + (((long long)lists.size() + 3) & ~3LL);
  if (total > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
  *needed_ints = (size_t)total;
  if (schedule == nullptr) return FA_OK;
  if (schedule_ints < (size_t)total) return FA_ERR_NO_WORKSPACE;
  int* s = schedule;
  std::fill(s, s + total, 0);
  s[FA_SCHED_MAGIC] = FA_SCHED_MAGIC_VALUE;
  s[FA_SCHED_HEADER_INTS] = FA_SCHED_HEADER;
  s[FA_SCHED_NB] = nb;
  s[FA_SCHED_CAUSAL] = causal;
  s[FA_SCHED_SEG] = (int)seg;
  s[FA_SCHED_N_ROWS] = (int)rows.size();
  s[FA_SCHED_N_COLS] = (int)cols.size();
  s[FA_SCHED_ROW_SLOTS] = row_slots;
  s[FA_SCHED_COL_SLOTS] = col_slots;
  s[FA_SCHED_N_LONG_ROWS] = (int)long_rows.size() / 4;
  s[FA_SCHED_N_LONG_COLS] = (int)long_cols.size() / 4;
  s[FA_SCHED_OFF_ROWS] = (int)off_rows;
  s[FA_SCHED_OFF_COLS] = (int)off_cols;
  s[FA_SCHED_OFF_LONG_ROWS] = (int)off_long_rows;
  s[FA_SCHED_OFF_LONG_COLS] = (int)off_long_cols;
  s[FA_SCHED_OFF_LISTS] = (int)off_lists;
  s[FA_SCHED_LIST_LEN] = (int)lists.size();
  s[FA_SCHED_TOTAL] = (int)total;
  s[FA_SCHED_NNZ] = (int)nnz;
  auto put = [&](long long at, const std::vector<Item>& items) {
    for (const Item& it : items) {
      s[at++] = it.t;
      s[at++] = it.off;
      s[at++] = it.cnt;
      s[at++] = it.slotw;
    }
  };
  put(off_rows, rows);
  put(off_cols, cols);
  std::copy(long_rows.begin(), long_rows.end(), s + off_long_rows);
  std::copy(long_cols.begin(), long_cols.end(), s + off_long_cols);
  std::copy(lists.begin(), lists.end(), s + off_lists);
  return FA_OK;
}

size_t fa_sparse_workspace_bytes(const int* schedule, int B, int H, int N, int d, int backward) {
  fa::SchedView v;
  if (!fa::read_schedule(schedule, v) || B < 1 || H < 1 || N < 1 ||
      v.nb != (N + 127) / 128 || (d != 64 && d != 128 && d != 256))
    return 0;
  const size_t tile = (size_t)B * H * 128;
  if (!backward)
    return align256((size_t)v.row_slots * tile * d * 4) + align256((size_t)v.row_slots * tile * 4);
  return align256(fa_backward_workspace_bytes(B, H, N, d, FA_BF16)) +
         align256((size_t)v.row_slots * tile * d * 4) +
         2 * align256((size_t)v.col_slots * tile * d * 4);
}

}  // extern "C"
