/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * What is computed (per batch b and head h, all N x d matrices row-major):
 *
 *   S   = scale * Q K^T                      (N x N, never stored)
 *   S_ij = -inf for j > i  when causal       (key j visible to query i iff j <= i)
 *   P   = softmax over each row of S         (never stored)
 *   O   = P V
 *   LSE_i = ln sum_j exp(S_ij)               (natural log, scaled + masked scores)
 *
 * This is standard attention as defined in "Lecture 8 . GPU Performance &
 * FlashAttention" (CS324 notes), section 5.1; the forward is computed tile by
 * tile with the online softmax of section 5.2 of those notes ("FlashAttention
 * and GPU memory", sections 07-08), so that only O and the per-row LSE reach
 * device memory.  The backward recomputes S and P tile by tile from Q, K and
 * LSE (CS324 notes section 5.4; "FlashAttention and GPU memory" section 09)
 * and returns the gradients of L = sum(dO * O):
 *
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Conventions shared by every entry point
 * --------------------------------------
 *  - Q, K, V, O, dO, dQ, dK, dV: contiguous [B, H, N, d] tensors of one
 *    element type (`dtype`): FA_BF16 (bfloat16, fp32 accumulation inside)
 *    or FA_F32 (float32 throughout).  LSE: contiguous float32 [B, H, N].
 *  - All pointers are DEVICE pointers, 16-byte aligned.  The caller owns
 *    every buffer; the library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is only enqueued; functions return once it is enqueued.
 *  - d must be 64, 128 or 256.  N >= 1 (any value; tails are masked),
 *    B >= 1, H >= 1; N*d <= 2^31 - 2^16 and B*H*N < 2^31.
 *  - `scale` must be finite and > 0 (the pages' scale is a positive factor,
 *    1/sqrt(d) in practice); `causal` is 0 or 1.
 *  - Errors are returned as codes (never thrown across the ABI); argument
 *    checks happen before anything is enqueued, so an error return means
 *    nothing was launched (except FA_ERR_HIP, reported by the launch itself).
 *  - No global mutable state: calls from several host threads are safe.
 *    Calls that write the same output buffers on different streams race,
 *    as any two kernels would.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, scale not finite and > 0, causal not 0/1 */
  FA_ERR_UNSUPPORTED = -2,  /* d not in {64,128,256}, unknown dtype, tensor too large */
  FA_ERR_MISALIGNED = -3,   /* a pointer is not 16-byte aligned */
  FA_ERR_NO_WORKSPACE = -4, /* workspace NULL or smaller than fa_backward_workspace_bytes() */
  FA_ERR_HIP = -5           /* a kernel launch reported an error */
};

/* Library version as an integer (major*10000 + minor*100 + patch). */
int fa_version(void);

/* Human-readable text for a return code; never NULL. */
const char* fa_strerror(int code);

/*
 * Forward pass.  Reads Q, K, V; writes O ([B,H,N,d], dtype) and LSE
 * ([B,H,N] float32, natural log).  Tiles Q into row blocks and streams K/V
 * blocks through on-chip memory with a running max / sum per row (CS324
 * notes sections 5.2-5.3, in the loop order of section 8.1's second
 * version: one Q block per workgroup, inner loop over K/V blocks).
 */
int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int H, int N, int d, float scale, int causal, int dtype,
               void* stream);

/*
 * Split-KV forward (the Flash-Decoding scheme of CS324 notes section 8.2):
 * the keys of every row are cut into `splits` contiguous ranges of
 * span = 64 * ceil(ceil(N / splits) / 64) keys (the last ranges may be
 * shorter or empty).  One workgroup per (head, query block, range) runs the
 * forward's tile loop over its range only, so that B*H*N/128 * splits
 * workgroups share the GPU when B*H*N/128 alone would leave it idle
 * (small batch, few heads).  Each writes a partial result -- the range's O,
 * normalised over the range (float32), and the range's log-sum-exp (-inf for
 * a row that sees no key of the range) -- to `workspace`, and a second
 * kernel merges the ranges of every row with the online-softmax merge
 * (exercises 3 and 7 of those notes; see fa_merge_partials).  O and LSE mean
 * exactly what fa_forward writes; the result differs from fa_forward's only
 * by rounding (the ranges are summed in float32 before O is rounded).
 *
 * splits: 1..256.  splits == 1 is fa_forward itself (workspace unused, may
 * be NULL; every dtype).  splits > 1 supports FA_BF16 only
 * (FA_ERR_UNSUPPORTED otherwise) and needs `workspace` of at least
 * fa_forward_split_workspace_bytes() bytes (contents ignored on entry):
 * partial outputs float32 [splits, B*H*N, d], then from the next 256-byte
 * boundary partial log-sum-exps float32 [splits, B*H*N].
 * fa_forward_split_workspace_bytes returns 0 for splits == 1 and for
 * invalid sizes.
 */
size_t fa_forward_split_workspace_bytes(int B, int H, int N, int d, int splits, int dtype);

int fa_forward_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     float scale, int causal, int splits, int dtype, void* stream);

/*
 * Merge of partial attention results over disjoint key sets (CS324 notes
 * exercises 3 and 7, section 8.2).  O_parts: float32 [splits, B*H*N, d],
 * part s's output for each row normalised over part s's keys; LSE_parts:
 * float32 [splits, B*H*N], part s's natural-log log-sum-exp L_s, -inf when
 * part s holds no key for the row (its O_parts row is then not read).  With
 * M = max_s L_s, writes LSE = M + ln sum_s e^{L_s - M} and
 * O = sum_s e^{L_s - LSE} O_s, rounded to `dtype` (FA_BF16 or FA_F32);
 * a row whose parts are all empty gets O = 0, LSE = -inf.  This is the
 * merge a sequence-parallel caller applies to the results of different
 * devices.  splits: 1..256; d in {64, 128, 256}; pointers 16-byte aligned.
 */
int fa_merge_partials(const float* O_parts, const float* LSE_parts, int splits, void* O,
                      float* LSE, int B, int H, int N, int d, int dtype, void* stream);

/*
 * Block-sparse attention (block-sparse FlashAttention, "FlashAttention and
 * GPU memory" section 10; CS324 notes section 5.7, where causal attention is
 * the same idea: blocks wholly in a query block's future are neither read
 * nor computed).  block_mask: device int32 [nb, nb], nb = ceil(N / 128),
 * row-major, shared by every (b, h): query i may see key j only if
 * block_mask[i / 128][j / 128] != 0, and, when causal, j <= i.  The kernels
 * visit only the set 128 x 128 tiles (query blocks and key blocks are one
 * tile wide), so the work and the K/V (Q/dO) traffic scale with the number
 * of set tiles.  A row that sees no key has nothing to normalise: its O is
 * 0, its LSE -inf, its dQ 0, and it adds nothing to dK, dV.
 *
 * fa_forward_sparse writes O and LSE as fa_forward does; fa_backward_sparse
 * takes the workspace of fa_backward (fa_backward_workspace_bytes) and
 * writes dQ, dK, dV completely.  Both need the same mask, FA_BF16
 * (FA_ERR_UNSUPPORTED otherwise) and a 16-byte aligned block_mask; the mask
 * is only read.  All-ones masks give fa_forward / fa_backward's results
 * bit for bit.
 */
int fa_forward_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      const int* block_mask, int B, int H, int N, int d, float scale, int causal,
                      int dtype, void* stream);

int fa_backward_sparse(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, const int* block_mask, void* dQ, void* dK, void* dV,
                       void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                       float scale, int causal, int dtype, void* stream);

/*
 * Balanced block-sparse attention.  fa_forward_sparse / fa_backward_sparse
 * run one workgroup per tile row (forward, dQ) and per tile column (dK, dV),
 * so a mask whose rows or columns differ much in length -- a sliding window
 * with global tokens -- leaves a long row's whole work on one workgroup.
 * The calls below take a schedule, built once per mask on the host, that
 * cuts every row and column longer than `seg` set tiles into segments of at
 * most `seg` tiles, one workgroup each, longest first; the segments of a
 * split row write float32 partial results that small kernels then combine
 * in a fixed order (forward: the merge of partial softmax results, CS324
 * notes exercises 3 and 7; gradients: plain sums).  The kernels walk each
 * item's list of tiles instead of scanning the mask.  Results are
 * deterministic; they equal fa_forward_sparse / fa_backward_sparse's bit
 * for bit when no row or column is split and to rounding otherwise.
 *
 * fa_sparse_schedule (host only; launches nothing): block_mask is a HOST
 * int32 [nb, nb] array with fa_forward_sparse's meaning, nb = ceil(N/128).
 * seg_tiles: the most tiles one item visits, >= 1, or 0 for the default
 * max(8, ceil(B*H*(set tiles in reach) / 1024)).  Writes the number of ints
 * the schedule takes to *needed_ints; writes the schedule itself only when
 * `schedule` is non-NULL and schedule_ints >= that number (otherwise
 * FA_ERR_NO_WORKSPACE; NULL schedule: FA_OK, size only).  The schedule
 * depends on the mask, N, causal and seg only (B and H enter the default
 * seg); its layout is the FA_SCHED_* header below followed by the items.
 *
 * fa_sparse_workspace_bytes: workspace of the balanced forward (backward =
 * 0: partial O and LSE of the split rows) or backward (backward = 1: the
 * workspace of fa_backward followed by the partial dQ, dK and dV of the
 * split rows and columns); 0 for an invalid schedule or sizes, and 0 for a
 * forward whose schedule splits nothing (workspace may then be NULL).
 *
 * fa_forward_sparse_balanced / fa_backward_sparse_balanced: as
 * fa_forward_sparse / fa_backward_sparse, with `schedule` the host copy
 * (read for the launch sizes and checked: FA_ERR_INVALID_ARG if it is not a
 * schedule of this N and causal) and `schedule_dev` a device copy of the
 * same ints (16-byte aligned; read by the kernels, which keep every access
 * inside the sizes of the host copy's header, but a device copy that differs
 * from the host copy gives undefined values).  FA_BF16 only.  Calls that
 * share a workspace must not overlap.
 */
#define FA_SCHED_MAGIC 0
#define FA_SCHED_HEADER_INTS 1
#define FA_SCHED_NB 2
#define FA_SCHED_CAUSAL 3
#define FA_SCHED_SEG 4
#define FA_SCHED_N_ROWS 5       /* row items (4 ints: tile, list offset, count, slot word) */
#define FA_SCHED_N_COLS 6       /* column items */
#define FA_SCHED_ROW_SLOTS 7    /* partial-result slots of split rows */
#define FA_SCHED_COL_SLOTS 8
#define FA_SCHED_N_LONG_ROWS 9  /* split rows (4 ints: tile, first slot, slots, 0) */
#define FA_SCHED_N_LONG_COLS 10
#define FA_SCHED_OFF_ROWS 11    /* int offsets of the sections */
#define FA_SCHED_OFF_COLS 12
#define FA_SCHED_OFF_LONG_ROWS 13
#define FA_SCHED_OFF_LONG_COLS 14
#define FA_SCHED_OFF_LISTS 15
#define FA_SCHED_LIST_LEN 16
#define FA_SCHED_TOTAL 17
#define FA_SCHED_NNZ 18         /* set tiles in reach (causal: at or below the diagonal) */
#define FA_SCHED_HEADER 20
#define FA_SCHED_MAGIC_VALUE 0x46534221

int fa_sparse_schedule(const int* block_mask, int N, int causal, int B, int H, int seg_tiles,
                       int* schedule, size_t schedule_ints, size_t* needed_ints);

size_t fa_sparse_workspace_bytes(const int* schedule, int B, int H, int N, int d, int backward);

int fa_forward_sparse_balanced(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const int* schedule, const int* schedule_dev, void* workspace,
                               size_t workspace_bytes, int B, int H, int N, int d, float scale,
                               int causal, int dtype, void* stream);

int fa_backward_sparse_balanced(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, const int* schedule,
                                const int* schedule_dev, void* dQ, void* dK, void* dV,
                                void* workspace, size_t workspace_bytes, int B, int H, int N,
                                int d, float scale, int causal, int dtype, void* stream);

/*
 * Attention with dropout on the weights (the fused dropout of "FlashAttention
 * and GPU memory", section 07: applied after the softmax, before the product
 * with V).  No mask is stored: the forward keeps only the generator's key
 * (`seed`), and the backward regenerates the same draws ("FlashAttention and
 * GPU memory", section 09; CS324 notes, section 5.4).
 *
 *   Z_ij  = [u_ij < t],  t = round((1 - p_drop) * 256)   (keep mask)
 *   O     = (P o Z) V * 256 / t
 *   LSE   as fa_forward (the softmax's normaliser; dropout does not touch it)
 *
 * u_ij (0..255) is the draw of query i and key j of head b*H + h: byte
 * (j mod 4) of word (i mod 4) of Philox4x32-10 (Salmon et al., "Parallel
 * random numbers: as easy as 1, 2, 3", SC 2011) at counter
 * (j / 4, i / 4, b*H + h, 0) under key (seed mod 2^32, seed / 2^32).  So the
 * drop probability actually applied is 1 - t/256 (p_drop rounded to a
 * multiple of 1/256), and the kept weights are scaled so that the expected
 * output is P V exactly.  The draws depend only on (seed, b, h, i, j): the
 * same seed gives the same mask for any causal flag and launch
 * configuration.
 *
 * fa_backward_dropout returns the gradients of L = sum(dO * O) for that O
 * with the mask fixed:
 *   dV = (P o Z)^T dO * 256/t,  dP = (dO V^T) o Z * 256/t,
 *   D_i = sum_k dO_ik O_ik,  dS = P o (dP - D),  dQ = scale dS K,
 *   dK = scale dS^T Q;
 * it takes fa_backward's workspace and writes dQ, dK, dV completely.  Pass
 * the seed and p_drop of the forward that produced O and LSE.
 *
 * p_drop: finite, 0 <= p_drop < 1 with t >= 1 (FA_ERR_INVALID_ARG
 * otherwise); p_drop = 0 gives fa_forward / fa_backward's results bit for
 * bit.  FA_BF16 only (FA_ERR_UNSUPPORTED otherwise).  Other arguments and
 * errors as fa_forward / fa_backward.
 */
int fa_forward_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int H, int N, int d, float scale, int causal, float p_drop,
                       unsigned long long seed, int dtype, void* stream);

int fa_backward_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                        const float* LSE, void* dQ, void* dK, void* dV, void* workspace,
                        size_t workspace_bytes, int B, int H, int N, int d, float scale,
                        int causal, float p_drop, unsigned long long seed, int dtype,
                        void* stream);

/*
 * Attention forward in 8-bit floating point with block quantisation (the FP8
 * variant of the third version of the kernel: CS324 notes, section 8.1;
 * "FlashAttention and GPU memory", section 11).
 *
 * Format: OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite 448), round to nearest even.  Every block of 32 elements
 * along a contraction axis shares a power-of-two scale 2^e, stored as the
 * byte e + 127; e is the smallest integer with max|x| <= 448 * 2^e (0 for an
 * all-zero block), so an element x is stored as E4M3(x / 2^e) and never
 * overflows.
 *
 * fa_quantize_fp8 converts a bfloat16 [B,H,N,d] tensor:
 *   layout FA_FP8_ROWS (Q and K): X8 [B,H,N,d] bytes, Xs [B,H,Np,d/32]; block
 *     = 32 consecutive head dims of a row (rows N .. Np-1 of Xs, padding,
 *     hold 127: the exponent of an all-zero block).
 *   layout FA_FP8_KEYS (V): X8 [B,H,d,Np] bytes (V transposed: keys
 *     contiguous, padding 0), Xs [B,H,Np/32,d]; block = 32 consecutive keys
 *     of one head dim.
 * Np = N rounded up to a multiple of 64.
 * fa_fp8_bytes / fa_fp8_scale_bytes give the sizes of X8 and Xs (0 for
 * invalid sizes or layout).
 *
 * fa_forward_fp8 computes O (bfloat16 [B,H,N,d]) and LSE (float32 [B,H,N])
 * of attention over the dequantised Q, K, V (Q and K in FA_FP8_ROWS, V in
 * FA_FP8_KEYS): S = scale Q K^T with the scales applied by the matrix
 * instructions, fp32 accumulation, the online softmax in fp32, and the
 * weights rounded to E4M3 (times 2^8) for the product with V.  Relative to
 * attention of the dequantised inputs, O differs by at most the E4M3
 * rounding of the weights (2^-4 relative, 2^-18 absolute per weight) plus the
 * bfloat16 rounding of O.
 *
 * All pointers 16-byte aligned device memory; other arguments and errors as
 * fa_forward (inputs are bfloat16 for fa_quantize_fp8).
 */
enum { FA_FP8_ROWS = 0, FA_FP8_KEYS = 1 };

size_t fa_fp8_bytes(int B, int H, int N, int d, int layout);

size_t fa_fp8_scale_bytes(int B, int H, int N, int d, int layout);

int fa_quantize_fp8(const void* X, void* X8, void* Xs, int B, int H, int N, int d, int layout,
                    void* stream);

int fa_forward_fp8(const void* Q8, const void* Qs, const void* K8, const void* Ks, const void* V8,
                   const void* Vs, void* O, float* LSE, int B, int H, int N, int d, float scale,
                   int causal, void* stream);

/*
 * Bytes of device workspace fa_backward needs: two float32 vectors of one
 * value per query row (B*H*N rows), each starting on a 256-byte boundary --
 * -D_i = -sum_k dO_ik O_ik (D is the vector of CS324 notes section 5.4;
 * stored negated so that it can start the dP accumulation) and
 * LSE_i * log2(e).  Returns 0 for invalid sizes.
 */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward pass.  Reads Q, K, V, O, dO and the forward's LSE; writes dQ, dK,
 * dV (all [B,H,N,d], dtype) completely (no accumulation into the caller's
 * buffers).  `workspace` (device memory of at least
 * fa_backward_workspace_bytes(), contents ignored on entry) receives -D and
 * LSE * log2(e).  Two kernels are enqueued on `stream`, in order: a dQ
 * kernel (one Q block per workgroup, loop over K/V blocks) that also forms
 * D = rowsum(dO * O) and LSE * log2(e) for its rows and stores them in
 * `workspace`; then a dK/dV kernel (one K/V block per workgroup, loop over
 * Q blocks) that reads them.  No atomics: results are bitwise reproducible
 * run to run.
 */
int fa_backward(const void* Q, const void* K, const void* V, const void* O,
                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, float scale, int causal, int dtype,
                void* stream);

/*
 * fa_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The two workspace vectors live in a
 * device scratch array compiled into the library, FA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, held from module load until the process ends; problems
 * whose fa_backward_workspace_bytes() exceeds it (more than about 2.09
 * million query rows B*H*N) return FA_ERR_NO_WORKSPACE before anything is
 * enqueued.  Nothing is allocated or freed: the call enqueues the same two
 * kernels as fa_backward (identical results, bit for bit) on `stream`, which
 * must belong to the current device (FA_ERR_INVALID_ARG otherwise).  The
 * scratch address is looked up once per device on the first call.  Every
 * call on a GPU shares that GPU's scratch and leaves its contents behind:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller; a call needs no cleared scratch (the dQ
 * kernel writes every value the dK/dV kernel reads).  Other arguments and
 * errors as fa_backward.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                        int B, int H, int N, int d, float scale, int causal, int dtype,
                        void* stream);

/*
 * The stages of fa_backward as separate calls, for callers that want to
 * schedule or time them individually.  Enqueuing fa_backward_dq and then
 * fa_backward_dkdv on one stream computes exactly what fa_backward computes
 * (the same kernels, bit for bit).
 *
 * fa_backward_dq:   reads Q, K, V, O, dO and LSE; writes dQ, and writes -D
 *   (D_i = sum_k dO_ik O_ik, float32: the identity of CS324 notes section
 *   5.4 that replaces sum_j P_ij dP_ij) and LSE * log2(e) into `workspace`.
 * fa_backward_dkdv: reads Q, K, V, dO and the two workspace vectors; writes
 *   dK, dV.  The workspace must have been filled by fa_backward_dq or
 *   fa_backward_preprocess on the same O, dO and LSE, enqueued earlier.
 * fa_backward_preprocess: the two workspace vectors alone (a streaming pass
 *   over O, dO and LSE), for callers that run fa_backward_dkdv without
 *   fa_backward_dq.  Its D may differ from fa_backward_dq's in the last bits
 *   (different summation order).
 * Errors and argument rules are those of fa_backward.
 */
int fa_backward_preprocess(const void* O, const void* dO, const float* LSE, void* workspace,
                           size_t workspace_bytes, int B, int H, int N, int d, int dtype,
                           void* stream);

int fa_backward_dq(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* workspace, size_t workspace_bytes, void* dQ, int B,
                   int H, int N, int d, float scale, int causal, int dtype, void* stream);

int fa_backward_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                     const void* workspace, size_t workspace_bytes, void* dK, void* dV, int B,
                     int H, int N, int d, float scale, int causal, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
