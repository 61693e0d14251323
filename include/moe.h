/*
 * moe.h - C ABI of an MI355X (gfx950) library for one GPU's share of an expert-parallel
 * Mixture-of-Experts layer:  route -> permute -> grouped SwiGLU FFN -> combine.
 *
 * The operation is the one the "Expert Parallelism" tutorial page describes in section 1
 * (What is it?: E expert FFNs per layer, each token routed to k of them) and section 4
 * (The All-to-All: the router names each token's experts; tokens are sorted by destination
 * expert and counted so that every expert holds a contiguous block of rows; a grouped GEMM
 * runs every expert over its rows; results return to the original token order and the k
 * expert outputs of a token are summed with their gate weights). On one GPU the exchange
 * steps are the identity, so dispatch is the expert sort and combine is its inverse.
 *
 * Conventions shared by every call
 *  - Memory: every pointer argument is a device pointer allocated by the caller (the
 *    library never allocates or frees device memory and keeps no per-call state). Buffers
 *    must not overlap unless stated.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call
 *    only enqueues work and returns; it never synchronises. Results are valid once the
 *    stream has reached that point. Prefill-sized calls of moe_grouped_ffn with bf16 weights
 *    (and the moe_layer calls that make them) may run the experts with few rows on a second
 *    stream, one that the library creates for each (device, caller stream) on first use and
 *    keeps until the process ends (for at most 64 such pairs per process; calls on further
 *    caller streams run on `stream` alone, with results equal up to rounding): it
 *    waits on an event recorded on `stream` at the start of
 *    the call, and `stream` waits on an event recorded on it at the end, so everything
 *    enqueued on `stream` afterwards sees the call's results, and the call can be captured in
 *    a graph. Calls on one caller stream must not be enqueued from several threads at once
 *    (they share that stream's two events).
 *  - Errors: all arguments are checked on the host before anything is enqueued; on any
 *    error nothing is enqueued and a status other than MOE_OK is returned. A failed kernel
 *    launch returns MOE_ERR_HIP. Device-side faults surface at the caller's next
 *    synchronisation. Device-resident index data produced by one call and consumed by
 *    another (ids, offsets, maps) must be what the producing call wrote; kernels clamp such
 *    indices so that corrupt values never address memory out of bounds, but the results
 *    are then unspecified.
 *  - Sizes: T tokens, E experts, k experts per token, d hidden size, d_ff expert width,
 *    R = T*k routed rows. Limits: 0 <= T, 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E,
 *    MOE_MAX_TOPK), T*k*max(d, d_ff) < 2^31. T = 0 is a valid empty call.
 *  - Alignment: every pointer 16-byte aligned.
 *  - Determinism: no floating-point atomics; repeated calls give bit-identical results.
 *
 * Number formats (moe_dtype_t): fp32, bf16, and OCP fp8 e4m3fn (1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, max 448) for weights only; and, for weights only,
 * MOE_BF16_BLOCKED and MOE_FP8_E4M3FN_BLOCKED: bf16 / fp8 e4m3fn values with each [N, K] matrix
 * (K its contraction axis) stored in blocks of 8 rows x 128 bytes (64 bf16 or 128 fp8
 * contraction elements), each block 1 KB contiguous: [N/8][K/64][8][64] for bf16,
 * [N/8][K/128][8][128] for fp8 (moe_block_weights writes them from the row-major layout). The
 * grouped FFN's tiles load a step of 8 weight rows x 128 bytes at a time, so in these layouts
 * each load reads one contiguous kilobyte instead of 128 bytes of each of 8 rows a row apart;
 * the results are bit-identical to the row-major formats with the same weight values (fp8
 * block scales keep their layout).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, size out of range, bad combination */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than the *_workspace_size */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3FN = 2,
  MOE_BF16_BLOCKED = 3,       /* weights only */
  MOE_FP8_E4M3FN_BLOCKED = 4  /* weights only */
} moe_dtype_t;

#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32

/* Text for a status code (static storage; never NULL). */
const char* moe_status_string(moe_status_t status);

/*
 * moe_route - router output to top-k experts and gate weights (tutorial page, section 4:
 * the router's per-token choice of experts; section 1: each token goes to k of E experts;
 * section 4, combine: the weights of the weighted sum).
 *
 *   logits     [T, E] fp32, row-major, finite (non-finite values give unspecified ids).
 *   topk_ids   [T, k] int32 out: for each token the k largest logits in descending order;
 *              equal logits go to the lower expert index (+0.0 equals -0.0).
 *   topk_gates [T, k] fp32 out: softmax over the k chosen logits,
 *              g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) (equal to the full softmax
 *              renormalised over the top k); sums to 1 within k * 2^-23.
 *   counts     [E] int32 out, or NULL: number of rows routed to each expert (the histogram
 *              of topk_ids; overwritten, not accumulated).
 */
moe_status_t moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                       float* topk_gates, int32_t* counts, void* stream);

/*
 * moe_route_gemm - the router's scores and the top-k gating in one launch, with no round trip
 * of the logits through memory (tutorial page, section 4: the router decides each token's
 * destination experts; section 1: each token goes to k of E experts; the scores are the
 * token's hidden state times one weight row per expert).
 *
 *   x          [T, d] bf16, row-major (the tokens' hidden states).
 *   w_router   [E, d] bf16, row-major (one row per expert, contraction-contiguous).
 *   logits     [T, E] fp32 out, or NULL: logits[t, e] = sum_i x[t, i] * w_router[e, i], exact
 *              products summed in fp32 (the order of that sum is the kernel's own).
 *   topk_ids, topk_gates, counts: as moe_route, computed from these fp32 logits (the same
 *              selection and gates moe_route gives on them).
 *   workspace  >= moe_route_gemm_workspace_size(T, E, k) bytes, 16-byte aligned (batches of
 *              up to 1024 tokens split the contraction over several workgroups and keep fp32
 *              partial scores there; larger batches need none and may pass NULL).
 *   Requires x_dtype = w_dtype = MOE_BF16, E <= 256 and d a multiple of 32
 *   (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status_t moe_route_gemm(const void* x, moe_dtype_t x_dtype, const void* w_router,
                            moe_dtype_t w_dtype, int T, int E, int k, int d, float* logits,
                            int32_t* topk_ids, float* topk_gates, int32_t* counts,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_route_gemm needs (0 for invalid sizes or large batches). */
size_t moe_route_gemm_workspace_size(int T, int E, int k);

/* Bytes of workspace moe_permute needs (0 is possible; then workspace may be NULL). */
size_t moe_permute_workspace_size(int T, int E, int k);

/*
 * moe_permute - sort the T*k assignments by destination expert, count them and copy every
 * token's row into expert-contiguous order (tutorial page, section 4, dispatch: sort by
 * destination expert, count per destination, contiguous rows per expert; section 9: unsorted
 * rows mean uncoalesced access).
 *
 *   x              [T, d] in x_dtype (MOE_F32 or MOE_BF16), row-major.
 *   topk_ids       [T, k] int32, each in [0, E) (as written by moe_route).
 *   counts         [E] int32 out: rows per expert.
 *   offsets        [E+1] int32 out: exclusive scan of counts; offsets[E] = T*k.
 *   sorted_to_flat [T*k] int32 out: sorted row r holds flat assignment i = t*k + j.
 *   flat_to_sorted [T*k] int32 out: inverse permutation of sorted_to_flat.
 *   x_sorted       [T*k, d] in x_dtype out: x_sorted[r] = x[sorted_to_flat[r] / k] (a bit
 *                  copy). Within one expert, rows are in increasing flat index (stable sort).
 *   workspace      >= moe_permute_workspace_size(T, E, k) bytes, 16-byte aligned.
 *   Requires d*sizeof(x_dtype) to be a multiple of 16.
 */
moe_status_t moe_permute(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids, int T,
                         int E, int k, int d, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute_noalloc - moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): no workspace
 * argument, and no allocation of any kind. Its scratch (the per-tile histograms and bases,
 * moe_permute_workspace_size(T, E, k) bytes) is a static device array of
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4 MiB) that each GPU holds from the first call on that
 * GPU until the process ends; sizes whose workspace would exceed it return MOE_ERR_WORKSPACE
 * before anything is enqueued (with E = 256 that is T*k above 1,048,576 assignments). The array keeps the last
 * call's contents and needs no clearing (every entry read is written first within the call).
 * All calls on one GPU share the array: calls that overlap on one GPU (on different streams,
 * without ordering between them) race and give undefined results. Arguments, outputs and
 * other errors as moe_permute; the first call on a GPU also looks up the array's device
 * address (MOE_ERR_HIP if that fails).
 */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status_t moe_permute_noalloc(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids,
                                 int T, int E, int k, int d, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                                 void* stream);

/*
 * moe_expert_capacity - ceil(C * T * k / E), the per-expert capacity for a capacity factor
 * C = factor_percent / 100 (tutorial page, section 5, mitigation 1: capacity = C x tokens / E,
 * here counting the T*k assignments; section 10, exercise D sweeps C from 1.0 to 2.0). Exact
 * integer arithmetic; returns -1 if T < 0, E < 1, k < 1 or factor_percent < 0, and INT_MAX if
 * the value does not fit an int.
 */
int moe_expert_capacity(int T, int E, int k, int factor_percent);

/*
 * moe_permute_capped - moe_permute with a capacity factor (same page, section 5, mitigation
 * 1: the excess of an over-full expert is dropped and passes the expert by). Each expert
 * keeps its first `capacity` assignments in flat order (capacity >= 0, else
 * MOE_ERR_INVALID_ARG):
 *   counts         [E] out: kept rows per expert, min(assignments, capacity).
 *   offsets        [E+1] out: exclusive scan of counts; offsets[E] = kept rows <= T*k.
 *   sorted_to_flat entries [0, offsets[E]) are written, the rest are left untouched.
 *   flat_to_sorted [T*k] out: the row of each kept assignment, -1 for a dropped one.
 *   x_sorted       rows [0, offsets[E]) are written.
 * moe_grouped_ffn then works on the kept rows only (it takes its rows from offsets) and
 * moe_combine skips the dropped slots. Other arguments as moe_permute.
 */
moe_status_t moe_permute_capped(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids,
                                int T, int E, int k, int d, int capacity, int32_t* counts,
                                int32_t* offsets, int32_t* sorted_to_flat,
                                int32_t* flat_to_sorted, void* x_sorted, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Bytes of workspace moe_grouped_ffn needs: the SwiGLU activations h [rows, d_ff] in act_dtype
 * between the two GEMMs, and, for launches small enough that the contraction is split across
 * workgroups (rows < 32 * E, bf16 activations and weights, and at most 256 tiles of 64 rows by
 * 64 h columns, or by 128 output columns, counting every expert that could hold a row), 16 MiB
 * of fp32 partial tiles after h; for prefill-sized launches (bf16 activations; bf16 weights
 * with rows >= 32 * E, or fp8 weights with rows > 8 * E and d and d_ff at most 65536) a
 * 256-byte header and 64 MiB
 * (bf16) or 32 MiB (fp8) of fp32 partial tiles for the last round's tiles, whose contraction is
 * split across workgroups. */
size_t moe_ffn_workspace_size(int rows, int E, int d, int d_ff, moe_dtype_t act_dtype,
                              moe_dtype_t w_dtype);

/*
 * moe_block_weights - copy weights from the row-major layout of moe_grouped_ffn ([E, N, K],
 * contraction axis K contiguous) into the blocked layout of the same format: with B = 64
 * (w_dtype MOE_BF16, giving MOE_BF16_BLOCKED) or B = 128 (MOE_FP8_E4M3FN, giving
 * MOE_FP8_E4M3FN_BLOCKED) contraction elements per block row, element (e, n, k) goes to
 *     ((e*(N/8) + n/8) * (K/B) + k/B) * 8*B + (n%8) * B + k%B.
 * Weights are prepared once (at load time); a bit copy, no arithmetic.
 *   src, dst  [E*N*K] device buffers in w_dtype, not overlapping; E >= 1, N a multiple of 8, K
 *             of B, each matrix under 2 GiB, E*N*K < 2^40. Other w_dtype values give
 *             MOE_ERR_UNSUPPORTED.
 */
moe_status_t moe_block_weights(const void* src, void* dst, moe_dtype_t w_dtype, int E, int N, int K,
                               void* stream);

/*
 * moe_grouped_ffn - every expert's SwiGLU FFN over its contiguous rows, all experts in one
 * grouped launch per GEMM (tutorial page, section 4, compute: a grouped GEMM, many
 * differently shaped GEMMs in one launch; section 8: grouped-GEMM quality matters; the
 * makespan-dispatcher abstract on the UltraEP-titled page: below roughly 156-168 rows an
 * expert's time is weight streaming, above it GEMM tiles).
 *
 * For expert e and rows r in [offsets[e], offsets[e+1]):
 *     h[r]        = silu(x_sorted[r] . Wg_e) * (x_sorted[r] . Wu_e),  silu(z) = z/(1+e^-z)
 *     y_sorted[r] = h[r] . Wd_e
 *
 *   x_sorted  [rows, d] in act_dtype (MOE_F32 or MOE_BF16).
 *   offsets   [E+1] int32, non-decreasing, offsets[0] = 0, offsets[E] = rows.
 *   w_gate, w_up [E, d_ff, d] in w_dtype; w_down [E, d, d_ff] in w_dtype. Each matrix is
 *             stored with its contraction axis contiguous (the transpose of the math-side
 *             Wg, Wu [d, d_ff] and Wd [d_ff, d]).
 *   w_dtype   MOE_F32 with act MOE_F32; MOE_BF16, MOE_FP8_E4M3FN, MOE_BF16_BLOCKED (each of the
 *             E matrices of w_gate, w_up, w_down in the blocked layout above; d and d_ff
 *             multiples of 64) or MOE_FP8_E4M3FN_BLOCKED (d and d_ff at most 65536) with act
 *             MOE_BF16.
 *   s_gate, s_up [E, ceil(d_ff/128), ceil(d/128)], s_down [E, ceil(d/128), ceil(d_ff/128)]
 *             fp32 per-128x128-block scales of the stored matrices (fp8 only, else NULL):
 *             the weight value is code * scale of its block.
 *   y_sorted  [rows, d] fp32 out.
 *   Arithmetic: fp32 accumulation; with act MOE_BF16, h is rounded to bf16 (RNE) between
 *   the two GEMMs; fp8 codes are converted exactly and the block scale multiplies the fp32
 *   partial sum of each 128-long contraction block.
 *   Requires d and d_ff multiples of 8 (of 128 for fp8). Experts with no rows are never read.
 */
moe_status_t moe_grouped_ffn(const void* x_sorted, moe_dtype_t act_dtype, const int32_t* offsets,
                             int rows, int E, int d, int d_ff, const void* w_gate,
                             const void* w_up, const void* w_down, moe_dtype_t w_dtype,
                             const float* s_gate, const float* s_up, const float* s_down,
                             float* y_sorted, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * moe_combine - return the expert outputs to token order and take each token's gate-weighted
 * sum (tutorial page, section 4, combine).
 *
 *   y[t] = sum_{j=0..k-1} topk_gates[t, j] * y_sorted[flat_to_sorted[t*k + j]]
 *   summed in fp32 in slot order j = 0..k-1. A slot whose flat_to_sorted entry is negative (an
 *   assignment dropped by moe_permute_capped) adds nothing; so does one at or past T*k.
 *
 *   y_sorted [T*k, d] fp32; flat_to_sorted [T*k] int32; topk_gates [T, k] fp32;
 *   y [T, d] out, in y_dtype: MOE_F32 (the fp32 sum itself) or MOE_BF16 (that fp32 sum rounded
 *   to the nearest bf16, ties to even: half the bytes written, and a final rounding of up to
 *   2^-9 of each value). MOE_FP8_E4M3FN gives MOE_ERR_UNSUPPORTED, any other value
 *   MOE_ERR_INVALID_ARG. Requires d a multiple of 4 and y 16-byte aligned.
 */
moe_status_t moe_combine(const float* y_sorted, const int32_t* flat_to_sorted,
                         const float* topk_gates, int T, int k, int d, void* y,
                         moe_dtype_t y_dtype, void* stream);

/* Bytes of workspace moe_layer needs. */
size_t moe_layer_workspace_size(int T, int E, int k, int d, int d_ff, moe_dtype_t act_dtype,
                                moe_dtype_t w_dtype);

/*
 * moe_layer - the whole layer on one stream: moe_route, moe_permute, moe_grouped_ffn and
 * moe_combine in order, with every intermediate written to a caller buffer so that each can
 * be checked. Arguments have the meanings given above; x and x_sorted are in act_dtype, y in
 * y_dtype (as moe_combine).
 */
moe_status_t moe_layer(const float* logits, const void* x, moe_dtype_t act_dtype, int T, int E,
                       int k, int d, int d_ff, const void* w_gate, const void* w_up,
                       const void* w_down, moe_dtype_t w_dtype, const float* s_gate,
                       const float* s_up, const float* s_down, int32_t* topk_ids,
                       float* topk_gates, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                       float* y_sorted, void* y, moe_dtype_t y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * moe_layer_capped - moe_layer with moe_permute_capped in place of moe_permute (each expert
 * keeps at most `capacity` assignments; see moe_expert_capacity). Dropped slots add nothing to
 * y; the gates are not renormalised. The workspace is that of moe_layer.
 */
moe_status_t moe_layer_capped(const float* logits, const void* x, moe_dtype_t act_dtype, int T,
                              int E, int k, int d, int d_ff, int capacity, const void* w_gate,
                              const void* w_up, const void* w_down, moe_dtype_t w_dtype,
                              const float* s_gate, const float* s_up, const float* s_down,
                              int32_t* topk_ids, float* topk_gates, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_to_flat, int32_t* flat_to_sorted,
                              void* x_sorted, float* y_sorted, void* y, moe_dtype_t y_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
