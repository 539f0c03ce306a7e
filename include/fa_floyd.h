/*
 * fa_floyd.h — C ABI of Floyd attention in libfa_bwd.so (MI355X, gfx950).
 *
 * What it computes (page "CANN Floyd注意力梯度算子", section 功能说明): the
 * scores add a product batched over n and one batched over m,
 *     S[n,m,k] = scale * (Q[n,m] . K1[n,k] + Q[n,m] . K2[k,m]),
 * masked positions (mask[b,0,n,0,k] != 0) take no part, P = softmax_k(S) and
 *     Y[n,m]   = sum_k P[n,m,k] (V1[n,k] + V2[k,m]).
 * The backward returns
 *     dV1 = P^T dY (summed over m),  dV2 = P^T dY (summed over n),
 *     dQ  = scale * (dS K1 + dS K2), dK1 = scale * dS^T Q (over m),
 *     dK2 = scale * dS^T Q (over n),
 * with dP = dY V1^T + dY V2^T, sfmg = rowsum(dY (.) Y), dS = P (.) (dP - sfmg)
 * and P rebuilt as exp(S - softmaxMax) / softmaxSum from the forward's
 * statistics.
 *
 * Shapes (the page's parameter table of
 * aclnnFusedFloydAttentionGradGetWorkspaceSize), all dense, row-major,
 * contiguous, in device memory, owned by the caller, 16-byte aligned:
 *     query, dy, attention_in, dq      [B, H, N, M, D]
 *     key1, value1, dk1, dv1           [B, H, N, K, D]
 *     key2, value2, dk2, dv2           [B, H, K, M, D]
 *     atten_mask (optional, uint8)     [B, 1, N, 1, K]; 1 = excluded, 0 = part
 *     softmax_max, softmax_sum (fp32)  [B, H, N, M, 8]; the 8 entries of a row
 *                                      hold one value, the first is read
 * Element type: bf16 or IEEE fp16 (FA_DTYPE_* of fa_bwd.h) for every 16-bit
 * tensor; the statistics and the workspace are float32.
 * Shape rules of the page's constraints section (约束说明), enforced here:
 *     1 <= B <= 2048, 1 <= H <= 256, 16 <= N <= 2^20 with N % 16 == 0,
 *     128 <= M, K <= 2^20 with M % 128 == 0 and K % 128 == 0,
 *     D in {32, 64, 128}.
 * A row whose every key is masked has softmax_max = -inf, softmax_sum = 0,
 * Y = 0 and receives no gradient.
 *
 * Status codes are those of fa_bwd.h (FA_OK, FA_ERR_*); nothing is printed.
 * Results are bitwise repeatable (no atomics).
 */
#ifndef FA_FLOYD_H
#define FA_FLOYD_H

#include <stddef.h>
#include <stdint.h>

#include "fa_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fa_floyd_desc {
  int32_t abi_version;   /* FA_BWD_ABI_VERSION                                 */
  int32_t dtype;         /* FA_DTYPE_BF16 or FA_DTYPE_FP16                      */
  int32_t B, H, N, M, K, D;
  float scale_value;     /* the page's scaleValue, used as given (finite)      */
} fa_floyd_desc;

/* Device workspace bytes that fa_floyd_bwd_run and fa_floyd_fwd_run need for
 * `desc` (pure host code).  The fp32 scores and dP of a group of heads, the
 * 16-bit P and dS and an fp32 dQ partial live there: 12*N*M*K + 4*N*M*D +
 * 8*N*M bytes per (b, h) pair, for as many pairs at a time as fit in 4 GiB
 * (at least one; the environment variable FA_FLOYD_CHUNK_BYTES, a positive
 * byte count, replaces the 4 GiB budget).  Errors: FA_ERR_NULLPTR, FA_ERR_PARAM_INVALID (abi_version,
 * dtype, non-finite scale), FA_ERR_SHAPE (a rule above), FA_ERR_UNSUPPORTED
 * (a problem whose launch grid or per-pair workspace exceeds what one launch
 * addresses). */
int fa_floyd_workspace_size(const fa_floyd_desc* desc, size_t* workspace_bytes);

/* Enqueue the Floyd attention backward on `stream` (hipStream_t; NULL = the
 * null stream).  Asynchronous, allocates nothing.  Inputs are only read;
 * dq, dk1, dv1, dk2, dv2 are fully overwritten.  atten_mask may be NULL (no
 * position masked).  `workspace` (at least fa_floyd_workspace_size bytes) is
 * owned by the call until it completes on `stream`.  Errors: those of
 * fa_floyd_workspace_size, FA_ERR_NULLPTR (a required tensor NULL),
 * FA_ERR_PARAM_INVALID (a pointer not 16-byte aligned), FA_ERR_WORKSPACE,
 * FA_ERR_RUNTIME (a launch failed). */
int fa_floyd_bwd_run(const fa_floyd_desc* desc,
                     const void* query, const void* key1, const void* value1,
                     const void* key2, const void* value2, const void* dy,
                     const uint8_t* atten_mask,
                     const float* softmax_max, const float* softmax_sum,
                     const void* attention_in,
                     void* dq, void* dk1, void* dv1, void* dk2, void* dv2,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Timing hook: the same launches as fa_floyd_bwd_run with a HIP event
 * recorded on `stream` before the first and after each stage; waits for them
 * and writes the stages' durations in milliseconds (summed over the groups of
 * heads) to stage_ms[0 .. FA_FLOYD_BWD_STAGES), in this order: row
 * statistics (sfmg, log-sum-exp), score products batched over n, score
 * products batched over m with P and dS, dV1, dK1, dV2, dK2, the dQ term of
 * K1, the dQ term of K2.  Synchronous; for benchmarks.  Errors: those of
 * fa_floyd_bwd_run, FA_ERR_NULLPTR (stage_ms NULL), FA_ERR_RUNTIME (an event
 * call failed). */
#define FA_FLOYD_BWD_STAGES 9
int fa_floyd_bwd_run_timed(const fa_floyd_desc* desc,
                           const void* query, const void* key1, const void* value1,
                           const void* key2, const void* value2, const void* dy,
                           const uint8_t* atten_mask,
                           const float* softmax_max, const float* softmax_sum,
                           const void* attention_in,
                           void* dq, void* dk1, void* dv1, void* dk2, void* dv2,
                           void* workspace, size_t workspace_bytes, void* stream,
                           float* stage_ms);

/* The forward that produces the backward's inputs (section 功能说明, forward
 * formula): attention_out (Y, 16-bit, query's shape) and the float32
 * statistics softmax_max (row max of the scaled, masked scores) and
 * softmax_sum (sum of exp(S - max) over the row), each written 8 times per
 * row.  Same pointer rules, workspace and errors as fa_floyd_bwd_run. */
int fa_floyd_fwd_run(const fa_floyd_desc* desc,
                     const void* query, const void* key1, const void* value1,
                     const void* key2, const void* value2,
                     const uint8_t* atten_mask,
                     void* attention_out, float* softmax_max, float* softmax_sum,
                     void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_FLOYD_H */
