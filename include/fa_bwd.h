/*
 * fa_bwd.h — C ABI of the MI355X (gfx950) FlashAttention backward library
 * (libfa_bwd.so).
 *
 * What it computes (page "CANN ops-transformer FlashAttnGrad 算子详解",
 * section 一, forward formulas and backward formulas): from the forward's
 * inputs q, k, v, its output attn_out (Y) and its per-row log-sum-exp
 * softmax_lse, and the upstream gradient dout (dY), the library rebuilds
 *     P = exp(scale * Q K^T - softmax_lse)            (never stored whole)
 * tile by tile and returns
 *     dV = P^T dY,  dP = dY V^T,  sfmg = rowsum(dY (.) Y),
 *     dS = P (.) (dP - sfmg),  dQ = scale * dS K,  dK = scale * dS^T Q.
 * Under GQA (N1 a multiple of N2) query head n1 uses key/value head
 * n1 / (N1/N2), and dK, dV of a key/value head sum over its N1/N2 query heads.
 *
 * The interface follows the page's PyTorch signature (section 四 4.2) and its
 * two-stage "size the workspace, then execute on a stream" aclnn pattern
 * (section 六): fa_bwd_create validates the problem, plans the launch and
 * reports the workspace size; fa_bwd_run enqueues the kernels on a stream.
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, row-major, contiguous, in device memory, owned by
 *    the caller.  Inputs are only read.  dq, dk, dv are fully overwritten
 *    (rows that receive no gradient are written as zeros).
 *  - The kernels move q, k, v, dout, attn_out, dq, dk and dv in 16-byte
 *    pieces: their pointers must be 16-byte aligned, and softmax_lse and the
 *    int32 arrays 4-byte aligned (FA_ERR_PARAM_INVALID otherwise, returned
 *    before any launch).
 *  - Element types (section 五 5.4 registers both): bf16 and IEEE fp16.  q, k,
 *    v, dout, attn_out and dq, dk, dv share the plan's type; softmax_lse and
 *    the workspace are float32.
 *  - Return value: FA_OK (0) or one of the FA_ERR_* codes below; nothing
 *    is thrown across the ABI and nothing is printed unless FA_BWD_LOG=1.
 *  - Plans hold host memory only; a plan may be used by one stream at a time.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_BWD_ABI_VERSION 3

/* Status codes.  The classes mirror the aclnn error families that page
 * "aclnnFusedFloydAttentionGrad" lists (null pointer 161001, invalid
 * parameter 161002, inner/tiling error 561002, runtime error 361001). */
enum {
  FA_OK = 0,
  FA_ERR_NULLPTR = 1,       /* a required pointer is NULL                      */
  FA_ERR_PARAM_INVALID = 2, /* unknown dtype / layout / mask_mode / flag, bad
                               abi_version, non-finite softmax_scale          */
  FA_ERR_SHAPE = 3,         /* a shape constraint of section 四 4.6 is broken,
                               cu_seqlens are inconsistent, or a row stride
                               (N*D elements in BSND/TND) reaches 2^23         */
  FA_ERR_UNSUPPORTED = 4,   /* valid on the page but not built here (head dims
                               outside the built set, flags)                   */
  FA_ERR_WORKSPACE = 5,     /* workspace pointer NULL or smaller than needed   */
  FA_ERR_RUNTIME = 6        /* a HIP call or kernel launch failed              */
};

/* element types of the page's two binaries (section 五 5.4) */
enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP16 = 1 };

/* Layouts of section 四 4.6; q, k, v, dout, attn_out, dq, dk, dv share one.
 *   BSND: q [B, S1, N1, D]   k [B, S2, N2, D]   v [B, S2, N2, Dv]
 *   BNSD: q [B, N1, S1, D]   k [B, N2, S2, D]   v [B, N2, S2, Dv]
 *   TND : q [T1, N1, D]      k [T2, N2, D]      v [T2, N2, Dv]
 * dout and attn_out have q's shape with Dv; dq/dk/dv have q/k/v's shapes.
 * softmax_lse (float32) is [B, N1, S1] for BSND and BNSD, [N1, T1] for TND. */
enum { FA_LAYOUT_BSND = 0, FA_LAYOUT_BNSD = 1, FA_LAYOUT_TND = 2 };

/* mask_mode (section 四 4.3; its value table was lost, this is the reading
 * used throughout): the diagonal of query i is key i + (s2 - s1) of the same
 * sequence (bottom-right alignment), and key j is visible to query i iff
 *   j >= i + (s2 - s1) - win_left   (skipped when win_left  == -1) and
 *   j <= i + (s2 - s1) + win_right  (skipped when win_right == -1).
 *   FA_MASK_NONE   : dense; win_left = win_right = -1 required.
 *   FA_MASK_CAUSAL : win_right forced to 0 (must be -1 or 0); win_left >= -1
 *                    optionally bounds the left side (a causal sliding window).
 *   FA_MASK_WINDOW : both bounds from win_left / win_right (each >= -1). */
enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1, FA_MASK_WINDOW = 2 };

/* flags */
/* Bitwise-repeatable results.  Every dQ mode but FA_DQ_ATOMIC already gives
 * them; with FA_DQ_AUTO the flag only keeps the plan off the atomic mode, and
 * asking for FA_DQ_ATOMIC together with it is FA_ERR_PARAM_INVALID. */
#define FA_FLAG_DETERMINISTIC 0x1u
/* fp32 debugging form (not on the page; it checks the arithmetic of section 一
 * at fp32 accuracy): dq, dk, dv are float32 arrays with the shapes and layouts
 * of q, k, v; P and dS are kept in fp32 and every product is an fp32 FMA, so
 * the only 16-bit roundings are those of the inputs.  Slow (VALU, untuned);
 * deterministic.  Takes dq_mode FA_DQ_AUTO only. */
#define FA_FLAG_FP32_OUT 0x2u

/* How dQ = scale * dS K is formed (fa_bwd_desc.dq_mode; fa_bwd_plan_dq_path
 * reports the plan's choice).  The page's own kernel adds dQ across key tiles
 * with atomic adds into an fp32 workspace (section 五 5.2); FA_DQ_ATOMIC is
 * that strategy.  The others write every dQ element once and are bitwise
 * repeatable.
 *   FA_DQ_AUTO      : desc only.  fa_bwd_create picks FA_DQ_FUSED for small
 *                     problems (below), else FA_DQ_STORED_DS when the dS of
 *                     at least one key/value head fits the workspace bound,
 *                     else FA_DQ_RECOMPUTE.
 *   FA_DQ_STORED_DS : the dK/dV kernel also stores dS (the element type, 2
 *                     bytes per (row, key) of each 32 x 32 tile a 128-row
 *                     query group sees) in the workspace and a GEMM kernel
 *                     reads it back; whole key/value heads are processed in
 *                     chunks that fit the bound.
 *   FA_DQ_RECOMPUTE : a query-tile-parallel kernel recomputes S and dP and
 *                     writes dQ; no dS in the workspace (the page's low-memory
 *                     property: nothing of size S1 x S2 is kept).
 *   FA_DQ_ATOMIC    : fp32 atomic adds into a dQ workspace, then a cast;
 *                     not bitwise repeatable; bf16 only and no seqused
 *                     (FA_ERR_UNSUPPORTED otherwise).
 *   FA_DQ_FUSED     : the page's per-head small-sequence schedule
 *                     (flash_attn_grad_bn2, section 五 5.2): one launch, one
 *                     workgroup per (sequence, key/value head) forms sfmg, dK,
 *                     dV and dQ for all the head group's query rows, with no
 *                     workspace.  Needs the longest key sequence <= 128,
 *                     G * ceil(S1 / 32) <= 64 (G = N1 / N2, S1 the longest
 *                     query sequence) and (D, Dv) in {(64, 64), (128, 64),
 *                     (128, 128)}, FA_ERR_UNSUPPORTED otherwise; AUTO takes
 *                     it whenever these hold.
 *   FA_DQ_FP32_FORM : reported only: the fp32 debugging form
 *                     (FA_FLAG_FP32_OUT), which takes FA_DQ_AUTO only. */
enum {
  FA_DQ_AUTO = 0,
  FA_DQ_STORED_DS = 1,
  FA_DQ_RECOMPUTE = 2,
  FA_DQ_ATOMIC = 3,
  FA_DQ_FUSED = 4,
  FA_DQ_FP32_FORM = 5
};

typedef struct fa_bwd_plan_s* fa_bwd_plan; /* opaque, host memory only */

/* Problem description (the page's attributes and shapes, section 四 4.2/4.6). */
typedef struct fa_bwd_desc {
  int32_t abi_version;   /* FA_BWD_ABI_VERSION                                    */
  int32_t dtype;         /* FA_DTYPE_BF16 or FA_DTYPE_FP16                         */
  int32_t layout;        /* FA_LAYOUT_*                                            */
  int32_t B;             /* batch (BSND/BNSD) or number of sequences (TND); 0 < B < 65536 */
  int32_t N1, N2;        /* query heads, key/value heads; N1 % N2 == 0           */
  int32_t S1, S2;        /* BSND/BNSD: sequence lengths (> 0).  TND: max_seqlen_q /
                            max_seqlen_kv, or -1 to derive them from the host
                            cu_seqlens copies below.  Both below 2^29            */
  int32_t D, Dv;         /* head dims, 0 < Dv <= D <= 192                         */
  int64_t T1, T2;        /* TND: total query / key rows (> 0); ignored otherwise  */
  const int32_t* host_cu_seqlens_q;  /* TND, optional: host copy of cu_seqlens_q
                                        (B+1 entries) used to validate and plan;
                                        read only during fa_bwd_create           */
  const int32_t* host_cu_seqlens_kv; /* TND, optional: same for cu_seqlens_kv    */
  float softmax_scale;   /* 0 selects 1/sqrt(D) (section 一, scale rule)         */
  int32_t mask_mode;     /* FA_MASK_*                                             */
  int32_t win_left, win_right; /* window bounds, -1 = unbounded; a bound wider
                                  than the sequences (left > S2, right > S1)
                                  acts as that width                          */
  uint32_t flags;        /* FA_FLAG_*                                             */
  /* ABI version 3 */
  int32_t dq_mode;       /* FA_DQ_* (FA_DQ_AUTO = 0: the planner's choice)        */
  int32_t num_cus;       /* compute units the job split fills; 0 = those of the
                            current HIP device, read once per process (256, an
                            MI355X, when no device is visible)                  */
  uint64_t max_workspace_bytes; /* upper bound on the workspace; 0 = none (the
                            stored dS is then kept below 4 GiB per chunk of
                            key/value heads).  The planner fits the dS chunk,
                            then the dK/dV partial sums, inside the bound and
                            falls back to FA_DQ_RECOMPUTE (under FA_DQ_AUTO)
                            when not even one head's dS fits              */
} fa_bwd_desc;

/* Validate `desc` (all rules of section 四 4.6 that this library enforces) and
 * build a plan.  On success *plan receives a new plan and *workspace_bytes the
 * device workspace size fa_bwd_run needs (never above max_workspace_bytes when
 * that is set).  Host code only; its one HIP call is the CU-count query when
 * num_cus = 0 (made once per process).
 * Workspace (float32 parts, 256-byte aligned, in this order):
 *   sfmg                 : 4 * (query rows x N1) bytes (not for FA_DQ_FUSED);
 *   dQ accumulator       : FA_DQ_ATOMIC only, 4 bytes per element of q;
 *   dK / dV partial sums : when the job split gives a key tile to several
 *                          workgroups (query heads of a GQA group or query
 *                          ranges), n_partials fp32 copies of k and of v;
 *   dS                   : FA_DQ_STORED_DS only, 8 KB per (128-row query
 *                          group, query head of a chunk, 32-key slice of the
 *                          group's band); the band is every slice of the
 *                          longest key sequence unless both window bounds are
 *                          given.
 * Errors: FA_ERR_NULLPTR (desc/plan/workspace_bytes NULL),
 * FA_ERR_PARAM_INVALID (also: dq_mode unknown, FA_DQ_ATOMIC with
 * FA_FLAG_DETERMINISTIC, an explicit dq_mode with FA_FLAG_FP32_OUT, num_cus
 * < 0), FA_ERR_SHAPE, FA_ERR_UNSUPPORTED (also: FA_DQ_ATOMIC with fp16,
 * FA_DQ_FUSED outside its limits), FA_ERR_WORKSPACE (max_workspace_bytes
 * below what the requested or any mode needs); *plan is left NULL. */
int fa_bwd_create(const fa_bwd_desc* desc, fa_bwd_plan* plan, size_t* workspace_bytes);

/* Enqueue the backward on `stream` (a hipStream_t; NULL = the null stream).
 * Asynchronous: no allocation, no host synchronisation.
 *   q, k, v, dout, attn_out : the plan's element type (bf16 or fp16), in the
 *                             plan's layout (see above)
 *   softmax_lse             : float32, [B, N1, S1] or [N1, T1]; -inf marks a
 *                             query row with no visible key (its dq row is 0)
 *   cu_seqlens_q/kv         : device int32 [B+1] prefix sums; required for TND
 *                             (cu[0] = 0, non-decreasing, cu[B] = T), NULL
 *                             otherwise (section 四 4.6)
 *   seqused_q/kv            : optional device int32 [B] (the page's seqused_q /
 *                             seqused_kv inputs, section 二 2.1; it names them
 *                             only): of sequence b only the first seqused[b]
 *                             query rows / keys take part (values clamped to
 *                             [0, the sequence's length]); masks align on those
 *                             used lengths; the rest is padding that nothing
 *                             attends and whose dq / dk / dv rows are written
 *                             as zeros.  NULL: every row takes part.  Any layout.
 *                             Not available with FA_DQ_ATOMIC
 *                             (FA_ERR_UNSUPPORTED, returned before any launch).
 *   dq, dk, dv              : outputs of the plan's element type, shapes of
 *                             q, k, v
 *   workspace               : device memory of at least *workspace_bytes from
 *                             fa_bwd_create, exclusively owned by this call
 *                             until it completes on `stream`
 * Errors: FA_ERR_NULLPTR (plan or a tensor pointer NULL), FA_ERR_SHAPE
 * (cu_seqlens given or missing against the layout), FA_ERR_PARAM_INVALID (a
 * pointer misaligned, see the conventions above), FA_ERR_WORKSPACE,
 * FA_ERR_RUNTIME (a launch failed).  Device cu_seqlens are trusted: they must
 * agree with T1/T2 and the max lengths in the plan. */
int fa_bwd_run(fa_bwd_plan plan,
               const void* q, const void* k, const void* v,
               const void* dout, const void* attn_out, const float* softmax_lse,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
               const int32_t* seqused_q, const int32_t* seqused_kv,
               void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes, void* stream);

/* Size of the library-owned device scratch that fa_bwd_run_noalloc uses in
 * place of a caller workspace (64 MiB on each device the library runs on,
 * held until the process ends). */
#define FA_BWD_SCRATCH_BYTES ((size_t)64 << 20)

/* fa_bwd_run for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as fa_bwd_run, without the workspace: the
 * kernels use a library-owned device array of FA_BWD_SCRATCH_BYTES on the
 * current device instead.  The call allocates nothing (no hipMalloc, no
 * library routine that allocates).  Create the plan with
 * max_workspace_bytes <= FA_BWD_SCRATCH_BYTES so that it fits; a plan whose
 * workspace is larger is refused with FA_ERR_WORKSPACE before any launch.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (several streams, host threads or processes' worth of
 * plans on the same array) race and must be ordered by the caller.  Nothing
 * in the array needs to start at zero: every part the kernels read is
 * written earlier in the same call.  Errors: those of fa_bwd_run, and
 * FA_ERR_RUNTIME when the array's address cannot be found on the current
 * device. */
int fa_bwd_run_noalloc(fa_bwd_plan plan,
                       const void* q, const void* k, const void* v,
                       const void* dout, const void* attn_out, const float* softmax_lse,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                       const int32_t* seqused_q, const int32_t* seqused_kv,
                       void* dq, void* dk, void* dv, void* stream);

/* The preprocess step alone (the page's first vector stage, section 五 5.2:
 * sfmg = rowsum(dY (.) Y)): writes float32 sfmg in softmax_lse's layout
 * ([B, N1, S1] or [N1, T1]) to `sfmg`, a caller buffer of that size.
 * Same pointer rules and errors as fa_bwd_run. */
int fa_bwd_sfmg(fa_bwd_plan plan, const void* dout, const void* attn_out,
                const int32_t* cu_seqlens_q, float* sfmg, void* stream);

/* Attention forward producing the two tensors the backward consumes
 * (section 一, S = scale*Q K^T, P = exp(S - softmax_lse), Y = P V, with
 * softmax_lse the natural-log row log-sum-exp): writes attn_out (the plan's
 * element type, q's layout with Dv) and float32 softmax_lse ([B, N1, S1] or
 * [N1, T1]) for the plan's problem, masks and layout.  A query row with no
 * visible key gets
 * attn_out = 0 and softmax_lse = -inf, and so does a row past seqused_q.
 * Same pointer rules and errors as fa_bwd_run; needs no workspace. */
int fa_fwd_run(fa_bwd_plan plan, const void* q, const void* k, const void* v,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
               const int32_t* seqused_q, const int32_t* seqused_kv,
               void* attn_out, float* softmax_lse, void* stream);

/* How the plan forms dQ: one of FA_DQ_STORED_DS, FA_DQ_RECOMPUTE,
 * FA_DQ_ATOMIC, FA_DQ_FUSED, FA_DQ_FP32_FORM (see fa_bwd_desc.dq_mode).
 * Writes it to *path.  Errors: FA_ERR_NULLPTR. */
int fa_bwd_plan_dq_path(fa_bwd_plan plan, int* path);

/* Timing hook.  With slots > 0, every later fa_bwd_run records one pair of
 * HIP events on its stream immediately before and after the main kernels
 * (the dK/dV kernel and the dQ kernel, or the single kernel of the other
 * forms),
 * into a ring of `slots` pairs owned by the plan (slots = 0 frees them and
 * stops recording).  Errors: FA_ERR_NULLPTR, FA_ERR_PARAM_INVALID
 * (slots < 0 or > 65536), FA_ERR_RUNTIME (event creation failed). */
int fa_bwd_profile_enable(fa_bwd_plan plan, int slots);

/* Wait for the recorded runs and write the main kernel's duration of each,
 * in milliseconds, oldest first, into ms[0 .. *count) (at most cap and at
 * most `slots` entries); the ring is then emptied.  Errors: FA_ERR_NULLPTR,
 * FA_ERR_RUNTIME (an event query failed). */
int fa_bwd_profile_read(fa_bwd_plan plan, float* ms, int cap, int* count);

/* The same recorded runs as fa_bwd_profile_read (and the same emptying of
 * the ring), each split at the boundary between its two main kernels, where
 * the run records a third event: first_ms[i] is the first kernel (the dK/dV
 * kernel under FA_DQ_STORED_DS, the dQ kernel under FA_DQ_RECOMPUTE) and
 * second_ms[i] the other.  Runs with a single main kernel (FA_DQ_FUSED,
 * FA_DQ_ATOMIC, the fp32 form) or with dS processed in several chunks of
 * key/value heads record no boundary: their whole span goes to first_ms[i]
 * and second_ms[i] is 0.  Errors: FA_ERR_NULLPTR, FA_ERR_RUNTIME. */
int fa_bwd_profile_read_split(fa_bwd_plan plan, float* first_ms, float* second_ms, int cap, int* count);

/* Free a plan (and its timing events).  NULL is a no-op.  Returns FA_OK. */
int fa_bwd_destroy(fa_bwd_plan plan);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_bwd_strerror(int status);

/* FA_BWD_ABI_VERSION of the loaded library. */
int fa_bwd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
