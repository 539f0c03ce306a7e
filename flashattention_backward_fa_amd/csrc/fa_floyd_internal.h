// Internal contract between the Floyd attention host code (fa_floyd_api.cpp,
// plain C++) and its gfx950 kernels (fa_floyd_kernels.hip).  Not public ABI.
//
// Index names follow page "CANN Floyd注意力梯度算子" (parameter table of
// aclnnFusedFloydAttentionGradGetWorkspaceSize): Q, dY, Y are [B, H, N, M, D],
// K1, V1 [B, H, N, K, D], K2, V2 [B, H, K, M, D], the mask [B, 1, N, 1, K].
// A "head" below is one (b, h) pair, numbered b * H + h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ffloyd {

// A strided batched product C(i, j) = alpha * sum_t A(i, t) B(t, j) over the
// heads [0, heads) of a launch and an inner batch index z in [0, nb):
//   A(i, t) at a[h*a_sh + z*a_sz + i*a_si + t*a_st]
//   B(t, j) at b[h*b_sh + z*b_sz + j*b_sj + t*b_st]
//   C(i, j) at c[h*c_sh + z*c_sz + i*c_si + j]
// One of a_si / a_st is 1 (a_tc = 1: t contiguous), likewise b_sj / b_st
// (b_tc = 1: t contiguous).  With `addend` (fp32, the offsets of C) the result
// is alpha * acc + addend.  C is fp32 when out_f32, else 16-bit elements.
struct GemmArgs {
  const void* a;
  int64_t a_si, a_st, a_sh, a_sz;
  const void* b;
  int64_t b_sj, b_st, b_sh, b_sz;
  void* c;
  int64_t c_si, c_sh, c_sz;
  const float* addend;
  int32_t I, J, T;   // extents of i, j and the contraction t
  int32_t nb;        // inner batch count
  int32_t heads;     // heads in this launch
  float alpha;
  int32_t out_f32;
  int32_t a_tc, b_tc;
  int32_t f16;       // 1: IEEE fp16 elements, 0: bf16
};

// The score products of one launch (heads [0, heads) of the chunk).
//   by_m = 0: for each n, C(m, k) = Q[n, m] . X[n, k]  (X = K1, and V1 with dY)
//   by_m = 1: for each m, C(n, k) = Q[n, m] . X[k, m]  (X = K2, and V2 with dY)
// C lives in the fp32 score workspace ws_s [heads][N][M][K] (and ws_p for dP).
// epi: 0 = store both (backward, by n); 1 = fused softmax gradient (backward,
// by m): P and dS written as 16-bit to ws_pe / ws_dse; 2 = store the score
// only (forward, by n); 3 = add the score into ws_s (forward, by m).
struct ScoreArgs {
  const void* q;     // Q of the chunk's first head
  const void* dy;    // dY (epi 0, 1)
  const void* x1;    // K1 (by n) or K2 (by m)
  const void* x2;    // V1 (by n) or V2 (by m) (epi 0, 1)
  float* ws_s;
  float* ws_p;
  void* ws_pe;       // P, 16-bit (epi 1)
  void* ws_dse;      // dS, 16-bit (epi 1)
  const float* sfmg; // [heads][N][M] (epi 1)
  const float* lse2; // [heads][N][M], log2-domain row log-sum-exp, +inf for dead rows (epi 1)
  const uint8_t* mask;  // [B][N][K] or null (epi 1)
  int32_t head0;     // index of the chunk's first head (for the mask's batch)
  int32_t heads, H, N, M, K, D;
  int32_t by_m, epi;
  float scale;
  int32_t f16;
};

// Per row (head, n, m) of the chunk: sfmg = sum_d dY * Y, and
// lse2 = (max + ln(sum)) * log2(e) from the forward's statistics (first of
// the 8 copies), +inf when the row has no live key (max = -inf or sum = 0).
struct RowStatsArgs {
  const void* dy;
  const void* y;
  const float* smax;  // [rows][8]
  const float* ssum;  // [rows][8]
  float* sfmg;
  float* lse2;
  int64_t rows;
  int32_t D;
  int32_t f16;
};

// Forward softmax over k of the chunk's scores: P (16-bit) and the 8-copy
// max / sum statistics.
struct SoftmaxArgs {
  const float* ws_s;
  void* p;
  float* smax;
  float* ssum;
  const uint8_t* mask;
  int32_t head0, heads, H, N, M, K;
  float scale;
  int32_t f16;
};

// HIP events between consecutive launches on one stream (timing hook).
struct StageTimer;
StageTimer* stage_timer_create(int marks);            // nullptr on failure
int stage_timer_mark(StageTimer* t, int i, void* stream);
int stage_timer_read(StageTimer* t, float* ms);       // waits; ms[i] = mark i -> i + 1
void stage_timer_destroy(StageTimer* t);

int launch_gemm(const GemmArgs& g, void* stream);
int launch_scores(const ScoreArgs& s, void* stream);
int launch_rowstats(const RowStatsArgs& r, void* stream);
int launch_softmax(const SoftmaxArgs& s, void* stream);

}  // namespace ffloyd
