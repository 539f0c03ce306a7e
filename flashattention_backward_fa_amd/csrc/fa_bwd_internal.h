// Internal contract between the host planner (fa_bwd_api.cpp, plain C++) and
// the gfx950 kernels (fa_bwd_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fabwd {

// Tile shape of the main kernel: each workgroup owns KV_TILE keys of one
// sequence and one key/value head (4 wavefronts x 32 keys); query rows stream
// through LDS Q_TILE at a time.
constexpr int KV_TILE = 128;
constexpr int Q_TILE = 64;      // query rows per step of the 4-wavefront kernel
constexpr int Q_TILE_2G = 32;   // query rows per step and group of the 8-wavefront kernel

// Everything a launch needs, plain old data, passed by value to the kernels.
struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* out;
  const float* lse;
  const int32_t* cu_q;   // TND only (device)
  const int32_t* cu_kv;  // TND only (device)
  const int32_t* seqused_q;   // optional (device, [B]): rows of each sequence that take part
  const int32_t* seqused_kv;  // optional (device, [B]): keys of each sequence that take part
  float* dq_acc;         // fp32, q's layout
  float* sfmg;           // fp32, lse's layout
  float* dk_acc;         // fp32, k's layout (only when query heads are split)
  float* dv_acc;         // fp32, v's layout (only when query heads are split)
  void* dq;
  void* dk;
  void* dv;

  int32_t B, N1, N2, G;
  int32_t S1, S2;        // dense lengths, or max lengths for TND
  int32_t D, Dv;
  int64_t T1, T2;
  int32_t varlen;        // 1 for TND
  int32_t f16;           // 1: elements are IEEE fp16, 0: bf16 (same 16-bit storage)
  int32_t layout;        // FA_LAYOUT_* of include/fa_bwd.h

  // element strides: batch (dense layouts), sequence row, head
  int64_t q_sb, q_ss, q_sn;   // q, dq, dq_acc
  int64_t k_sb, k_ss, k_sn;   // k, dk
  int64_t v_sb, v_ss, v_sn;   // v, dv
  int64_t o_sb, o_ss, o_sn;   // dout, attn_out
  int64_t l_sb, l_sn;         // lse, sfmg (row stride 1)

  float scale;           // softmax scale actually used
  float scale_log2;      // scale * log2(e)
  int32_t win_left;      // -1 = unbounded
  int32_t win_right;     // -1 = unbounded
  int32_t has_mask;      // any bound present

  int32_t variant;        // 0 = 4-wavefront atomic kernel, 1 = 8-wavefront atomic kernel,
                          // 2 = atomic-free pair (dK/dV kernel + dQ kernel),
                          // 3 = fp32 debugging form (fp32 outputs),
                          // 4 = dS-store pair (dK/dV kernel storing dS + dQ GEMM),
                          // 5 = fused small-sequence kernel (one launch)
  int32_t heads_per_job;  // query heads of a GQA group handled by one workgroup
  int32_t q_splits;       // query-range splits of one key tile (atomic-free pair only)
  int32_t n_partials;     // fp32 dK/dV partial sums per key tile (atomic-free pair only)
  int64_t k_part_stride;  // elements between dK partials (= elements of k)
  int64_t v_part_stride;  // elements between dV partials (= elements of v)

  // dS-store form (variant 4): the dK/dV kernel stores dS, bf16 (or fp16), as
  // [ds_groups][N1][ds_w][4][1024] elements: per 128-row query group, per
  // query head, per 32-key slice counted from the first slice the group sees
  // (a band of ds_w slices), the four 32 x 32 tiles of the group's query
  // blocks; a GEMM kernel then forms dQ = scale * dS K from them.  Group of
  // row group R of sequence b: b * ds_nr + R (dense layouts) or
  // cu_q[b] / 128 + b + R (TND; distinct for every (b, R) since cu_q does not
  // decrease).
  void* ds;
  int32_t ds_nr;          // dense layouts: 128-row groups per sequence (ceil(S1 / 128))
  int32_t ds_w;           // slices per group: a bound on the 32-key slices one group sees
  int64_t ds_groups;      // groups the workspace holds
  int32_t ds_heads;       // query heads the workspace holds per group (G * KV heads of a chunk)
  // KV heads [n2_begin, n2_begin + n2_count) handled by one dK/dV launch (and
  // their query heads by the dQ launch): the whole range, or one chunk when
  // the stored dS is processed a few KV heads at a time
  int32_t n2_begin, n2_count;
  // 1: the dQ GEMM launch also adds the fp32 dK/dV partial sums (extra
  // workgroups after the GEMM's, which the dispatcher starts as the GEMM's
  // last ones drain), in place of a separate reduce launch
  int32_t reduce_tail;
  // dQ GEMM workgroups: 1 = 4 wavefronts; 2 = two groups of 4 that share a row
  // group and take alternate key steps (D <= 128, no reduce tail)
  int32_t dq_groups;
  // dK/dV kernel: workgroups that the device holds at once (one per CU), the
  // unit of the engine-order reversal of its job order; 0 = no reversal
  int32_t round_wgs;
  // dK/dV kernel job order: 0 = key tile slowest (longest first under a causal
  // mask), 1 = sequence slowest and key tile fastest (varlen: a sequence's
  // tiles are consecutive)
  int32_t seq_major;
};

// True when dK/dV of one key/value head are summed over several workgroups
// (through the fp32 dk_acc / dv_acc workspace) instead of in registers.
inline bool split_heads(const KernelArgs& a) { return a.variant < 2 && a.heads_per_job < a.G; }

// Launchers (fa_bwd_kernels.hip).  Each returns 0 or a hipError_t value.
int launch_preprocess(const KernelArgs& a, bool zero_dq_acc, void* stream);
int launch_main(const KernelArgs& a, void* stream);
bool main_v2_instantiated(int D, int Dv);

// Atomic-free pair (fa_bwd_det_kernels.hip).
bool det_instantiated(int D, int Dv);
int det_keys_per_wave(int D);
int launch_dkdv(const KernelArgs& a, void* stream);
int launch_dq(const KernelArgs& a, void* stream);
int launch_dq_ds(const KernelArgs& a, void* stream);
int launch_reduce_parts(const KernelArgs& a, void* stream);
int launch_dq_finalize(const KernelArgs& a, void* stream);
int launch_forward(const KernelArgs& a, void* out, float* lse, void* stream);

// Fused small-sequence kernel (fa_bwd_fused_kernels.hip): one workgroup per
// (sequence, KV head) holds the whole key range (at most FUSED_MAX_KEYS keys)
// and forms sfmg, dK, dV and dQ for the G query heads in one launch.  The
// planner takes it by default when a workgroup has at most FUSED_MAX_BLOCKS
// (query head, 32-row block) items.
constexpr int FUSED_MAX_KEYS = 128;
constexpr int FUSED_MAX_BLOCKS = 64;
bool fused_instantiated(int D, int Dv);
int launch_fused(const KernelArgs& a, void* stream);

// Compute units of the current HIP device, or 0 when it cannot be read.
int device_cu_count();

// Library-owned device scratch of fa_bwd_run_noalloc (fa_bwd_scratch.hip):
// SCRATCH_BYTES on each device, its device address on the current device
// looked up once per device.  Returns 0 or a hipError_t value.
constexpr size_t SCRATCH_BYTES = size_t(64) << 20;
int scratch_ptr(void** ptr);

// fp32 debugging form (fa_bwd_f32_kernels.hip): dK/dV and dQ, fp32 outputs.
int launch_f32_debug(const KernelArgs& a, void* stream);
bool main_instantiated(int D, int Dv);

// Ring of HIP event pairs bracketing the main kernel (timing hook).
struct Profiler;
Profiler* profiler_create(int slots);   // nullptr on failure
void profiler_destroy(Profiler* p);
int profiler_begin(Profiler* p, void* stream);
int profiler_mark(Profiler* p, void* stream);  // boundary between the two main kernels
int profiler_end(Profiler* p, void* stream);
// second == nullptr: whole spans into ms; else the parts before and after the
// mark (ms, second), or the whole span and 0 for runs without a mark
int profiler_read(Profiler* p, float* ms, float* second, int cap, int* count);

}  // namespace fabwd
