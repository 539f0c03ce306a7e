// Host side of libfa_bwd.so: validation, planning, workspace sizing and the
// C ABI declared in include/fa_bwd.h.  Plain C++ (no HIP headers): every
// device call (the launches and the CU-count query) goes through the
// functions of the .hip sources declared in fa_bwd_internal.h.
//
// The checks follow page "CANN ops-transformer FlashAttnGrad 算子详解",
// section 四 4.6 (constraints) and section 五 5.1 (host tiling: parse, check,
// plan, write back).

#include "fa_bwd.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <new>

#include "fa_bwd_internal.h"

using fabwd::KernelArgs;

struct fa_bwd_plan_s {
  fa_bwd_desc desc;
  KernelArgs args;         // pointers left NULL; filled per run
  int64_t q_elems;         // elements of q (and of the fp32 dQ accumulator)
  int64_t lse_elems;       // elements of softmax_lse / sfmg
  size_t off_dq_acc, off_sfmg, off_dk_acc, off_dv_acc, off_ds, ws_bytes;
  int32_t n2_chunk;        // stored-dS chain: KV heads per dK/dV + dQ launch pair
  fabwd::Profiler* prof = nullptr;  // timing hook, off by default
};

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxSeqLen = int64_t(1) << 29;  // bound on S1, S2 (exclusive)
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// CU count of the current HIP device (256, an MI355X, when none is visible)
int device_cus() {
  const int n = fabwd::device_cu_count();
  return n > 0 ? n : 256;
}

bool log_enabled() {
  const char* e = std::getenv("FA_BWD_LOG");
  return e && e[0] == '1';
}

// Validate host cu_seqlens: B+1 entries, cu[0] = 0, non-decreasing, cu[B] = T.
// Returns the longest sequence or -1 when invalid.
int64_t check_cu(const int32_t* cu, int B, int64_t T) {
  if (cu[0] != 0) return -1;
  int64_t mx = 0;
  for (int b = 0; b < B; ++b) {
    if (cu[b + 1] < cu[b]) return -1;
    int64_t len = (int64_t)cu[b + 1] - cu[b];
    if (len > mx) mx = len;
  }
  if ((int64_t)cu[B] != T) return -1;
  return mx;
}

int validate_and_plan(const fa_bwd_desc& d, fa_bwd_plan_s& p) {
  if (d.abi_version != FA_BWD_ABI_VERSION) return FA_ERR_PARAM_INVALID;
  if (d.dtype != FA_DTYPE_BF16 && d.dtype != FA_DTYPE_FP16) return FA_ERR_PARAM_INVALID;
  if (d.layout < FA_LAYOUT_BSND || d.layout > FA_LAYOUT_TND) return FA_ERR_PARAM_INVALID;
  if (d.mask_mode < FA_MASK_NONE || d.mask_mode > FA_MASK_WINDOW) return FA_ERR_PARAM_INVALID;
  if (!std::isfinite(d.softmax_scale)) return FA_ERR_PARAM_INVALID;
  if (d.flags & ~(FA_FLAG_DETERMINISTIC | FA_FLAG_FP32_OUT)) return FA_ERR_PARAM_INVALID;
  if (d.dq_mode < FA_DQ_AUTO || d.dq_mode > FA_DQ_FUSED) return FA_ERR_PARAM_INVALID;
  if (d.num_cus < 0) return FA_ERR_PARAM_INVALID;
  if ((d.flags & FA_FLAG_FP32_OUT) && d.dq_mode != FA_DQ_AUTO) return FA_ERR_PARAM_INVALID;
  if ((d.flags & FA_FLAG_DETERMINISTIC) && d.dq_mode == FA_DQ_ATOMIC) return FA_ERR_PARAM_INVALID;

  // section 四 4.6: positive sizes, 0 < B < 65536, N1 % N2 == 0, 0 < Dv <= D <= 192
  if (d.B <= 0 || d.B >= 65536) return FA_ERR_SHAPE;
  if (d.N1 <= 0 || d.N2 <= 0 || d.N1 % d.N2 != 0) return FA_ERR_SHAPE;
  if (d.D <= 0 || d.Dv <= 0 || d.Dv > d.D || d.D > 192) return FA_ERR_SHAPE;
  // dense attention iff mask_mode 0 with no window; causal closes the right side
  if (d.win_left < -1 || d.win_right < -1) return FA_ERR_SHAPE;
  if (d.mask_mode == FA_MASK_NONE && (d.win_left != -1 || d.win_right != -1)) return FA_ERR_SHAPE;
  if (d.mask_mode == FA_MASK_CAUSAL && d.win_right > 0) return FA_ERR_SHAPE;

  const bool tnd = d.layout == FA_LAYOUT_TND;
  int64_t S1 = d.S1, S2 = d.S2;
  if (tnd) {
    if (d.T1 <= 0 || d.T2 <= 0) return FA_ERR_SHAPE;
    if (d.T1 > INT32_MAX || d.T2 > INT32_MAX) return FA_ERR_SHAPE;
    if ((d.host_cu_seqlens_q == nullptr) != (d.host_cu_seqlens_kv == nullptr)) return FA_ERR_SHAPE;
    if (d.host_cu_seqlens_q) {
      int64_t m1 = check_cu(d.host_cu_seqlens_q, d.B, d.T1);
      int64_t m2 = check_cu(d.host_cu_seqlens_kv, d.B, d.T2);
      if (m1 < 0 || m2 < 0) return FA_ERR_SHAPE;
      if (S1 == -1) S1 = m1; else if (S1 < m1) return FA_ERR_SHAPE;
      if (S2 == -1) S2 = m2; else if (S2 < m2) return FA_ERR_SHAPE;
    } else if (S1 == -1 || S2 == -1) {
      return FA_ERR_SHAPE;  // max lengths needed when no host copy is given
    }
    if (S1 < 0 || S2 < 0 || S1 > d.T1 || S2 > d.T2) return FA_ERR_SHAPE;
  } else {
    if (d.host_cu_seqlens_q || d.host_cu_seqlens_kv) return FA_ERR_SHAPE;
    if (S1 <= 0 || S2 <= 0) return FA_ERR_SHAPE;
  }
  // row and key indices, their differences and window sums are 32-bit
  if (S1 >= kMaxSeqLen || S2 >= kMaxSeqLen) return FA_ERR_SHAPE;

  if (!fabwd::main_instantiated(d.D, d.Dv) || !fabwd::det_instantiated(d.D, d.Dv)) return FA_ERR_UNSUPPORTED;
  if (d.dq_mode == FA_DQ_ATOMIC && d.dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;  // bf16 kernels only

  KernelArgs& a = p.args;
  std::memset(&a, 0, sizeof(a));
  a.B = d.B; a.N1 = d.N1; a.N2 = d.N2; a.G = d.N1 / d.N2;
  a.S1 = (int32_t)S1; a.S2 = (int32_t)S2;
  a.D = d.D; a.Dv = d.Dv;
  a.varlen = tnd ? 1 : 0;
  a.f16 = d.dtype == FA_DTYPE_FP16 ? 1 : 0;
  a.layout = d.layout;
  a.T1 = tnd ? d.T1 : 0; a.T2 = tnd ? d.T2 : 0;
  const int64_t N1 = d.N1, N2 = d.N2, D = d.D, Dv = d.Dv;
  switch (d.layout) {
    case FA_LAYOUT_BSND:
      a.q_sb = S1 * N1 * D;  a.q_ss = N1 * D;  a.q_sn = D;
      a.k_sb = S2 * N2 * D;  a.k_ss = N2 * D;  a.k_sn = D;
      a.v_sb = S2 * N2 * Dv; a.v_ss = N2 * Dv; a.v_sn = Dv;
      a.o_sb = S1 * N1 * Dv; a.o_ss = N1 * Dv; a.o_sn = Dv;
      a.l_sb = N1 * S1;      a.l_sn = S1;
      break;
    case FA_LAYOUT_BNSD:
      a.q_sb = N1 * S1 * D;  a.q_ss = D;  a.q_sn = S1 * D;
      a.k_sb = N2 * S2 * D;  a.k_ss = D;  a.k_sn = S2 * D;
      a.v_sb = N2 * S2 * Dv; a.v_ss = Dv; a.v_sn = S2 * Dv;
      a.o_sb = N1 * S1 * Dv; a.o_ss = Dv; a.o_sn = S1 * Dv;
      a.l_sb = N1 * S1;      a.l_sn = S1;
      break;
    default:  // TND
      a.q_sb = 0; a.q_ss = N1 * D;  a.q_sn = D;
      a.k_sb = 0; a.k_ss = N2 * D;  a.k_sn = D;
      a.v_sb = 0; a.v_ss = N2 * Dv; a.v_sn = Dv;
      a.o_sb = 0; a.o_ss = N1 * Dv; a.o_sn = Dv;
      a.l_sb = 0; a.l_sn = d.T1;
      break;
  }
  // The kernels address a tile of up to 128 rows by 32-bit byte offsets from
  // its first row: the distance between consecutive rows of q, k, v, dout
  // must stay below 2^23 elements.
  constexpr int64_t kMaxRowStride = int64_t(1) << 23;
  if (a.q_ss >= kMaxRowStride || a.k_ss >= kMaxRowStride || a.v_ss >= kMaxRowStride || a.o_ss >= kMaxRowStride)
    return FA_ERR_SHAPE;
  const double scale = d.softmax_scale != 0.0f ? (double)d.softmax_scale : 1.0 / std::sqrt((double)d.D);
  a.scale = (float)scale;
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  if (d.mask_mode == FA_MASK_NONE) { a.win_left = -1; a.win_right = -1; }
  else if (d.mask_mode == FA_MASK_CAUSAL) { a.win_left = d.win_left; a.win_right = 0; }
  else { a.win_left = d.win_left; a.win_right = d.win_right; }
  // A left bound of at least S2 - 1 (a right bound of at least S1 - 1) masks
  // nothing that the sequence ends do not: clamp wider bounds to S2 (S1), so
  // that the kernels' index sums i + (s2 - s1) +- bound stay within 32 bits
  // (with S1, S2 < 2^29 they stay below 3 * 2^29).
  if (a.win_left > a.S2) a.win_left = a.S2;
  if (a.win_right > a.S1) a.win_right = a.S1;
  a.has_mask = (a.win_left >= 0 || a.win_right >= 0) ? 1 : 0;

  // Kernel choice (the dQ modes of include/fa_bwd.h):
  //  - variant 5, FA_DQ_FUSED: one workgroup per (sequence, KV head) forms
  //    sfmg, dK, dV and dQ in one launch (small problems: the longest key
  //    sequence fits one 128-key tile);
  //  - variant 4, FA_DQ_STORED_DS: the dK/dV kernel also stores dS (2 bytes
  //    per query/key pair of every 32 x 32 tile a 128-row query group sees)
  //    and a GEMM kernel forms dQ = scale * dS K from it, reading dS once
  //    instead of recomputing S and dP.  KV heads are processed in chunks
  //    whose dS fits the workspace bound (4 GiB per chunk when none is set);
  //  - variant 2, FA_DQ_RECOMPUTE: a query-tile-parallel dQ kernel recomputes
  //    S and dP; taken under FA_DQ_AUTO when not even one KV head's dS fits;
  //  - variants 0/1, FA_DQ_ATOMIC: fp32 atomic adds into a dQ workspace;
  //  - variant 3: the fp32 debugging form.
  const int64_t k_elems = tnd ? d.T2 * N2 * D : (int64_t)d.B * S2 * N2 * D;
  const int64_t v_elems = tnd ? d.T2 * N2 * Dv : (int64_t)d.B * S2 * N2 * Dv;
  p.q_elems = tnd ? d.T1 * N1 * D : (int64_t)d.B * S1 * N1 * D;
  p.lse_elems = tnd ? N1 * d.T1 : (int64_t)d.B * N1 * S1;
  // dS band: a 128-row group sees at most 128 + left + right keys under a
  // two-sided window, i.e. ceil((128 + left + right) / 32) + 1 slices of 32
  // (one more for misalignment); otherwise up to every slice of the longest
  // key sequence.
  {
    const int64_t all = (S2 + 31) / 32;
    int64_t w = all;
    if (a.win_left >= 0 && a.win_right >= 0)
      w = std::min<int64_t>(all, (128 + (int64_t)a.win_left + a.win_right + 31) / 32 + 1);
    a.ds_w = (int32_t)std::max<int64_t>(w, 1);
    a.ds_nr = (int32_t)((S1 + 127) / 128);
    // TND group indices cu_q[b] / 128 + b + R stay below T1 / 128 + B + 1
    a.ds_groups = tnd ? d.T1 / 128 + d.B + 1 : (int64_t)d.B * a.ds_nr;
  }
  const uint64_t bound = d.max_workspace_bytes;  // 0: no bound
  const int cus = d.num_cus > 0 ? d.num_cus : device_cus();
  const size_t sfmg_bytes = align_up((size_t)p.lse_elems * sizeof(float));
  // the fused kernel holds the whole key range in one tile and the row
  // statistics of all its (query head, 32-row block) items in LDS
  // (and addresses a head's dq rows by 32-bit byte offsets)
  const bool fused_ok = fabwd::fused_instantiated(d.D, d.Dv) && S2 <= fabwd::FUSED_MAX_KEYS &&
                        (int64_t)a.G * ((S1 + 31) / 32) <= fabwd::FUSED_MAX_BLOCKS &&
                        (S1 + 32) * a.q_ss * 2 < (int64_t(1) << 31);

  // Job split of the pair kernels for launches over n2l KV heads: halve the
  // query heads of a GQA group per job, then split the query range of a key
  // tile (up to 4 ways), until there are at least 2 jobs per CU, so that
  // causal work (a 32:1 skew between the first and last key tile at
  // S = 4096) balances; each split adds an fp32 partial sum of dK and dV per
  // key that a reduce kernel adds up.  A split whose partials would pass
  // part_budget bytes (when >= 0) is not taken.
  const int64_t tiles = (S2 + 127) / 128;  // 128-key tiles of the dK/dV kernel
  auto partial_bytes = [&](int hpj, int qs) -> size_t {
    const int64_t np = (int64_t)(a.G / hpj) * qs;
    return np > 1 ? align_up((size_t)np * (size_t)k_elems * sizeof(float)) +
                        align_up((size_t)np * (size_t)v_elems * sizeof(float))
                  : 0;
  };
  auto split_for = [&](int64_t n2l, int64_t part_budget) {
    a.heads_per_job = a.G;
    a.q_splits = 1;
    const int64_t target = 2 * (int64_t)cus;
    while (tiles * (a.G / a.heads_per_job) * a.q_splits * a.B * n2l < target) {
      int h2 = a.heads_per_job, q2 = a.q_splits;
      if (h2 > 1 && h2 % 2 == 0) h2 /= 2;
      else if (q2 < 4) q2 *= 2;
      else break;
      if (part_budget >= 0 && (int64_t)partial_bytes(h2, q2) > part_budget) break;
      a.heads_per_job = h2;
      a.q_splits = q2;
    }
    if (const char* e = std::getenv("FA_BWD_SPLIT")) {  // tuning override "heads_per_job,q_splits"
      int h = 0, q = 0;
      if (std::sscanf(e, "%d,%d", &h, &q) == 2 && h >= 1 && a.G % h == 0 && q >= 1 && q <= 64) {
        a.heads_per_job = h;
        a.q_splits = q;
      }
    }
  };
  const double per_kv = (double)a.ds_groups * (double)a.G * (double)a.ds_w * 8192.0;  // dS bytes of one KV head
  auto ds_bytes = [&](int64_t n2l) {
    return align_up((size_t)a.ds_groups * (size_t)(a.G * n2l) * (size_t)a.ds_w * 8192u);
  };

  a.heads_per_job = a.G;
  a.q_splits = 1;
  p.n2_chunk = (int32_t)N2;
  const int mode = d.dq_mode;
  if (d.flags & FA_FLAG_FP32_OUT) {
    a.variant = 3;  // fp32 debugging form: sfmg + two VALU kernels
  } else if (mode == FA_DQ_FUSED || (mode == FA_DQ_AUTO && fused_ok)) {
    if (!fused_ok) return FA_ERR_UNSUPPORTED;
    a.variant = 5;
  } else if (mode == FA_DQ_ATOMIC) {
    a.variant = fabwd::main_v2_instantiated(d.D, d.Dv) ? 1 : 0;
    if (a.variant == 1 && a.G > 1) a.heads_per_job = 1;
  } else {
    a.variant = 0;
    if (mode == FA_DQ_STORED_DS || mode == FA_DQ_AUTO) {
      // the largest chunk of whole KV heads whose dS fits (4 GiB, or what the
      // bound leaves beside sfmg), then the split for launches of that many
      // heads in what remains
      const double room = bound ? (double)bound - (double)sfmg_bytes : 4.0 * 1024 * 1024 * 1024;
      int64_t chunk = room > 0 ? (int64_t)std::min<double>((double)N2, std::floor(room / per_kv)) : 0;
      while (chunk >= 1 && bound && (uint64_t)(sfmg_bytes + ds_bytes(chunk)) > bound) --chunk;  // alignment
      if (chunk < 1 && mode == FA_DQ_STORED_DS && !bound) chunk = 1;  // forced: one KV head at a time
      if (chunk >= 1) {
        a.variant = 4;
        p.n2_chunk = (int32_t)chunk;
        split_for(chunk, bound ? (int64_t)bound - (int64_t)(sfmg_bytes + ds_bytes(chunk)) : -1);
      } else if (mode == FA_DQ_STORED_DS) {
        return FA_ERR_WORKSPACE;
      }
    }
    if (a.variant == 0) {  // recompute: sfmg and the partial sums only
      if (bound && sfmg_bytes > bound) return FA_ERR_WORKSPACE;
      a.variant = 2;
      split_for(N2, bound ? (int64_t)(bound - sfmg_bytes) : -1);
    }
  }
  a.n2_begin = 0;
  a.n2_count = (int32_t)N2;
  a.ds_heads = (int32_t)(a.G * p.n2_chunk);
  const bool pair = a.variant == 2 || a.variant == 4;
  a.n_partials = pair ? (a.G / a.heads_per_job) * a.q_splits : 1;
  a.k_part_stride = k_elems;
  a.v_part_stride = v_elems;
  // dQ GEMM: two step groups per workgroup when its grid fits one round of two
  // workgroups per CU (the longest row groups of a causal mask then take half
  // as long) and no partial-sum reduce runs in its tail
  a.dq_groups = 1;
  if (a.variant == 4 && d.D <= 128) {
    const bool tail = p.n2_chunk >= N2 && a.n_partials > 1;
    const int64_t wgs = (S1 + 127) / 128 * a.G * p.n2_chunk * d.B;
    if (!tail && wgs <= 2 * (int64_t)cus) a.dq_groups = 2;
  }
  a.round_wgs = pair ? cus : 0;  // the dK/dV kernel holds one workgroup per CU
  // Varlen grids run each sequence's key tiles together: sequences of unequal
  // lengths then spread over every shader engine (in key-tile order the
  // sequence index alone picks the engine pair), and neighbouring tiles of a
  // sequence share their query rows in L2.
  a.seq_major = pair && tnd ? 1 : 0;

  // workspace: sfmg, [dQ accumulator], [dK / dV partial sums], [dS]
  p.off_sfmg = 0;
  p.off_dq_acc = 0;
  size_t cur = a.variant == 5 ? 0 : sfmg_bytes;  // the fused kernel forms sfmg itself
  if (a.variant < 2) {
    p.off_dq_acc = cur;
    cur += align_up((size_t)p.q_elems * sizeof(float));
  }
  p.off_dk_acc = p.off_dv_acc = cur;
  if (fabwd::split_heads(a) || (pair && a.n_partials > 1)) {
    const size_t parts = pair ? (size_t)a.n_partials : 1;
    p.off_dk_acc = cur;
    cur += align_up(parts * (size_t)k_elems * sizeof(float));
    p.off_dv_acc = cur;
    cur += align_up(parts * (size_t)v_elems * sizeof(float));
  }
  p.off_ds = cur;
  if (a.variant == 4) cur += ds_bytes(p.n2_chunk);  // 4 tiles of 32 x 32 elements per (group, head of a chunk, slot)
  if (bound && cur > bound) return FA_ERR_WORKSPACE;  // e.g. the atomic kernels' dQ accumulator
  p.ws_bytes = cur;
  p.desc = d;
  p.desc.S1 = (int32_t)S1;
  p.desc.S2 = (int32_t)S2;
  p.desc.host_cu_seqlens_q = nullptr;   // host copies are not kept
  p.desc.host_cu_seqlens_kv = nullptr;
  return FA_OK;
}

int check_run_pointers(const fa_bwd_plan_s& p, const int32_t* cu_q, const int32_t* cu_kv) {
  const bool tnd = p.desc.layout == FA_LAYOUT_TND;
  if (tnd && (!cu_q || !cu_kv)) return FA_ERR_SHAPE;
  if (!tnd && (cu_q || cu_kv)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Element tensors move in 16-byte pieces (copies to LDS, vector loads, row
// stores); float32 and int32 arrays in 4-byte words.  NULL passes (optional
// arrays).
bool aligned(std::initializer_list<const void*> t16, std::initializer_list<const void*> t4) {
  for (const void* p : t16)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  for (const void* p : t4)
    if (reinterpret_cast<uintptr_t>(p) & 3) return false;
  return true;
}

}  // namespace

extern "C" {

int fa_bwd_create(const fa_bwd_desc* desc, fa_bwd_plan* plan, size_t* workspace_bytes) {
  if (!desc || !plan || !workspace_bytes) return FA_ERR_NULLPTR;
  *plan = nullptr;
  fa_bwd_plan_s* p = new (std::nothrow) fa_bwd_plan_s();
  if (!p) return FA_ERR_RUNTIME;
  int st = validate_and_plan(*desc, *p);
  if (st != FA_OK) {
    delete p;
    return st;
  }
  *plan = p;
  *workspace_bytes = p->ws_bytes;
  if (log_enabled()) {
    const KernelArgs& a = p->args;
    std::fprintf(stderr,
                 "[fa_bwd] plan layout=%d B=%d N1=%d N2=%d S1=%d S2=%d D=%d Dv=%d T1=%lld T2=%lld "
                 "scale=%g window=(%d,%d) variant=%d heads_per_job=%d q_splits=%d partials=%d kv_chunk=%d "
                 "dq_groups=%d round_wgs=%d seq_major=%d workspace=%zu B\n",
                 p->desc.layout, a.B, a.N1, a.N2, a.S1, a.S2, a.D, a.Dv, (long long)a.T1,
                 (long long)a.T2, (double)a.scale, a.win_left, a.win_right, a.variant,
                 a.heads_per_job, a.q_splits, a.n_partials, p->n2_chunk, a.dq_groups, a.round_wgs, a.seq_major,
                 p->ws_bytes);
  }
  return FA_OK;
}

int fa_bwd_run(fa_bwd_plan plan, const void* q, const void* k, const void* v, const void* dout,
               const void* attn_out, const float* softmax_lse, const int32_t* cu_seqlens_q,
               const int32_t* cu_seqlens_kv, const int32_t* seqused_q, const int32_t* seqused_kv, void* dq,
               void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !q || !k || !v || !dout || !attn_out || !softmax_lse || !dq || !dk || !dv)
    return FA_ERR_NULLPTR;
  int st = check_run_pointers(*plan, cu_seqlens_q, cu_seqlens_kv);
  if (st != FA_OK) return st;
  if (!aligned({q, k, v, dout, attn_out, dq, dk, dv}, {softmax_lse, cu_seqlens_q, cu_seqlens_kv, seqused_q, seqused_kv}))
    return FA_ERR_PARAM_INVALID;
  if (plan->ws_bytes > 0 && (!workspace || workspace_bytes < plan->ws_bytes)) return FA_ERR_WORKSPACE;
  // the atomic kernels do not read seqused
  if ((seqused_q || seqused_kv) && plan->args.variant < 2) return FA_ERR_UNSUPPORTED;

  KernelArgs a = plan->args;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.out = attn_out; a.lse = softmax_lse;
  a.cu_q = cu_seqlens_q; a.cu_kv = cu_seqlens_kv;
  a.seqused_q = seqused_q; a.seqused_kv = seqused_kv;
  a.dq = dq; a.dk = dk; a.dv = dv;
  char* ws = static_cast<char*>(workspace);
  a.sfmg = reinterpret_cast<float*>(ws + plan->off_sfmg);
  if (a.variant < 2) a.dq_acc = reinterpret_cast<float*>(ws + plan->off_dq_acc);
  a.dk_acc = reinterpret_cast<float*>(ws + plan->off_dk_acc);
  a.dv_acc = reinterpret_cast<float*>(ws + plan->off_dv_acc);
  a.ds = a.variant == 4 ? ws + plan->off_ds : nullptr;

  if (a.variant == 5) {  // one launch: sfmg, dK/dV and dQ per (sequence, KV head)
    if (plan->prof && fabwd::profiler_begin(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (fabwd::launch_fused(a, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_end(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    return FA_OK;
  }
  if (a.variant == 3) {
    if (fabwd::launch_preprocess(a, false, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_begin(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (fabwd::launch_f32_debug(a, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_end(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    return FA_OK;
  }
  if (a.variant == 4) {
    // sfmg -> dK/dV kernel (which also stores dS) -> dQ GEMM over the stored
    // dS -> partial-sum reduce (when a key tile is split over jobs)
    if (fabwd::launch_preprocess(a, false, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_begin(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    // unchunked, the dQ GEMM launch also adds the partial sums (in its last
    // workgroups); chunked, the reduce runs once after the last chunk
    const bool one_pass = plan->n2_chunk >= a.N2;
    a.reduce_tail = one_pass && a.n_partials > 1 ? 1 : 0;
    for (int32_t n2b = 0; n2b < a.N2; n2b += plan->n2_chunk) {  // one pass unless dS is chunked
      a.n2_begin = n2b;
      a.n2_count = std::min(plan->n2_chunk, a.N2 - n2b);
      if (fabwd::launch_dkdv(a, stream) != 0) return FA_ERR_RUNTIME;
      if (plan->prof && one_pass && fabwd::profiler_mark(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
      if (fabwd::launch_dq_ds(a, stream) != 0) return FA_ERR_RUNTIME;
    }
    a.n2_begin = 0;
    a.n2_count = a.N2;
    if (plan->prof && fabwd::profiler_end(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (!a.reduce_tail && fabwd::launch_reduce_parts(a, stream) != 0) return FA_ERR_RUNTIME;
    return FA_OK;
  }
  if (a.variant == 2) {
    // dQ kernel (which also forms sfmg) -> dK/dV kernel (which reads it) ->
    // partial-sum reduce (when a key tile is split over jobs)
    if (plan->prof && fabwd::profiler_begin(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (fabwd::launch_dq(a, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_mark(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (fabwd::launch_dkdv(a, stream) != 0) return FA_ERR_RUNTIME;
    if (plan->prof && fabwd::profiler_end(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
    if (fabwd::launch_reduce_parts(a, stream) != 0) return FA_ERR_RUNTIME;
    return FA_OK;
  }
  if (fabwd::launch_preprocess(a, true, stream) != 0) return FA_ERR_RUNTIME;
  if (plan->prof && fabwd::profiler_begin(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
  if (fabwd::launch_main(a, stream) != 0) return FA_ERR_RUNTIME;
  if (plan->prof && fabwd::profiler_end(plan->prof, stream) != 0) return FA_ERR_RUNTIME;
  if (fabwd::launch_dq_finalize(a, stream) != 0) return FA_ERR_RUNTIME;
  return FA_OK;
}

int fa_bwd_run_noalloc(fa_bwd_plan plan, const void* q, const void* k, const void* v, const void* dout,
                       const void* attn_out, const float* softmax_lse, const int32_t* cu_seqlens_q,
                       const int32_t* cu_seqlens_kv, const int32_t* seqused_q, const int32_t* seqused_kv, void* dq,
                       void* dk, void* dv, void* stream) {
  static_assert(fabwd::SCRATCH_BYTES == FA_BWD_SCRATCH_BYTES, "one scratch size");
  if (!plan) return FA_ERR_NULLPTR;
  if (plan->ws_bytes > FA_BWD_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  // the argument checks of fa_bwd_run come first, before any device call
  if (!q || !k || !v || !dout || !attn_out || !softmax_lse || !dq || !dk || !dv) return FA_ERR_NULLPTR;
  const int st = check_run_pointers(*plan, cu_seqlens_q, cu_seqlens_kv);
  if (st != FA_OK) return st;
  if (!aligned({q, k, v, dout, attn_out, dq, dk, dv}, {softmax_lse, cu_seqlens_q, cu_seqlens_kv, seqused_q, seqused_kv}))
    return FA_ERR_PARAM_INVALID;
  if ((seqused_q || seqused_kv) && plan->args.variant < 2) return FA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (plan->ws_bytes > 0 && fabwd::scratch_ptr(&scratch) != 0) return FA_ERR_RUNTIME;
  return fa_bwd_run(plan, q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q, cu_seqlens_kv, seqused_q, seqused_kv,
                    dq, dk, dv, scratch, plan->ws_bytes > 0 ? FA_BWD_SCRATCH_BYTES : 0, stream);
}

int fa_fwd_run(fa_bwd_plan plan, const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
               const int32_t* cu_seqlens_kv, const int32_t* seqused_q, const int32_t* seqused_kv, void* attn_out,
               float* softmax_lse, void* stream) {
  if (!plan || !q || !k || !v || !attn_out || !softmax_lse) return FA_ERR_NULLPTR;
  int st = check_run_pointers(*plan, cu_seqlens_q, cu_seqlens_kv);
  if (st != FA_OK) return st;
  if (!aligned({q, k, v, attn_out}, {softmax_lse, cu_seqlens_q, cu_seqlens_kv, seqused_q, seqused_kv}))
    return FA_ERR_PARAM_INVALID;
  KernelArgs a = plan->args;
  a.q = q; a.k = k; a.v = v;
  a.cu_q = cu_seqlens_q; a.cu_kv = cu_seqlens_kv;
  a.seqused_q = seqused_q; a.seqused_kv = seqused_kv;
  if (fabwd::launch_forward(a, attn_out, softmax_lse, stream) != 0) return FA_ERR_RUNTIME;
  return FA_OK;
}

int fa_bwd_plan_dq_path(fa_bwd_plan plan, int* path) {
  if (!plan || !path) return FA_ERR_NULLPTR;
  switch (plan->args.variant) {
    case 5: *path = FA_DQ_FUSED; break;
    case 4: *path = FA_DQ_STORED_DS; break;
    case 2: *path = FA_DQ_RECOMPUTE; break;
    case 3: *path = FA_DQ_FP32_FORM; break;
    default: *path = FA_DQ_ATOMIC; break;
  }
  return FA_OK;
}

int fa_bwd_profile_enable(fa_bwd_plan plan, int slots) {
  if (!plan) return FA_ERR_NULLPTR;
  if (slots < 0 || slots > 65536) return FA_ERR_PARAM_INVALID;
  fabwd::profiler_destroy(plan->prof);
  plan->prof = nullptr;
  if (slots == 0) return FA_OK;
  plan->prof = fabwd::profiler_create(slots);
  return plan->prof ? FA_OK : FA_ERR_RUNTIME;
}

int fa_bwd_profile_read(fa_bwd_plan plan, float* ms, int cap, int* count) {
  if (!plan || !ms || !count) return FA_ERR_NULLPTR;
  *count = 0;
  if (!plan->prof) return FA_OK;
  return fabwd::profiler_read(plan->prof, ms, nullptr, cap, count) == 0 ? FA_OK : FA_ERR_RUNTIME;
}

int fa_bwd_profile_read_split(fa_bwd_plan plan, float* first_ms, float* second_ms, int cap, int* count) {
  if (!plan || !first_ms || !second_ms || !count) return FA_ERR_NULLPTR;
  *count = 0;
  if (!plan->prof) return FA_OK;
  return fabwd::profiler_read(plan->prof, first_ms, second_ms, cap, count) == 0 ? FA_OK : FA_ERR_RUNTIME;
}

int fa_bwd_sfmg(fa_bwd_plan plan, const void* dout, const void* attn_out,
                const int32_t* cu_seqlens_q, float* sfmg, void* stream) {
  if (!plan || !dout || !attn_out || !sfmg) return FA_ERR_NULLPTR;
  const bool tnd = plan->desc.layout == FA_LAYOUT_TND;
  if (tnd != (cu_seqlens_q != nullptr)) return FA_ERR_SHAPE;
  if (!aligned({dout, attn_out}, {cu_seqlens_q, sfmg})) return FA_ERR_PARAM_INVALID;
  KernelArgs a = plan->args;
  a.dout = dout; a.out = attn_out; a.cu_q = cu_seqlens_q; a.sfmg = sfmg;
  if (fabwd::launch_preprocess(a, false, stream) != 0) return FA_ERR_RUNTIME;
  return FA_OK;
}

int fa_bwd_destroy(fa_bwd_plan plan) {
  if (plan) fabwd::profiler_destroy(plan->prof);
  delete plan;
  return FA_OK;
}

const char* fa_bwd_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_PARAM_INVALID: return "invalid parameter (dtype, layout, mask_mode, flags, abi_version or scale)";
    case FA_ERR_SHAPE: return "shape constraint violated (sizes, N1 % N2, Dv <= D <= 192, window, cu_seqlens)";
    case FA_ERR_UNSUPPORTED: return "combination not built in this library";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_RUNTIME: return "HIP runtime or kernel launch failure";
    default: return "unknown status";
  }
}

int fa_bwd_abi_version(void) { return FA_BWD_ABI_VERSION; }

}  // extern "C"
