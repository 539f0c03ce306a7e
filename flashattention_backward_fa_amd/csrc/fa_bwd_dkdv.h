// gfx950 (MI355X) FlashAttention backward: the dK/dV kernel (key tiles in
// parallel), which in the stored-dS chain also writes dS for the dQ GEMM
// (fa_bwd_det_kernels.hip).  The template lives here; fa_bwd_dkdv_kernels.hip
// instantiates it for D <= 128 and fa_bwd_dkdv192_kernels.hip for D = 192, so
// that each is compiled with the scheduling strategy that suits it.
//
// Formulas: page "CANN ops-transformer FlashAttnGrad 算子详解", section 一
// (P = exp(scale*QK^T - softmax_lse), dV = P^T dY, dP = dY V^T,
// sfmg = rowsum(dY (.) Y), dS = P (.) (dP - sfmg), dK = scale*dS^T Q).
//
// One workgroup owns a 128-key tile of one (sequence, key/value head): 4
// wavefronts of 32 keys in each of QG query groups (QG = 2 at D <= 128, two
// wavefronts per SIMD; QG = 1 at D = 192).  K and V stay in LDS; the groups
// take alternate 32-row query blocks, whose Q and dY tiles are copied global ->
// LDS one block ahead (double-buffered).  S = Q K^T and dP = dY V^T use query
// rows as M and keys as N of v_mfma_f32_32x32x16_bf16, so each lane holds one
// key and 16 query rows: exactly the A-operand layout of the key-major products
// dV += P^T dY and dK += dS^T Q, whose B operands (dY and Q read down their
// columns) come from ds_read_b64_tr_b16.  A job is (key tile, query-head slot,
// query-range split, sequence, key/value head).  When a key tile is split over
// several jobs (GQA heads, or query ranges for balance) each job stores fp32
// partial sums and a reduce kernel adds them; otherwise the job writes 16-bit
// dK/dV directly.

#pragma once

#include <hip/hip_runtime.h>

#include "fa_bwd_tiles.h"

namespace fabwd {
namespace dkdv {

// ------------------------------------------------------------------ dK / dV

// QG query groups of NWG wavefronts share one tile of NWG*KPW keys; wavefront
// w of each group owns keys w*KPW .. w*KPW+KPW-1 of the tile.  The groups take
// alternate 32-row query blocks; each group double-buffers its Q/dY tile so a
// step needs one barrier.  K/V tiles use a padded pitch (16-byte row reads
// only); Q/dY tiles are swizzled (row reads and transposing reads).
// Instantiated with NWG = 4, KPW = 32: 8 wavefronts in two query groups (two
// per SIMD) at D <= 128, 4 wavefronts in one group at D = 192.
// DS: also store each (32-row block, 32-key slice) tile of dS for the dQ GEMM
// (dq_ds_kernel), as row-major [32 keys][128 rows] tiles of a 128-row group.
template <int HD, int HDV, int KPW, int NWG, int QG, bool F16, bool DS>
__global__ __launch_bounds__(64 * NWG * QG, 1) void dkdv_kernel(KernelArgs a) {
  constexpr int BC = NWG * KPW;       // keys per workgroup
  constexpr int NKB = KPW / 32;       // 32-key blocks per wavefront
  static_assert(!DS || NKB == 1, "the dS stores assume one 32-key slice per wavefront");
  constexpr int BR = 32;              // query rows per step and group
  constexpr int KP = HD + 8;          // padded pitches of the K and V tiles
  constexpr int VP = HDV + 8;
  constexpr int NKQ = HD / 16;
  constexpr int NKV = HDV / 16;
  constexpr int NBK = HD / 32;
  constexpr int NBV = HDV / 32;
  constexpr int QTB = BR * HD * 2;    // bytes of one Q / dY tile buffer
  constexpr int YTB = BR * HDV * 2;

  __shared__ __attribute__((aligned(1024))) bf16 Ks[BC * KP];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[BC * VP];
  __shared__ __attribute__((aligned(1024))) bf16 Qs[QG][2][BR * HD];
  __shared__ __attribute__((aligned(1024))) bf16 Ys[QG][2][BR * HDV];
  __shared__ __attribute__((aligned(16))) float lse_s[QG][2][BR];
  __shared__ __attribute__((aligned(16))) float sfm_s[QG][2][BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave / NWG;     // query group
  const int kw = wave % NWG;     // key slice
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // job = ((((tile * HJ + hslot) * QS + qs) * B + b) * N2 + n2), longest first
  // under a causal mask, or for varlen grids (seq_major)
  // ((((b * HJ + hslot) * QS + qs) * tiles + tile) * N2 + n2), so that a
  // sequence's tiles run together.
  // The dispatcher sends workgroup i to XCD i % 8 and, within the XCD, to its
  // four shader engines in turn ((i / 8) % 4), each workgroup waiting for a CU
  // of its own engine while the XCD's later ones wait behind it.  In the even
  // rounds of the grid (round_wgs workgroups each, one per CU) the engines
  // take the jobs of each 32 in reverse (i ^ 24 flips bits 3-4), so that the
  // shortest job of the round, whose CU frees first, sits in the engine that
  // the next round's first workgroup asks for.  XCD placement is unchanged.
  // Sequence-major grids, whose jobs are of near-equal length under a window,
  // keep the plain order (measured slightly faster there).
  const int hpj = a.heads_per_job;
  const int HJ = a.G / hpj;
  const int QS = a.q_splits;
  int r = blockIdx.x;
  if (a.round_wgs > 0 && !a.seq_major && ((r / a.round_wgs) & 1) == 0 && (r | 31) < (int)gridDim.x) r ^= 24;
  // The two orders differ only in which of (b, tile) is the fast index, so one
  // decomposition serves both (selects, no branches).
  const int nfast = a.seq_major ? (a.S2 + BC - 1) / BC : a.B;
  const int n2 = a.n2_begin + r % a.n2_count; r /= a.n2_count;
  const int fast = r % nfast; r /= nfast;
  const int qs = r % QS; r /= QS;
  const int hslot = r % HJ;
  const int slow = r / HJ;
  const int b = a.seq_major ? slow : fast;
  const int tile = a.seq_major ? fast : slow;
  const int part = hslot * QS + qs;

  const SeqBounds sb = seq_bounds(a, b);
  const int s1 = sb.s1, s2 = sb.s2;
  const int j0 = tile * BC;
  if (j0 >= sb.s2a) return;
  // a tile past the used keys (seqused_kv) computes nothing and writes zeros
  const bool live = j0 < s2;
  const int j1 = min(j0 + BC, s2);
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;

  // K and V tiles, asynchronously (rows past the sequence end repeat its last key)
  const int kvalid = (live ? s2 : sb.s2a) - j0;
  padded_copy<HD, BC, NWG * QG>(lds_addr(Ks), static_cast<const bf16*>(a.k) + sb.kbase + (int64_t)n2 * a.k_sn + (int64_t)j0 * a.k_ss,
                                (int)a.k_ss * 2, kvalid, wave, lane);
  padded_copy<HDV, BC, NWG * QG>(lds_addr(Vs), static_cast<const bf16*>(a.v) + sb.vbase + (int64_t)n2 * a.v_sn + (int64_t)j0 * a.v_ss,
                               (int)a.v_ss * 2, kvalid, wave, lane);

  // query blocks that see a key of [j0, j1); this job takes split qs of them
  const fa_sched::Span blks =
      live ? fa_sched::split_part(fa_sched::blocks_covering(fa_sched::rows_seeing(s1, j0, j1, off, wl, wr), BR), qs, QS)
           : fa_sched::Span{0, 0};
  const int bs_lo = blks.lo;
  const int nblk = blks.hi - blks.lo;
  const int T = hpj * nblk;  // items: (query head, query block) pairs
  const int g0 = hslot * hpj;

  // Item t = it*QG + qg of this group is query head g0 + t / nblk, block
  // bs_lo + t % nblk; a cursor walks it without divisions.
  struct Cursor { int h, blk; };
  auto step_cursor = [&](Cursor& c, int n) {
    if (nblk == 0) return;  // no items at all (the loop below would not end)
    c.blk += n;
    while (c.blk >= nblk) { c.blk -= nblk; ++c.h; }
  };

  // Q/dY tiles of an item go straight to LDS (async); lse and sfmg of its rows
  // go through registers of wavefront kw = 0, raw and loaded first, so that
  // nothing waits for them before the tile itself is awaited.
  TileCopy<HD, BR, NWG> qcp;
  TileCopy<HDV, BR, NWG> ycp;
  const uint32_t q_lds = lds_addr(Qs) + qg * 2 * QTB;  // this group's Q / dY buffers
  const uint32_t y_lds = lds_addr(Ys) + qg * 2 * YTB;
  qcp.init(kw, lane, (int)a.q_ss * 2);
  ycp.init(kw, lane, (int)a.o_ss * 2);
  float pl = 0.f, pf = 0.f;
  // The fetch side walks its items with running pointers to the Q and dY
  // tiles and to the head's lse / sfmg rows, advanced by additions only.
  struct FetchCursor { int h, blk; const bf16* qp; const bf16* yp; const float* lp; const float* sp; };
  const int64_t q_adv = (int64_t)QG * BR * a.q_ss, y_adv = (int64_t)QG * BR * a.o_ss;
  const int64_t q_wrap = a.q_sn - (int64_t)nblk * BR * a.q_ss, y_wrap = a.o_sn - (int64_t)nblk * BR * a.o_ss;
  auto fc_init = [&](FetchCursor& f) {
    const int n1 = n2 * a.G + g0 + f.h;
    const int i0 = (bs_lo + f.blk) * BR;
    f.qp = static_cast<const bf16*>(a.q) + sb.qbase + (int64_t)n1 * a.q_sn + (int64_t)i0 * a.q_ss;
    f.yp = static_cast<const bf16*>(a.dout) + sb.obase + (int64_t)n1 * a.o_sn + (int64_t)i0 * a.o_ss;
    f.lp = a.lse + sb.lbase + (int64_t)n1 * a.l_sn;
    f.sp = a.sfmg + sb.lbase + (int64_t)n1 * a.l_sn;
  };
  auto fc_step = [&](FetchCursor& f) {  // to the group's next item
    if (nblk == 0) return;  // no items at all (the loop below would not end)
    f.blk += QG;
    f.qp += q_adv;
    f.yp += y_adv;
    while (f.blk >= nblk) {
      f.blk -= nblk;
      ++f.h;
      f.qp += q_wrap;
      f.yp += y_wrap;
      f.lp += a.l_sn;
      f.sp += a.l_sn;
    }
  };
  auto fetch = [&](const FetchCursor& f, int t, int buf) {
    if (t < T) {
      const int i0 = (bs_lo + f.blk) * BR;
      if (kw == 0) {
        const int lrow = min(i0 + l32, s1 - 1);
        pl = f.lp[lrow];
        pf = f.sp[lrow];
      }
      qcp.issue(q_lds + buf * QTB, f.qp, s1 - i0, kw, lane);
      ycp.issue(y_lds + buf * YTB, f.yp, s1 - i0, kw, lane);
    }
  };
  // lse in base 2 for the rows of the block at i0; a row past the end or an
  // empty row (lse = -inf) gets +inf, so that its P is 0
  auto put_row_stats = [&](int i0, int buf) {
    if (kw == 0 && lane < BR) {
      lse_s[qg][buf][lane] = (i0 + lane >= s1 || pl == -__builtin_inff()) ? __builtin_inff() : pl * kLog2e;
      sfm_s[qg][buf][lane] = pf;
    }
  };

  floatx16 dKr[NKB][NBK], dVr[NKB][NBV];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int i = 0; i < NBK; ++i) dKr[kb][i] = floatx16{};
#pragma unroll
    for (int i = 0; i < NBV; ++i) dVr[kb][i] = floatx16{};
  }

  SwzTile<HD, BR> qadr;
  SwzTile<HDV, BR> yadr;
  qadr.init(q_lds, lane);
  yadr.init(y_lds, lane);
  const int kw0 = kw * KPW;  // first key of this wavefront within the tile
  const uint32_t k_lane = lds_addr(Ks) + ((kw0 + l32) * KP + 8 * hi) * 2;
  const uint32_t v_lane = lds_addr(Vs) + ((kw0 + l32) * VP + 8 * hi) * 2;

  // DS form: the dS of the last item, kept until the next step has passed its
  // barrier and issued its prefetch, so that the stores have a whole step to
  // drain before the next s_waitcnt vmcnt(0), which also counts them.
  bf16x8 ds_keep[NKB][2];
  int ds_i0 = -1, ds_n1 = 0;
  // Tile (query block qb, 32-key slice ks) of dS is the register image of the
  // wavefront that formed it: 2 halves x 64 lanes x 8 elements, half h of lane
  // p holding rows 16h + 8*(e/4) + 4*(p/32) + e%4 (e = 0..7) of key p%32.
  // Each half is one 1 KB store instruction.  The 4 tiles of a 128-row query
  // group and slice are consecutive, at slot ks - (the group's first slice).
  // (The group and slot guards keep the stores inside the workspace even for a
  // sequence longer than the maximum length the plan was made for.)
  // Per job: this wavefront's slice, the query blocks that see a key of it
  // (the tiles that are stored), the group of row group 0 and the group stride.
  const int ds_ks = (j0 + kw0) >> 5;
  const fa_sched::Span ds_vis =
      ds_ks * 32 < s2 ? fa_sched::blocks_covering(fa_sched::rows_seeing(s1, ds_ks * 32, min(ds_ks * 32 + 32, s2), off, wl, wr), 32)
                      : fa_sched::Span{0, 0};
  const int64_t ds_g0 = ds_group(a, sb, 0);  // the group of row group R is ds_g0 + R
  const int64_t ds_gstride = (int64_t)a.ds_heads * a.ds_w * 4;
  auto ds_flush = [&]() {
    if (DS && ds_i0 >= 0) {
      const int qb = ds_i0 >> 5, R = ds_i0 >> 7;
      const int slot = ds_ks - ds_band_lo(R, s1, s2, off, wl, wr);
      const int64_t g = ds_g0 + R;
      if ((a.varlen || R < a.ds_nr) && g < a.ds_groups && (unsigned)slot < (unsigned)a.ds_w && qb >= ds_vis.lo &&
          qb < ds_vis.hi) {
        const int64_t tile0 = g * ds_gstride + (int64_t)(((ds_n1 - a.n2_begin * a.G) * a.ds_w + slot) * 4 + (qb & 3));
        bf16* dsg = static_cast<bf16*>(a.ds) + tile0 * 1024 + lane * 8;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            __builtin_nontemporal_store(ds_keep[kb][h], reinterpret_cast<bf16x8*>(dsg + kb * 4096 + h * 512));
        }
      }
    }
    ds_i0 = -1;
  };

  floatx16 sacc[NKB], pacc[NKB];
  // S = Q K^T and dP = dY V^T for this wavefront's KPW keys
  // Each run of MFMAs raises the wavefront's issue priority, so that on a SIMD
  // shared by two wavefronts the one with matrix work issues first and the
  // other's exp / LDS work fills the MFMA pipe's shadow.
  auto phase_a = [&](int buf) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = floatx16{};
      pacc[kb] = floatx16{};
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < NKQ; ++kk) {
      const bf16x8 qa = lds_load16(qadr.row_read_c(kk, buf * QTB));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = mfma32<F16>(qa, lds_load16(k_lane + (kb * 32 * KP + 16 * kk) * 2), sacc[kb]);
    }
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) {
      const bf16x8 ya = lds_load16(yadr.row_read_c(kk, buf * YTB));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) pacc[kb] = mfma32<F16>(ya, lds_load16(v_lane + (kb * 32 * VP + 16 * kk) * 2), pacc[kb]);
    }
    // instruction grouping for the scheduler (0x100: LDS reads, 0x008: MFMAs):
    // eight reads ahead, then each MFMA followed by the two reads of a later one
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < (NKQ + NKV) * NKB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // The 32-row blocks at i0 that see every key of the tile (fa_sched::tile_full
  // as one range of i0): fully inside the sequence, at or past the right
  // window's (causal) edge and not past the left window's.  The D = 192 form
  // tests the range (1.7 % shorter there); the others evaluate tile_full per
  // step, which measured 0.3 % shorter for them.
  int full_lo = 0, full_hi = -1;
  if constexpr (HD == 192) {
    full_lo = wr >= 0 ? j0 + BC - 1 - off - wr : INT_MIN;
    full_hi = j0 + BC > s2 ? INT_MIN : min(s1 - BR, wl >= 0 ? j0 - (BR - 1) - off + wl : INT_MAX);
  }
  // P, dS (masked when the tile is partial), then dV += P^T dY and dK += dS^T Q
  auto phase_b = [&](int buf, int i0, int n1) {
    // P = exp(S*scale - lse) (masked), dS = P (dP - sfmg), packed as bf16 A operands.
    // A tile that every (row, key) pair sees takes the unmasked path; otherwise
    // row i is kept iff it lies in [vis_lo, vis_hi] of the lane's key (one
    // unsigned compare per element, no branches).
    bool full;
    if constexpr (HD == 192)
      full = i0 >= full_lo && i0 <= full_hi;
    else
      full = fa_sched::tile_full(i0, BR, j0, BC, s1, s2, off, wl, wr);
    bf16x8 pa[NKB][2], da[NKB][2];
    if (full) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ib = r4 * 8 + hi * 4;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[qg][buf][ib]);
        const floatx4 f4 = *reinterpret_cast<const floatx4*>(&sfm_s[qg][buf][ib]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if constexpr (F16) {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const int rg = r4 * 4 + e;
              const float p0 = __builtin_amdgcn_exp2f(sacc[kb][rg] * a.scale_log2 - l4[e]);
              const float p1 = __builtin_amdgcn_exp2f(sacc[kb][rg + 1] * a.scale_log2 - l4[e + 1]);
              put_f16_pair(pa[kb][rg >> 3], (rg & 7) >> 1, p0, p1);
              put_f16_pair(da[kb][rg >> 3], (rg & 7) >> 1, p0 * (pacc[kb][rg] - f4[e]),
                           p1 * (pacc[kb][rg + 1] - f4[e + 1]));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rg = r4 * 4 + e;
              const float p = __builtin_amdgcn_exp2f(sacc[kb][rg] * a.scale_log2 - l4[e]);
              pa[kb][rg >> 3][rg & 7] = to_elem<F16>(p);
              da[kb][rg >> 3][rg & 7] = to_elem<F16>(p * (pacc[kb][rg] - f4[e]));
            }
          }
        }
      }
    } else {
      fa_sched::Window vis[NKB];  // visible rows of this lane's key, relative to i0
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        vis[kb] = fa_sched::window(fa_sched::rows_of_key(j0 + kw0 + kb * 32 + l32, s1, s2, off, wl, wr), i0);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ib = r4 * 8 + hi * 4;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[qg][buf][ib]);
        const floatx4 f4 = *reinterpret_cast<const floatx4*>(&sfm_s[qg][buf][ib]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if constexpr (F16) {
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const int rg = r4 * 4 + e;
              float p0 = __builtin_amdgcn_exp2f(sacc[kb][rg] * a.scale_log2 - l4[e]);
              float p1 = __builtin_amdgcn_exp2f(sacc[kb][rg + 1] * a.scale_log2 - l4[e + 1]);
              p0 = fa_sched::in_window(vis[kb], ib + e) ? p0 : 0.f;
              p1 = fa_sched::in_window(vis[kb], ib + e + 1) ? p1 : 0.f;
              put_f16_pair(pa[kb][rg >> 3], (rg & 7) >> 1, p0, p1);
              put_f16_pair(da[kb][rg >> 3], (rg & 7) >> 1, p0 * (pacc[kb][rg] - f4[e]),
                           p1 * (pacc[kb][rg + 1] - f4[e + 1]));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rg = r4 * 4 + e;
              float p = __builtin_amdgcn_exp2f(sacc[kb][rg] * a.scale_log2 - l4[e]);
              p = fa_sched::in_window(vis[kb], ib + e) ? p : 0.f;
              pa[kb][rg >> 3][rg & 7] = to_elem<F16>(p);
              da[kb][rg >> 3][rg & 7] = to_elem<F16>(p * (pacc[kb][rg] - f4[e]));
            }
          }
        }
      }
    }

    if constexpr (DS) {  // stored at the start of the next step (ds_flush)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        ds_keep[kb][0] = da[kb][0];
        ds_keep[kb][1] = da[kb][1];
      }
      ds_i0 = i0;
      ds_n1 = n1;
    }

    // dV += P^T dY, dK += dS^T Q; one transposing read serves all key blocks
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) {
        const bf16x8 yb = join(lds_load_tr(yadr.tr_read_c(kc, 0, nb, buf * YTB)), lds_load_tr(yadr.tr_read_c(kc, 1, nb, buf * YTB)));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) dVr[kb][nb] = mfma32<F16>(pa[kb][kc], yb, dVr[kb][nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) {
        const bf16x8 qb = join(lds_load_tr(qadr.tr_read_c(kc, 0, nb, buf * QTB)), lds_load_tr(qadr.tr_read_c(kc, 1, nb, buf * QTB)));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) dKr[kb][nb] = mfma32<F16>(da[kb][kc], qb, dKr[kb][nb]);
      }
    }
    // the same for the transposing reads: four ahead, then two per MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * (NBV + NBK) * NKB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Step it: wait for item t's tile (buffer buf), prefetch item t + QG into
  // the other buffer, compute item t.
  const int iters = (T + QG - 1) / QG;
  Cursor cc{0, qg};                  // item t being computed
  FetchCursor cf{0, qg, nullptr, nullptr, nullptr, nullptr};  // item being fetched
  step_cursor(cc, 0);
  {
    Cursor c0{0, qg};
    step_cursor(c0, 0);
    cf.h = c0.h;
    cf.blk = c0.blk;
    fc_init(cf);
  }
  fetch(cf, qg, 0);
  fc_step(cf);
  auto step = [&](int it, int buf) {
    const int t = it * QG + qg;
    const int i0 = (bs_lo + cc.blk) * BR;
    if (QG == 1 || t < T) put_row_stats(i0, buf);  // with one group every step has an item
    wait_vmem();    // this wavefront's copies of item t landed
    lds_barrier();  // ... and everyone's; buffer buf ^ 1 is no longer read
    fetch(cf, t + QG, buf ^ 1);
    fc_step(cf);
    if constexpr (DS) ds_flush();
    if (QG == 1 || t < T) {
      phase_a(buf);
      phase_b(buf, i0, n2 * a.G + g0 + cc.h);
    }
    step_cursor(cc, QG);
  };
  // two steps per iteration, so that the buffer offsets are constants
  int it = 0;
  for (; it + 1 < iters; it += 2) {
    step(it, 0);
    step(it + 1, 1);
  }
  if (it < iters) step(it, 0);
  if constexpr (DS) ds_flush();
  wait_vmem();  // no copy may still be landing when LDS is reused below

  // ---- QG = 2: the groups swap halves through LDS (group 1 hands its dK to
  // group 0, group 0 its dV to group 1); each adds the half it received and
  // stores it.  The K, V, Q and dY tiles are no longer read; 32-column block c
  // of [dK | dV] takes 16 KB in the first of them with room left.
  if constexpr (QG > 1) {
    static_assert(QG == 2 && NKB == 1, "two groups of one 32-key slice per wavefront");
    constexpr int CH = NWG * 16 * 64 * 4;
    constexpr int nK = (int)sizeof(Ks) / CH, nV = (int)sizeof(Vs) / CH, nQ = (int)sizeof(Qs) / CH;
    static_assert(nK + nV + nQ + (int)sizeof(Ys) / CH >= NBK + NBV, "LDS room for one group's dK and dV");
    auto chunk = [&](int c) -> float* {
      char* p = c < nK             ? reinterpret_cast<char*>(Ks) + c * CH
                : c < nK + nV      ? reinterpret_cast<char*>(Vs) + (c - nK) * CH
                : c < nK + nV + nQ ? reinterpret_cast<char*>(&Qs[0][0][0]) + (c - nK - nV) * CH
                                   : reinterpret_cast<char*>(&Ys[0][0][0]) + (c - nK - nV - nQ) * CH;
      return reinterpret_cast<float*>(p);
    };
    __syncthreads();
    if (qg == 1) {
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) xput(chunk(nb), kw, lane, dKr[0][nb]);
    } else {
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) xput(chunk(NBK + nb), kw, lane, dVr[0][nb]);
    }
    __syncthreads();
    if (qg == 0) {
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) xadd(chunk(nb), kw, lane, dKr[0][nb]);
    } else {
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) xadd(chunk(NBK + nb), kw, lane, dVr[0][nb]);
    }
  }
  const bool st_k = QG == 1 || qg == 0, st_v = QG == 1 || qg == 1;

  // ---- output: 16-bit dK / dV when this job alone covers the key tile, as
  // 16-byte row pieces (the accumulators transposed on MFMA first); else fp32
  // partial sums, one column per lane
  static_assert(NKB == 1, "one 32-key slice per wavefront");
  if (a.n_partials == 1) {
    bf16x8 eye[2];
    eye_operand<F16>(lane, eye);
    const int jr = j0 + kw0 + l32;  // the key of this lane's row
    const bool ok = jr < sb.s2a;    // keys past the used ones hold zeros
    auto put = [&](bf16* row, const floatx16& acc, float mul, int nb) {
      u32x4 piece[2];
      row_pieces<F16>(transpose_acc<F16>(acc, mul, eye), 1.f, piece);
      if (ok) {
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) *reinterpret_cast<u32x4*>(row + nb * 32 + pc * 16 + hi * 8) = piece[pc];
      }
    };
    if (st_k) {
      bf16* row = static_cast<bf16*>(a.dk) + sb.kbase + (int64_t)n2 * a.k_sn + (int64_t)jr * a.k_ss;
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) put(row, dKr[0][nb], a.scale, nb);
    }
    if (st_v) {
      bf16* row = static_cast<bf16*>(a.dv) + sb.vbase + (int64_t)n2 * a.v_sn + (int64_t)jr * a.v_ss;
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) put(row, dVr[0][nb], 1.f, nb);
    }
    return;
  }
  const int64_t kpart = (int64_t)part * a.k_part_stride;
  const int64_t vpart = (int64_t)part * a.v_part_stride;
#pragma unroll
  for (int rg = 0; rg < 16; ++rg) {
    const int j = j0 + kw0 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
    if (j >= sb.s2a) continue;  // keys past the used ones hold zeros
    const int64_t ko = sb.kbase + (int64_t)n2 * a.k_sn + (int64_t)j * a.k_ss;
    const int64_t vo = sb.vbase + (int64_t)n2 * a.v_sn + (int64_t)j * a.v_ss;
    if (st_k) {
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) a.dk_acc[kpart + ko + nb * 32 + l32] = dKr[0][nb][rg] * a.scale;
    }
    if (st_v) {
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) a.dv_acc[vpart + vo + nb * 32 + l32] = dVr[0][nb][rg];
    }
  }
}

// The D = 192 instantiations (fa_bwd_dkdv192_kernels.hip).
int launch_d192(const KernelArgs& a, bool ds, dim3 grid, hipStream_t s);

}  // namespace dkdv
}  // namespace fabwd
