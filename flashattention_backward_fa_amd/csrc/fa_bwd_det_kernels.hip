// gfx950 (MI355X) FlashAttention backward, atomic-free dQ paths (query tiles
// in parallel): a GEMM over the dS that the dK/dV kernel stored (dq_ds_kernel,
// the default), or a pass that recomputes S and dP (dq_kernel); and the reduce
// of split dK/dV partial sums.  The dK/dV kernel is in fa_bwd_dkdv_kernels.hip.
//
// Formulas: page "CANN ops-transformer FlashAttnGrad 算子详解", section 一
// (P = exp(scale*QK^T - softmax_lse), dV = P^T dY, dP = dY V^T,
// sfmg = rowsum(dY (.) Y), dS = P (.) (dP - sfmg), dQ = scale*dS K,
// dK = scale*dS^T Q).  The page's own kernel reduces dQ across key tiles with
// atomic adds into an fp32 workspace (section 五 5.2).  On MI355X fp32
// atomics reach about 1.35 TB/s against about 7.5 TB/s for plain stores, so
// here dQ gets its own query-tile-parallel pass that writes every dQ element
// once: from dS stored by the dK/dV kernel (2 bytes per pair written and read
// back), or by recomputing S and dP (two extra GEMMs); results are bitwise
// repeatable.
//
// dQ kernel: one workgroup = 4 wavefronts owning 32 query rows each.  Q and
// dY fragments stay in VGPRs; 64-key blocks of K and V stream through LDS.
// S^T = K Q^T and dP^T = V dY^T put keys on M and query rows on N, so each lane
// owns one query row (its lse and sfmg are lane-local) and 16 keys; dS packed
// to bf16 is then the A operand of dQ += dS K as it stands, with K read down
// its columns through ds_read_b64_tr_b16.

#include <hip/hip_runtime.h>

#include "fa_bwd_tiles.h"

namespace fabwd {
namespace {

// ------------------------------------------------------------------ dQ

constexpr int DQ_BQ = 128;  // query rows per workgroup (4 wavefronts x 32)
constexpr int DQ_BK = 64;   // keys per step

template <int HD, int HDV, bool F16>
__global__ __launch_bounds__(256, HD > 128 ? 1 : 2) void dq_kernel(KernelArgs a) {
  constexpr int NKQ = HD / 16;
  constexpr int NKV = HDV / 16;
  constexpr int NBK = HD / 32;
  constexpr int KTB = DQ_BK * HD * 2;  // bytes of one K / V tile buffer
  constexpr int VTB = DQ_BK * HDV * 2;
  __shared__ __attribute__((aligned(1024))) bf16 Ks[2][DQ_BK * HD];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[2][DQ_BK * HDV];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // job -> (query tile, query head, sequence); the query tile varies slowest
  // and counts down, so the causal tiles with the most keys start first
  const int per_tile = a.N1 * a.B;
  const int ntiles = (a.S1 + DQ_BQ - 1) / DQ_BQ;
  const int tile = ntiles - 1 - (int)(blockIdx.x / per_tile);
  const int rem = blockIdx.x % per_tile;
  const int n1 = rem % a.N1;
  const int b = rem / a.N1;
  const int n2 = n1 / a.G;

  const SeqBounds sb = seq_bounds(a, b);
  const int s1 = sb.s1, s2 = sb.s2;
  const int i0 = tile * DQ_BQ;
  if (i0 >= sb.s1a) return;  // a tile past the used rows (seqused_q) writes zeros
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;
  const int iq = i0 + wave * 32 + l32;  // this lane's query row

  const bf16* __restrict__ Qg = static_cast<const bf16*>(a.q) + sb.qbase + (int64_t)n1 * a.q_sn;
  const bf16* __restrict__ Yg = static_cast<const bf16*>(a.dout) + sb.obase + (int64_t)n1 * a.o_sn;
  const bf16* __restrict__ Kg = static_cast<const bf16*>(a.k) + sb.kbase + (int64_t)n2 * a.k_sn;
  const bf16* __restrict__ Vg = static_cast<const bf16*>(a.v) + sb.vbase + (int64_t)n2 * a.v_sn;

  // keys that any row of [i0, i0 + DQ_BQ) can see
  const fa_sched::Span kblk = i0 < s1 ? fa_sched::blocks_covering(
                                             fa_sched::keys_seen(s2, i0, min(i0 + DQ_BQ, s1), off, wl, wr), DQ_BK)
                                       : fa_sched::Span{0, 0};
  const int jb0 = kblk.lo * DQ_BK;
  const int nsteps = kblk.hi - kblk.lo;

  // K/V blocks go straight to LDS (async), double-buffered
  TileCopy<HD, DQ_BK, 4> kcp;
  TileCopy<HDV, DQ_BK, 4> vcp;
  kcp.init(wave, lane, (int)a.k_ss * 2);
  vcp.init(wave, lane, (int)a.v_ss * 2);
  auto fetch = [&](int jb, int buf) {
    kcp.issue(lds_addr(Ks) + buf * KTB, Kg + (int64_t)jb * a.k_ss, s2 - jb, wave, lane);
    vcp.issue(lds_addr(Vs) + buf * VTB, Vg + (int64_t)jb * a.v_ss, s2 - jb, wave, lane);
  };
  if (nsteps > 0) fetch(jb0, 0);

  bf16x8 qf[NKQ], yf[NKV];  // B operands: query row iq, dims 16*kk + 8*hi + 0..7
#pragma unroll
  for (int kk = 0; kk < NKQ; ++kk) {
    bf16x8 val = {};
    if (iq < s1) val = *reinterpret_cast<const bf16x8*>(Qg + (int64_t)iq * a.q_ss + 16 * kk + 8 * hi);
    qf[kk] = val;
  }
#pragma unroll
  for (int kk = 0; kk < NKV; ++kk) {
    bf16x8 val = {};
    if (iq < s1) val = *reinterpret_cast<const bf16x8*>(Yg + (int64_t)iq * a.o_ss + 16 * kk + 8 * hi);
    yf[kk] = val;
  }
  // sfmg = rowsum(dY * Y) of this lane's row: the dY fragments above times Y
  // read in the same layout (lanes l and l ^ 32 hold the two halves of the
  // row's columns), in fp32; written out for the dK/dV kernel, which runs next
  const int64_t lrow = sb.lbase + (int64_t)n1 * a.l_sn + iq;
  float l2 = __builtin_inff(), sf = 0.f;
  if (iq < s1) {
    const bf16* __restrict__ Og =
        static_cast<const bf16*>(a.out) + sb.obase + (int64_t)n1 * a.o_sn + (int64_t)iq * a.o_ss;
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) {
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(Og + 16 * kk + 8 * hi);
      if constexpr (F16) {  // reinterpret whole vectors (element-wise casts of bf16 lanes miscompile)
        const halfx8 gh = __builtin_bit_cast(halfx8, yf[kk]), yh = __builtin_bit_cast(halfx8, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) sf += (float)gh[e] * (float)yh[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sf += (float)yf[kk][e] * (float)y[e];
      }
    }
    const float l = a.lse[lrow];
    l2 = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;
  }
  sf += __shfl_xor(sf, 32);
  if (iq < s1 && hi == 0) a.sfmg[lrow] = sf;

  SwzTile<HD, DQ_BK> kadr;
  SwzTile<HDV, DQ_BK> vadr;
  kadr.init(lds_addr(Ks), lane);
  vadr.init(lds_addr(Vs), lane);

  floatx16 dq[NBK];
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) dq[nb] = floatx16{};

  // Step st: wait for key block st (buffer buf), prefetch block st + 1 into the
  // other buffer, compute.
  auto step = [&](int st, int buf) {
    const int j0 = jb0 + st * DQ_BK;
    wait_vmem();    // this wavefront's copies of block st landed
    lds_barrier();  // ... and everyone's; buffer buf ^ 1 is no longer read
    if (st + 1 < nsteps) fetch(j0 + DQ_BK, buf ^ 1);

    const bool full = fa_sched::tile_full(i0, DQ_BQ, j0, DQ_BK, s1, s2, off, wl, wr);
    // keys visible to this lane's row, relative to j0 (used on partial tiles):
    // one unsigned compare per element
    fa_sched::Window kvis{0u, 0xffffffffu};
    if (!full) kvis = fa_sched::window(fa_sched::keys_of_row(iq, s1, s2, off, wl, wr), j0);
    // two halves of 32 keys: S^T, dP^T, dS, then dQ += dS K for that half;
    // the MFMA runs raise the wavefront's issue priority as in the dK/dV kernel
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      floatx16 s = {}, dp = {};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk) s = mfma32<F16>(lds_load16(kadr.row_read_at(kk, mb * 32, buf * KTB)), qf[kk], s);
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk) dp = mfma32<F16>(lds_load16(vadr.row_read_at(kk, mb * 32, buf * VTB)), yf[kk], dp);
      __builtin_amdgcn_s_setprio(0);
      bf16x8 da[2];
      if (full) {
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const float p = __builtin_amdgcn_exp2f(s[rg] * a.scale_log2 - l2);
          da[rg >> 3][rg & 7] = to_elem<F16>(p * (dp[rg] - sf));
        }
      } else {
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const int jj = mb * 32 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
          float p = __builtin_amdgcn_exp2f(s[rg] * a.scale_log2 - l2);
          p = fa_sched::in_window(kvis, jj) ? p : 0.f;
          da[rg >> 3][rg & 7] = to_elem<F16>(p * (dp[rg] - sf));
        }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kc = mb * 2 + c;
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const bf16x8 kb = join(lds_load_tr(kadr.tr_read(kc, 0, nb, buf * KTB)),
                                 lds_load_tr(kadr.tr_read(kc, 1, nb, buf * KTB)));
          dq[nb] = mfma32<F16>(da[c], kb, dq[nb]);
        }
      }
      // scheduler grouping (0x100: LDS reads, 0x008: MFMAs): the transposing
      // reads of two MFMAs ahead, then each MFMA followed by a later one's two
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NBK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };
  for (int st = 0; st < nsteps; ++st) step(st, st & 1);

  // dq = bf16(scale * acc): lane holds head-dim column nb*32 + l32 of 16 rows
  bf16* __restrict__ dQg = static_cast<bf16*>(a.dq) + sb.qbase + (int64_t)n1 * a.q_sn;
#pragma unroll
  for (int rg = 0; rg < 16; ++rg) {
    const int i = i0 + wave * 32 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
    if (i < sb.s1a) {  // rows past the used ones hold zeros
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) dQg[(int64_t)i * a.q_ss + nb * 32 + l32] = to_elem<F16>(dq[nb][rg] * a.scale);
    }
  }
}

// ------------------------------------------------------------------ partial sums

// dk = bf16(sum over parts) and dv likewise: blocks [0, kblocks) of the
// nblocks take dK, the rest dV; 8 elements per thread, parts added in index
// order (so the result is repeatable).
template <bool F16>
__device__ __forceinline__ void reduce_parts_body(const float* __restrict__ kpart, int64_t k_stride,
                                                  bf16* __restrict__ kout, const float* __restrict__ vpart,
                                                  int64_t v_stride, bf16* __restrict__ vout, int nparts, int kblocks,
                                                  int blk_id, int nblocks) {
  const bool is_k = blk_id < kblocks;
  const float* __restrict__ part = is_k ? kpart : vpart;
  const int64_t stride = is_k ? k_stride : v_stride;
  bf16* __restrict__ out = is_k ? kout : vout;
  const int64_t n8 = stride / 8;
  const int64_t nblk = is_k ? kblocks : (int64_t)nblocks - kblocks;
  const int64_t blk = is_k ? blk_id : blk_id - kblocks;
  for (int64_t i = blk * 256 + threadIdx.x; i < n8; i += nblk * 256) {
    floatx4 s0 = reinterpret_cast<const floatx4*>(part)[2 * i];
    floatx4 s1 = reinterpret_cast<const floatx4*>(part)[2 * i + 1];
    for (int p = 1; p < nparts; ++p) {
      const float* q = part + (int64_t)p * stride;
      s0 += reinterpret_cast<const floatx4*>(q)[2 * i];
      s1 += reinterpret_cast<const floatx4*>(q)[2 * i + 1];
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = to_elem<F16>(s0[e]);
      o[e + 4] = to_elem<F16>(s1[e]);
    }
    reinterpret_cast<bf16x8*>(out)[i] = o;
  }
}

template <bool F16>
__global__ __launch_bounds__(256) void reduce_parts_kernel(const float* __restrict__ kpart, int64_t k_stride,
                                                           bf16* __restrict__ kout, const float* __restrict__ vpart,
                                                           int64_t v_stride, bf16* __restrict__ vout, int nparts,
                                                           int kblocks) {
  reduce_parts_body<F16>(kpart, k_stride, kout, vpart, v_stride, vout, nparts, kblocks, blockIdx.x, gridDim.x);
}

// Blocks of the reduce: at most 4096 per tensor, 8 elements per thread.
__host__ __device__ inline int64_t reduce_blocks(int64_t elems) {
  const int64_t b = (elems / 8 + 255) / 256;
  return b > 4096 ? 4096 : b;
}

// ------------------------------------------------------------------ dQ from stored dS

// dQ = scale * dS K with dS read back from the tiles the dK/dV kernel stored
// (DS form): a GEMM per (sequence, query head, 128-row group) over the 32-key
// slices the group sees, bound by the HBM reads of dS.  One workgroup = 4
// wavefronts owning 32 query rows (one stored query block) each; a step
// brings 64 keys: the K rows (swizzled tile) and the 8 dS tiles of the two
// slices (16 KB, contiguous in the workspace) go straight to LDS,
// double-buffered.  Both MFMA operands are transposing reads with the same key
// order inside each 16-key chunk: B = K through SwzTile, A = dS through
// per-lane addresses into the stored register images (below).
// QG = 2 (grids of at most one round): two such groups of 4 wavefronts share
// the row group and take alternate steps, each with its own buffers; at the end
// they swap halves of the columns through LDS and each stores its half.  The
// longest row groups of a causal mask then take half as long.
constexpr int DQS_BK = 64;  // keys per step: two 32-key slices


template <int HD, int QG, bool F16>
__global__ __launch_bounds__(256 * QG, 2 / QG) void dq_ds_kernel(KernelArgs a) {
  constexpr int NBK = HD / 32;
  constexpr int KTB = DQS_BK * HD * 2;  // bytes of one K tile buffer
  constexpr int STB = 16384;            // bytes of one dS buffer: 2 slices x 4 query blocks x 2 KB
  __shared__ __attribute__((aligned(1024))) bf16 Ks[QG][2][DQS_BK * HD];
  __shared__ __attribute__((aligned(1024))) bf16 Ss[QG][2][STB / 2];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wv >> 2;   // step group: takes steps qg, qg + QG, ...
  const int wave = wv & 3;  // query block of the row group
  const uint32_t ks_lds = lds_addr(Ks) + qg * 2 * KTB, ss_lds = lds_addr(Ss) + qg * 2 * STB;
  // job -> (query group, query head, sequence), the longest groups first
  const int nh = a.G * a.n2_count;  // query heads of this launch's KV heads
  const int per_tile = nh * a.B;
  const int ntiles = (a.S1 + DQ_BQ - 1) / DQ_BQ;
  if (a.reduce_tail) {  // workgroups past the GEMM's add the dK/dV partial sums
    const int gemm_blocks = ntiles * per_tile;
    if ((int)blockIdx.x >= gemm_blocks) {
      reduce_parts_body<F16>(a.dk_acc, a.k_part_stride, static_cast<bf16*>(a.dk), a.dv_acc, a.v_part_stride,
                             static_cast<bf16*>(a.dv), a.n_partials, (int)reduce_blocks(a.k_part_stride),
                             (int)blockIdx.x - gemm_blocks, (int)gridDim.x - gemm_blocks);
      return;
    }
  }
  // engines in reverse in even rounds, as in the dK/dV grid (rounds of one
  // workgroup per CU at QG = 2, two at QG = 1)
  int bid = blockIdx.x;
  const int rw = a.round_wgs * (2 / QG);
  if (rw > 0 && ((bid / rw) & 1) == 0 && (bid | 31) < ntiles * per_tile) bid ^= 24;
  const int tile = ntiles - 1 - bid / per_tile;
  const int rem = bid % per_tile;
  const int hl = rem % nh;          // head within the chunk (its index in the workspace)
  const int n1 = a.n2_begin * a.G + hl;
  const int b = rem / nh;
  const int n2 = n1 / a.G;

  const SeqBounds sb = seq_bounds(a, b);
  const int s1 = sb.s1, s2 = sb.s2;
  const int i0 = tile * DQ_BQ;
  if (i0 >= sb.s1a) return;  // no rows of this sequence here
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;
  const int qb = tile * 4 + wave;  // this wavefront's 32-row query block

  const bf16* __restrict__ Kg = static_cast<const bf16*>(a.k) + sb.kbase + (int64_t)n2 * a.k_sn;
  // this group's band of slices: slot x holds slice ksl.lo + x
  const int64_t grp = ds_group(a, sb, tile);
  const bf16* __restrict__ Sg = static_cast<const bf16*>(a.ds) + (grp * a.ds_heads + hl) * a.ds_w * 4096;

  // 32-key slices that any row of [i0, i0 + 128) sees (slices past the band,
  // and groups past the workspace, possible only with a sequence longer than
  // the planned maximum, are left out)
  const fa_sched::Span ksl = i0 < s1 ? fa_sched::blocks_covering(
                                            fa_sched::keys_seen(s2, i0, min(i0 + DQ_BQ, s1), off, wl, wr), 32)
                                      : fa_sched::Span{0, 0};
  const bool grp_ok = (a.varlen || tile < a.ds_nr) && grp < a.ds_groups;
  const int ks_end = grp_ok ? min(ksl.hi, ksl.lo + a.ds_w) : ksl.lo;
  const int nsteps = (ks_end - ksl.lo + 1) / 2;

  TileCopy<HD, DQS_BK, 4> kcp;
  kcp.init(wave, lane, (int)a.k_ss * 2);
  // dS copy: instruction u (wavefront u % 4) fills LDS bytes [1024u, 1024u + 1024)
  // = half u % 2 of tile u / 2; lane t brings the chunk that the placement puts
  // in slot t.  A lone last slice re-reads itself for the second one.
  const uint32_t s_voff = (uint32_t)ds_chunk_slot(lane, wave & 1) * 16;
  auto fetch = [&](int st, int buf) {
    const int ks = ksl.lo + 2 * st;
    kcp.issue(ks_lds + buf * KTB, Kg + (int64_t)ks * 32 * a.k_ss, s2 - ks * 32, wave, lane);
    const bf16* src = Sg + (int64_t)(ks - ksl.lo) * 4096;
    const bool two = ks + 1 < ks_end;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int u = wave + 4 * x;  // half u % 2 == wave % 2 of tile u / 2
      const int usrc = (u >= 8 && !two) ? u - 8 : u;
      dma16_nt(src + usrc * 512, s_voff, ss_lds + buf * STB + u * 1024);
    }
  };
  if (qg < nsteps) fetch(qg, 0);

  SwzTile<HD, DQS_BK> kadr;
  kadr.init(ks_lds, lane);
  // A operand: lane i of a 16-lane group gets, as element e of a transposing
  // read, element i % 4 of the 8 bytes that lane 4e + i/4 of its group loads.
  // For query row m = 16*(g % 2) + i (g = lane / 16) and keys
  // 16kc + 8s + 4*(g / 2) + e, lane L = 4e + q loads rows 16*(g % 2) + 4q + 0..3
  // of key 16kc + 8s + 4*(g / 2) + e: producer lane 32*(q % 2) + key, half
  // g % 2, elements 4*(q / 2) + 0..3.
  uint32_t a_base[2];
  {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3, h = g & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 32 * (q & 1) + 8 * s + 4 * (g >> 1) + e;  // chunk at kc = 0
      a_base[s] = ss_lds + wave * 2048 + h * 1024 + ds_chunk_slot(c, h) * 16 + (q >> 1) * 8;
    }
  }

  // The tile of (qb, slice ks) was stored iff some row of qb sees a key of the
  // slice (the dK/dV kernel runs every such pair); otherwise it adds nothing.
  auto stored = [&](int ks) { return ds_tile_visible(qb, ks, s1, s2, off, wl, wr); };

  floatx16 dq[NBK];
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) dq[nb] = floatx16{};

  // iteration it: group qg computes step st = it * QG + qg (if there is one)
  auto step = [&](int st, int buf) {
    wait_vmem();    // this wavefront's copies of step st landed
    lds_barrier();  // ... and everyone's; buffer buf ^ 1 is no longer read
    if (st + QG < nsteps) fetch(st + QG, buf ^ 1);
    if (st >= nsteps) return;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int ks = ksl.lo + 2 * st + sl;
      if (ks < ks_end && stored(ks)) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t ao = buf * STB + sl * 8192 + c * 256;  // slice sl, chunk bit 4 = c
          const bf16x8 da = join(lds_load_tr(a_base[0] + ao), lds_load_tr(a_base[1] + ao));
          const int kc = 2 * sl + c;
#pragma unroll
          for (int nb = 0; nb < NBK; ++nb) {
            const bf16x8 kb = join(lds_load_tr(kadr.tr_read_c(kc, 0, nb, buf * KTB)),
                                   lds_load_tr(kadr.tr_read_c(kc, 1, nb, buf * KTB)));
            dq[nb] = mfma32<F16>(da, kb, dq[nb]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
  };
  const int iters = (nsteps + QG - 1) / QG;
  int it = 0;  // two steps per iteration, so that the buffer offsets are constants
  for (; it + 1 < iters; it += 2) {
    step(it * QG + qg, 0);
    step((it + 1) * QG + qg, 1);
  }
  if (it < iters) step(it * QG + qg, 0);

  // QG = 2: group 1 hands column blocks [0, NBK/2) to group 0, group 0 hands
  // the rest to group 1 (16 KB of LDS per block); each adds what it received
  constexpr int NLO = QG > 1 ? NBK / 2 : NBK;  // blocks that group 0 stores
  if constexpr (QG > 1) {
    static_assert(NBK % 2 == 0 && QG == 2, "two halves");
    static_assert(sizeof(Ks) >= (size_t)NBK * 16384, "LDS room for the swap");
    wait_vmem();
    __syncthreads();  // every LDS read of the steps is done
    float* area = reinterpret_cast<float*>(&Ks[0][0][0]);
    if (qg == 1) {
#pragma unroll
      for (int nb = 0; nb < NLO; ++nb) xput(area + nb * 4096, wave, lane, dq[nb]);
    } else {
#pragma unroll
      for (int nb = NLO; nb < NBK; ++nb) xput(area + nb * 4096, wave, lane, dq[nb]);
    }
    __syncthreads();
    if (qg == 0) {
#pragma unroll
      for (int nb = 0; nb < NLO; ++nb) xadd(area + nb * 4096, wave, lane, dq[nb]);
    } else {
#pragma unroll
      for (int nb = NLO; nb < NBK; ++nb) xadd(area + nb * 4096, wave, lane, dq[nb]);
    }
  }
  const int nb_lo = qg == 0 ? 0 : NLO, nb_hi = qg == 0 ? NLO : NBK;

  bf16* __restrict__ dQg = static_cast<bf16*>(a.dq) + sb.qbase + (int64_t)n1 * a.q_sn;
  if constexpr (QG > 1) {
    // dq = bf16(scale * acc), each 32 x 32 block turned row-major by two MFMAs
    // against a permuted identity (exact: every output is one input times 1),
    // then stored as 16-byte row pieces (lane = query row).  Measured faster
    // only for the one-round grids of this form (MHA -3.5 %; the QG = 1 grids
    // of GQA, varlen and wide_qk +0.5 to +2.6 %).
    bf16x8 eye[2];
    eye_operand<F16>(lane, eye);
    const int row = i0 + wave * 32 + l32;
    bf16* __restrict__ dq_row = dQg + (int64_t)row * a.q_ss;
    const bool row_ok = row < sb.s1a;  // rows past the used ones hold zeros
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      if (nb >= nb_lo && nb < nb_hi) {
        u32x4 piece[2];
        row_pieces<F16>(transpose_acc<F16>(dq[nb], a.scale, eye), 1.f, piece);
        if (row_ok) {
#pragma unroll
          for (int pc = 0; pc < 2; ++pc) *reinterpret_cast<u32x4*>(dq_row + nb * 32 + pc * 16 + hi * 8) = piece[pc];
        }
      }
    }
  } else {
    // dq = bf16(scale * acc): lane holds head-dim column nb*32 + l32 of 16 rows
#pragma unroll
    for (int rg = 0; rg < 16; ++rg) {
      const int i = i0 + wave * 32 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
      if (i < sb.s1a) {  // rows past the used ones hold zeros
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb)
          if (nb >= nb_lo && nb < nb_hi) dQg[(int64_t)i * a.q_ss + nb * 32 + l32] = to_elem<F16>(dq[nb][rg] * a.scale);
      }
    }
  }
}

}  // namespace

bool det_instantiated(int D, int Dv) {
  return (D == 64 && Dv == 64) || (D == 128 && (Dv == 64 || Dv == 128)) || (D == 192 && (Dv == 64 || Dv == 128));
}

// Keys per tile of the dK/dV kernel divided by 4 (every shape uses 128-key
// tiles: 8 wavefronts x 32 keys in two query groups, 4 x 32 at D = 192).
int det_keys_per_wave(int D) { (void)D; return 32; }

namespace {

template <bool F16>
int launch_dq_ds_t(const KernelArgs& a, dim3 grid, hipStream_t s) {
  const bool two = a.dq_groups == 2;
  const dim3 b1(256), b2(512);
  if (a.D == 64) return two ? launch(dq_ds_kernel<64, 2, F16>, grid, b2, s, a) : launch(dq_ds_kernel<64, 1, F16>, grid, b1, s, a);
  if (a.D == 128)
    return two ? launch(dq_ds_kernel<128, 2, F16>, grid, b2, s, a) : launch(dq_ds_kernel<128, 1, F16>, grid, b1, s, a);
  if (a.D == 192 && !two) return launch(dq_ds_kernel<192, 1, F16>, grid, b1, s, a);
  return (int)hipErrorInvalidValue;
}

template <bool F16>
int launch_dq_t(const KernelArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (a.D == 64 && a.Dv == 64) return launch(dq_kernel<64, 64, F16>, grid, block, s, a);
  if (a.D == 128 && a.Dv == 64) return launch(dq_kernel<128, 64, F16>, grid, block, s, a);
  if (a.D == 128 && a.Dv == 128) return launch(dq_kernel<128, 128, F16>, grid, block, s, a);
  if (a.D == 192 && a.Dv == 64) return launch(dq_kernel<192, 64, F16>, grid, block, s, a);
  if (a.D == 192 && a.Dv == 128) return launch(dq_kernel<192, 128, F16>, grid, block, s, a);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_dq(const KernelArgs& a, void* stream) {
  const int64_t tiles = (a.S1 + DQ_BQ - 1) / DQ_BQ;
  const int64_t blocks = tiles * a.N1 * a.B;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks);
  return a.f16 ? launch_dq_t<true>(a, grid, s) : launch_dq_t<false>(a, grid, s);
}

int launch_dq_ds(const KernelArgs& a, void* stream) {
  const int64_t tiles = (a.S1 + DQ_BQ - 1) / DQ_BQ;
  const int64_t blocks = tiles * a.G * a.n2_count * a.B +
                         (a.reduce_tail ? reduce_blocks(a.k_part_stride) + reduce_blocks(a.v_part_stride) : 0);
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks);
  return a.f16 ? launch_dq_ds_t<true>(a, grid, s) : launch_dq_ds_t<false>(a, grid, s);
}

int launch_reduce_parts(const KernelArgs& a, void* stream) {
  if (a.n_partials <= 1) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kb = reduce_blocks(a.k_part_stride), vb = reduce_blocks(a.v_part_stride);
  if (kb <= 0 || vb <= 0) return 0;
  return launch(a.f16 ? reduce_parts_kernel<true> : reduce_parts_kernel<false>, dim3((unsigned)(kb + vb)), dim3(256), s,
                (const float*)a.dk_acc, a.k_part_stride, static_cast<bf16*>(a.dk), (const float*)a.dv_acc,
                a.v_part_stride, static_cast<bf16*>(a.dv), a.n_partials, (int)kb);
}

}  // namespace fabwd
