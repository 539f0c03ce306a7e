// gfx950 (MI355X) kernels of the FlashAttention backward: the sfmg
// preprocess used by every path, and the two fp32-atomic forms of the main
// kernel (selected with FA_BWD_VARIANT=0/1; the default path is the
// atomic-free pair of fa_bwd_det_kernels.hip).
//
// Formulas: page "CANN ops-transformer FlashAttnGrad 算子详解", section 一
// (P = exp(scale*QK^T - softmax_lse), dV = P^T dY, dP = dY V^T,
// sfmg = rowsum(dY (.) Y), dS = P (.) (dP - sfmg), dQ = scale*dS K,
// dK = scale*dS^T Q).  Section 五 5.2 describes the page's own kernel as five
// cube matmuls plus vector stages, with dQ reduced through an fp32 workspace by
// atomic adds and dK/dV accumulated on chip across query blocks; the design
// below keeps those two ideas and is otherwise laid out for CDNA4:
//
//   preprocess  sfmg = rowsum(dY (.) Y) in fp32, one 16-byte load per lane,
//               cross-lane sums; also clears the fp32 dQ accumulator.
//   main        one workgroup = 4 wavefronts = 128 keys of one key/value head
//               (32 keys per wavefront).  K and V fragments stay in VGPRs for
//               the whole kernel; Q and dY stream through LDS 64 rows at a
//               time.  Per block of 64 query rows each wavefront computes
//               S = Q K^T and dP = dY V^T for its 32 keys with
//               v_mfma_f32_32x32x16_bf16 (query rows as M, keys as N), so every
//               lane holds one key and 16 query rows.  That accumulator layout is
//               exactly the A-operand layout of the key-major products, so P and
//               dS feed dV += P^T dY and dK += dS^T Q from registers; the
//               B operands (dY and Q read down their columns) come from LDS with
//               ds_read_b64_tr_b16.  dS^T goes to LDS once and the four
//               wavefronts then form dQ = dS K for the block and add it into the
//               fp32 accumulator with hardware float atomics.  The G query heads
//               of a GQA group run inside the same workgroup, so dK/dV are
//               complete in registers when the loop ends.
//   finalize    dq = bf16(scale * dq_acc).
//
// exp is v_exp_f32 (base 2) with log2(e) folded into the scale and the lse.

#include <hip/hip_runtime.h>

#include <new>
#include <type_traits>

#include "fa_bwd.h"
#include "fa_bwd_internal.h"
#include "fa_bwd_schedule.h"

namespace fabwd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
typedef unsigned uintx2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane i receives element
// (i % 4) of the 8 bytes addressed by lane 4*e + i/4, for e = 0..3.  With lane
// i of the group pointing at row (r0 + i/4), column (c0 + 4*(i%4)) of a
// row-major bf16 tile, lane i gets column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ shortx4 lds_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(p));
}

__device__ __forceinline__ bf16x8 join(shortx4 lo, shortx4 hi) {
  shortx8 s = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, s);
}

// ---------------------------------------------------------------- preprocess

// One row = Dv contiguous bf16 of dout / attn_out.  DV/8 lanes per row, each
// with one 16-byte load of each tensor.  BNSD and TND: a block takes RPB
// consecutive rows.  BSND: a block takes RPB consecutive rows of one (batch,
// head) pair, the pair the faster block index, so that its sfmg values
// ([b][n][s]) are one contiguous store instead of RPB scattered 4-byte ones
// while the blocks in flight together still read whole rows of heads
// (measured: GQA 13.8 -> 12.3 us, MHA 8.7 -> 7.1 us; the same for TND, or
// the pair as the slower index, made varlen and BNSD slower).  One
// instantiation per layout; TND and BNSD form the sfmg index after the loads.
template <int DV, bool F16, int LAYOUT>
__global__ __launch_bounds__(256) void preprocess_kernel(KernelArgs a, int64_t rows, uint32_t pairs, int zero_dq,
                                                          int64_t dq_elems, int64_t dk_elems, int64_t dv_elems) {
  constexpr int LPR = DV / 8;             // lanes per row
  constexpr int RPB = 256 / LPR;          // rows per block
  const int tid = threadIdx.x;
  int64_t row, o = 0;  // the row's index in dout / attn_out (rows of Dv elements) and in sfmg
  bool ok;
  if constexpr (LAYOUT == FA_LAYOUT_BSND) {  // block -> (chunk, pair = b * N1 + n); row (b * S1 + s) * N1 + n
    const uint32_t chunk = blockIdx.x / pairs, pair = blockIdx.x - chunk * pairs;
    const uint32_t b = pair / (uint32_t)a.N1, n = pair - b * (uint32_t)a.N1;
    const int64_t si = (int64_t)chunk * RPB + tid / LPR;
    row = ((int64_t)b * a.S1 + si) * a.N1 + n;
    o = (int64_t)pair * a.S1 + si;  // [b][n][s]: l_sb = N1 * S1, l_sn = S1
    ok = si < a.S1;
  } else {
    row = (int64_t)blockIdx.x * RPB + tid / LPR;
    ok = row < rows;
  }
  const int part = tid % LPR;
  float s = 0.f;
  if (ok) {
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.out) + row * DV + part * 8);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.dout) + row * DV + part * 8);
    if constexpr (F16) {  // fp16 in the same storage: reinterpret whole vectors (element-wise casts of
                          // bf16 lanes miscompile)
      typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
      const halfx8 yh = __builtin_bit_cast(halfx8, y), gh = __builtin_bit_cast(halfx8, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)gh[e] * (float)yh[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s += (float)g[e] * (float)y[e];
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, LPR);
  if (ok && part == 0) {  // (the other layouts' sfmg index is formed after the loads)
    if constexpr (LAYOUT == FA_LAYOUT_BNSD) {  // row = (b*N1 + n)*S1 + s  ->  same order
      o = row;
    } else if constexpr (LAYOUT == FA_LAYOUT_TND) {  // row = t*N1 + n  ->  [n][t]
      const int64_t n = row % a.N1, t = row / a.N1;
      o = n * a.l_sn + t;
    }
    a.sfmg[o] = s;
  }
  if (zero_dq) {  // clear the fp32 accumulators (dQ, and dK/dV when heads are split)
    const floatx4 z = {0.f, 0.f, 0.f, 0.f};
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t first = (int64_t)blockIdx.x * 256 + tid;
    floatx4* p = reinterpret_cast<floatx4*>(a.dq_acc);
    for (int64_t i = first; i < dq_elems / 4; i += stride) p[i] = z;
    if (dk_elems) {
      p = reinterpret_cast<floatx4*>(a.dk_acc);
      for (int64_t i = first; i < dk_elems / 4; i += stride) p[i] = z;
      p = reinterpret_cast<floatx4*>(a.dv_acc);
      for (int64_t i = first; i < dv_elems / 4; i += stride) p[i] = z;
    }
  }
}

// ---------------------------------------------------------------- finalize

__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                          int64_t n8, float scale) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const floatx4 x0 = reinterpret_cast<const floatx4*>(acc)[2 * i];
    const floatx4 x1 = reinterpret_cast<const floatx4*>(acc)[2 * i + 1];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[e] = (bf16)(x0[e] * scale);
      o[e + 4] = (bf16)(x1[e] * scale);
    }
    reinterpret_cast<bf16x8*>(dq)[i] = o;
  }
}

// ---------------------------------------------------------------- main

template <int HD, int HDV>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(KernelArgs a) {
  constexpr int BC = KV_TILE;   // keys per workgroup
  constexpr int BR = Q_TILE;    // query rows per step
  constexpr int QP = HD + 8;    // padded LDS row pitch (elements) of K and Q tiles
  constexpr int YP = HDV + 8;   // dY tile
  constexpr int SP = BR + 8;    // dS^T tile (rows = keys)
  constexpr int NMB = BR / 32;  // 32-row query blocks per step
  constexpr int NKQ = HD / 16;  // k-steps over D
  constexpr int NKV = HDV / 16; // k-steps over Dv
  constexpr int NDQ = NMB * (HD / 32);  // dQ output tiles per step

  __shared__ __attribute__((aligned(16))) bf16 Ks[BC * QP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[BR * QP];
  __shared__ __attribute__((aligned(16))) bf16 Ys[BR * YP];
  __shared__ __attribute__((aligned(16))) bf16 St[BC * SP];
  __shared__ __attribute__((aligned(16))) float lse_s[BR];
  __shared__ __attribute__((aligned(16))) float sfm_s[BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // workgroup -> (key tile, key/value head, sequence).  The key tile varies
  // slowest, so the tiles with the most causal work are dispatched first.
  const int bid = blockIdx.x;
  const int per_tile = a.N2 * a.B;
  const int tile = bid / per_tile;
  const int rem = bid - tile * per_tile;
  const int n2 = rem % a.N2;
  const int b = rem / a.N2;

  int s1, s2;
  int64_t qbase, kbase, vbase, obase, lbase;
  if (a.varlen) {
    const int q0 = a.cu_q[b], k0 = a.cu_kv[b];
    s1 = a.cu_q[b + 1] - q0;
    s2 = a.cu_kv[b + 1] - k0;
    qbase = (int64_t)q0 * a.q_ss;
    obase = (int64_t)q0 * a.o_ss;
    kbase = (int64_t)k0 * a.k_ss;
    vbase = (int64_t)k0 * a.v_ss;
    lbase = q0;
  } else {
    s1 = a.S1;
    s2 = a.S2;
    qbase = (int64_t)b * a.q_sb;
    obase = (int64_t)b * a.o_sb;
    kbase = (int64_t)b * a.k_sb;
    vbase = (int64_t)b * a.v_sb;
    lbase = (int64_t)b * a.l_sb;
  }
  const int j0 = tile * BC;
  if (j0 >= s2) return;  // whole workgroup: this sequence has fewer keys
  const int j1 = min(j0 + BC, s2);
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;

  const bf16* __restrict__ Kg = static_cast<const bf16*>(a.k) + kbase + (int64_t)n2 * a.k_sn;
  const bf16* __restrict__ Vg = static_cast<const bf16*>(a.v) + vbase + (int64_t)n2 * a.v_sn;

  // K tile -> LDS (row-major, zero rows past the sequence end)
  for (int c = tid; c < BC * (HD / 8); c += 256) {
    const int r = c / (HD / 8), cc = (c % (HD / 8)) * 8;
    bf16x8 val = {};
    if (j0 + r < s2) val = *reinterpret_cast<const bf16x8*>(Kg + (int64_t)(j0 + r) * a.k_ss + cc);
    *reinterpret_cast<bf16x8*>(&Ks[r * QP + cc]) = val;
  }
  // V fragments (B operand of dP = dY V^T): lane holds key kw, dims 16*kk + 8*hi + 0..7
  const int kw = wave * 32 + l32;
  bf16x8 vf[NKV];
#pragma unroll
  for (int kk = 0; kk < NKV; ++kk) {
    bf16x8 val = {};
    if (j0 + kw < s2) val = *reinterpret_cast<const bf16x8*>(Vg + (int64_t)(j0 + kw) * a.v_ss + 16 * kk + 8 * hi);
    vf[kk] = val;
  }
  __syncthreads();
  bf16x8 kf[NKQ];  // B operand of S = Q K^T
#pragma unroll
  for (int kk = 0; kk < NKQ; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(&Ks[kw * QP + 16 * kk + 8 * hi]);

  floatx16 dk_acc[HD / 32], dv_acc[HDV / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) dk_acc[i] = floatx16{};
#pragma unroll
  for (int i = 0; i < HDV / 32; ++i) dv_acc[i] = floatx16{};

  // lane offsets of the transposing reads
  const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column within a 32-wide block
  const int tr_r4 = 4 * hi + ((lane & 15) >> 2);             // row pattern of P/dS-ordered chunks
  const int tr_r8 = 8 * hi + ((lane & 15) >> 2);             // row pattern of contiguous chunks

  // query rows that see at least one key of [j0, j1)
  const fa_sched::Span qblk = fa_sched::blocks_covering(fa_sched::rows_seeing(s1, j0, j1, off, wl, wr), BR);

  for (int g = 0; g < a.G; ++g) {
    const int n1 = n2 * a.G + g;
    const bf16* __restrict__ Qg = static_cast<const bf16*>(a.q) + qbase + (int64_t)n1 * a.q_sn;
    const bf16* __restrict__ Yg = static_cast<const bf16*>(a.dout) + obase + (int64_t)n1 * a.o_sn;
    float* __restrict__ dQa = a.dq_acc + qbase + (int64_t)n1 * a.q_sn;
    const float* __restrict__ Lg = a.lse + lbase + (int64_t)n1 * a.l_sn;
    const float* __restrict__ Fg = a.sfmg + lbase + (int64_t)n1 * a.l_sn;

    for (int i0 = qblk.lo * BR; i0 < qblk.hi * BR; i0 += BR) {
      // ---- stage Q, dY, lse, sfmg of rows [i0, i0 + BR) in LDS
      for (int c = tid; c < BR * (HD / 8); c += 256) {
        const int r = c / (HD / 8), cc = (c % (HD / 8)) * 8;
        bf16x8 val = {};
        if (i0 + r < s1) val = *reinterpret_cast<const bf16x8*>(Qg + (int64_t)(i0 + r) * a.q_ss + cc);
        *reinterpret_cast<bf16x8*>(&Qs[r * QP + cc]) = val;
      }
      for (int c = tid; c < BR * (HDV / 8); c += 256) {
        const int r = c / (HDV / 8), cc = (c % (HDV / 8)) * 8;
        bf16x8 val = {};
        if (i0 + r < s1) val = *reinterpret_cast<const bf16x8*>(Yg + (int64_t)(i0 + r) * a.o_ss + cc);
        *reinterpret_cast<bf16x8*>(&Ys[r * YP + cc]) = val;
      }
      if (tid < BR) {
        const int i = i0 + tid;
        float l2 = __builtin_inff(), f = 0.f;
        if (i < s1) {
          const float l = Lg[i];
          // a row with no visible key (lse = -inf) must give P = 0
          l2 = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;
          f = Fg[i];
        }
        lse_s[tid] = l2;
        sfm_s[tid] = f;
      }
      __syncthreads();

      // ---- S = Q K^T and dP = dY V^T for this wavefront's 32 keys
      floatx16 sacc[NMB], pacc[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        sacc[mb] = floatx16{};
        pacc[mb] = floatx16{};
#pragma unroll
        for (int kk = 0; kk < NKQ; ++kk) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[(mb * 32 + l32) * QP + 16 * kk + 8 * hi]);
          sacc[mb] = mfma32(qa, kf[kk], sacc[mb]);
        }
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
          const bf16x8 ya = *reinterpret_cast<const bf16x8*>(&Ys[(mb * 32 + l32) * YP + 16 * kk + 8 * hi]);
          pacc[mb] = mfma32(ya, vf[kk], pacc[mb]);
        }
      }

      // ---- P = exp(S*scale - lse) (masked), dS = P (dP - sfmg), both packed as bf16
      const bool full = fa_sched::tile_full(i0, BR, j0, BC, s1, s2, off, wl, wr);
      const int jk = j0 + kw;
      bf16x8 pa[2 * NMB], da[2 * NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ib = mb * 32 + r4 * 8 + hi * 4;  // first of 4 consecutive query rows
          const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[ib]);
          const floatx4 f4 = *reinterpret_cast<const floatx4*>(&sfm_s[ib]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r4 * 4 + e;
            float p = __builtin_amdgcn_exp2f(sacc[mb][r] * a.scale_log2 - l4[e]);
            if (!full) {
              const int i = i0 + ib + e;
              const bool vis = fa_sched::visible(i, jk, s1, s2, off, wl, wr);
              p = vis ? p : 0.f;
            }
            const float ds = p * (pacc[mb][r] - f4[e]);
            pa[mb * 2 + (r >> 3)][r & 7] = (bf16)p;
            da[mb * 2 + (r >> 3)][r & 7] = (bf16)ds;
          }
        }
      }

      // ---- dV += P^T dY and dK += dS^T Q  (M = keys, N = head dim, K = query rows)
#pragma unroll
      for (int kc = 0; kc < 2 * NMB; ++kc) {
#pragma unroll
        for (int nb = 0; nb < HDV / 32; ++nb) {
          const bf16* p0 = &Ys[(16 * kc + tr_r4) * YP + nb * 32 + tr_c];
          const bf16x8 yb = join(lds_tr(p0), lds_tr(p0 + 8 * YP));
          dv_acc[nb] = mfma32(pa[kc], yb, dv_acc[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < HD / 32; ++nb) {
          const bf16* p0 = &Qs[(16 * kc + tr_r4) * QP + nb * 32 + tr_c];
          const bf16x8 qb = join(lds_tr(p0), lds_tr(p0 + 8 * QP));
          dk_acc[nb] = mfma32(da[kc], qb, dk_acc[nb]);
        }
      }

      // ---- dS^T -> LDS: row = key, 4 consecutive query rows per 8-byte store.
      // (Whole-vector bit casts only: this compiler mis-lowers a bit cast of a
      // single bf16 vector element.)
#pragma unroll
      for (int kc = 0; kc < 2 * NMB; ++kc) {
        const uintx4 u = __builtin_bit_cast(uintx4, da[kc]);
        bf16* row = &St[kw * SP + kc * 16 + hi * 4];
        *reinterpret_cast<uintx2*>(row) = uintx2{u[0], u[1]};
        *reinterpret_cast<uintx2*>(row + 8) = uintx2{u[2], u[3]};
      }
      __syncthreads();

      // ---- dQ(rows i0..) += dS K, added into the fp32 accumulator
#pragma unroll
      for (int t = wave; t < NDQ; t += 4) {
        const int mq = t % NMB, nd = t / NMB;
        floatx16 acc = {};
#pragma unroll
        for (int kc = 0; kc < BC / 16; ++kc) {
          const bf16* pa0 = &St[(16 * kc + tr_r8) * SP + mq * 32 + tr_c];
          const bf16* pb0 = &Ks[(16 * kc + tr_r8) * QP + nd * 32 + tr_c];
          const bf16x8 av = join(lds_tr(pa0), lds_tr(pa0 + 4 * SP));
          const bf16x8 bv = join(lds_tr(pb0), lds_tr(pb0 + 4 * QP));
          acc = mfma32(av, bv, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + mq * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          if (i < s1) unsafeAtomicAdd(dQa + (int64_t)i * a.q_ss + nd * 32 + l32, acc[r]);
        }
      }
      __syncthreads();
    }
  }

  // ---- write dK = scale * acc and dV (bf16); keys past the sequence end are skipped
  bf16* __restrict__ dKg = static_cast<bf16*>(a.dk) + kbase + (int64_t)n2 * a.k_sn;
  bf16* __restrict__ dVg = static_cast<bf16*>(a.dv) + vbase + (int64_t)n2 * a.v_sn;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = j0 + wave * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
    if (j < s2) {
#pragma unroll
      for (int nb = 0; nb < HD / 32; ++nb) dKg[(int64_t)j * a.k_ss + nb * 32 + l32] = (bf16)(dk_acc[nb][r] * a.scale);
#pragma unroll
      for (int nb = 0; nb < HDV / 32; ++nb) dVg[(int64_t)j * a.v_ss + nb * 32 + l32] = (bf16)dv_acc[nb][r];
    }
  }
}

// ---------------------------------------------------------------- main, 8 wavefronts

// One workgroup = 8 wavefronts = two query groups of 4 wavefronts sharing one
// 128-key tile of K and V in LDS.  Wavefront (group, w) owns keys 32w..32w+31 of
// the tile for its group's work; the groups take alternate 32-row query blocks
// (over the query heads of the job), so every SIMD runs two wavefronts that
// interleave their MFMA, exp and LDS work.  The next block of each group is
// prefetched into registers while the current one is computed.  When the loop
// ends the second group's dK/dV partials are added into the first group's
// through LDS.  Jobs are (key tile, query-head slot, sequence, key/value head),
// the key tile slowest, so long causal tiles are dispatched first and the
// query heads of one key/value head sit on the same XCD (blockIdx mod 8) when
// N2 is a multiple of 8.
template <int HD, int HDV>
__global__ __launch_bounds__(512, 1) void bwd_main_v2_kernel(KernelArgs a) {
  constexpr int BC = KV_TILE;
  constexpr int BR = Q_TILE_2G;
  constexpr int KP = HD + 8;
  constexpr int VP = HDV + 8;
  constexpr int SP = BR + 8;
  constexpr int NKQ = HD / 16;
  constexpr int NKV = HDV / 16;
  constexpr int NBK = HD / 32;
  constexpr int NBV = HDV / 32;
  constexpr int NQC = BR * HD / 8 / 256;    // 16-byte Q chunks per thread and block
  constexpr int NYC = BR * HDV / 8 / 256;   // 16-byte dY chunks per thread and block
  static_assert(NQC * 256 * 8 == BR * HD && NYC * 256 * 8 == BR * HDV, "tile split");

  __shared__ __attribute__((aligned(16))) bf16 Ks[BC * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[BC * VP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BR * KP];
  __shared__ __attribute__((aligned(16))) bf16 Ys[2][BR * VP];
  __shared__ __attribute__((aligned(16))) bf16 St[2][BC * SP];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BR];
  __shared__ __attribute__((aligned(16))) float sfm_s[2][BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qg = wave >> 2;       // query group
  const int kw = wave & 3;        // key slice of the tile
  const int gt = tid & 255;       // thread index within the group
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- job
  const int hpj = a.heads_per_job;
  const int HJ = a.G / hpj;
  int r = blockIdx.x;
  const int n2 = r % a.N2; r /= a.N2;
  const int b = r % a.B; r /= a.B;
  const int gslot = r % HJ;
  const int tile = r / HJ;

  int s1, s2;
  int64_t qbase, kbase, vbase, obase, lbase;
  if (a.varlen) {
    const int q0 = a.cu_q[b], k0 = a.cu_kv[b];
    s1 = a.cu_q[b + 1] - q0;
    s2 = a.cu_kv[b + 1] - k0;
    qbase = (int64_t)q0 * a.q_ss;
    obase = (int64_t)q0 * a.o_ss;
    kbase = (int64_t)k0 * a.k_ss;
    vbase = (int64_t)k0 * a.v_ss;
    lbase = q0;
  } else {
    s1 = a.S1;
    s2 = a.S2;
    qbase = (int64_t)b * a.q_sb;
    obase = (int64_t)b * a.o_sb;
    kbase = (int64_t)b * a.k_sb;
    vbase = (int64_t)b * a.v_sb;
    lbase = (int64_t)b * a.l_sb;
  }
  const int j0 = tile * BC;
  if (j0 >= s2) return;
  const int j1 = min(j0 + BC, s2);
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;

  // ---- K and V tiles -> LDS
  {
    const bf16* Kg = static_cast<const bf16*>(a.k) + kbase + (int64_t)n2 * a.k_sn;
    const bf16* Vg = static_cast<const bf16*>(a.v) + vbase + (int64_t)n2 * a.v_sn;
    for (int c = tid; c < BC * (HD / 8); c += 512) {
      const int rr = c / (HD / 8), cc = (c % (HD / 8)) * 8;
      bf16x8 val = {};
      if (j0 + rr < s2) val = *reinterpret_cast<const bf16x8*>(Kg + (int64_t)(j0 + rr) * a.k_ss + cc);
      *reinterpret_cast<bf16x8*>(&Ks[rr * KP + cc]) = val;
    }
    for (int c = tid; c < BC * (HDV / 8); c += 512) {
      const int rr = c / (HDV / 8), cc = (c % (HDV / 8)) * 8;
      bf16x8 val = {};
      if (j0 + rr < s2) val = *reinterpret_cast<const bf16x8*>(Vg + (int64_t)(j0 + rr) * a.v_ss + cc);
      *reinterpret_cast<bf16x8*>(&Vs[rr * VP + cc]) = val;
    }
  }

  // ---- query blocks that see a key of [j0, j1), for each head of the job
  const fa_sched::Span qblk = fa_sched::blocks_covering(fa_sched::rows_seeing(s1, j0, j1, off, wl, wr), BR);
  const int blk_lo = qblk.lo;
  const int nblk = qblk.hi - qblk.lo;
  const int T = hpj * nblk;
  const int g0 = gslot * hpj;

  // prefetch registers of the group's next item
  bf16x8 pq[NQC], py[NYC];
  float pl = __builtin_inff(), pf = 0.f;
  auto fetch = [&](int t) {
    if (t < T) {
      const int n1 = n2 * a.G + g0 + t / nblk;
      const int i0 = (blk_lo + t % nblk) * BR;
      const bf16* Qg = static_cast<const bf16*>(a.q) + qbase + (int64_t)n1 * a.q_sn;
      const bf16* Yg = static_cast<const bf16*>(a.dout) + obase + (int64_t)n1 * a.o_sn;
#pragma unroll
      for (int u = 0; u < NQC; ++u) {
        const int c = gt + 256 * u, rr = c / (HD / 8), cc = (c % (HD / 8)) * 8;
        bf16x8 val = {};
        if (i0 + rr < s1) val = *reinterpret_cast<const bf16x8*>(Qg + (int64_t)(i0 + rr) * a.q_ss + cc);
        pq[u] = val;
      }
#pragma unroll
      for (int u = 0; u < NYC; ++u) {
        const int c = gt + 256 * u, rr = c / (HDV / 8), cc = (c % (HDV / 8)) * 8;
        bf16x8 val = {};
        if (i0 + rr < s1) val = *reinterpret_cast<const bf16x8*>(Yg + (int64_t)(i0 + rr) * a.o_ss + cc);
        py[u] = val;
      }
      if (gt < BR) {
        const int i = i0 + gt;
        pl = __builtin_inff();
        pf = 0.f;
        if (i < s1) {
          const float l = a.lse[lbase + (int64_t)n1 * a.l_sn + i];
          pl = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;  // empty row -> P = 0
          pf = a.sfmg[lbase + (int64_t)n1 * a.l_sn + i];
        }
      }
    }
  };
  fetch(qg);

  floatx16 dKr[NBK], dVr[NBV];
#pragma unroll
  for (int i = 0; i < NBK; ++i) dKr[i] = floatx16{};
#pragma unroll
  for (int i = 0; i < NBV; ++i) dVr[i] = floatx16{};

  const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int tr_r4 = 4 * hi + ((lane & 15) >> 2);
  const int tr_r8 = 8 * hi + ((lane & 15) >> 2);
  const int krow = kw * 32 + l32;  // this lane's key within the tile
  const int jk = j0 + krow;
  bf16* Qg_s = Qs[qg];
  bf16* Yg_s = Ys[qg];
  bf16* St_s = St[qg];

  const int iters = (T + 1) / 2;
  for (int it = 0; it < iters; ++it) {
    const int t = 2 * it + qg;
    const bool valid = t < T;
    int n1 = 0, i0 = 0;
    if (valid) {
      n1 = n2 * a.G + g0 + t / nblk;
      i0 = (blk_lo + t % nblk) * BR;
#pragma unroll
      for (int u = 0; u < NQC; ++u) {
        const int c = gt + 256 * u, rr = c / (HD / 8), cc = (c % (HD / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&Qg_s[rr * KP + cc]) = pq[u];
      }
#pragma unroll
      for (int u = 0; u < NYC; ++u) {
        const int c = gt + 256 * u, rr = c / (HDV / 8), cc = (c % (HDV / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&Yg_s[rr * VP + cc]) = py[u];
      }
      if (gt < BR) {
        lse_s[qg][gt] = pl;
        sfm_s[qg][gt] = pf;
      }
    }
    fetch(t + 2);
    __syncthreads();

    if (valid) {
      // S = Q K^T and dP = dY V^T for this wavefront's 32 keys (B operands from LDS)
      floatx16 sacc = {}, pacc = {};
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk) {
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&Ks[krow * KP + 16 * kk + 8 * hi]);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qg_s[l32 * KP + 16 * kk + 8 * hi]);
        sacc = mfma32(qa, kb, sacc);
      }
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk) {
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&Vs[krow * VP + 16 * kk + 8 * hi]);
        const bf16x8 ya = *reinterpret_cast<const bf16x8*>(&Yg_s[l32 * VP + 16 * kk + 8 * hi]);
        pacc = mfma32(ya, vb, pacc);
      }
      const bool full = fa_sched::tile_full(i0, BR, j0, BC, s1, s2, off, wl, wr);
      bf16x8 pa[2], da[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ib = r4 * 8 + hi * 4;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[qg][ib]);
        const floatx4 f4 = *reinterpret_cast<const floatx4*>(&sfm_s[qg][ib]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rg = r4 * 4 + e;
          float p = __builtin_amdgcn_exp2f(sacc[rg] * a.scale_log2 - l4[e]);
          if (!full) {
            const int i = i0 + ib + e;
            const bool vis = fa_sched::visible(i, jk, s1, s2, off, wl, wr);
            p = vis ? p : 0.f;
          }
          const float ds = p * (pacc[rg] - f4[e]);
          pa[rg >> 3][rg & 7] = (bf16)p;
          da[rg >> 3][rg & 7] = (bf16)ds;
        }
      }
      // dV += P^T dY, dK += dS^T Q (B operands by transposing LDS reads)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
          const bf16* p0 = &Yg_s[(16 * kc + tr_r4) * VP + nb * 32 + tr_c];
          dVr[nb] = mfma32(pa[kc], join(lds_tr(p0), lds_tr(p0 + 8 * VP)), dVr[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const bf16* p0 = &Qg_s[(16 * kc + tr_r4) * KP + nb * 32 + tr_c];
          dKr[nb] = mfma32(da[kc], join(lds_tr(p0), lds_tr(p0 + 8 * KP)), dKr[nb]);
        }
      }
      // dS^T -> LDS (whole-vector bit casts only)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const uintx4 u = __builtin_bit_cast(uintx4, da[kc]);
        bf16* row = &St_s[krow * SP + kc * 16 + hi * 4];
        *reinterpret_cast<uintx2*>(row) = uintx2{u[0], u[1]};
        *reinterpret_cast<uintx2*>(row + 8) = uintx2{u[2], u[3]};
      }
    }
    __syncthreads();

    if (valid) {
      // dQ(rows i0..i0+31) += dS K: wavefront kw takes head-dim blocks kw, kw+4, ...
      float* dQa = a.dq_acc + qbase + (int64_t)n1 * a.q_sn;
#pragma unroll
      for (int nd = kw; nd < NBK; nd += 4) {
        floatx16 acc = {};
#pragma unroll
        for (int kc = 0; kc < BC / 16; ++kc) {
          const bf16* pa0 = &St_s[(16 * kc + tr_r8) * SP + tr_c];
          const bf16* pb0 = &Ks[(16 * kc + tr_r8) * KP + nd * 32 + tr_c];
          acc = mfma32(join(lds_tr(pa0), lds_tr(pa0 + 4 * SP)), join(lds_tr(pb0), lds_tr(pb0 + 4 * KP)), acc);
        }
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const int i = i0 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
          if (i < s1) unsafeAtomicAdd(dQa + (int64_t)i * a.q_ss + nd * 32 + l32, acc[rg]);
        }
      }
    }
  }

  // ---- add the second group's dK/dV into the first group's, 32 columns at a time
  float* red = reinterpret_cast<float*>(Ks);  // K/V tiles are no longer read
#pragma unroll
  for (int nb = 0; nb < NBK; ++nb) {
    __syncthreads();
    if (qg == 1) {
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) red[(kw * 16 + rg) * 64 + lane] = dKr[nb][rg];
    }
    __syncthreads();
    if (qg == 0) {
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) dKr[nb][rg] += red[(kw * 16 + rg) * 64 + lane];
    }
  }
#pragma unroll
  for (int nb = 0; nb < NBV; ++nb) {
    __syncthreads();
    if (qg == 1) {
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) red[(kw * 16 + rg) * 64 + lane] = dVr[nb][rg];
    }
    __syncthreads();
    if (qg == 0) {
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) dVr[nb][rg] += red[(kw * 16 + rg) * 64 + lane];
    }
  }
  const bool split = a.heads_per_job < a.G;  // other workgroups share this key/value head
  if (qg != 0 || (T == 0 && split)) return;

  // ---- output: bf16 directly, or fp32 adds when other workgroups share the key/value head
#pragma unroll
  for (int rg = 0; rg < 16; ++rg) {
    const int j = j0 + kw * 32 + (rg >> 2) * 8 + hi * 4 + (rg & 3);
    if (j >= s2) continue;
    if (split) {
      float* dKa = a.dk_acc + kbase + (int64_t)n2 * a.k_sn + (int64_t)j * a.k_ss;
      float* dVa = a.dv_acc + vbase + (int64_t)n2 * a.v_sn + (int64_t)j * a.v_ss;
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) unsafeAtomicAdd(dKa + nb * 32 + l32, dKr[nb][rg] * a.scale);
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) unsafeAtomicAdd(dVa + nb * 32 + l32, dVr[nb][rg]);
    } else {
      bf16* dKg = static_cast<bf16*>(a.dk) + kbase + (int64_t)n2 * a.k_sn + (int64_t)j * a.k_ss;
      bf16* dVg = static_cast<bf16*>(a.dv) + vbase + (int64_t)n2 * a.v_sn + (int64_t)j * a.v_ss;
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) dKg[nb * 32 + l32] = (bf16)(dKr[nb][rg] * a.scale);
#pragma unroll
      for (int nb = 0; nb < NBV; ++nb) dVg[nb * 32 + l32] = (bf16)dVr[nb][rg];
    }
  }
}

// ---------------------------------------------------------------- launchers

namespace {
// Launch and return the status of this launch only (hipLaunchKernel's own
// return value), never a stale error left in the runtime by another call.
template <typename T> struct same_type { using type = T; };
template <typename... KArgs>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

int64_t q_elems(const KernelArgs& a) {
  return a.varlen ? a.T1 * a.N1 * a.D : (int64_t)a.B * a.S1 * a.N1 * a.D;
}
int64_t k_elems(const KernelArgs& a) {
  return a.varlen ? a.T2 * a.N2 * a.D : (int64_t)a.B * a.S2 * a.N2 * a.D;
}
int64_t v_elems(const KernelArgs& a) {
  return a.varlen ? a.T2 * a.N2 * a.Dv : (int64_t)a.B * a.S2 * a.N2 * a.Dv;
}
}  // namespace

int launch_preprocess(const KernelArgs& a, bool zero_dq_acc, void* stream) {
  const int lpr = a.Dv / 8;
  const int64_t rpb = 256 / lpr;
  const int64_t rows = a.varlen ? a.T1 * a.N1 : (int64_t)a.B * a.S1 * a.N1;
  // BSND: blocks of rpb rows of one (batch, head) pair; otherwise of rpb rows
  const int64_t pairs = (int64_t)a.B * a.N1;
  const int64_t blocks = a.layout == 0 ? pairs * ((a.S1 + rpb - 1) / rpb) : (rows + rpb - 1) / rpb;
  if (blocks <= 0) return 0;
  if (blocks > UINT32_MAX) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t dqe = zero_dq_acc ? q_elems(a) : 0;
  const int64_t dke = zero_dq_acc && split_heads(a) ? k_elems(a) : 0;
  const int64_t dve = zero_dq_acc && split_heads(a) ? v_elems(a) : 0;
  const dim3 grid((unsigned)blocks), block(256);
  const int z = zero_dq_acc ? 1 : 0;
  auto go = [&](auto kernel) { return launch(kernel, grid, block, s, a, rows, (uint32_t)pairs, z, dqe, dke, dve); };
  auto by_layout = [&](auto dv, auto f16) {
    constexpr int DV = decltype(dv)::value;
    constexpr bool F16 = decltype(f16)::value;
    if (a.layout == FA_LAYOUT_BSND) return go(preprocess_kernel<DV, F16, FA_LAYOUT_BSND>);
    if (a.layout == FA_LAYOUT_BNSD) return go(preprocess_kernel<DV, F16, FA_LAYOUT_BNSD>);
    return go(preprocess_kernel<DV, F16, FA_LAYOUT_TND>);
  };
  using T = std::true_type;
  using F = std::false_type;
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  if (a.Dv == 128) return a.f16 ? by_layout(D128{}, T{}) : by_layout(D128{}, F{});
  if (a.Dv == 64) return a.f16 ? by_layout(D64{}, T{}) : by_layout(D64{}, F{});
  return (int)hipErrorInvalidValue;
}

int launch_dq_finalize(const KernelArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto one = [&](const float* acc, void* out, int64_t elems, float scale) -> int {
    const int64_t n8 = elems / 8;
    int64_t blocks = (n8 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks <= 0) return 0;
    return launch(dq_finalize_kernel, dim3((unsigned)blocks), dim3(256), s, acc, static_cast<bf16*>(out), n8, scale);
  };
  int e = one(a.dq_acc, a.dq, q_elems(a), a.scale);
  if (e == 0 && split_heads(a)) e = one(a.dk_acc, a.dk, k_elems(a), 1.f);
  if (e == 0 && split_heads(a)) e = one(a.dv_acc, a.dv, v_elems(a), 1.f);
  return e;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

bool main_instantiated(int D, int Dv) {
  return (D == 64 && Dv == 64) || (D == 128 && (Dv == 64 || Dv == 128)) || (D == 192 && (Dv == 64 || Dv == 128));
}

bool main_v2_instantiated(int D, int Dv) {
  return (D == 64 && Dv == 64) || (D == 128 && (Dv == 64 || Dv == 128));
}

int launch_main(const KernelArgs& a, void* stream) {
  const int64_t tiles = (a.S2 + KV_TILE - 1) / KV_TILE;
  if (a.variant == 1) {
    const int64_t blocks = tiles * (a.G / a.heads_per_job) * a.B * a.N2;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(512);
    if (a.D == 64 && a.Dv == 64) return launch(bwd_main_v2_kernel<64, 64>, grid, block, s, a);
    if (a.D == 128 && a.Dv == 64) return launch(bwd_main_v2_kernel<128, 64>, grid, block, s, a);
    if (a.D == 128 && a.Dv == 128) return launch(bwd_main_v2_kernel<128, 128>, grid, block, s, a);
    return (int)hipErrorInvalidValue;
  }
  const int64_t blocks = tiles * a.N2 * a.B;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks), block(256);
  if (a.D == 64 && a.Dv == 64) return launch(bwd_main_kernel<64, 64>, grid, block, s, a);
  else if (a.D == 128 && a.Dv == 64) return launch(bwd_main_kernel<128, 64>, grid, block, s, a);
  else if (a.D == 128 && a.Dv == 128) return launch(bwd_main_kernel<128, 128>, grid, block, s, a);
  else if (a.D == 192 && a.Dv == 64) return launch(bwd_main_kernel<192, 64>, grid, block, s, a);
  else if (a.D == 192 && a.Dv == 128) return launch(bwd_main_kernel<192, 128>, grid, block, s, a);
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------- timing hook

struct Profiler {
  int slots = 0;
  int next = 0;    // slot of the next begin/end pair
  int count = 0;   // recorded pairs not yet read
  hipEvent_t* start = nullptr;
  hipEvent_t* mid = nullptr;   // boundary between the two main kernels
  hipEvent_t* stop = nullptr;
  bool* has_mid = nullptr;
};

Profiler* profiler_create(int slots) {
  Profiler* p = new (std::nothrow) Profiler();
  if (!p) return nullptr;
  p->start = new (std::nothrow) hipEvent_t[slots]();
  p->mid = new (std::nothrow) hipEvent_t[slots]();
  p->stop = new (std::nothrow) hipEvent_t[slots]();
  p->has_mid = new (std::nothrow) bool[slots]();
  if (!p->start || !p->mid || !p->stop || !p->has_mid) { profiler_destroy(p); return nullptr; }
  for (int i = 0; i < slots; ++i) {
    if (hipEventCreate(&p->start[i]) != hipSuccess || hipEventCreate(&p->mid[i]) != hipSuccess ||
        hipEventCreate(&p->stop[i]) != hipSuccess) {
      p->slots = i + 1;
      profiler_destroy(p);
      return nullptr;
    }
  }
  p->slots = slots;
  return p;
}

void profiler_destroy(Profiler* p) {
  if (!p) return;
  for (int i = 0; i < p->slots; ++i) {
    if (p->start && p->start[i]) (void)hipEventDestroy(p->start[i]);
    if (p->mid && p->mid[i]) (void)hipEventDestroy(p->mid[i]);
    if (p->stop && p->stop[i]) (void)hipEventDestroy(p->stop[i]);
  }
  delete[] p->start;
  delete[] p->mid;
  delete[] p->stop;
  delete[] p->has_mid;
  delete p;
}

int profiler_begin(Profiler* p, void* stream) {
  p->has_mid[p->next] = false;
  return (int)hipEventRecord(p->start[p->next], static_cast<hipStream_t>(stream));
}

int profiler_mark(Profiler* p, void* stream) {
  p->has_mid[p->next] = true;
  return (int)hipEventRecord(p->mid[p->next], static_cast<hipStream_t>(stream));
}

int profiler_end(Profiler* p, void* stream) {
  const int e = (int)hipEventRecord(p->stop[p->next], static_cast<hipStream_t>(stream));
  p->next = (p->next + 1) % p->slots;
  if (p->count < p->slots) ++p->count;
  return e;
}

int profiler_read(Profiler* p, float* ms, float* second, int cap, int* count) {
  const int n = p->count < cap ? p->count : cap;
  const int first = (p->next - p->count + p->slots) % p->slots;  // oldest recorded slot
  for (int i = 0; i < n; ++i) {
    const int k = (first + (p->count - n) + i) % p->slots;     // newest n, oldest first
    if (hipEventSynchronize(p->stop[k]) != hipSuccess) return 1;
    if (!second) {
      if (hipEventElapsedTime(&ms[i], p->start[k], p->stop[k]) != hipSuccess) return 1;
    } else if (p->has_mid[k]) {
      if (hipEventElapsedTime(&ms[i], p->start[k], p->mid[k]) != hipSuccess) return 1;
      if (hipEventElapsedTime(&second[i], p->mid[k], p->stop[k]) != hipSuccess) return 1;
    } else {
      if (hipEventElapsedTime(&ms[i], p->start[k], p->stop[k]) != hipSuccess) return 1;
      second[i] = 0.f;
    }
  }
  *count = n;
  p->count = 0;
  return 0;
}

}  // namespace fabwd
