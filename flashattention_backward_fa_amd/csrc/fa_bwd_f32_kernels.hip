// gfx950 FlashAttention backward, fp32 debug form: the same bf16 inputs, but
// P and dS are never rounded to bf16, every product is an fp32 FMA on the
// VALU and dq, dk, dv are written as fp32 in the layouts of q, k, v.  It is
// there to check the arithmetic of the formulas of page "CANN ops-transformer
// FlashAttnGrad 算子详解", section 一, at fp32 accuracy; it is not tuned.
//
// dkdv_f32_kernel: one workgroup (256 threads) per 32-key tile of one
// (sequence, key/value head).  K and V of the tile sit in LDS as fp32; the
// query rows that can see the tile stream through LDS 8 at a time, for every
// query head of the GQA group.  Thread (r, j) forms S, P, dP, dS of row r and
// key j; thread (key, slice) then accumulates dK and dV of its key over the
// 8 rows, for every 8th column starting at the slice.
//
// dq_f32_kernel: one workgroup per 32 query rows of one query head; the keys
// the rows can see stream through LDS 8 at a time; thread (row, slice)
// accumulates dQ of its row.

#include <hip/hip_runtime.h>

#include "fa_bwd_internal.h"
#include "fa_bwd_schedule.h"

namespace fabwd {
namespace {

typedef __bf16 bf16;

// Inputs are bf16, or IEEE fp16 when F16 (same 16-bit storage).
template <bool F16>
__device__ __forceinline__ float from_elem(bf16 v) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, v);
  else return (float)v;
}

constexpr int F32_BK = 32;   // keys per dK/dV workgroup
constexpr int F32_BQ = 32;   // query rows per dQ workgroup
constexpr int F32_CH = 8;    // rows (dK/dV) or keys (dQ) per LDS chunk
constexpr int F32_MAXD = 192;

// s1, s2: rows / keys that take part (seqused_q / seqused_kv when given);
// s1a, s2a: rows / keys the sequence holds.
struct Seq {
  int s1, s2, s1a, s2a;
  int64_t qbase, kbase, vbase, obase, lbase;
};

__device__ Seq seq_of(const KernelArgs& a, int b) {
  Seq r;
  if (a.varlen) {
    const int q0 = a.cu_q[b], k0 = a.cu_kv[b];
    r.s1 = a.cu_q[b + 1] - q0;
    r.s2 = a.cu_kv[b + 1] - k0;
    r.qbase = (int64_t)q0 * a.q_ss;
    r.obase = (int64_t)q0 * a.o_ss;
    r.kbase = (int64_t)k0 * a.k_ss;
    r.vbase = (int64_t)k0 * a.v_ss;
    r.lbase = q0;
  } else {
    r.s1 = a.S1;
    r.s2 = a.S2;
    r.qbase = (int64_t)b * a.q_sb;
    r.obase = (int64_t)b * a.o_sb;
    r.kbase = (int64_t)b * a.k_sb;
    r.vbase = (int64_t)b * a.v_sb;
    r.lbase = (int64_t)b * a.l_sb;
  }
  r.s1a = r.s1;
  r.s2a = r.s2;
  if (a.seqused_q) r.s1 = fa_sched::used_len(r.s1a, a.seqused_q[b]);
  if (a.seqused_kv) r.s2 = fa_sched::used_len(r.s2a, a.seqused_kv[b]);
  return r;
}


template <bool F16>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(KernelArgs a) {
  __shared__ float Ks[F32_BK][F32_MAXD + 1];   // +1: conflict-free column walks
  __shared__ float Vs[F32_BK][F32_MAXD + 1];
  __shared__ float Qr[F32_CH][F32_MAXD + 1];
  __shared__ float Yr[F32_CH][F32_MAXD + 1];
  __shared__ float Ps[F32_CH][F32_BK];
  __shared__ float dSs[F32_CH][F32_BK];
  __shared__ float lse_s[F32_CH], sfm_s[F32_CH];

  const int t = threadIdx.x;
  const int D = a.D, Dv = a.Dv;
  int r = blockIdx.x;
  const int n2 = r % a.N2; r /= a.N2;
  const int b = r % a.B;
  const int tile = r / a.B;
  const Seq sq = seq_of(a, b);
  const int j0 = tile * F32_BK;
  if (j0 >= sq.s2a) return;  // keys past the used ones get zeros below
  const int off = sq.s2 - sq.s1;

  const bf16* K = static_cast<const bf16*>(a.k) + sq.kbase + (int64_t)n2 * a.k_sn;
  const bf16* V = static_cast<const bf16*>(a.v) + sq.vbase + (int64_t)n2 * a.v_sn;
  for (int e = t; e < F32_BK * F32_MAXD; e += 256) {
    const int jj = e / F32_MAXD, d = e % F32_MAXD;
    const int j = j0 + jj;
    Ks[jj][d] = (j < sq.s2 && d < D) ? from_elem<F16>(K[(int64_t)j * a.k_ss + d]) : 0.f;
    Vs[jj][d] = (j < sq.s2 && d < Dv) ? from_elem<F16>(V[(int64_t)j * a.v_ss + d]) : 0.f;
  }

  // rows that can see a key of the tile
  const fa_sched::Span rows = j0 < sq.s2 ? fa_sched::rows_seeing(sq.s1, j0, min(j0 + F32_BK, sq.s2), off,
                                                                  a.win_left, a.win_right)
                                         : fa_sched::Span{0, 0};
  const int i_lo = rows.lo, i_hi = rows.hi;

  const int pr = t / F32_BK, pj = t % F32_BK;   // pair role: row pr of the chunk, key pj
  const int ak = t / 8, sl = t % 8;             // accumulation role: key ak, columns sl, sl+8, ...
  float dk[F32_MAXD / 8], dv[F32_MAXD / 8];
#pragma unroll
  for (int m = 0; m < F32_MAXD / 8; ++m) dk[m] = dv[m] = 0.f;

  for (int g = 0; g < a.G; ++g) {
    const int n1 = n2 * a.G + g;
    const bf16* Q = static_cast<const bf16*>(a.q) + sq.qbase + (int64_t)n1 * a.q_sn;
    const bf16* Y = static_cast<const bf16*>(a.dout) + sq.obase + (int64_t)n1 * a.o_sn;
    const float* L = a.lse + sq.lbase + (int64_t)n1 * a.l_sn;
    const float* F = a.sfmg + sq.lbase + (int64_t)n1 * a.l_sn;
    for (int c0 = i_lo; c0 < i_hi; c0 += F32_CH) {
      __syncthreads();  // the previous chunk is consumed
      for (int e = t; e < F32_CH * F32_MAXD; e += 256) {
        const int rr = e / F32_MAXD, d = e % F32_MAXD;
        const int i = c0 + rr;
        Qr[rr][d] = (i < i_hi && d < D) ? from_elem<F16>(Q[(int64_t)i * a.q_ss + d]) : 0.f;
        Yr[rr][d] = (i < i_hi && d < Dv) ? from_elem<F16>(Y[(int64_t)i * a.o_ss + d]) : 0.f;
      }
      if (t < F32_CH) {
        const int i = c0 + t;
        lse_s[t] = i < i_hi ? L[i] : -__builtin_inff();
        sfm_s[t] = i < i_hi ? F[i] : 0.f;
      }
      __syncthreads();
      {
        const int i = c0 + pr, j = j0 + pj;
        float p = 0.f, ds = 0.f;
        if (i < i_hi && fa_sched::visible(i, j, sq.s1, sq.s2, off, a.win_left, a.win_right) &&
            lse_s[pr] != -__builtin_inff()) {
          float s = 0.f, dp = 0.f;
          for (int d = 0; d < D; ++d) s = fmaf(Qr[pr][d], Ks[pj][d], s);
          for (int d = 0; d < Dv; ++d) dp = fmaf(Yr[pr][d], Vs[pj][d], dp);
          p = expf(s * a.scale - lse_s[pr]);
          ds = p * (dp - sfm_s[pr]);
        }
        Ps[pr][pj] = p;
        dSs[pr][pj] = ds;
      }
      __syncthreads();
      for (int rr = 0; rr < F32_CH; ++rr) {
        const float p = Ps[rr][ak], ds = dSs[rr][ak];
#pragma unroll
        for (int m = 0; m < F32_MAXD / 8; ++m) {
          const int d = sl + 8 * m;
          if (d < Dv) dv[m] = fmaf(p, Yr[rr][d], dv[m]);
          if (d < D) dk[m] = fmaf(ds, Qr[rr][d], dk[m]);
        }
      }
    }
  }
  const int j = j0 + ak;
  if (j < sq.s2a) {
    float* dK = static_cast<float*>(a.dk) + sq.kbase + (int64_t)n2 * a.k_sn + (int64_t)j * a.k_ss;
    float* dV = static_cast<float*>(a.dv) + sq.vbase + (int64_t)n2 * a.v_sn + (int64_t)j * a.v_ss;
#pragma unroll
    for (int m = 0; m < F32_MAXD / 8; ++m) {
      const int d = sl + 8 * m;
      if (d < D) dK[d] = dk[m] * a.scale;
      if (d < Dv) dV[d] = dv[m];
    }
  }
}

template <bool F16>
__global__ __launch_bounds__(256) void dq_f32_kernel(KernelArgs a) {
  __shared__ float Qs[F32_BQ][F32_MAXD + 1];
  __shared__ float Ys[F32_BQ][F32_MAXD + 1];
  __shared__ float Kc[F32_CH][F32_MAXD + 1];
  __shared__ float Vc[F32_CH][F32_MAXD + 1];
  __shared__ float dSs[F32_BQ][F32_CH];
  __shared__ float lse_s[F32_BQ], sfm_s[F32_BQ];

  const int t = threadIdx.x;
  const int D = a.D, Dv = a.Dv;
  int r = blockIdx.x;
  const int n1 = r % a.N1; r /= a.N1;
  const int b = r % a.B;
  const int tile = r / a.B;
  const int n2 = n1 / a.G;
  const Seq sq = seq_of(a, b);
  const int i0 = tile * F32_BQ;
  if (i0 >= sq.s1a) return;  // rows past the used ones get zeros below
  const int off = sq.s2 - sq.s1;

  const bf16* Q = static_cast<const bf16*>(a.q) + sq.qbase + (int64_t)n1 * a.q_sn;
  const bf16* Y = static_cast<const bf16*>(a.dout) + sq.obase + (int64_t)n1 * a.o_sn;
  const bf16* K = static_cast<const bf16*>(a.k) + sq.kbase + (int64_t)n2 * a.k_sn;
  const bf16* V = static_cast<const bf16*>(a.v) + sq.vbase + (int64_t)n2 * a.v_sn;
  for (int e = t; e < F32_BQ * F32_MAXD; e += 256) {
    const int rr = e / F32_MAXD, d = e % F32_MAXD;
    const int i = i0 + rr;
    Qs[rr][d] = (i < sq.s1 && d < D) ? from_elem<F16>(Q[(int64_t)i * a.q_ss + d]) : 0.f;
    Ys[rr][d] = (i < sq.s1 && d < Dv) ? from_elem<F16>(Y[(int64_t)i * a.o_ss + d]) : 0.f;
  }
  if (t < F32_BQ) {
    const int i = i0 + t;
    lse_s[t] = i < sq.s1 ? a.lse[sq.lbase + (int64_t)n1 * a.l_sn + i] : -__builtin_inff();
    sfm_s[t] = i < sq.s1 ? a.sfmg[sq.lbase + (int64_t)n1 * a.l_sn + i] : 0.f;
  }

  // keys that a row of the tile can see
  const fa_sched::Span keys = i0 < sq.s1 ? fa_sched::keys_seen(sq.s2, i0, min(i0 + F32_BQ, sq.s1), off,
                                                                a.win_left, a.win_right)
                                         : fa_sched::Span{0, 0};
  const int j_lo = keys.lo, j_hi = keys.hi;

  const int pr = t / F32_CH, pc = t % F32_CH;   // pair role: row pr, key pc of the chunk
  const int ar = t / 8, sl = t % 8;             // accumulation role: row ar, columns sl, sl+8, ...
  float dq[F32_MAXD / 8];
#pragma unroll
  for (int m = 0; m < F32_MAXD / 8; ++m) dq[m] = 0.f;

  for (int c0 = j_lo; c0 < j_hi; c0 += F32_CH) {
    __syncthreads();  // the previous chunk is consumed (and the Q/dY tile is in place)
    for (int e = t; e < F32_CH * F32_MAXD; e += 256) {
      const int cc = e / F32_MAXD, d = e % F32_MAXD;
      const int j = c0 + cc;
      Kc[cc][d] = (j < j_hi && d < D) ? from_elem<F16>(K[(int64_t)j * a.k_ss + d]) : 0.f;
      Vc[cc][d] = (j < j_hi && d < Dv) ? from_elem<F16>(V[(int64_t)j * a.v_ss + d]) : 0.f;
    }
    __syncthreads();
    {
      const int i = i0 + pr, j = c0 + pc;
      float ds = 0.f;
      if (j < j_hi && fa_sched::visible(i, j, sq.s1, sq.s2, off, a.win_left, a.win_right) &&
          lse_s[pr] != -__builtin_inff()) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(Qs[pr][d], Kc[pc][d], s);
        for (int d = 0; d < Dv; ++d) dp = fmaf(Ys[pr][d], Vc[pc][d], dp);
        const float p = expf(s * a.scale - lse_s[pr]);
        ds = p * (dp - sfm_s[pr]);
      }
      dSs[pr][pc] = ds;
    }
    __syncthreads();
    for (int cc = 0; cc < F32_CH; ++cc) {
      const float ds = dSs[ar][cc];
#pragma unroll
      for (int m = 0; m < F32_MAXD / 8; ++m) {
        const int d = sl + 8 * m;
        if (d < D) dq[m] = fmaf(ds, Kc[cc][d], dq[m]);
      }
    }
  }
  const int i = i0 + ar;
  if (i < sq.s1a) {
    float* dQ = static_cast<float*>(a.dq) + sq.qbase + (int64_t)n1 * a.q_sn + (int64_t)i * a.q_ss;
#pragma unroll
    for (int m = 0; m < F32_MAXD / 8; ++m) {
      const int d = sl + 8 * m;
      if (d < D) dQ[d] = dq[m] * a.scale;
    }
  }
}

}  // namespace

int launch_f32_debug(const KernelArgs& a, void* stream) {
  if (a.D > F32_MAXD || a.Dv > F32_MAXD) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t kb = (int64_t)((a.S2 + F32_BK - 1) / F32_BK) * a.B * a.N2;
  const int64_t qb = (int64_t)((a.S1 + F32_BQ - 1) / F32_BQ) * a.B * a.N1;
  if (kb > 0x7fffffff || qb > 0x7fffffff) return (int)hipErrorInvalidValue;
  KernelArgs args = a;
  if (kb > 0) {
    void* argv[] = {&args};
    const void* k = reinterpret_cast<const void*>(a.f16 ? dkdv_f32_kernel<true> : dkdv_f32_kernel<false>);
    const hipError_t e = hipLaunchKernel(k, dim3((unsigned)kb), dim3(256), argv, 0, s);
    if (e != hipSuccess) return (int)e;
  }
  if (qb > 0) {
    void* argv[] = {&args};
    const void* k = reinterpret_cast<const void*>(a.f16 ? dq_f32_kernel<true> : dq_f32_kernel<false>);
    const hipError_t e = hipLaunchKernel(k, dim3((unsigned)qb), dim3(256), argv, 0, s);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace fabwd
