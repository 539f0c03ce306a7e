// gfx950 attention forward: attn_out Y and softmax_lse, the two saved tensors
// the backward consumes.
//
// Formulas: page "CANN ops-transformer FlashAttnGrad 算子详解", section 一
// (S = scale * Q K^T, P_ij = exp(S_ij - softmax_lse_i), Y = P V; the lse is
// the per-row log-sum-exp that makes P sum to one).  Masks, layouts and GQA
// mapping are the ones of the backward (include/fa_bwd.h).
//
// Layout: one workgroup = 4 wavefronts = 128 query rows of one query head
// (32 rows per wavefront).  Keys stream through LDS 64 at a time.  Each
// wavefront computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as M,
// query rows as N), so every lane owns one query row and the online softmax
// (running max m and sum l) stays inside the lane plus its partner lane 32
// apart.  P then feeds O^T += V^T P^T as the B operand straight from
// registers; V^T comes from LDS through ds_read_b64_tr_b16.  O^T's
// accumulator keeps the query row per lane, so the rescale by exp(m_old -
// m_new) is lane-local.

#include <hip/hip_runtime.h>

#include "fa_bwd_internal.h"
#include "fa_bwd_schedule.h"

namespace fabwd {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Elements are bf16, or IEEE fp16 when F16 (same 16-bit storage).
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
template <bool F16>
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ bf16 to_elem(float x) {  // round to nearest even
  if constexpr (F16) return __builtin_bit_cast(bf16, (_Float16)x);
  else return (bf16)x;
}
__device__ __forceinline__ shortx4 lds_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(p));
}
__device__ __forceinline__ bf16x8 join(shortx4 lo, shortx4 hi) {
  shortx8 s = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, s);
}

constexpr int FQ = 128;  // query rows per workgroup
constexpr int FK = 64;   // keys per step

template <int HD, int HDV, bool F16>
__global__ __launch_bounds__(256, 1) void fwd_kernel(KernelArgs a, bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int KP = HD + 8;
  constexpr int VP = HDV + 8;
  constexpr int NKQ = HD / 16;
  constexpr int NB = HDV / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[FK * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[FK * VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int bid = blockIdx.x;
  const int per_tile = a.N1 * a.B;
  const int tile = bid / per_tile;
  const int rem = bid - tile * per_tile;
  const int n1 = rem % a.N1;
  const int b = rem / a.N1;
  const int n2 = n1 / a.G;

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
    s1 = a.S1; s2 = a.S2;
    qbase = (int64_t)b * a.q_sb; obase = (int64_t)b * a.o_sb;
    kbase = (int64_t)b * a.k_sb; vbase = (int64_t)b * a.v_sb;
    lbase = (int64_t)b * a.l_sb;
  }
  // rows / keys that take part (seqused_q / seqused_kv); rows past them
  // (s1 <= row < s1a) get attn_out = 0 and softmax_lse = -inf
  const int s1a = s1;
  if (a.seqused_q) s1 = fa_sched::used_len(s1a, a.seqused_q[b]);
  if (a.seqused_kv) s2 = fa_sched::used_len(s2, a.seqused_kv[b]);
  const int i0 = tile * FQ;
  if (i0 >= s1a) return;
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;
  const int iq = i0 + wave * 32 + l32;  // this lane's query row

  const bf16* __restrict__ Qg = static_cast<const bf16*>(a.q) + qbase + (int64_t)n1 * a.q_sn;
  const bf16* __restrict__ Kg = static_cast<const bf16*>(a.k) + kbase + (int64_t)n2 * a.k_sn;
  const bf16* __restrict__ Vg = static_cast<const bf16*>(a.v) + vbase + (int64_t)n2 * a.v_sn;

  bf16x8 qf[NKQ];  // B operand of S^T = K Q^T: query iq, dims 16*kk + 8*hi + 0..7
#pragma unroll
  for (int kk = 0; kk < NKQ; ++kk) {
    bf16x8 val = {};
    if (iq < s1) val = *reinterpret_cast<const bf16x8*>(Qg + (int64_t)iq * a.q_ss + 16 * kk + 8 * hi);
    qf[kk] = val;
  }

  // keys that any row of [i0, i0 + FQ) can see
  const fa_sched::Span kblk =
      i0 < s1 ? fa_sched::blocks_covering(fa_sched::keys_seen(s2, i0, min(i0 + FQ, s1), off, wl, wr), FK)
              : fa_sched::Span{0, 0};

  const int tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int tr_r4 = 4 * hi + ((lane & 15) >> 2);

  floatx16 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = floatx16{};
  float m = -__builtin_inff(), l = 0.f;

  for (int j0 = kblk.lo * FK; j0 < kblk.hi * FK; j0 += FK) {
    __syncthreads();
    for (int c = tid; c < FK * (HD / 8); c += 256) {
      const int r = c / (HD / 8), cc = (c % (HD / 8)) * 8;
      bf16x8 val = {};
      if (j0 + r < s2) val = *reinterpret_cast<const bf16x8*>(Kg + (int64_t)(j0 + r) * a.k_ss + cc);
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + cc]) = val;
    }
    for (int c = tid; c < FK * (HDV / 8); c += 256) {
      const int r = c / (HDV / 8), cc = (c % (HDV / 8)) * 8;
      bf16x8 val = {};
      if (j0 + r < s2) val = *reinterpret_cast<const bf16x8*>(Vg + (int64_t)(j0 + r) * a.v_ss + cc);
      *reinterpret_cast<bf16x8*>(&Vs[r * VP + cc]) = val;
    }
    __syncthreads();

    // S^T for 64 keys (2 blocks of 32) x this wavefront's 32 query rows
    floatx16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = floatx16{};
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(mb * 32 + l32) * KP + 16 * kk + 8 * hi]);
        s[mb] = mfma32<F16>(ka, qf[kk], s[mb]);
      }
    }
    // scores in log2 units, masked to -inf
    const bool full = fa_sched::tile_full(i0, FQ, j0, FK, s1, s2, off, wl, wr);
    float mx = -__builtin_inff();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[mb][r] * a.scale_log2;
        if (!full) {
          const int j = j0 + mb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const bool vis = fa_sched::visible(iq, j, s1, s2, off, wl, wr);
          x = vis ? x : -__builtin_inff();
        }
        s[mb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    float rs = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[mb][r] - m_use);
        rs += p;
        pb[mb * 2 + (r >> 3)][r & 7] = to_elem<F16>(p);
      }
    }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
    }
    // O^T[dv][query] += V^T P^T over 4 chunks of 16 keys
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16* p0 = &Vs[(16 * kc + tr_r4) * VP + nb * 32 + tr_c];
        const bf16x8 va = join(lds_tr(p0), lds_tr(p0 + 8 * VP));
        o[nb] = mfma32<F16>(va, pb[kc], o[nb]);
      }
    }
  }

  if (iq < s1a) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    bf16* __restrict__ Og = out + obase + (int64_t)n1 * a.o_sn + (int64_t)iq * a.o_ss;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = to_elem<F16>(o[nb][r4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(Og + nb * 32 + r4 * 8 + hi * 4) = w;
      }
    }
    if (hi == 0) {
      const float v = (l > 0.f) ? (m + __log2f(l)) * kLn2 : -__builtin_inff();
      lse[lbase + (int64_t)n1 * a.l_sn + iq] = v;
    }
  }
}

}  // namespace

// Launch and return the status of this launch only (hipLaunchKernel's own
// return value), never a stale error left in the runtime by another call.
template <typename T> struct same_type { using type = T; };
template <typename... KArgs>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

namespace {
template <bool F16>
int launch_forward_t(const KernelArgs& a, dim3 grid, hipStream_t s, bf16* o, float* lse) {
  const dim3 block(256);
  if (a.D == 64 && a.Dv == 64) return launch(fwd_kernel<64, 64, F16>, grid, block, s, a, o, lse);
  if (a.D == 128 && a.Dv == 64) return launch(fwd_kernel<128, 64, F16>, grid, block, s, a, o, lse);
  if (a.D == 128 && a.Dv == 128) return launch(fwd_kernel<128, 128, F16>, grid, block, s, a, o, lse);
  if (a.D == 192 && a.Dv == 64) return launch(fwd_kernel<192, 64, F16>, grid, block, s, a, o, lse);
  if (a.D == 192 && a.Dv == 128) return launch(fwd_kernel<192, 128, F16>, grid, block, s, a, o, lse);
  return (int)hipErrorInvalidValue;
}
}  // namespace

int launch_forward(const KernelArgs& a, void* out, float* lse, void* stream) {
  const int64_t tiles = (a.S1 + FQ - 1) / FQ;
  const int64_t blocks = tiles * a.N1 * a.B;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bf16* o = static_cast<bf16*>(out);
  const dim3 grid((unsigned)blocks);
  return a.f16 ? launch_forward_t<true>(a, grid, s, o, lse) : launch_forward_t<false>(a, grid, s, o, lse);
}

}  // namespace fabwd
