// gfx950 (MI355X) FlashAttention backward for short key sequences in one
// launch: the per-head schedule of page "CANN ops-transformer FlashAttnGrad
// 算子详解", section 五 5.2 (template flash_attn_grad_bn2: one core per
// (batch, key/value head), no separate pre- or post-processing pass).
//
// One workgroup owns one (sequence, key/value head) and the whole key range of
// that sequence (at most 128 keys in LDS, 32 per wavefront of a group of 4).
// At D = 64 it holds two such groups (8 wavefronts, two per SIMD) that take
// alternate query blocks and add their dK / dV up at the end; at D = 128 one.
// It forms every quantity of section 一 for the G query heads of the group:
//   sfmg = rowsum(dY (.) Y)        for all of its query rows, first;
//   S = scale * Q K^T, P = exp(S - lse), dP = dY V^T, dS = P (.) (dP - sfmg)
//                                  per 32-row query block;
//   dV += P^T dY, dK += dS^T Q     in registers over all blocks and heads;
//   dQ = scale * dS K              per block, one step later: the four
//                                  wavefronts' dS tiles meet in LDS and D / 32
//                                  of the four wavefronts form 32 columns of
//                                  dQ each over all 128 keys.
// Every dQ row sees its whole key range inside the workgroup, so dQ is
// written once, with no atomics and no workspace, and the result is bitwise
// repeatable.  S and dP put query rows on M and keys on N, as in the dK/dV
// kernel (fa_bwd_det_kernels.hip), so P and dS packed to 16 bits are MFMA
// operands of the key products as they stand.  dV, dK and dQ accumulate
// transposed (the key or query row on N), so that every lane ends with
// 16-byte pieces of its own row; the dQ product reads the dS register images
// back through transposing LDS reads, like the GEMM over stored dS.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_bwd_kernarg.h"
#include "fa_bwd_tiles.h"

namespace fabwd {
namespace {

// s_waitcnt vmcnt(N): all but this wavefront's N most recent vector-memory
// instructions have completed (gfx9 retires loads and stores in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  asm volatile("" ::: "memory");
}

constexpr int FK = FUSED_MAX_KEYS;  // keys per workgroup: 4 wavefronts x 32
constexpr int FR = 32;              // query rows per step
static_assert(FK == 128, "one 32-key slice per wavefront");

// QG query groups of 4 wavefronts take alternate items (two groups at
// D = 64, where two wavefronts fit a SIMD; one at D = 128); the groups' dK / dV
// are added up at the end.
template <int HD, int HDV, int QG, bool F16>
__global__ __launch_bounds__(256 * QG, 1) void fused_kernel(KernelArgs a) {
  constexpr int NT = 256 * QG;       // threads
  constexpr int NKQ = HD / 16;
  constexpr int NKV = HDV / 16;
  constexpr int NBK = HD / 32;
  constexpr int NBV = HDV / 32;
  constexpr int QTB = FR * HD * 2;   // bytes of one Q / dY tile buffer
  constexpr int YTB = FR * HDV * 2;
  constexpr int MAXR = FUSED_MAX_BLOCKS * FR;  // query rows whose statistics fit
  static_assert(HD == 64 || HD == 128, "swizzled tiles of 64 or 128 columns");

  __shared__ __attribute__((aligned(1024))) bf16 Ks[FK * HD];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[FK * HDV];
  __shared__ __attribute__((aligned(1024))) bf16 Qs[QG][2][FR * HD];
  __shared__ __attribute__((aligned(1024))) bf16 Ys[QG][2][FR * HDV];
  // per group, double-buffered: dS images of the 4 key slices (2 KB each)
  __shared__ __attribute__((aligned(1024))) bf16 Ss[QG][2][4 * 1024];
  // with two groups: the rest of the dK / dV exchange area (below)
  __shared__ __attribute__((aligned(1024))) float Xs[QG == 2 ? 4096 : 1];
  __shared__ __attribute__((aligned(16))) float lse_s[MAXR];    // lse * log2(e) (+inf: row sees nothing)
  __shared__ __attribute__((aligned(16))) float sfm_s[MAXR];

  prefetch_args();
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave >> 2;   // query group
  const int kw = wave & 3;    // key slice
  const int n2 = blockIdx.x % a.N2;
  const int b = blockIdx.x / a.N2;
  const int G = a.G;
  const SeqBounds sb = seq_bounds(a, b);
  const int s1 = sb.s1, s2 = sb.s2;
  const int off = s2 - s1;
  const int wl = a.win_left, wr = a.win_right;
  const int kw0 = kw * 32;  // this wavefront's keys within the tile
  // the 32-column block of dQ this wavefront forms (when below D / 32): with
  // two groups at D = 64, group 1 uses wavefronts 2 and 3, so that every SIMD
  // runs one dQ product per step
  const int cb = (kw - qg * NBK) & 3;

  bf16* __restrict__ dQ = static_cast<bf16*>(a.dq) + sb.qbase;
  // blocks of 32 rows over every row the sequence holds (rows past the used
  // ones are masked and get zero gradients); a sequence longer than the plan's
  // maximum is cut to what the row statistics hold
  const int nblk = min((sb.s1a + FR - 1) / FR, FUSED_MAX_BLOCKS / G);
  const int T = G * nblk;  // items (query head, block), head-major

  if (sb.s2a == 0) {  // no keys at all: every dq row of the group is zero
    for (int h = 0; h < G; ++h) {
      const int64_t hb = (int64_t)(n2 * G + h) * a.q_sn;
      for (int x = tid; x < sb.s1a * HD; x += NT) dQ[hb + (int64_t)(x / HD) * a.q_ss + x % HD] = to_elem<F16>(0.f);
    }
    return;
  }

  // K and V (rows past the sequence's keys repeat its last key; the masks
  // ignore them), and the first item's Q / dY tiles, asynchronously
  {
    TileCopy<HD, FK, 4 * QG> kcp;
    TileCopy<HDV, FK, 4 * QG> vcp;
    kcp.init(wave, lane, (int)a.k_ss * 2);
    vcp.init(wave, lane, (int)a.v_ss * 2);
    const int kvalid = min(sb.s2a, FK);
    kcp.issue(lds_addr(Ks), static_cast<const bf16*>(a.k) + sb.kbase + (int64_t)n2 * a.k_sn, kvalid, wave, lane);
    vcp.issue(lds_addr(Vs), static_cast<const bf16*>(a.v) + sb.vbase + (int64_t)n2 * a.v_sn, kvalid, wave, lane);
  }
  TileCopy<HD, FR, 4> qcp;
  TileCopy<HDV, FR, 4> ycp;
  qcp.init(kw, lane, (int)a.q_ss * 2);
  ycp.init(kw, lane, (int)a.o_ss * 2);
  const uint32_t q_lds = lds_addr(Qs) + qg * 2 * QTB;  // this group's Q / dY buffers
  const uint32_t y_lds = lds_addr(Ys) + qg * 2 * YTB;
  auto fetch = [&](int t, int buf) {  // item t, by this group's 4 wavefronts
    const int n1 = n2 * G + t / nblk;
    const int i0 = (t % nblk) * FR;
    qcp.issue(q_lds + buf * QTB, static_cast<const bf16*>(a.q) + sb.qbase + (int64_t)n1 * a.q_sn + (int64_t)i0 * a.q_ss,
              sb.s1a - i0, kw, lane);
    ycp.issue(y_lds + buf * YTB, static_cast<const bf16*>(a.dout) + sb.obase + (int64_t)n1 * a.o_sn + (int64_t)i0 * a.o_ss,
              sb.s1a - i0, kw, lane);
  };
  if (qg < T) fetch(qg, 0);

  // Row statistics of every item: lse in base 2 (+inf for rows past the used
  // ones or with lse = -inf, so that their P is 0) and sfmg = rowsum(dY * Y).
  // Every load is issued unconditionally (rows clamped into the sequence) and
  // the row's validity applied to the value, so that a lane's loads are all
  // in flight together.
  const int R = T * FR;  // statistics rows: item r / 32, row r % 32 of its block
  auto row_of = [&](int r, int& n1, int& i) {
    const int rc = min(r, R - 1);
    n1 = n2 * G + (rc / FR) / nblk;
    i = ((rc / FR) % nblk) * FR + rc % FR;
  };
  {
    constexpr int LPR = HDV / 8;      // lanes per row
    constexpr int RPP = NT / LPR;     // rows per pass
    const int part = tid % LPR;
    // UN passes in flight per round: no more than the rows need (a clamped
    // pass would only repeat the last row's loads)
    auto stats = [&](auto un) {
      constexpr int UN = decltype(un)::value;
      for (int r0 = tid / LPR; r0 < R; r0 += RPP * UN) {
        bf16x8 y[UN], g[UN];
        float x[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          int n1, i;
          row_of(r0 + u * RPP, n1, i);
          const int ic = max(min(i, sb.s1a - 1), 0);
          const int64_t o = sb.obase + (int64_t)n1 * a.o_sn + (int64_t)ic * a.o_ss + part * 8;
          y[u] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.out) + o);
          g[u] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.dout) + o);
          x[u] = a.lse[sb.lbase + (int64_t)n1 * a.l_sn + ic];
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          float acc = 0.f;
          if constexpr (F16) {  // reinterpret whole vectors (element casts of bf16 lanes miscompile)
            const halfx8 yh = __builtin_bit_cast(halfx8, y[u]), gh = __builtin_bit_cast(halfx8, g[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)gh[e] * (float)yh[e];
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)g[u][e] * (float)y[u][e];
          }
#pragma unroll
          for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
          int n1, i;
          const int r = r0 + u * RPP;
          row_of(r, n1, i);
          if (part == 0 && r < R) {
            sfm_s[r] = i < sb.s1a ? acc : 0.f;
            lse_s[r] = (i < s1 && x[u] != -__builtin_inff()) ? x[u] * kLog2e : __builtin_inff();
          }
        }
      }
    };
    if (R <= RPP) stats(std::integral_constant<int, 1>{});
    else if (R <= 2 * RPP) stats(std::integral_constant<int, 2>{});
    else if (R <= 4 * RPP) stats(std::integral_constant<int, 4>{});
    else stats(std::integral_constant<int, 8>{});
  }

  // dK and dV accumulate transposed (lane = key, elements = columns), so
  // that each lane ends with pieces of its key's rows
  floatx16 dKr[NBK], dVr[NBV];
#pragma unroll
  for (int i = 0; i < NBK; ++i) dKr[i] = floatx16{};
#pragma unroll
  for (int i = 0; i < NBV; ++i) dVr[i] = floatx16{};

  SwzTile<HD, FK> kadr;
  SwzTile<HDV, FK> vadr;
  SwzTile<HD, FR> qadr;
  SwzTile<HDV, FR> yadr;
  kadr.init(lds_addr(Ks), lane);
  vadr.init(lds_addr(Vs), lane);
  qadr.init(q_lds, lane);
  yadr.init(y_lds, lane);

  // B operand of dQ^T = K^T dS^T (keys on K, query rows on N) read back from
  // the dS register images in Ss: lane i of a 16-lane group receives, as
  // element e of a transposing read, element i % 4 of the 8 bytes that lane
  // 4e + i/4 of the group loads; lane L = 4e + q (g = lane / 16) loads rows
  // 16*(g % 2) + 4q + 0..3 of key 16kc + 8s + 4*(g / 2) + e, which the
  // producing wavefront's lane 32*(q % 2) + key holds in half g % 2, elements
  // 4*(q / 2) + 0..3.  Within each 1 KB half h, chunk c (the producer lane)
  // sits at ds_chunk_slot(c, h), which spreads these reads over all banks.
  constexpr uint32_t SGB = 2 * 8192;  // bytes of one group's two dS buffers
  uint32_t a_base[2];
  {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3, h = g & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 32 * (q & 1) + 8 * s + 4 * (g >> 1) + e;  // producer chunk at kc = 0
      a_base[s] = lds_addr(Ss) + qg * SGB + h * 1024 + ds_chunk_slot(c, h) * 16 + (q >> 1) * 8;
    }
  }
  // where this lane puts half h of its own dS image (buffer 0)
  const uint32_t s_put = lds_addr(Ss) + qg * SGB + kw * 2048;
  // dq rows of a head leave as buffer stores whose range ends with the last
  // row the sequence holds, so that rows past it are dropped by the range
  // check: every storing lane issues the same 2 store instructions per item,
  // and the wait two steps later can leave exactly those in flight (the
  // planner keeps the byte offsets below 2^31)
  constexpr int NST = 2;
  const int64_t dq_bytes = sb.s1a > 0 ? ((int64_t)(sb.s1a - 1) * a.q_ss + HD) * 2 : 0;

  wait_vmem();    // K, V, the first tiles and the statistics' loads landed
  lds_barrier();  // ... everyone's

  const int j_key = kw0 + l32;  // this lane's key
  const int nsteps = (T + QG - 1) / QG;
  // Step k: group g forms S, dP, dS, dK, dV of item t = k*QG + g and dQ of
  // its item of step k - 1, whose dS images the step's one barrier made
  // visible; one more step forms the last dQ.
  for (int k = 0; k <= nsteps; ++k) {
    const int t = k * QG + qg;
    const bool has = k < nsteps && t < T;
    const int tp = t - QG;  // the item whose dQ is formed now
    const bool hasp = k > 0 && tp < T;
    const int buf = k & 1;
    if (k > 0) {
      // this wavefront's copies of item t landed; its dq stores of step
      // k - 1, issued after those copies, may stay in flight (at step 1 it
      // has stored nothing yet)
      if (cb < NBK && k >= 2) wait_vmem_keep<NST>();
      else wait_vmem();
      lds_barrier();  // ... everyone's, and every dS image of step k - 1
    }
    if (k < nsteps && t + QG < T) fetch(t + QG, buf ^ 1);

    // dQ^T of item tp, 32 head-dim columns per wavefront, over all 128 keys
    if (hasp && cb < NBK) {
      floatx16 dq = floatx16{};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t ao = (buf ^ 1) * 8192 + sl * 2048 + c * 256;  // buffer, slice sl, chunk bit 4 = c
          const bf16x8 dsb = join(lds_load_tr(a_base[0] + ao), lds_load_tr(a_base[1] + ao));
          const int kc = 2 * sl + c;
          const bf16x8 ka = join(lds_load_tr(kadr.tr_read(kc, 0, cb)), lds_load_tr(kadr.tr_read(kc, 1, cb)));
          dq = mfma32<F16>(ka, dsb, dq);
        }
      }
      u32x4 piece[2];
      row_pieces<F16>(dq, a.scale, piece);
      const int n1p = n2 * G + tp / nblk;
      const int ip = (tp % nblk) * FR + l32;  // this lane's query row
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(dQ + (int64_t)n1p * a.q_sn, (short)0, (int)dq_bytes, 0x00020000);
#pragma unroll
      for (int pc = 0; pc < NST; ++pc) {
        const uint32_t off = (uint32_t)(((int64_t)ip * a.q_ss + cb * 32 + pc * 16 + hi * 8) * 2);
        __builtin_amdgcn_raw_buffer_store_b128(piece[pc], rsrc, (int)off, 0, 0);
      }
    }

    if constexpr (QG == 2) {
      if (k == nsteps) {
        // dK / dV exchange, while the dQ above runs: group 1's dK goes to
        // group 0 through the Q and dY buffers, group 0's dV to group 1
        // through the V tile and Xs (none of them is read or filled in the
        // last step)
        static_assert(HD == 64 && HDV == 64, "16 KB exchange areas per 32-column block");
        if (qg == 1) {
          xput(reinterpret_cast<float*>(&Qs[0][0][0]), kw, lane, dKr[0]);
          xput(reinterpret_cast<float*>(&Ys[0][0][0]), kw, lane, dKr[1]);
        } else {
          xput(reinterpret_cast<float*>(Vs), kw, lane, dVr[0]);
          xput(Xs, kw, lane, dVr[1]);
        }
      }
    }

    if (has) {
      const int i0 = (t % nblk) * FR;
      // S = Q K^T, dP = dY V^T for this wavefront's 32 keys
      floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
      for (int kk = 0; kk < NKQ; ++kk)
        sacc = mfma32<F16>(lds_load16(qadr.row_read(kk, buf * QTB)), lds_load16(kadr.row_read_at(kk, kw0)), sacc);
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk)
        pacc = mfma32<F16>(lds_load16(yadr.row_read(kk, buf * YTB)), lds_load16(vadr.row_read_at(kk, kw0)), pacc);

      // P = exp(S * scale - lse) masked, dS = P (dP - sfmg), packed to 16 bits:
      // lane = key, element rg of the accumulator = row 8*(rg/4) + 4*hi + rg%4
      const fa_sched::Window vis = fa_sched::window(fa_sched::rows_of_key(j_key, s1, s2, off, wl, wr), i0);
      bf16x8 pa[2], da[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ib = r4 * 8 + hi * 4;
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[t * FR + ib]);
        const floatx4 f4 = *reinterpret_cast<const floatx4*>(&sfm_s[t * FR + ib]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rg = r4 * 4 + e;
          float p = __builtin_amdgcn_exp2f(sacc[rg] * a.scale_log2 - l4[e]);
          p = fa_sched::in_window(vis, ib + e) ? p : 0.f;
          pa[rg >> 3][rg & 7] = to_elem<F16>(p);
          da[rg >> 3][rg & 7] = to_elem<F16>(p * (pacc[rg] - f4[e]));
        }
      }
      // this wavefront's dS image for the dQ product of the next step
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *(LDS_AS bf16x8*)(uintptr_t)(s_put + buf * 8192 + hh * 1024 + ds_chunk_slot(lane, hh) * 16) = da[hh];

      // dV^T += dY^T P, dK^T += Q^T dS (A operands: dY and Q read down their columns)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int nb = 0; nb < NBV; ++nb) {
          const bf16x8 ya = join(lds_load_tr(yadr.tr_read(kc, 0, nb, buf * YTB)), lds_load_tr(yadr.tr_read(kc, 1, nb, buf * YTB)));
          dVr[nb] = mfma32<F16>(ya, pa[kc], dVr[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < NBK; ++nb) {
          const bf16x8 qa = join(lds_load_tr(qadr.tr_read(kc, 0, nb, buf * QTB)), lds_load_tr(qadr.tr_read(kc, 1, nb, buf * QTB)));
          dKr[nb] = mfma32<F16>(qa, da[kc], dKr[nb]);
        }
      }
    }
  }

  // dK = scale * acc and dV = acc of this lane's key, 16-byte row pieces
  // (keys past the used ones hold zeros: no row sees them)
  const bool key_ok = j_key < sb.s2a;
  bf16* __restrict__ dK = static_cast<bf16*>(a.dk) + sb.kbase + (int64_t)n2 * a.k_sn + (int64_t)j_key * a.k_ss;
  bf16* __restrict__ dV = static_cast<bf16*>(a.dv) + sb.vbase + (int64_t)n2 * a.v_sn + (int64_t)j_key * a.v_ss;
  if constexpr (QG == 1) {
    store_rows<F16>(dK, dKr, a.scale, hi, key_ok);
    store_rows<F16>(dV, dVr, 1.f, hi, key_ok);
  } else {
    lds_barrier();  // the exchange areas are filled
    if (qg == 0) {
      xadd(reinterpret_cast<const float*>(&Qs[0][0][0]), kw, lane, dKr[0]);
      xadd(reinterpret_cast<const float*>(&Ys[0][0][0]), kw, lane, dKr[1]);
      store_rows<F16>(dK, dKr, a.scale, hi, key_ok);
    } else {
      xadd(reinterpret_cast<const float*>(Vs), kw, lane, dVr[0]);
      xadd(Xs, kw, lane, dVr[1]);
      store_rows<F16>(dV, dVr, 1.f, hi, key_ok);
    }
  }
}

template <bool F16>
int launch_fused_t(const KernelArgs& a, dim3 grid, hipStream_t s) {
  if (a.D == 64 && a.Dv == 64) return launch(fused_kernel<64, 64, 2, F16>, grid, dim3(512), s, a);
  if (a.D == 128 && a.Dv == 64) return launch(fused_kernel<128, 64, 1, F16>, grid, dim3(256), s, a);
  if (a.D == 128 && a.Dv == 128) return launch(fused_kernel<128, 128, 1, F16>, grid, dim3(256), s, a);
  return (int)hipErrorInvalidValue;
}

}  // namespace

bool fused_instantiated(int D, int Dv) { return (D == 64 && Dv == 64) || (D == 128 && (Dv == 64 || Dv == 128)); }

int launch_fused(const KernelArgs& a, void* stream) {
  const int64_t blocks = (int64_t)a.B * a.N2;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return a.f16 ? launch_fused_t<true>(a, dim3((unsigned)blocks), s) : launch_fused_t<false>(a, dim3((unsigned)blocks), s);
}

}  // namespace fabwd
