// gfx950 (MI355X) kernels of Floyd attention, forward and backward.
//
// Page "CANN Floyd注意力梯度算子", section 功能说明: the scores add two
// products, S[n,m,k] = scale * (Q[n,m].K1[n,k] + Q[n,m].K2[k,m]), the first a
// batch matmul over n and the second one over m; P = softmax_k(S) and
// Y = P V1 + P V2 with the same two batch axes.  The backward's five
// gradients reduce over three different axes (dQ over k, dK1 / dV1 over m,
// dK2 / dV2 over n).
//
// Design.  A score element needs one product from each batch orientation, and
// an MFMA tile of one orientation holds (m, k) for a fixed n while the other
// holds (n, k) for a fixed m.  The two meet through the fp32 score workspace
// in HBM, [head][n][m][k]:
//   1. score_kernel, by n: Q[n] K1[n]^T and dY[n] V1[n]^T into ws_s / ws_p;
//   2. score_grad_kernel, by m: Q[:,m] K2[:,m]^T completes S, and pointwise
//      P = exp(S - max)/sum from the forward's statistics is written as
//      16-bit; then dY[:,m] V2[:,m]^T completes dP and dS = P (dP - sfmg)
//      (P in fp32) is written as 16-bit;
//   3. gemm_kernel for dV1 = P^T dY and dK1 = scale dS^T Q (batched over n),
//      dV2, dK2 (batched over m), dQ = scale (dS K1 + dS K2) (two launches,
//      the second adding the first's fp32 result).
// No row reduction over k is needed in the backward (the statistics come
// from the forward), so P and dS are formed where the second score product
// ends.  Every product is a v_mfma_f32_32x32x16 tile fed from LDS.  In the
// general kernels each operand tile is copied global -> registers -> LDS one
// k-step ahead (double-buffered LDS, one barrier per step): an operand whose
// contraction index t is contiguous in memory is stored [x][t] and read 16
// bytes per lane; one whose row index x is contiguous is stored [t][x] and
// read with ds_read_b64_tr_b16, which hands each lane a column of four rows.
// The fixed-m score kernel (D = 64, 128) and the gradient GEMMs whose
// operands are both row-contiguous copy their tiles straight to LDS instead
// (global_load_lds into the attention kernels' swizzled tiles).

#include <hip/hip_runtime.h>

#include "fa_bwd_tiles.h"
#include "fa_floyd_internal.h"

namespace ffloyd {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr int NT = 256;  // threads per workgroup (4 wavefronts)
constexpr int BM = 128;  // tile rows (i) of every kernel but score_grad_kernel
constexpr int BK = 32;   // contraction step

template <bool F16>
__device__ __forceinline__ floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ bf16 to_elem(float x) {
  if constexpr (F16) return __builtin_bit_cast(bf16, (_Float16)x);
  else return (bf16)x;
}
template <bool F16>
__device__ __forceinline__ float from_elem(bf16 x) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, x);
  else return (float)x;
}

// Operand view of one block: element (x, t) at p[x*sx + t*st]; X rows and T
// contraction entries exist (both multiples of 8 along the contiguous axis).
struct Op {
  const bf16* p;
  int64_t sx, st;
  int X, T;
};

// One operand's tile of BX rows x BK contraction entries.
//  TC (t contiguous): LDS [x][t], pitch BK + 8 (80 bytes): the 16-byte reads
//     of 8 consecutive rows fall in distinct banks.
//  XC (x contiguous): LDS [t][x], pitch 16 banks (mod 64) apart per row
//     (BX + 32 elements; 48 for BX = 32), so the four rows of one
//     transposing read of a 16-lane group fall in distinct banks.
template <bool TC, int BX>
struct Tile {
  static constexpr int PITCH = TC ? BK + 8 : (BX == 32 ? 48 : BX + 32);
  static constexpr int ELEMS = TC ? BX * PITCH : BK * PITCH;
  static constexpr int CHUNKS = BX * BK / 8;
  static constexpr int PER = (CHUNKS + NT - 1) / NT;
  uint4 r[PER];

  __device__ __forceinline__ void chunk_pos(int c, int& x, int& t) const {
    if constexpr (TC) {
      x = c / (BK / 8);
      t = (c % (BK / 8)) * 8;
    } else {
      t = c / (BX / 8);
      x = (c % (BX / 8)) * 8;
    }
  }
  __device__ __forceinline__ void load(const Op& o, int x0, int t0, int tid) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      int x, t;
      chunk_pos(c, x, t);
      const bool ok = c < CHUNKS && x0 + x < o.X && t0 + t < o.T;
      r[u] = ok ? *reinterpret_cast<const uint4*>(o.p + (int64_t)(x0 + x) * o.sx + (int64_t)(t0 + t) * o.st)
                : uint4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(bf16* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * NT;
      if (c < CHUNKS) {
        int x, t;
        chunk_pos(c, x, t);
        *reinterpret_cast<uint4*>(lds + (TC ? x * PITCH + t : t * PITCH + x)) = r[u];
      }
    }
  }
  // MFMA operand of 32-row block bx, contraction slice kk (16 entries): lane l
  // gets row x = 32*bx + l%32 and t = 16*kk + 8*(l/32) + 0..7.
  __device__ __forceinline__ bf16x8 frag(const bf16* lds, int bx, int kk, int lane) const {
    if constexpr (TC) {
      return *reinterpret_cast<const bf16x8*>(lds + (bx * 32 + (lane & 31)) * PITCH + kk * 16 + 8 * (lane >> 5));
    } else {
      // 16-lane group g = lane/16 covers rows x0 .. x0+15, x0 = 32*bx + 16*(g%2);
      // lane i of the group points at contraction row t + i/4, column x0 + 4*(i%4)
      // and receives column x0 + i of four contraction rows.
      const int row = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
      const int col = bx * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const bf16* p = lds + row * PITCH + col;
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(p));
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(p + 4 * PITCH));
      const shortx8 s = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, s);
    }
  }
};

// Wavefront arrangement of a TBM x BN tile over 4 wavefronts.
template <int BN, int TBM = BM>
struct Cfg {
  // 128 x 128: 2 x 2 wavefronts of 64 x 64; 128 x 64 and 128 x 32: 4 x 1;
  // 64 x 128: 2 x 2 of 32 x 64; 32 x 128: 1 x 4 of 32 x 32
  static constexpr int WAVES_M = TBM / 32 >= 4 ? (BN == 128 ? 2 : 4) : TBM / 32;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WN = BN / WAVES_N;  // columns per wavefront
  static constexpr int WM = TBM / WAVES_M;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && WAVES_M * WAVES_N == 4, "wavefront arrangement");
};

constexpr int LDS_ELEMS = 2 * 2 * 5120;  // two buffers of the largest A and B tiles

// acc += A(i0.., :) B(:, j0..) over the whole contraction.  Every thread of
// the workgroup calls it; it ends with a barrier, so the LDS may be reused.
template <bool ATC, bool BTC, int BN, bool F16, int TBM = BM>
__device__ __forceinline__ void gemm_tile(const Op& A, const Op& B, int i0, int j0,
                                          floatx16 (&acc)[Cfg<BN, TBM>::TM][Cfg<BN, TBM>::TN], bf16* lds) {
  using C = Cfg<BN, TBM>;
  using TA = Tile<ATC, TBM>;
  using TB = Tile<BTC, BN>;
  static_assert(TA::ELEMS <= 5120 && TB::ELEMS <= 5120, "LDS tile size");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  bf16* la[2] = {lds, lds + 5120};
  bf16* lb[2] = {lds + 2 * 5120, lds + 3 * 5120};
  TA ta;
  TB tb;
  const int nk = (A.T + BK - 1) / BK;
  ta.load(A, i0, 0, tid);
  tb.load(B, j0, 0, tid);
  ta.store(la[0], tid);
  tb.store(lb[0], tid);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      ta.load(A, i0, (it + 1) * BK, tid);
      tb.load(B, j0, (it + 1) * BK, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) af[tm] = ta.frag(la[cur], wm * C::TM + tm, kk, lane);
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) bfr[tn] = tb.frag(lb[cur], wn * C::TN + tn, kk, lane);
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = mfma<F16>(af[tm], bfr[tn], acc[tm][tn]);
    }
    if (more) {
      ta.store(la[cur ^ 1], tid);
      tb.store(lb[cur ^ 1], tid);
    }
    __syncthreads();
  }
}

// Workgroup -> (inner batch, tile) with the tiles of one batch entry on one
// XCD: workgroup w runs on XCD w % 8, so logical index (w % 8) * (n / 8) + w / 8
// gives every XCD a contiguous range of logical tiles.
__device__ __forceinline__ int logical_block() {
  const int w = blockIdx.x, n = gridDim.x;
  return (n & 7) == 0 ? (w & 7) * (n >> 3) + (w >> 3) : w;
}

template <bool ATC, bool BTC, int BN, bool F16, int TBM>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs g) {
  using C = Cfg<BN, TBM>;
  __shared__ __attribute__((aligned(16))) bf16 lds[LDS_ELEMS];
  const int tiles_j = (g.J + BN - 1) / BN, tiles_i = (g.I + TBM - 1) / TBM;
  const int L = logical_block();
  const int z = L / (tiles_i * tiles_j), tile = L % (tiles_i * tiles_j);
  const int i0 = (tile / tiles_j) * TBM, j0 = (tile % tiles_j) * BN;
  const int h = blockIdx.y;
  Op A{static_cast<const bf16*>(g.a) + h * g.a_sh + z * g.a_sz, g.a_si, g.a_st, g.I, g.T};
  Op B{static_cast<const bf16*>(g.b) + h * g.b_sh + z * g.b_sz, g.b_sj, g.b_st, g.J, g.T};
  floatx16 acc[C::TM][C::TN];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = floatx16{};
  gemm_tile<ATC, BTC, BN, F16, TBM>(A, B, i0, j0, acc, lds);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int64_t cb = h * g.c_sh + z * g.c_sz;
  // A tile inside the output (the usual case) issues a block's 16 addend
  // loads before any store; edge tiles check every element.
  const bool full = i0 + TBM <= g.I && j0 + BN <= g.J;
  const float* __restrict__ add = g.addend;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int j = j0 + (wn * C::TN + tn) * 32 + (lane & 31);
      const int ib = i0 + (wm * C::TM + tm) * 32 + 4 * (lane >> 5);
      if (full) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = add ? add[cb + (ib + 8 * (r >> 2) + (r & 3)) * g.c_si + j] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t off = cb + (ib + 8 * (r >> 2) + (r & 3)) * g.c_si + j;
          const float x = g.alpha * acc[tm][tn][r] + v[r];
          if (g.out_f32) static_cast<float*>(g.c)[off] = x;
          else static_cast<bf16*>(g.c)[off] = to_elem<F16>(x);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = ib + 8 * (r >> 2) + (r & 3);
          if (i < g.I && j < g.J) {
            const int64_t off = cb + i * g.c_si + j;
            float x = g.alpha * acc[tm][tn][r];
            if (add) x += add[off];
            if (g.out_f32) static_cast<float*>(g.c)[off] = x;
            else static_cast<bf16*>(g.c)[off] = to_elem<F16>(x);
          }
        }
      }
    }
}

// The same product for B operands whose row index x is contiguous in memory
// (B[x][t] at x + t*b_st) and A operands of either kind (A[x][t] at x +
// t*a_st: dV1, dK1, dV2, dK2; or at x*a_si + t, ATC: the dQ terms), on whole
// 128 x 128 tiles with a contraction that is a multiple of 64: each 64-deep
// step of both operands goes straight to LDS as a swizzled tile (the
// attention kernels' copy), double-buffered, the next step's copy issued as
// soon as every wavefront has finished the previous one.  B, and an A of the
// first kind, are transposing reads of [t][x] tiles; an ATC A is read from its
// [x][t] tile in the same order of t inside each 16-deep chunk (two 8-byte
// reads: t = 4h..4h+3 and 8+4h..8+4h+3 for lane half h).
constexpr int GKB = 64;  // contraction per step of gemm_dma_kernel

template <bool ATC, bool F16>
__global__ __launch_bounds__(NT, 2) void gemm_dma_kernel(GemmArgs g) {
  using C = Cfg<128, 128>;
  static_assert(C::TM == 2 && C::TN == 2 && C::WAVES_N == 2, "2 x 2 wavefronts of 64 x 64");
  constexpr int TB = GKB * 128 * 2;  // bytes of one operand tile
  __shared__ __attribute__((aligned(1024))) bf16 As[2][GKB * 128];
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][GKB * 128];
  const int tiles_j = g.J / 128, tiles_i = g.I / 128;
  const int L = logical_block();
  const int z = L / (tiles_i * tiles_j), tile = L % (tiles_i * tiles_j);
  const int i0 = (tile / tiles_j) * 128, j0 = (tile % tiles_j) * 128;
  const int h = blockIdx.y;
  const bf16* __restrict__ Ag = static_cast<const bf16*>(g.a) + h * g.a_sh + z * g.a_sz + i0 * (ATC ? g.a_si : 1);
  const bf16* __restrict__ Bg = static_cast<const bf16*>(g.b) + h * g.b_sh + z * g.b_sz + j0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // A: rows t, 128 columns x (or, ATC, rows x, 64 columns t); B: rows t
  fabwd::TileCopy<ATC ? GKB : 128, ATC ? 128 : GKB, 4> acp;
  fabwd::TileCopy<128, GKB, 4> bcp;
  acp.init(wave, lane, (int)((ATC ? g.a_si : g.a_st) * 2));
  bcp.init(wave, lane, (int)(g.b_st * 2));
  const uint32_t a_lds = fabwd::lds_addr(As), b_lds = fabwd::lds_addr(Bs);
  fabwd::SwzTile<ATC ? GKB : 128, ATC ? 128 : GKB> aadr;
  fabwd::SwzTile<128, GKB> badr;
  aadr.init(a_lds, lane);
  badr.init(b_lds, lane);
  auto fetch = [&](int st, int buf) {
    acp.issue(a_lds + buf * TB, Ag + (int64_t)st * GKB * (ATC ? 1 : g.a_st), ATC ? 128 : GKB, wave, lane);
    bcp.issue(b_lds + buf * TB, Bg + (int64_t)st * GKB * g.b_st, GKB, wave, lane);
  };
  floatx16 acc[C::TM][C::TN];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = floatx16{};
  const int nk = g.T / GKB;
  fetch(0, 0);
  auto step = [&](int st, int buf) {
    fabwd::wait_vmem();     // this wavefront's copies of step st landed
    fabwd::lds_barrier();   // ... and everyone's; buffer buf ^ 1 is no longer read
    if (st + 1 < nk) fetch(st + 1, buf ^ 1);
#pragma unroll
    for (int kc = 0; kc < GKB / 16; ++kc) {
      bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        if constexpr (ATC) {
          // logical 16-byte chunk 2kc (t = 16kc..16kc+7) of row 64wm + 32tm + l32
          // and chunk 2kc + 1, each read at the lane half's 8-byte half
          const int hi = lane >> 5;
          const uint32_t c0 = aadr.row_read_at(kc, 64 * wm + 32 * tm, buf * TB) ^ (16 * hi);
          const shortx4 lo4 = *(LDS_AS const shortx4*)(uintptr_t)(c0 + 8 * hi);
          const shortx4 hi4 = *(LDS_AS const shortx4*)(uintptr_t)((c0 ^ 16) + 8 * hi);
          af[tm] = fabwd::join(lo4, hi4);
        } else {
          af[tm] = fabwd::join(fabwd::lds_load_tr(aadr.tr_read_c(kc, 0, 2 * wm + tm, buf * TB)),
                               fabwd::lds_load_tr(aadr.tr_read_c(kc, 1, 2 * wm + tm, buf * TB)));
        }
      }
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
        bfr[tn] = fabwd::join(fabwd::lds_load_tr(badr.tr_read_c(kc, 0, 2 * wn + tn, buf * TB)),
                              fabwd::lds_load_tr(badr.tr_read_c(kc, 1, 2 * wn + tn, buf * TB)));
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = fabwd::mfma32<F16>(af[tm], bfr[tn], acc[tm][tn]);
    }
  };
  int st = 0;  // two steps per iteration, so that the buffer offsets are constants
  for (; st + 1 < nk; st += 2) {
    step(st, 0);
    step(st + 1, 1);
  }
  if (st < nk) step(st, 0);

  const int64_t cb = h * g.c_sh + z * g.c_sz;
  const float* __restrict__ add = g.addend;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int j = j0 + (wn * C::TN + tn) * 32 + (lane & 31);
      const int ib = i0 + (wm * C::TM + tm) * 32 + 4 * (lane >> 5);
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = add ? add[cb + (ib + 8 * (r >> 2) + (r & 3)) * g.c_si + j] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t off = cb + (ib + 8 * (r >> 2) + (r & 3)) * g.c_si + j;
        const float x = g.alpha * acc[tm][tn][r] + v[r];
        if (g.out_f32) static_cast<float*>(g.c)[off] = x;
        else static_cast<bf16*>(g.c)[off] = to_elem<F16>(x);
      }
    }
}

// Score products (see ScoreArgs), epilogues 0, 2 and 3.  Rows i of the tile
// are m (by n) or n (by m), columns j are keys k; the inner batch index z is
// n (by n) or m (by m).
constexpr int SBM = 128;  // tile rows of score_kernel (64 re-reads K1 / V1 tiles twice as often: slower)

template <bool F16, int EPI>
__global__ __launch_bounds__(NT) void score_kernel(ScoreArgs s) {
  using C = Cfg<128, SBM>;
  __shared__ __attribute__((aligned(16))) bf16 lds[LDS_ELEMS];
  const bool by_m = EPI == 1 || EPI == 3;
  const int I = by_m ? s.N : s.M, J = s.K;
  const int tiles_j = (J + 127) / 128, tiles_i = (I + SBM - 1) / SBM;
  const int L = logical_block();
  const int z = L / (tiles_i * tiles_j), tile = L % (tiles_i * tiles_j);
  const int i0 = (tile / tiles_j) * SBM, j0 = (tile % tiles_j) * 128;
  const int h = blockIdx.y;
  const int64_t MD = (int64_t)s.M * s.D, NMD = (int64_t)s.N * MD;
  const int64_t KD = (int64_t)s.K * s.D;
  // Q / dY rows: by n, row m of batch n at (n*M + m)*D; by m, row n of batch m at n*M*D + m*D
  const int64_t q_off = h * NMD + (by_m ? (int64_t)z * s.D : (int64_t)z * MD);
  const int64_t q_sx = by_m ? MD : s.D;
  // K1/V1 [N][K][D]: by n, row k of batch n at n*K*D + k*D
  // K2/V2 [K][M][D]: by m, row k of batch m at k*M*D + m*D
  const int64_t x_off = by_m ? h * (int64_t)s.K * MD + (int64_t)z * s.D : h * (int64_t)s.N * KD + (int64_t)z * KD;
  const int64_t x_sx = by_m ? MD : s.D;

  floatx16 acs[C::TM][C::TN], acp[C::TM][C::TN];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acs[tm][tn] = acp[tm][tn] = floatx16{};
  {
    Op A{static_cast<const bf16*>(s.q) + q_off, q_sx, 1, I, s.D};
    Op B{static_cast<const bf16*>(s.x1) + x_off, x_sx, 1, J, s.D};
    gemm_tile<true, true, 128, F16, SBM>(A, B, i0, j0, acs, lds);
  }
  if constexpr (EPI == 0) {
    Op A{static_cast<const bf16*>(s.dy) + q_off, q_sx, 1, I, s.D};
    Op B{static_cast<const bf16*>(s.x2) + x_off, x_sx, 1, J, s.D};
    gemm_tile<true, true, 128, F16, SBM>(A, B, i0, j0, acp, lds);
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int64_t MK = (int64_t)s.M * s.K, NMK = (int64_t)s.N * MK;
  // element (i, j) of the tile in the [head][n][m][k] workspace
  const int64_t wbase = h * NMK + (by_m ? (int64_t)z * s.K : (int64_t)z * MK);
  const int64_t w_si = by_m ? MK : s.K;
  const float sl2 = s.scale * kLog2e;
  const int bb = (s.head0 + h) / s.H;  // batch index of the mask
  float* __restrict__ ws_s = s.ws_s;
  float* __restrict__ ws_p = s.ws_p;
  const bool full = i0 + SBM <= I && j0 + 128 <= J;
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const int j = j0 + (wn * C::TN + tn) * 32 + (lane & 31);
      const int ib = i0 + (wm * C::TM + tm) * 32 + 4 * (lane >> 5);
      auto row_of = [&](int r) { return ib + 8 * (r >> 2) + (r & 3); };
      auto off_of = [&](int r) { return wbase + row_of(r) * w_si + j; };
      if constexpr (EPI == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (full || (row_of(r) < I && j < J)) {
            ws_s[off_of(r)] = acs[tm][tn][r];
            ws_p[off_of(r)] = acp[tm][tn][r];
          }
      } else if constexpr (EPI == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (full || (row_of(r) < I && j < J)) ws_s[off_of(r)] = acs[tm][tn][r];
      } else if constexpr (EPI == 3) {
        if (full) {
          float old[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) old[r] = ws_s[off_of(r)];
#pragma unroll
          for (int r = 0; r < 16; ++r) ws_s[off_of(r)] = old[r] + acs[tm][tn][r];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (row_of(r) < I && j < J) ws_s[off_of(r)] += acs[tm][tn][r];
        }
      }
    }
}

// Epilogue 1 (backward, by m): for each m, the (n, k) tile of Q K2^T completes
// the scores with the by-n partial in ws_s, P = exp(scale*S - lse) is stored
// as 16-bit and kept in fp32 registers; then the tile of dY V2^T completes dP
// with ws_p and dS = P (dP - sfmg) is stored.  Forming P before the second product
// frees the score accumulators for it.  Each epilogue's loads are issued
// before the product that precedes it (edge tiles check each element).
constexpr int GBM = 64;  // tile rows (n) of score_grad_kernel

template <bool F16>
__global__ __launch_bounds__(NT) void score_grad_kernel(ScoreArgs s) {
  using C = Cfg<128, GBM>;
  __shared__ __attribute__((aligned(16))) bf16 lds[LDS_ELEMS];
  const int I = s.N, J = s.K;
  const int tiles_j = (J + 127) / 128, tiles_i = (I + GBM - 1) / GBM;
  // consecutive workgroups of an XCD take consecutive m of one (n, k) tile:
  // their rows of Q, dY and of the workspace lie side by side in memory
  const int L = logical_block();
  const int z = L % s.M, tile = L / s.M;
  const int i0 = (tile / tiles_j) * GBM, j0 = (tile % tiles_j) * 128;
  const int h = blockIdx.y;
  const int64_t MD = (int64_t)s.M * s.D, NMD = (int64_t)s.N * MD;
  // Q / dY row n of batch m at n*M*D + m*D; K2 / V2 row k of batch m at k*M*D + m*D
  const int64_t q_off = h * NMD + (int64_t)z * s.D;
  const int64_t x_off = h * (int64_t)s.K * MD + (int64_t)z * s.D;
  const int64_t MK = (int64_t)s.M * s.K, NMK = (int64_t)s.N * MK;
  const int64_t wbase = h * NMK + (int64_t)z * s.K;   // element (n, m = z, k) at wbase + n*MK + k
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const float sl2 = s.scale * kLog2e;
  const int bb = (s.head0 + h) / s.H;
  const bool full = i0 + GBM <= I && j0 + 128 <= J;
  const float* __restrict__ ws_s = s.ws_s;
  const float* __restrict__ ws_p = s.ws_p;
  bf16* __restrict__ pe = static_cast<bf16*>(s.ws_pe);
  bf16* __restrict__ dse = static_cast<bf16*>(s.ws_dse);

  floatx16 acc[C::TM][C::TN];
  float pf[C::TM][C::TN][16];  // P in fp32 for dS (the stored P is 16-bit)
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) acc[tm][tn] = floatx16{};
  auto row_of = [&](int tm, int r) { return i0 + (wm * C::TM + tm) * 32 + 4 * (lane >> 5) + 8 * (r >> 2) + (r & 3); };
  auto col_of = [&](int tn) { return j0 + (wn * C::TN + tn) * 32 + (lane & 31); };
  auto inside = [&](int tm, int tn, int r) { return full || (row_of(tm, r) < I && col_of(tn) < J); };

  // the by-n partial scores, the rows' log-sum-exp and the mask are loaded
  // before the first product, so that their latency overlaps it
  float sv[C::TM][C::TN][16], l2[C::TM][16];
  bool live[C::TM][C::TN][16];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row_of(tm, r);
      l2[tm][r] = (full || i < I) ? s.lse2[((int64_t)h * s.N + i) * s.M + z] : 0.f;
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = row_of(tm, r), j = col_of(tn);
        const bool in = inside(tm, tn, r);
        sv[tm][tn][r] = in ? ws_s[wbase + i * MK + j] : 0.f;
        live[tm][tn][r] = in && (s.mask == nullptr || s.mask[((int64_t)bb * s.N + i) * s.K + j] == 0);
      }
  }
  {
    Op A{static_cast<const bf16*>(s.q) + q_off, MD, 1, I, s.D};
    Op B{static_cast<const bf16*>(s.x1) + x_off, MD, 1, J, s.D};
    gemm_tile<true, true, 128, F16, GBM>(A, B, i0, j0, acc, lds);
  }
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p =
            live[tm][tn][r] ? __builtin_amdgcn_exp2f((acc[tm][tn][r] + sv[tm][tn][r]) * sl2 - l2[tm][r]) : 0.f;
        pf[tm][tn][r] = p;
        if (inside(tm, tn, r)) pe[wbase + row_of(tm, r) * MK + col_of(tn)] = to_elem<F16>(p);
      }
      acc[tm][tn] = floatx16{};
    }
  // the by-n partial dP and the rows' sfmg, loaded before the second product
  float pv[C::TM][C::TN][16], sf[C::TM][16];
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row_of(tm, r);
      sf[tm][r] = (full || i < I) ? s.sfmg[((int64_t)h * s.N + i) * s.M + z] : 0.f;
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pv[tm][tn][r] = inside(tm, tn, r) ? ws_p[wbase + row_of(tm, r) * MK + col_of(tn)] : 0.f;
  }
  {
    Op A{static_cast<const bf16*>(s.dy) + q_off, MD, 1, I, s.D};
    Op B{static_cast<const bf16*>(s.x2) + x_off, MD, 1, J, s.D};
    gemm_tile<true, true, 128, F16, GBM>(A, B, i0, j0, acc, lds);
  }
#pragma unroll
  for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (inside(tm, tn, r))
          dse[wbase + row_of(tm, r) * MK + col_of(tn)] =
              to_elem<F16>(pf[tm][tn][r] * (acc[tm][tn][r] + pv[tm][tn][r] - sf[tm][r]));
      }
}

// The same stage with its product operands copied straight to LDS, each
// tile whole (the contraction is D <= 128 deep), as in the attention
// kernels' swizzled tiles: Q, K2 and dY are in flight together, V2 is
// fetched while the first epilogue runs.  The plain form above fetches each
// operand one 32-deep step ahead through registers, a memory round trip per
// step.  D = 64 or 128; the tile's row offsets must fit 32 bits.
template <bool F16, int HD>
__global__ __launch_bounds__(NT) void score_grad_dma_kernel(ScoreArgs s) {
  using C = Cfg<128, GBM>;
  static_assert(C::TM == 1 && C::TN == 2 && C::WAVES_N == 2, "2 x 2 wavefronts of 32 x 64");
  constexpr int ATB = GBM * HD * 2;  // bytes of an n-row tile (Q or dY)
  __shared__ __attribute__((aligned(1024))) bf16 As[2][GBM * HD];  // Q, dY
  __shared__ __attribute__((aligned(1024))) bf16 Bs[128 * HD];     // K2, then V2
  const int I = s.N, J = s.K;
  const int tiles_j = (J + 127) / 128, tiles = ((I + GBM - 1) / GBM) * tiles_j;
  // consecutive workgroups of an XCD take the (n, k) tiles of one m: each Q /
  // dY tile is read by the tiles_j of them and each K2 / V2 tile by the n
  // tiles while it is still in the XCD's L2
  const int L = logical_block();
  const int z = L / tiles, tile = L % tiles;
  const int i0 = (tile / tiles_j) * GBM, j0 = (tile % tiles_j) * 128;
  const int h = blockIdx.y;
  const int64_t MD = (int64_t)s.M * s.D, NMD = (int64_t)s.N * MD;
  const int64_t q_off = h * NMD + (int64_t)z * s.D + (int64_t)i0 * MD;               // row n = i0 of batch m = z
  const int64_t x_off = h * (int64_t)s.K * MD + (int64_t)z * s.D + (int64_t)j0 * MD;  // row k = j0 of batch m = z
  const int64_t MK = (int64_t)s.M * s.K, NMK = (int64_t)s.N * MK;
  const int64_t wbase = h * NMK + (int64_t)z * s.K;  // element (n, m = z, k) at wbase + n*MK + k
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const float sl2 = s.scale * kLog2e;
  const int bb = (s.head0 + h) / s.H;
  const bool full = i0 + GBM <= I && j0 + 128 <= J;
  const float* __restrict__ ws_s = s.ws_s;
  const float* __restrict__ ws_p = s.ws_p;
  bf16* __restrict__ pe = static_cast<bf16*>(s.ws_pe);
  bf16* __restrict__ dse = static_cast<bf16*>(s.ws_dse);
  auto row_of = [&](int r) { return i0 + wm * 32 + 4 * (lane >> 5) + 8 * (r >> 2) + (r & 3); };
  auto col_of = [&](int tn) { return j0 + (wn * C::TN + tn) * 32 + (lane & 31); };
  auto inside = [&](int tn, int r) { return full || (row_of(r) < I && col_of(tn) < J); };

  // the first epilogue's by-n partial scores, log-sum-exp and mask, loaded
  // before the operand copies (they complete first)
  float sv[C::TN][16], l2[16];
  bool live[C::TN][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = row_of(r);
    l2[r] = (full || i < I) ? s.lse2[((int64_t)h * s.N + i) * s.M + z] : 0.f;
  }
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row_of(r), j = col_of(tn);
      const bool in = inside(tn, r);
      sv[tn][r] = in ? ws_s[wbase + i * MK + j] : 0.f;
      live[tn][r] = in && (s.mask == nullptr || s.mask[((int64_t)bb * s.N + i) * s.K + j] == 0);
    }

  // operand tiles, rows past the end repeating the last one (masked above)
  fabwd::TileCopy<HD, GBM, 4> acp;
  fabwd::TileCopy<HD, 128, 4> bcp;
  acp.init(wave, lane, (int)(MD * 2));
  bcp.init(wave, lane, (int)(MD * 2));
  const uint32_t a_lds = fabwd::lds_addr(As), b_lds = fabwd::lds_addr(Bs);
  acp.issue(a_lds, static_cast<const bf16*>(s.q) + q_off, I - i0, wave, lane);
  bcp.issue(b_lds, static_cast<const bf16*>(s.x1) + x_off, J - j0, wave, lane);
  acp.issue(a_lds + ATB, static_cast<const bf16*>(s.dy) + q_off, I - i0, wave, lane);
  fabwd::SwzTile<HD, GBM> aadr;
  fabwd::SwzTile<HD, 128> badr;
  aadr.init(a_lds, lane);
  badr.init(b_lds, lane);
  // acc += A (rows 32*wm..) B^T (rows 64*wn + 32*tn..), both 16-byte row reads
  auto product = [&](floatx16 (&acc)[C::TN], uint32_t a_off) {
#pragma unroll
    for (int kk = 0; kk < HD / 16; ++kk) {
      const bf16x8 a = fabwd::lds_load16(aadr.row_read_at(kk, 32 * wm, a_off));
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
        acc[tn] = fabwd::mfma32<F16>(a, fabwd::lds_load16(badr.row_read_at(kk, 64 * wn + 32 * tn)), acc[tn]);
    }
  };
  fabwd::wait_vmem();
  fabwd::lds_barrier();
  floatx16 acc[C::TN] = {floatx16{}, floatx16{}};
  product(acc, 0);
  fabwd::lds_barrier();  // every wavefront's reads of K2 are done
  bcp.issue(b_lds, static_cast<const bf16*>(s.x2) + x_off, J - j0, wave, lane);
  // the second epilogue's by-n partial dP and the rows' sfmg
  float pv[C::TN][16], sf[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = row_of(r);
    sf[r] = (full || i < I) ? s.sfmg[((int64_t)h * s.N + i) * s.M + z] : 0.f;
  }
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[tn][r] = inside(tn, r) ? ws_p[wbase + row_of(r) * MK + col_of(tn)] : 0.f;
  // P = exp(scale*S - lse), stored 16-bit, kept in fp32 for dS
  float pf[C::TN][16];
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = live[tn][r] ? __builtin_amdgcn_exp2f((acc[tn][r] + sv[tn][r]) * sl2 - l2[r]) : 0.f;
      pf[tn][r] = p;
      if (inside(tn, r)) pe[wbase + row_of(r) * MK + col_of(tn)] = to_elem<F16>(p);
    }
    acc[tn] = floatx16{};
  }
  fabwd::wait_vmem();
  fabwd::lds_barrier();
  product(acc, ATB);
#pragma unroll
  for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (inside(tn, r))
        dse[wbase + row_of(r) * MK + col_of(tn)] = to_elem<F16>(pf[tn][r] * (acc[tn][r] + pv[tn][r] - sf[r]));
}

// 16 lanes per row: sfmg = sum_d dY*Y in fp32, lse2 from the statistics.
// V = D / 16 contiguous elements of a row per lane, one vector load each.
template <bool F16, int V>
__device__ __forceinline__ float row_part(const bf16* g, const bf16* y) {
  typedef __bf16 vec __attribute__((ext_vector_type(V)));
  const vec a = *reinterpret_cast<const vec*>(g), b = *reinterpret_cast<const vec*>(y);
  float acc = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) acc += from_elem<F16>(a[v]) * from_elem<F16>(b[v]);
  return acc;
}

template <bool F16>
__global__ __launch_bounds__(NT) void rowstats_kernel(RowStatsArgs a) {
  const int64_t row = (int64_t)blockIdx.x * (NT / 16) + (threadIdx.x >> 4);
  const int e = threadIdx.x & 15;
  float acc = 0.f;
  if (row < a.rows) {
    const int V = a.D / 16;  // D is 32, 64 or 128
    const bf16* g = static_cast<const bf16*>(a.dy) + row * a.D + e * V;
    const bf16* y = static_cast<const bf16*>(a.y) + row * a.D + e * V;
    acc = V == 8 ? row_part<F16, 8>(g, y) : V == 4 ? row_part<F16, 4>(g, y) : row_part<F16, 2>(g, y);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (row < a.rows && e == 0) {
    a.sfmg[row] = acc;
    const float mx = a.smax[row * 8], sm = a.ssum[row * 8];
    const bool live = mx > -__builtin_inff() && sm > 0.f;
    a.lse2[row] = live ? (mx + __logf(sm)) * kLog2e : __builtin_inff();
  }
}

// One wavefront per row (head, n, m): max and sum over the live keys of the
// scaled scores, then P = exp(S - max) / sum.
template <bool F16>
__global__ __launch_bounds__(NT) void softmax_kernel(SoftmaxArgs a) {
  const int64_t rows = (int64_t)a.heads * a.N * a.M;
  const int64_t row = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int n = (int)((row / a.M) % a.N), h = (int)(row / ((int64_t)a.M * a.N));
  const float* srow = a.ws_s + row * a.K;
  const uint8_t* mrow = a.mask ? a.mask + ((int64_t)((a.head0 + h) / a.H) * a.N + n) * a.K : nullptr;
  const float sl2 = a.scale * kLog2e;
  float mx = -__builtin_inff();
  for (int k = lane; k < a.K; k += 64)
    if (!mrow || mrow[k] == 0) mx = fmaxf(mx, srow[k] * sl2);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const bool live = mx > -__builtin_inff();
  float sum = 0.f;
  if (live)
    for (int k = lane; k < a.K; k += 64)
      if (!mrow || mrow[k] == 0) sum += __builtin_amdgcn_exp2f(srow[k] * sl2 - mx);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const float inv = live ? 1.f / sum : 0.f;
  bf16* prow = static_cast<bf16*>(a.p) + row * a.K;
  for (int k = lane; k < a.K; k += 64) {
    const bool ok = live && (!mrow || mrow[k] == 0);
    prow[k] = to_elem<F16>(ok ? __builtin_amdgcn_exp2f(srow[k] * sl2 - mx) * inv : 0.f);
  }
  if (lane < 8) {
    // statistics in the natural-log domain: max of scale*S, sum of exp(scale*S - max)
    a.smax[row * 8 + lane] = live ? mx / kLog2e : -__builtin_inff();
    a.ssum[row * 8 + lane] = live ? sum : 0.f;
  }
}

template <bool ATC, bool BTC, bool F16>
int launch_gemm_bn(const GemmArgs& g, hipStream_t st) {
  constexpr int R = BM;
  const int ti = (g.I + R - 1) / R;
  if (g.J <= 32) {
    const int64_t nx = (int64_t)ti * ((g.J + 31) / 32) * g.nb;
    hipLaunchKernelGGL((gemm_kernel<ATC, BTC, 32, F16, R>), dim3((unsigned)nx, g.heads), dim3(NT), 0, st, g);
  } else if (g.J <= 64) {
    const int64_t nx = (int64_t)ti * ((g.J + 63) / 64) * g.nb;
    hipLaunchKernelGGL((gemm_kernel<ATC, BTC, 64, F16, R>), dim3((unsigned)nx, g.heads), dim3(NT), 0, st, g);
  } else {
    const int64_t nx = (int64_t)ti * ((g.J + 127) / 128) * g.nb;
    // both operands row-contiguous, whole tiles, 64-deep steps, and a step's
    // 64 rows addressed by 32-bit byte offsets: copies straight to LDS
    const bool dma = !BTC && (ATC ? g.a_st == 1 : g.a_si == 1) && g.b_sj == 1 && g.I % 128 == 0 &&
                     g.J % 128 == 0 && g.T % GKB == 0 &&
                     (int64_t)(ATC ? 128 * g.a_si : GKB * g.a_st) * 2 < (int64_t(1) << 31) &&
                     (int64_t)GKB * g.b_st * 2 < (int64_t(1) << 31);
    if (dma) hipLaunchKernelGGL((gemm_dma_kernel<ATC, F16>), dim3((unsigned)nx, g.heads), dim3(NT), 0, st, g);
    else hipLaunchKernelGGL((gemm_kernel<ATC, BTC, 128, F16, R>), dim3((unsigned)nx, g.heads), dim3(NT), 0, st, g);
  }
  return (int)hipGetLastError();
}

template <bool F16>
int launch_gemm_t(const GemmArgs& g, hipStream_t st) {
  if (g.a_tc && !g.b_tc) return launch_gemm_bn<true, false, F16>(g, st);
  if (!g.a_tc && !g.b_tc) return launch_gemm_bn<false, false, F16>(g, st);
  if (g.a_tc && g.b_tc) return launch_gemm_bn<true, true, F16>(g, st);
  return launch_gemm_bn<false, true, F16>(g, st);
}

template <bool F16>
int launch_scores_t(const ScoreArgs& s, hipStream_t st) {
  const bool by_m = s.epi == 1 || s.epi == 3;
  const int I = by_m ? s.N : s.M, rows = s.epi == 1 ? GBM : SBM;
  const int64_t nx = (int64_t)((I + rows - 1) / rows) * ((s.K + 127) / 128) * (by_m ? s.M : s.N);
  const dim3 grid((unsigned)nx, s.heads);
  switch (s.epi) {
    case 0: hipLaunchKernelGGL((score_kernel<F16, 0>), grid, dim3(NT), 0, st, s); break;
    case 1:
      // operand tiles straight to LDS when D allows it and a tile's row
      // offsets (128 rows of M*D elements) fit 32 bits
      if ((s.D == 64 || s.D == 128) && 128 * (int64_t)s.M * s.D * 2 < (int64_t(1) << 31)) {
        if (s.D == 128) hipLaunchKernelGGL((score_grad_dma_kernel<F16, 128>), grid, dim3(NT), 0, st, s);
        else hipLaunchKernelGGL((score_grad_dma_kernel<F16, 64>), grid, dim3(NT), 0, st, s);
      } else {
        hipLaunchKernelGGL((score_grad_kernel<F16>), grid, dim3(NT), 0, st, s);
      }
      break;
    case 2: hipLaunchKernelGGL((score_kernel<F16, 2>), grid, dim3(NT), 0, st, s); break;
    default: hipLaunchKernelGGL((score_kernel<F16, 3>), grid, dim3(NT), 0, st, s); break;
  }
  return (int)hipGetLastError();
}

}  // namespace

struct StageTimer {
  int marks;
  hipEvent_t* ev;
};

StageTimer* stage_timer_create(int marks) {
  StageTimer* t = new StageTimer{marks, new hipEvent_t[marks]};
  for (int i = 0; i < marks; ++i) {
    if (hipEventCreate(&t->ev[i]) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(t->ev[j]);
      delete[] t->ev;
      delete t;
      return nullptr;
    }
  }
  return t;
}

int stage_timer_mark(StageTimer* t, int i, void* stream) {
  return (int)hipEventRecord(t->ev[i], static_cast<hipStream_t>(stream));
}

int stage_timer_read(StageTimer* t, float* ms) {
  if (hipEventSynchronize(t->ev[t->marks - 1]) != hipSuccess) return 1;
  for (int i = 0; i + 1 < t->marks; ++i)
    if (hipEventElapsedTime(&ms[i], t->ev[i], t->ev[i + 1]) != hipSuccess) return 1;
  return 0;
}

void stage_timer_destroy(StageTimer* t) {
  if (!t) return;
  for (int i = 0; i < t->marks; ++i) (void)hipEventDestroy(t->ev[i]);
  delete[] t->ev;
  delete t;
}

int launch_gemm(const GemmArgs& g, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return g.f16 ? launch_gemm_t<true>(g, st) : launch_gemm_t<false>(g, st);
}

int launch_scores(const ScoreArgs& s, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  return s.f16 ? launch_scores_t<true>(s, st) : launch_scores_t<false>(s, st);
}

int launch_rowstats(const RowStatsArgs& r, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t blocks = (r.rows + NT / 16 - 1) / (NT / 16);
  if (r.f16) hipLaunchKernelGGL(rowstats_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, st, r);
  else hipLaunchKernelGGL(rowstats_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, st, r);
  return (int)hipGetLastError();
}

int launch_softmax(const SoftmaxArgs& s, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)s.heads * s.N * s.M;
  const int64_t blocks = (rows + NT / 64 - 1) / (NT / 64);
  if (s.f16) hipLaunchKernelGGL(softmax_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, st, s);
  else hipLaunchKernelGGL(softmax_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, st, s);
  return (int)hipGetLastError();
}

}  // namespace ffloyd
