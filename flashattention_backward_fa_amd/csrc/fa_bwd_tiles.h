// Device-side building blocks shared by the gfx950 backward kernels
// (fa_bwd_det_kernels.hip, fa_bwd_fused_kernels.hip): element types and the
// MFMA wrapper, the swizzled LDS tile layout and its per-lane addressing,
// asynchronous global -> LDS copies, sequence bounds, and the placement of
// the stored dS tiles.  Everything sits in an unnamed namespace: each
// translation unit gets its own copy.
#pragma once

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
typedef float floatx4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Elements are 16-bit: bf16, or IEEE fp16 when F16, held in the same storage
// type; only the MFMA and the conversions to and from fp32 differ.
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
// Transposing LDS read (see fa_bwd_kernels.hip): lane i of a 16-lane group,
// pointing at row r0 + i/4, column c0 + 4*(i%4) of a row-major bf16 tile,
// receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ shortx4 lds_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(p));
}
__device__ __forceinline__ bf16x8 join(shortx4 lo, shortx4 hi) {
  shortx8 s = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, s);
}

// LDS tile layout.  Tiles are stored without padding; the 16-byte chunk
// (8 bf16) holding element (r, c) is permuted within its row by an XOR with a
// function of r, chosen so that both access patterns of the kernels are free
// of bank conflicts on gfx950 (measured: 16-byte row reads ~200 B/clk/CU and
// transposing 8-byte reads ~130 B/clk/CU, against ~59 B/clk/CU for the
// transposing reads on a 272-byte padded pitch):
//  * 16 consecutive rows, same chunk (the A/B fragments of row-major reads);
//  * 4 consecutive rows x 64 bytes (one transposing read of 32 lanes).
// A 128-column block uses f(r) = 4*(r%4) + (r/4)%4 over its 16 chunks, a
// 64-column block (128-byte rows, two per bank cycle) uses
// g(r) = 4*((r/2)%2) + (r/4)%4 over its 8 chunks; 192 columns are a
// 128-column block followed by a 64-column block.
template <int COLS, int ROWS>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (COLS == 128) {
    return r * 128 + ((((c >> 3) ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 3) | (c & 7));
  } else if constexpr (COLS == 64) {
    return r * 64 + ((((c >> 3) ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))) << 3) | (c & 7));
  } else {
    static_assert(COLS == 192, "tile width");
    return c < 128 ? swz<128, ROWS>(r, c) : ROWS * 128 + swz<64, ROWS>(r, c - 128);
  }
}

// s1, s2: rows / keys that take part; s1a, s2a: rows / keys the sequence
// holds (they differ only when seqused_q / seqused_kv are given).
struct SeqBounds {
  int b;  // sequence index
  int s1, s2, s1a, s2a;
  int64_t qbase, kbase, vbase, obase, lbase;
};

__device__ __forceinline__ SeqBounds seq_bounds(const KernelArgs& a, int b) {
  SeqBounds r;
  r.b = b;
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

// LDS addressing.  LDS addresses are 32-bit byte offsets; reads go through
// them directly, so that per-lane parts are computed once and the rest (tile
// buffer, k-step) lands in the instructions' immediate offsets.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t) reinterpret_cast<uintptr_t>((LDS_AS const void*)p);
}
__device__ __forceinline__ bf16x8 lds_load16(uint32_t addr) { return *(LDS_AS const bf16x8*)(uintptr_t)addr; }
__device__ __forceinline__ shortx4 lds_load_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS shortx4*)(uintptr_t)addr);
}

// Per-lane LDS byte addresses of a swizzled tile block of width W (128 or 64
// columns) starting at LDS address blk (a multiple of 512), computed once: a
// 16-byte row read of (row l32, column 16*kk+8*hi) is at a_base ^ (kk*32); a
// transposing read of rows 16*kc + 8*s + tr_r4, columns nb*32 + tr_c is at
// (t_base[s] ^ (nb*64)) + kc*16*W*2.  Both equal blk + the swz() offsets (the
// XOR acts on bits 5..7 that the other terms leave clear or, for blk, do not
// carry into).
template <int W>
struct SwzBlock {
  uint32_t a_base;
  uint32_t t_base[2];
  __device__ __forceinline__ void init(uint32_t blk, int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    const int f = (W == 128) ? (((l32 & 3) << 2) | ((l32 >> 2) & 3)) : ((((l32 >> 1) & 1) << 2) | ((l32 >> 2) & 3));
    a_base = (blk + l32 * W * 2 + 16 * (hi ^ (f & 1))) | ((f >> 1) << 5);
    const int q = (W == 128) ? ((lane & 15) >> 2) : ((lane >> 3) & 1);
    const int tr_r4 = 4 * hi + ((lane & 15) >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      t_base[s] = (blk + tr_r4 * W * 2 + 8 * (lane & 1) + s * 8 * W * 2 + 16 * (cl ^ ((2 * s + hi) & 3))) | (q << 6);
  }
};

// Addressing of a swizzled tile of COLS (64, 128 or 192) columns and ROWS rows.
template <int COLS, int ROWS>
struct SwzTile {
  static constexpr int W0 = COLS == 64 ? 64 : 128;
  SwzBlock<W0> b0;
  SwzBlock<64> b1;  // second block of a 192-column tile
  __device__ __forceinline__ void init(uint32_t tile, int lane) {
    b0.init(tile, lane);
    if constexpr (COLS == 192) b1.init(tile + ROWS * 128 * 2, lane);
  }
  // LDS address of the 16-byte row read for k-step kk (columns 16*kk + 8*hi)
  // of the tile copy boff bytes further on (boff a multiple of 512)
  __device__ __forceinline__ uint32_t row_read(int kk, uint32_t boff = 0) const {
    if constexpr (COLS == 192) return kk < 8 ? ((b0.a_base + boff) ^ (kk * 32)) : ((b1.a_base + boff) ^ ((kk - 8) * 32));
    else return (b0.a_base + boff) ^ (kk * 32);
  }
  // the same for rows r0 + l32 (r0 a multiple of 16)
  __device__ __forceinline__ uint32_t row_read_at(int kk, int r0, uint32_t boff = 0) const {
    if constexpr (COLS == 192) return kk < 8 ? row_read(kk, boff) + r0 * 256 : row_read(kk, boff) + r0 * 128;
    else return row_read(kk, boff) + r0 * W0 * 2;
  }
  // The same two reads with boff added after the XOR (equal, since boff is a
  // multiple of 512 and the XOR acts on bits 5..7 only), for loops whose
  // buffer offset is a constant: it then becomes the instruction's offset.
  __device__ __forceinline__ uint32_t row_read_c(int kk, uint32_t boff) const { return row_read(kk) + boff; }
  __device__ __forceinline__ uint32_t tr_read_c(int kc, int s, int nb, uint32_t boff) const {
    return tr_read(kc, s, nb) + boff;
  }
  // LDS address of the transposing read for row chunk kc, half s, column block nb
  __device__ __forceinline__ uint32_t tr_read(int kc, int s, int nb, uint32_t boff = 0) const {
    if constexpr (COLS == 192) {
      return nb < 4 ? (((b0.t_base[s] + boff) ^ (nb * 64)) + kc * 16 * 128 * 2)
                    : (((b1.t_base[s] + boff) ^ ((nb - 4) * 64)) + kc * 16 * 64 * 2);
    } else {
      return ((b0.t_base[s] + boff) ^ (nb * 64)) + kc * 16 * W0 * 2;
    }
  }
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Elements 2k and 2k + 1 of an fp16 operand held in the 16-bit vector type:
// a and b rounded to nearest even as one packed conversion
// (v_cvt_pk_f16_f32), which element-wise conversions through the storage
// type do not always become.
__device__ __forceinline__ void put_f16_pair(bf16x8& v, int k, float a, float b) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t w = __builtin_bit_cast(u32x4_t, v);
  w[k] = __builtin_bit_cast(unsigned, __builtin_convertvector((float2_t){a, b}, half2_t));
  v = __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ uint32_t pack2(bf16 lo, bf16 hi) {
  return (uint32_t)__builtin_bit_cast(unsigned short, lo) | ((uint32_t)__builtin_bit_cast(unsigned short, hi) << 16);
}

// A 32 x 32 block held transposed (lane = row l % 32, element rg = column
// 8*(rg/4) + 4*(l/32) + rg%4), times mul, as two 16-byte pieces per lane:
// after a swap of halves between lanes l and l + 32, piece p of lane l holds
// columns 16p + 8*(l/32) .. +7 of its row.
template <bool F16>
__device__ __forceinline__ void row_pieces(const floatx16& acc, float mul, u32x4 (&piece)[2]) {
  uint32_t w[8];  // w[2*c4 + e]: columns 8*c4 + 4*hi + 2e, +1
#pragma unroll
  for (int x = 0; x < 8; ++x) w[x] = pack2(to_elem<F16>(acc[2 * x] * mul), to_elem<F16>(acc[2 * x + 1] * mul));
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      // lanes 32..63 of the first operand trade places with lanes 0..31 of the second
      const auto r = __builtin_amdgcn_permlane32_swap(w[4 * p + e], w[4 * p + 2 + e], false, false);
      w[4 * p + e] = r[0];
      w[4 * p + 2 + e] = r[1];
    }
    piece[p] = u32x4{w[4 * p], w[4 * p + 1], w[4 * p + 2], w[4 * p + 3]};
  }
}

// One key row of a transposed accumulator of NB 32-column blocks, times mul,
// in 16-byte pieces at row (when ok).
template <bool F16, int NB>
__device__ __forceinline__ void store_rows(bf16* row, const floatx16 (&acc)[NB], float mul, int hi, bool ok) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    u32x4 piece[2];
    row_pieces<F16>(acc[nb], mul, piece);
    if (ok) {
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) *reinterpret_cast<u32x4*>(row + nb * 32 + pc * 16 + hi * 8) = piece[pc];
    }
  }
}

// A key-major 32 x 32 accumulator (lane = column l % 32, element rg = key
// 8*(rg/4) + 4*(l/32) + rg%4), times mul and rounded to 16 bits, in the
// transposed form that row_pieces takes (lane = key).  Two MFMAs against a
// permutation of the identity: A is the accumulator as it stands (column =
// M, key = K; rg 8s..8s+7 are the K-slots of product s), and each output
// element is one input times 1 plus zeros, so the values come through
// unchanged.  eye[s] is this lane's B operand of product s (eye_operand).
template <bool F16>
__device__ __forceinline__ floatx16 transpose_acc(const floatx16& acc, float mul, const bf16x8 (&eye)[2]) {
  floatx16 d = floatx16{};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    bf16x8 x;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = to_elem<F16>(acc[8 * s + j] * mul);
    d = mfma32<F16>(x, eye[s], d);
  }
  return d;
}
// B operand of product s of transpose_acc for lane `lane`: K-slot 8*(lane/32)
// + j holds key 16s + 8*(j/4) + 4*(lane/32) + j%4; column n = lane % 32 takes
// a 1 at the slot of key n.
template <bool F16>
__device__ __forceinline__ void eye_operand(int lane, bf16x8 (&eye)[2]) {
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int m = n - 16 * s;
    const int jj = (m >= 0 && m < 16 && ((m >> 2) & 1) == h) ? 4 * (m >> 3) + (m & 3) : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) eye[s][j] = to_elem<F16>(j == jj ? 1.f : 0.f);
  }
}

// A 32 x 32 fp32 block of each of the 4 wavefronts of a group in 16 KB of
// LDS: lane-contiguous 16-byte pieces, element rg of lane l of wavefront w at
// float 4 * ((4w + rg/4) * 64 + l) + rg % 4.
__device__ __forceinline__ void xput(float* area, int w, int lane, const floatx16& acc) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
    *reinterpret_cast<floatx4*>(area + 4 * ((4 * w + r4) * 64 + lane)) =
        floatx4{acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
}
__device__ __forceinline__ void xadd(const float* area, int w, int lane, floatx16& acc) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const floatx4 x = *reinterpret_cast<const floatx4*>(area + 4 * ((4 * w + r4) * 64 + lane));
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[4 * r4 + e] += x[e];
  }
}

// Workgroup barrier for LDS-only hand-offs: waits for this wavefront's own LDS
// operations, then s_barrier.  Unlike __syncthreads it does not drain
// outstanding global loads (the compiler's release fence would), so a
// prefetch issued before it stays in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(0) as the compiler's own instruction (gfx9 encoding: vmcnt
// 0, expcnt 7, lgkmcnt 15), so that its wait insertion knows that every
// earlier global load has completed and adds no wait of its own later.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// One global_load_lds_dwordx4: lane t copies the 16 bytes at base + voff (base
// the same in all lanes, voff the lane's byte offset) to LDS byte lds + 16t
// (lds the same in all lanes).
// Issued as inline assembly so that the compiler's wait insertion does not see
// a pending LDS write: it would otherwise wait for every such copy before each
// later LDS read, whichever buffer the read targets, and a prefetch into the
// other half of a double buffer would stall the reads of the current half.
// Completion is therefore always awaited explicitly: s_waitcnt vmcnt(0), then
// a barrier.  M0 is set here and used by nothing else in these kernels.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)),
               "s"(m0)
               : "memory");
}

// The same with the non-temporal hint: for data read once (the stored dS), so
// that it does not displace reused tiles from the caches.
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(uniform_ptr(base)),
               "s"(m0)
               : "memory");
}

// Asynchronous copy of rows [0, ROWS) of a W-column block (columns col0 ..
// col0+W-1 of the source rows) into a swizzled LDS block: each instruction
// fills 1 KB of LDS, lane t writing bytes 16t..16t+15, so each lane loads the
// logical chunk that the swizzle puts in its slot.  Source row r is at
// g + r*ldb bytes; rows at or past nvalid repeat row nvalid-1 (the masks
// ignore them).  The NW wavefronts of a group share the NI instructions; the
// lane offsets of full tiles are kept from init().
template <int W>
__device__ __forceinline__ int swz_f(int r) {
  return (W == 128) ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int W, int ROWS, int NW>
struct BlockCopy {
  static constexpr int RPI = 1024 / (W * 2);  // rows per instruction
  static constexpr int CPR = W / 8;           // chunks per row
  static constexpr int NI = ROWS / RPI;
  static_assert(NI % NW == 0, "whole instructions per wavefront");
  static constexpr int PER = NI / NW;
  // Instruction wave + x*NW covers rows x*STEP further down than instruction
  // wave.  The swizzle repeats every 16 rows, so for full tiles the lane
  // offsets of x and x + Q (Q*STEP a multiple of 16) differ by a uniform row
  // shift that goes to the scalar base: Q lane offsets serve all x.
  static constexpr int STEP = NW * RPI;
  static constexpr int Q = STEP % 16 == 0 ? 1 : 16 / STEP;
  static_assert(Q * STEP % 16 == 0, "swizzle period");
  uint32_t voff[Q];
  __device__ __forceinline__ static uint32_t lane_off(int u, int lane, int ldb, int col0, int nvalid) {
    const int row = u * RPI + lane / CPR;
    const int chunk = (lane % CPR) ^ swz_f<W>(row);
    return (uint32_t)(min(row, nvalid - 1) * ldb + col0 * 2 + chunk * 16);
  }
  __device__ __forceinline__ void init(int wave, int lane, int ldb, int col0) {
#pragma unroll
    for (int q = 0; q < Q; ++q) voff[q] = lane_off(wave + q * NW, lane, ldb, col0, ROWS);
  }
  __device__ __forceinline__ void issue(uint32_t lds_blk, const void* g, int ldb, int col0, int nvalid, int wave,
                                        int lane) const {
    const char* gb = static_cast<const char*>(g);
    if (nvalid >= ROWS) {
#pragma unroll
      for (int x = 0; x < PER; ++x)
        dma16(gb + (int64_t)(x / Q) * Q * STEP * ldb, voff[x % Q], lds_blk + (wave + x * NW) * 1024);
    } else {
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int u = wave + x * NW;
        dma16(gb, lane_off(u, lane, ldb, col0, nvalid), lds_blk + u * 1024);
      }
    }
  }
};

// A swizzled tile of COLS (64, 128 or 192 = 128 + 64) columns.
template <int COLS, int ROWS, int NW>
struct TileCopy {
  BlockCopy<COLS == 64 ? 64 : 128, ROWS, NW> c0;
  BlockCopy<64, ROWS, NW> c1;  // second block of a 192-column tile
  int ldb;
  __device__ __forceinline__ void init(int wave, int lane, int ld_bytes) {
    ldb = ld_bytes;
    c0.init(wave, lane, ldb, 0);
    if constexpr (COLS == 192) c1.init(wave, lane, ldb, 128);
  }
  __device__ __forceinline__ void issue(uint32_t lds_tile, const void* g, int nvalid, int wave, int lane) const {
    c0.issue(lds_tile, g, ldb, 0, nvalid, wave, lane);
    if constexpr (COLS == 192) c1.issue(lds_tile + ROWS * 128 * 2, g, ldb, 128, nvalid, wave, lane);
  }
};

// The same into a padded tile (row pitch COLS + 8 elements, 16-byte row reads
// only): ROWS*(COLS/8 + 1) 16-byte slots, a multiple of 64 for ROWS % 64 == 0;
// a lane whose slot is the pad loads a valid dummy chunk.
template <int COLS, int ROWS, int NW>
__device__ __forceinline__ void padded_copy(uint32_t lds_tile, const void* g, int ldb, int nvalid, int wave, int lane) {
  constexpr int PC = COLS / 8 + 1;  // 16-byte slots per padded row
  constexpr int NI = ROWS * PC / 64;
  static_assert(NI * 64 == ROWS * PC, "whole instructions");
  for (int u = wave; u < NI; u += NW) {
    const int slot = u * 64 + lane;
    const int row = slot / PC;
    const int ch = slot % PC;
    dma16(g, (uint32_t)(min(row, nvalid - 1) * ldb + (ch < COLS / 8 ? ch * 16 : 0)), lds_tile + u * 1024);
  }
}

// DS form: whether query block qb (32 rows) sees a key of 32-key slice ks.
// Only such (block, slice) tiles of dS are stored and read back; the others
// are zero.
__device__ __forceinline__ bool ds_tile_visible(int qb, int ks, int s1, int s2, int off, int wl, int wr) {
  if (ks * 32 >= s2) return false;
  const fa_sched::Span blks =
      fa_sched::blocks_covering(fa_sched::rows_seeing(s1, ks * 32, min(ks * 32 + 32, s2), off, wl, wr), 32);
  return qb >= blks.lo && qb < blks.hi;
}

// DS form: workspace group of the 128-row query group R of a sequence, and
// the first 32-key slice that group sees (the origin of its band of slots).
__device__ __forceinline__ int64_t ds_group(const KernelArgs& a, const SeqBounds& sb, int R) {
  return a.varlen ? (sb.lbase >> 7) + sb.b + R : (int64_t)sb.b * a.ds_nr + R;
}
__device__ __forceinline__ int ds_band_lo(int R, int s1, int s2, int off, int wl, int wr) {
  return fa_sched::blocks_covering(fa_sched::keys_seen(s2, R * 128, min(R * 128 + 128, s1), off, wl, wr), 32).lo;
}


// LDS placement of a stored dS tile: within each 1 KB half h, the 16-byte
// chunk c (the lane of the producing wavefront) sits at chunk
// c ^ 4*(2h + bit 5 of c), which makes the transposing A reads below free of
// bank conflicts (an involution: the XOR leaves bit 5 alone).
__device__ __forceinline__ int ds_chunk_slot(int c, int h) { return c ^ (4 * ((2 * h + ((c >> 5) & 1)) & 3)); }

// Launch and return the status of this launch only.
template <typename T> struct same_type { using type = T; };
template <typename... KArgs>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
}

}  // namespace
}  // namespace fabwd
