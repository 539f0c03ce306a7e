// Argument-block prefetch for gfx950 kernels that take KernelArgs and are
// short enough for their prologue to count (the fused small-sequence kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd_internal.h"

namespace fabwd {

// One scalar load per 64-byte line of the first 448 bytes of the kernel's
// argument segment (KernelArgs, passed first, spans seven lines), waited for
// in the same statement.  The compiler places a kernel's own argument loads
// next to their uses and spreads them over several dependent waits (the
// branches on layout, seqused and masks); after this they hit the scalar
// cache, so the first wavefront on a CU waits for memory once, not four times.
__device__ __forceinline__ void prefetch_args() {
  static_assert(sizeof(KernelArgs) > 6 * 64, "the seventh line is inside the argument block");
  uint32_t x0, x1, x2, x3, x4, x5, x6;
  asm volatile(
      "s_load_dword %0, %7, 0x0\n\ts_load_dword %1, %7, 0x40\n\ts_load_dword %2, %7, 0x80\n\t"
      "s_load_dword %3, %7, 0xc0\n\ts_load_dword %4, %7, 0x100\n\ts_load_dword %5, %7, 0x140\n\t"
      "s_load_dword %6, %7, 0x180\n\ts_waitcnt lgkmcnt(0)"
      : "=s"(x0), "=s"(x1), "=s"(x2), "=s"(x3), "=s"(x4), "=s"(x5), "=s"(x6)
      : "s"(__builtin_amdgcn_kernarg_segment_ptr()));
  asm volatile("" ::"s"(x0 | x1 | x2 | x3 | x4 | x5 | x6));
}

}  // namespace fabwd
