// gfx950 (MI355X) FlashAttention backward: the D = 192 instantiations of the
// dK/dV kernel (template in fa_bwd_dkdv.h), compiled on their own so that they
// take the scheduling strategy that suits one wavefront per SIMD.

#include "fa_bwd_dkdv.h"

namespace fabwd {
namespace dkdv {
namespace {

template <bool F16, bool DS>
int launch_t(const KernelArgs& a, dim3 grid, hipStream_t s) {
  if (a.Dv == 64) return launch(dkdv_kernel<192, 64, 32, 4, 1, F16, DS>, grid, dim3(256), s, a);
  if (a.Dv == 128) return launch(dkdv_kernel<192, 128, 32, 4, 1, F16, DS>, grid, dim3(256), s, a);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_d192(const KernelArgs& a, bool ds, dim3 grid, hipStream_t s) {
  if (ds) return a.f16 ? launch_t<true, true>(a, grid, s) : launch_t<false, true>(a, grid, s);
  return a.f16 ? launch_t<true, false>(a, grid, s) : launch_t<false, false>(a, grid, s);
}

}  // namespace dkdv
}  // namespace fabwd
