// gfx950 (MI355X) FlashAttention backward: the dK/dV kernel (template in
// fa_bwd_dkdv.h) for D <= 128, and its launch for every head dimension.

#include "fa_bwd_dkdv.h"

namespace fabwd {
namespace dkdv {
namespace {

template <bool F16, bool DS>
int launch_t(const KernelArgs& a, dim3 grid, hipStream_t s) {
  if (a.D == 64 && a.Dv == 64) return launch(dkdv_kernel<64, 64, 32, 4, 2, F16, DS>, grid, dim3(512), s, a);
  if (a.D == 128 && a.Dv == 64) return launch(dkdv_kernel<128, 64, 32, 4, 2, F16, DS>, grid, dim3(512), s, a);
  if (a.D == 128 && a.Dv == 128) return launch(dkdv_kernel<128, 128, 32, 4, 2, F16, DS>, grid, dim3(512), s, a);
  return (int)hipErrorInvalidValue;
}

}  // namespace
}  // namespace dkdv

int launch_dkdv(const KernelArgs& a, void* stream) {
  const int64_t tiles = (a.S2 + 127) / 128;  // 128-key tiles in every shape
  const int64_t blocks = tiles * (a.G / a.heads_per_job) * a.q_splits * a.B * a.n2_count;
  if (blocks <= 0) return 0;
  if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)blocks);
  const bool ds = a.variant == 4;
  if (a.D == 192) return dkdv::launch_d192(a, ds, grid, s);
  if (ds) return a.f16 ? dkdv::launch_t<true, true>(a, grid, s) : dkdv::launch_t<false, true>(a, grid, s);
  return a.f16 ? dkdv::launch_t<true, false>(a, grid, s) : dkdv::launch_t<false, false>(a, grid, s);
}

}  // namespace fabwd
