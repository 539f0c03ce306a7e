"""MI355X (gfx950) FlashAttention backward: HIP kernels behind a C ABI
(include/fa_bwd.h, lib/libfa_bwd.so) and a thin ctypes binding."""

from .fa_bwd import (  # noqa: F401
    MaskMode, FaBwdError, Plan, PreparedGrad, flash_attn, flash_attn_grad, prepare_grad, sfmg, load_library,
    make_desc, strerror,
    FA_OK, FA_ERR_NULLPTR, FA_ERR_PARAM_INVALID, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED,
    FA_ERR_WORKSPACE, FA_ERR_RUNTIME, EXPORTED,
)
