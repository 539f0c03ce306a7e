"""Thin Python binding of Floyd attention (include/fa_floyd.h in
libfa_bwd.so).  Argument marshalling only: the forward and the backward run
in the library's HIP kernels; PyTorch provides device memory and the current
stream.  There is no fallback.

Names and shapes follow page "CANN Floyd注意力梯度算子" (parameter table of
aclnnFusedFloydAttentionGradGetWorkspaceSize): query / dy / attention_in
[B, H, N, M, D], key1 / value1 [B, H, N, K, D], key2 / value2 [B, H, K, M, D],
atten_mask [B, 1, N, 1, K] (1 = excluded), softmax_max / softmax_sum
[B, H, N, M, 8] float32.
"""

import ctypes
import math

from . import fa_bwd as fb


class FloydDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("M", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("scale_value", ctypes.c_float),
    ]


def make_desc(B, H, N, M, K, D, scale_value, dtype=fb.DTYPE_BF16):
    d = FloydDesc()
    d.abi_version = fb.ABI_VERSION
    d.dtype = dtype
    d.B, d.H, d.N, d.M, d.K, d.D = B, H, N, M, K, D
    d.scale_value = scale_value
    return d


def workspace_size(desc):
    lib = fb.load_library()
    n = ctypes.c_size_t(0)
    st = lib.fa_floyd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != fb.FA_OK:
        raise fb.FaBwdError(st, "fa_floyd_workspace_size")
    return n.value


def _shapes(q, k1, k2):
    if q.dim() != 5 or k1.dim() != 5 or k2.dim() != 5:
        raise ValueError("query, key1 and key2 must be 5-D ([B, H, N, M, D], [B, H, N, K, D], [B, H, K, M, D])")
    B, H, N, M, D = q.shape
    K = k1.shape[3]
    if tuple(k1.shape) != (B, H, N, K, D) or tuple(k2.shape) != (B, H, K, M, D):
        raise ValueError(f"shape mismatch: query {tuple(q.shape)}, key1 {tuple(k1.shape)}, key2 {tuple(k2.shape)}")
    return B, H, N, M, K, D


def _check(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} is {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.contiguous()


def _mask(mask, B, N, K, device):
    import torch

    if mask is None:
        return None
    if tuple(mask.shape) != (B, 1, N, 1, K):
        raise ValueError(f"atten_mask has shape {tuple(mask.shape)}, expected {(B, 1, N, 1, K)}")
    if mask.device != device:
        raise ValueError("atten_mask is on another device")
    return mask.to(torch.uint8).contiguous()


def _prepare(query, key1, value1, key2, value2, scale_value):
    B, H, N, M, K, D = _shapes(query, key1, key2)
    dt, dev = query.dtype, query.device
    code = fb._dtype_code(query)
    key1 = _check("key1", key1, (B, H, N, K, D), dt, dev)
    value1 = _check("value1", value1, (B, H, N, K, D), dt, dev)
    key2 = _check("key2", key2, (B, H, K, M, D), dt, dev)
    value2 = _check("value2", value2, (B, H, K, M, D), dt, dev)
    scale = 1.0 / math.sqrt(D) if scale_value is None else float(scale_value)
    desc = make_desc(B, H, N, M, K, D, scale, code)
    return desc, (B, H, N, M, K, D), query.contiguous(), key1, value1, key2, value2


def _workspace(desc, device, workspace):
    import torch

    need = workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {need}")
    return workspace


def floyd_attn(query, key1, value1, key2, value2, atten_mask=None, scale_value=None, workspace=None):
    """Forward: (attention_out, softmax_max, softmax_sum) on the current
    stream.  scale_value None means 1/sqrt(D), the value of the page's
    example."""
    import torch

    desc, (B, H, N, M, K, D), q, k1, v1, k2, v2 = _prepare(query, key1, value1, key2, value2, scale_value)
    dev = q.device
    mask = _mask(atten_mask, B, N, K, dev)
    out = torch.empty_like(q)
    smax = torch.empty((B, H, N, M, 8), dtype=torch.float32, device=dev)
    ssum = torch.empty_like(smax)
    ws = _workspace(desc, dev, workspace)
    lib = fb.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    p = fb._ptr
    st = lib.fa_floyd_fwd_run(ctypes.byref(desc), p(q), p(k1), p(v1), p(k2), p(v2), p(mask), p(out), p(smax),
                              p(ssum), p(ws), ws.numel() * ws.element_size(), stream)
    if st != fb.FA_OK:
        raise fb.FaBwdError(st, "fa_floyd_fwd_run")
    return out, smax, ssum


STAGES = ("rowstats", "scores_by_n", "scores_by_m_softmax_grad", "dv1", "dk1", "dv2", "dk2", "dq_k1", "dq_k2")


def floyd_attn_grad(query, key1, value1, key2, value2, dy, atten_mask, softmax_max, softmax_sum, attention_in,
                    scale_value=None, workspace=None, out=None, stage_ms=None):
    """Backward: (dq, dk1, dv1, dk2, dv2) on the current stream, in the
    inputs' element type (written into `out` when given).  With a list
    `stage_ms` the call goes through fa_floyd_bwd_run_timed, waits, and the
    list receives the duration of each stage of STAGES in milliseconds."""
    import torch

    desc, (B, H, N, M, K, D), q, k1, v1, k2, v2 = _prepare(query, key1, value1, key2, value2, scale_value)
    dev = q.device
    dy = _check("dy", dy, (B, H, N, M, D), q.dtype, dev)
    y = _check("attention_in", attention_in, (B, H, N, M, D), q.dtype, dev)
    smax = _check("softmax_max", softmax_max, (B, H, N, M, 8), torch.float32, dev)
    ssum = _check("softmax_sum", softmax_sum, (B, H, N, M, 8), torch.float32, dev)
    mask = _mask(atten_mask, B, N, K, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k1), torch.empty_like(v1), torch.empty_like(k2),
               torch.empty_like(v2))
    dq, dk1, dv1, dk2, dv2 = out
    for name, t, ref in (("dq", dq, q), ("dk1", dk1, k1), ("dv1", dv1, v1), ("dk2", dk2, k2), ("dv2", dv2, v2)):
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != ref.dtype or t.device != dev or not t.is_contiguous():
            raise ValueError(f"out[{name}] must be a contiguous {ref.dtype} tensor of shape {tuple(ref.shape)}")
    ws = _workspace(desc, dev, workspace)
    lib = fb.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    p = fb._ptr
    args = (ctypes.byref(desc), p(q), p(k1), p(v1), p(k2), p(v2), p(dy), p(mask), p(smax), p(ssum), p(y), p(dq),
            p(dk1), p(dv1), p(dk2), p(dv2), p(ws), ws.numel() * ws.element_size(), stream)
    if stage_ms is None:
        st = lib.fa_floyd_bwd_run(*args)
    else:
        buf = (ctypes.c_float * len(STAGES))()
        st = lib.fa_floyd_bwd_run_timed(*args, buf)
        stage_ms[:] = list(buf)
    if st != fb.FA_OK:
        raise fb.FaBwdError(st, "fa_floyd_bwd_run")
    return dq, dk1, dv1, dk2, dv2
