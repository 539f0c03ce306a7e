"""Thin Python binding of libfa_bwd.so (include/fa_bwd.h).

Argument marshalling only: every step of the backward runs in the library's
HIP kernels.  PyTorch provides device memory (outputs, workspace) and the
current stream.  If the library is missing this module raises on use; there
is no fallback.

The signature of flash_attn_grad follows the page "CANN ops-transformer
FlashAttnGrad 算子详解", section 四 4.2 (function prototype), with
seqused_q / seqused_kv, without the options this library does not build
(sinks, attn_mask, metadata), with one layout for q, kv and out (section 四
4.6 requires them equal), and with the library's own choices appended: the dQ
strategy (dq_mode), a workspace bound and the fp32 debugging form.
"""

import ctypes
import enum
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libfa_bwd.so")

ABI_VERSION = 3

FA_OK = 0
FA_ERR_NULLPTR = 1
FA_ERR_PARAM_INVALID = 2
FA_ERR_SHAPE = 3
FA_ERR_UNSUPPORTED = 4
FA_ERR_WORKSPACE = 5
FA_ERR_RUNTIME = 6

SCRATCH_BYTES = 64 << 20  # FA_BWD_SCRATCH_BYTES: the device scratch of fa_bwd_run_noalloc

LAYOUTS = {"BSND": 0, "BNSD": 1, "TND": 2}
FLAG_DETERMINISTIC = 0x1
FLAG_FP32_OUT = 0x2
DTYPE_BF16 = 0
DTYPE_FP16 = 1

# FA_DQ_* of include/fa_bwd.h: fa_bwd_desc.dq_mode takes the names, and
# fa_bwd_plan_dq_path reports one of them (never "auto")
DQ_MODES = {"auto": 0, "stored_ds": 1, "recompute": 2, "atomic": 3, "fused": 4}
DQ_PATHS = {1: "stored_ds", 2: "recompute", 3: "atomic", 4: "fused", 5: "fp32_form"}

EXPORTED = ("fa_bwd_create", "fa_bwd_run", "fa_bwd_run_noalloc", "fa_bwd_sfmg", "fa_fwd_run", "fa_bwd_plan_dq_path", "fa_bwd_profile_enable",
            "fa_bwd_profile_read", "fa_bwd_profile_read_split", "fa_bwd_destroy", "fa_bwd_strerror", "fa_bwd_abi_version",
            "fa_floyd_workspace_size", "fa_floyd_bwd_run", "fa_floyd_bwd_run_timed", "fa_floyd_fwd_run")


class MaskMode(enum.IntEnum):
    """mask_mode (section 四 4.3: IntEnum, int, or case-insensitive name)."""
    NONE = 0
    CAUSAL = 1
    WINDOW = 2


def mask_mode_value(m):
    if isinstance(m, str):
        try:
            return int(MaskMode[m.upper()])
        except KeyError:
            raise ValueError(f"unknown mask_mode name {m!r}") from None
    return int(m)


class FaBwdDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("N1", ctypes.c_int32),
        ("N2", ctypes.c_int32),
        ("S1", ctypes.c_int32),
        ("S2", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("Dv", ctypes.c_int32),
        ("T1", ctypes.c_int64),
        ("T2", ctypes.c_int64),
        ("host_cu_seqlens_q", ctypes.POINTER(ctypes.c_int32)),
        ("host_cu_seqlens_kv", ctypes.POINTER(ctypes.c_int32)),
        ("softmax_scale", ctypes.c_float),
        ("mask_mode", ctypes.c_int32),
        ("win_left", ctypes.c_int32),
        ("win_right", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("dq_mode", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("max_workspace_bytes", ctypes.c_uint64),
    ]


class FaBwdError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status}: {strerror(status)}")


_lib = None


def load_library(path=LIB_PATH):
    """Load libfa_bwd.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m flashattention_backward_fa_amd.build`")
    # PyTorch ships its own HIP runtime.  Import it first so that this
    # library binds to that same runtime: with two runtimes in one process,
    # device pointers allocated by torch are invalid for our launches.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the library itself needs no torch
        pass
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.fa_bwd_create.argtypes = [ctypes.POINTER(FaBwdDesc), ctypes.POINTER(vp), ctypes.POINTER(sz)]
    lib.fa_bwd_create.restype = ctypes.c_int
    lib.fa_bwd_run.argtypes = [vp] * 11 + [vp] * 3 + [vp, sz, vp]
    lib.fa_bwd_run.restype = ctypes.c_int
    lib.fa_bwd_run_noalloc.argtypes = [vp] * 11 + [vp] * 3 + [vp]
    lib.fa_bwd_run_noalloc.restype = ctypes.c_int
    lib.fa_bwd_sfmg.argtypes = [vp] * 6
    lib.fa_bwd_sfmg.restype = ctypes.c_int
    lib.fa_fwd_run.argtypes = [vp] * 11
    lib.fa_fwd_run.restype = ctypes.c_int
    lib.fa_bwd_plan_dq_path.argtypes = [vp, ctypes.POINTER(ctypes.c_int)]
    lib.fa_bwd_plan_dq_path.restype = ctypes.c_int
    lib.fa_bwd_profile_enable.argtypes = [vp, ctypes.c_int]
    lib.fa_bwd_profile_enable.restype = ctypes.c_int
    lib.fa_bwd_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]
    lib.fa_bwd_profile_read.restype = ctypes.c_int
    lib.fa_bwd_profile_read_split.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float),
                                              ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.fa_bwd_profile_read_split.restype = ctypes.c_int
    lib.fa_bwd_destroy.argtypes = [vp]
    lib.fa_bwd_destroy.restype = ctypes.c_int
    lib.fa_bwd_strerror.argtypes = [ctypes.c_int]
    lib.fa_bwd_strerror.restype = ctypes.c_char_p
    lib.fa_bwd_abi_version.argtypes = []
    lib.fa_bwd_abi_version.restype = ctypes.c_int
    # Floyd attention (include/fa_floyd.h); the descriptor is passed by pointer
    lib.fa_floyd_workspace_size.argtypes = [vp, ctypes.POINTER(sz)]
    lib.fa_floyd_workspace_size.restype = ctypes.c_int
    lib.fa_floyd_bwd_run.argtypes = [vp] * 16 + [vp, sz, vp]
    lib.fa_floyd_bwd_run.restype = ctypes.c_int
    lib.fa_floyd_bwd_run_timed.argtypes = [vp] * 16 + [vp, sz, vp, ctypes.POINTER(ctypes.c_float)]
    lib.fa_floyd_bwd_run_timed.restype = ctypes.c_int
    lib.fa_floyd_fwd_run.argtypes = [vp] * 10 + [vp, sz, vp]
    lib.fa_floyd_fwd_run.restype = ctypes.c_int
    if lib.fa_bwd_abi_version() != ABI_VERSION:
        raise RuntimeError("libfa_bwd.so ABI version mismatch")
    _lib = lib
    return lib


def strerror(status):
    return load_library().fa_bwd_strerror(int(status)).decode()


def dq_mode_value(m):
    """FA_DQ_* code of a dq_mode given by name ("auto", "stored_ds",
    "recompute", "atomic", "fused") or number."""
    if isinstance(m, str):
        try:
            return DQ_MODES[m.lower()]
        except KeyError:
            raise ValueError(f"unknown dq_mode {m!r}; one of {sorted(DQ_MODES)}") from None
    return int(m)


def make_desc(layout, B, N1, N2, S1, S2, D, Dv, T1=0, T2=0, softmax_scale=0.0, mask_mode=0,
              win_left=-1, win_right=-1, flags=0, host_cu_q=None, host_cu_kv=None, dtype=0, dq_mode=0,
              num_cus=0, max_workspace_bytes=0):
    """Fill an fa_bwd_desc.  host_cu_q/kv: optional int32 ctypes arrays kept
    alive by the caller until fa_bwd_create returns."""
    d = FaBwdDesc()
    d.abi_version = ABI_VERSION
    d.dtype = dtype
    d.layout = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    d.B, d.N1, d.N2, d.S1, d.S2, d.D, d.Dv = B, N1, N2, S1, S2, D, Dv
    d.T1, d.T2 = T1, T2
    P = ctypes.POINTER(ctypes.c_int32)
    d.host_cu_seqlens_q = ctypes.cast(host_cu_q, P) if host_cu_q is not None else P()
    d.host_cu_seqlens_kv = ctypes.cast(host_cu_kv, P) if host_cu_kv is not None else P()
    d.softmax_scale = softmax_scale
    d.mask_mode = mask_mode_value(mask_mode)
    d.win_left, d.win_right = win_left, win_right
    d.flags = flags
    d.dq_mode = dq_mode_value(dq_mode)
    d.num_cus = int(num_cus)
    d.max_workspace_bytes = int(max_workspace_bytes)
    return d


class Plan:
    """Owns an fa_bwd_plan handle; the library validates and sizes in create."""

    def __init__(self, desc):
        lib = load_library()
        h = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        st = lib.fa_bwd_create(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(ws))
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_create")
        self._lib = lib  # the handle belongs to this library instance
        self.handle = h
        self.workspace_bytes = ws.value
        self.layout = desc.layout

    def __del__(self):
        h = getattr(self, "handle", None)
        lib = getattr(self, "_lib", None)
        if h is not None and lib is not None:
            lib.fa_bwd_destroy(h)
            self.handle = None

    def run(self, q, k, v, dout, attn_out, lse, cu_q, cu_kv, dq, dk, dv, workspace, workspace_bytes, stream,
            seqused_q=None, seqused_kv=None):
        st = self._lib.fa_bwd_run(self.handle, q, k, v, dout, attn_out, lse, cu_q, cu_kv, seqused_q, seqused_kv,
                                  dq, dk, dv, workspace, workspace_bytes, stream)
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_run")

    def forward(self, q, k, v, cu_q, cu_kv, attn_out, lse, stream, seqused_q=None, seqused_kv=None):
        st = self._lib.fa_fwd_run(self.handle, q, k, v, cu_q, cu_kv, seqused_q, seqused_kv, attn_out, lse, stream)
        if st != FA_OK:
            raise FaBwdError(st, "fa_fwd_run")

    def dq_path(self):
        """One of DQ_PATHS' keys: how this plan forms dQ."""
        out = ctypes.c_int()
        st = self._lib.fa_bwd_plan_dq_path(self.handle, ctypes.byref(out))
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_plan_dq_path")
        return DQ_PATHS[out.value]

    def profile_enable(self, slots):
        st = self._lib.fa_bwd_profile_enable(self.handle, int(slots))
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_profile_enable")

    def profile_read(self, cap):
        buf = (ctypes.c_float * max(int(cap), 1))()
        n = ctypes.c_int()
        st = self._lib.fa_bwd_profile_read(self.handle, buf, int(cap), ctypes.byref(n))
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_profile_read")
        return [buf[i] for i in range(n.value)]

    def profile_read_split(self, cap):
        """[(first kernel ms, second kernel ms)] of the recorded runs; see
        fa_bwd_profile_read_split."""
        a = (ctypes.c_float * max(int(cap), 1))()
        b = (ctypes.c_float * max(int(cap), 1))()
        n = ctypes.c_int()
        st = self._lib.fa_bwd_profile_read_split(self.handle, a, b, int(cap), ctypes.byref(n))
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_profile_read_split")
        return [(a[i], b[i]) for i in range(n.value)]

    def sfmg(self, dout, attn_out, cu_q, out, stream):
        st = self._lib.fa_bwd_sfmg(self.handle, dout, attn_out, cu_q, out, stream)
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_sfmg")


# ------------------------------------------------------------------ torch-facing API

_plans = {}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shapes(q, k, v, layout):
    if layout == "TND":
        T1, N1, D = q.shape
        T2, N2, _ = k.shape
        return dict(N1=N1, N2=N2, D=D, Dv=v.shape[-1], T1=T1, T2=T2)
    if layout == "BSND":
        B, S1, N1, D = q.shape
        _, S2, N2, _ = k.shape
    else:
        B, N1, S1, D = q.shape
        _, N2, S2, _ = k.shape
    return dict(B=B, N1=N1, N2=N2, S1=S1, S2=S2, D=D, Dv=v.shape[-1])


def _dtype_code(t):
    """FA_DTYPE_* of a tensor's element type (bf16 or fp16)."""
    import torch

    codes = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}
    if t.dtype not in codes:
        raise TypeError(f"elements must be bfloat16 or float16, got {t.dtype}")
    return codes[t.dtype]


def _seqused(t, device):
    """Validate an optional seqused tensor (int32 on the inputs' device)."""
    import torch

    if t is None:
        return None
    _check("seqused", t, torch.int32, device)
    return t.contiguous()


def _check(name, t, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def get_plan(q, k, v, layout="BSND", cu_seqlens_q=None, cu_seqlens_kv=None, softmax_scale=0.0,
             mask_mode=0, win_left=-1, win_right=-1, max_seqlen_q=-1, max_seqlen_kv=-1,
             deterministic=False, host_cu_seqlens=None, fp32_out=False, dq_mode="auto", max_workspace_bytes=0):
    """Create (or reuse) the plan for these shapes, element type and attributes."""
    sh = _shapes(q, k, v, layout)
    dt = _dtype_code(q)
    flags = (FLAG_DETERMINISTIC if deterministic else 0) | (FLAG_FP32_OUT if fp32_out else 0)
    mm = mask_mode_value(mask_mode)
    dm = dq_mode_value(dq_mode)
    extra = dict(dq_mode=dm, max_workspace_bytes=int(max_workspace_bytes))
    if layout == "TND":
        if cu_seqlens_q is None or cu_seqlens_kv is None:
            raise ValueError("TND needs cu_seqlens_q and cu_seqlens_kv")
        B = cu_seqlens_q.numel() - 1
        hq = hk = None
        if host_cu_seqlens is not None:
            hq, hk = host_cu_seqlens
        elif max_seqlen_q < 0 or max_seqlen_kv < 0:
            # deriving the max lengths needs a host copy (this synchronises)
            hq = [int(x) for x in cu_seqlens_q.cpu().tolist()]
            hk = [int(x) for x in cu_seqlens_kv.cpu().tolist()]
        key = ("TND", B, sh["N1"], sh["N2"], sh["D"], sh["Dv"], sh["T1"], sh["T2"], max_seqlen_q,
               max_seqlen_kv, tuple(hq) if hq else None, tuple(hk) if hk else None, float(softmax_scale),
               mm, win_left, win_right, flags, dt, dm, int(max_workspace_bytes))
        if key not in _plans:
            aq = (ctypes.c_int32 * len(hq))(*hq) if hq else None
            ak = (ctypes.c_int32 * len(hk))(*hk) if hk else None
            d = make_desc("TND", B, sh["N1"], sh["N2"], max_seqlen_q, max_seqlen_kv, sh["D"], sh["Dv"],
                          sh["T1"], sh["T2"], softmax_scale, mm, win_left, win_right, flags, aq, ak, dtype=dt,
                          **extra)
            _plans[key] = Plan(d)
        return _plans[key]
    if cu_seqlens_q is not None or cu_seqlens_kv is not None:
        raise ValueError("cu_seqlens are only accepted with the TND layout")
    key = (layout, sh["B"], sh["N1"], sh["N2"], sh["S1"], sh["S2"], sh["D"], sh["Dv"], float(softmax_scale), mm,
           win_left, win_right, flags, dt, dm, int(max_workspace_bytes))
    if key not in _plans:
        d = make_desc(layout, sh["B"], sh["N1"], sh["N2"], sh["S1"], sh["S2"], sh["D"], sh["Dv"], 0, 0,
                      softmax_scale, mm, win_left, win_right, flags, dtype=dt, **extra)
        _plans[key] = Plan(d)
    return _plans[key]


def _bind_grad(q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q, cu_seqlens_kv, softmax_scale, mask_mode,
               win_left, win_right, max_seqlen_q, max_seqlen_kv, layout, deterministic, workspace, out, fp32_out,
               seqused_q, seqused_kv, dq_mode, max_workspace_bytes):
    """Validation, plan lookup and allocation shared by flash_attn_grad and
    prepare_grad: (plan, run arguments before the stream, outputs, tensors to
    keep alive)."""
    import torch

    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    dev = q.device
    _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("attn_out", attn_out)):
        _check(name, t, q.dtype, dev)
    _check("softmax_lse", softmax_lse, torch.float32, dev)
    q, k, v, dout, attn_out, softmax_lse = (t.contiguous() for t in (q, k, v, dout, attn_out, softmax_lse))
    if cu_seqlens_q is not None:
        _check("cu_seqlens_q", cu_seqlens_q, torch.int32, dev)
        _check("cu_seqlens_kv", cu_seqlens_kv, torch.int32, dev)
        cu_seqlens_q, cu_seqlens_kv = cu_seqlens_q.contiguous(), cu_seqlens_kv.contiguous()
    if dout.shape != attn_out.shape:
        raise ValueError("dout and attn_out must have the same shape")
    seqused_q, seqused_kv = _seqused(seqused_q, dev), _seqused(seqused_kv, dev)
    plan = get_plan(q, k, v, layout, cu_seqlens_q, cu_seqlens_kv, softmax_scale, mask_mode, win_left, win_right,
                    max_seqlen_q, max_seqlen_kv, deterministic, fp32_out=fp32_out, dq_mode=dq_mode,
                    max_workspace_bytes=max_workspace_bytes)
    odt = torch.float32 if fp32_out else q.dtype
    if out is None:
        dq, dk, dv = (torch.empty(t.shape, dtype=odt, device=dev) for t in (q, k, v))
    else:
        dq, dk, dv = out
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            _check(name, t, odt, dev)
            if t.shape != ref.shape or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(ref.shape)}")
    if workspace is None or workspace.numel() < plan.workspace_bytes:
        workspace = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
    args = (plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(attn_out), _ptr(softmax_lse),
            _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(seqused_q), _ptr(seqused_kv), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), ctypes.c_size_t(workspace.numel()))
    keep = (q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q, cu_seqlens_kv, seqused_q, seqused_kv, workspace)
    return plan, args, (dq, dk, dv), keep


def flash_attn_grad(q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q=None, cu_seqlens_kv=None,
                    softmax_scale=0.0, mask_mode=0, win_left=-1, win_right=-1, max_seqlen_q=-1,
                    max_seqlen_kv=-1, layout="BSND", deterministic=False, workspace=None, out=None,
                    fp32_out=False, seqused_q=None, seqused_kv=None, dq_mode="auto", max_workspace_bytes=0):
    """dq, dk, dv of attention on the current HIP stream, in the inputs' element
    type (bf16 or fp16).

    q, k, v, dout, attn_out: bf16 or fp16 CUDA(HIP) tensors of one type in
    `layout`; softmax_lse:
    float32, (B, N1, S1) or (N1, T1); cu_seqlens_*: int32 device tensors for
    TND only.  Non-contiguous inputs are made contiguous first.  `workspace`
    (uint8 tensor) and `out` ((dq, dk, dv)) may be passed to avoid allocation.
    fp32_out=True selects the fp32 debugging form (float32 outputs, P and dS
    kept in fp32; slow).  seqused_q / seqused_kv: optional int32 device
    tensors [B]; only the first seqused[b] rows / keys of sequence b take part
    and the gradients of the rest are zero.  dq_mode: how dQ is formed
    ("auto", "stored_ds", "recompute", "atomic" or "fused"; see FA_DQ_* in
    include/fa_bwd.h); max_workspace_bytes: an upper bound on the workspace
    the plan may ask for (0 = none).
    """
    import torch

    plan, args, outs, _keep = _bind_grad(q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q, cu_seqlens_kv,
                                         softmax_scale, mask_mode, win_left, win_right, max_seqlen_q, max_seqlen_kv,
                                         layout, deterministic, workspace, out, fp32_out, seqused_q, seqused_kv,
                                         dq_mode, max_workspace_bytes)
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    st = plan._lib.fa_bwd_run(*args, stream)
    if st != FA_OK:
        raise FaBwdError(st, "fa_bwd_run")
    return outs


class PreparedGrad:
    """The backward bound to fixed tensors (from prepare_grad): validation,
    plan lookup, output / workspace allocation and pointer marshalling are done
    once, and each call only enqueues fa_bwd_run.  The bound tensors may change
    in value between calls but not be reallocated; the object keeps them alive.
    Calling it returns (dq, dk, dv), the same tensors every time."""

    def __init__(self, plan, args, outs, keep, device, stream):
        self.plan = plan
        self.outputs = outs
        self._run = plan._lib.fa_bwd_run
        self._args = args
        self._keep = keep
        self._device = device
        self._stream = None if stream is None else ctypes.c_void_p(stream.cuda_stream)

    def __call__(self, stream=None):
        """Enqueue one backward on `stream` (a torch stream), else on the stream
        fixed at preparation, else on the current stream."""
        if stream is not None:
            s = ctypes.c_void_p(stream.cuda_stream)
        elif self._stream is not None:
            s = self._stream
        else:
            import torch

            s = ctypes.c_void_p(torch.cuda.current_stream(self._device).cuda_stream)
        st = self._run(*self._args, s)
        if st != FA_OK:
            raise FaBwdError(st, "fa_bwd_run")
        return self.outputs


def prepare_grad(q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q=None, cu_seqlens_kv=None, softmax_scale=0.0,
                 mask_mode=0, win_left=-1, win_right=-1, max_seqlen_q=-1, max_seqlen_kv=-1, layout="BSND",
                 deterministic=False, workspace=None, out=None, fp32_out=False, seqused_q=None, seqused_kv=None,
                 dq_mode="auto", max_workspace_bytes=0, stream=None):
    """flash_attn_grad's arguments bound once into a PreparedGrad, for loops
    that run the same backward many times (the per-call host cost of
    flash_attn_grad is a large share of a short backward).  `stream`: a torch
    stream to enqueue on (default: the current stream at each call)."""
    plan, args, outs, keep = _bind_grad(q, k, v, dout, attn_out, softmax_lse, cu_seqlens_q, cu_seqlens_kv,
                                        softmax_scale, mask_mode, win_left, win_right, max_seqlen_q, max_seqlen_kv,
                                        layout, deterministic, workspace, out, fp32_out, seqused_q, seqused_kv,
                                        dq_mode, max_workspace_bytes)
    return PreparedGrad(plan, args, outs, keep, q.device, stream)


def flash_attn(q, k, v, cu_seqlens_q=None, cu_seqlens_kv=None, softmax_scale=0.0, mask_mode=0, win_left=-1,
               win_right=-1, max_seqlen_q=-1, max_seqlen_kv=-1, layout="BSND", seqused_q=None, seqused_kv=None):
    """Forward (attn_out in the inputs' element type, softmax_lse float32) with
    the same conventions as flash_attn_grad; its outputs are what
    flash_attn_grad expects."""
    import torch

    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    dev = q.device
    _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, q.dtype, dev)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    plan = get_plan(q, k, v, layout, cu_seqlens_q, cu_seqlens_kv, softmax_scale, mask_mode, win_left, win_right,
                    max_seqlen_q, max_seqlen_kv)
    sh = _shapes(q, k, v, layout)
    out = torch.empty(tuple(q.shape[:-1]) + (sh["Dv"],), dtype=q.dtype, device=dev)
    if layout == "TND":
        lse = torch.empty((sh["N1"], sh["T1"]), dtype=torch.float32, device=dev)
    else:
        lse = torch.empty((sh["B"], sh["N1"], sh["S1"]), dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    plan.forward(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_kv), _ptr(out), _ptr(lse), stream,
                 _ptr(_seqused(seqused_q, dev)), _ptr(_seqused(seqused_kv, dev)))
    return out, lse


def sfmg(dout, attn_out, layout="BSND", cu_seqlens_q=None, N2=None, max_seqlen_q=-1):
    """The preprocess kernel alone: float32 rowsum(dout * attn_out) in
    softmax_lse's layout."""
    import torch

    # a plan needs key shapes; use a self-attention stand-in with N2 = N1 / 1
    if layout == "TND":
        T1, N1, Dv = dout.shape
        q = torch.empty((T1, N1, Dv), dtype=dout.dtype, device="meta")
        plan = get_plan(q, q, q, "TND", cu_seqlens_q, cu_seqlens_q, max_seqlen_q=max_seqlen_q,
                        max_seqlen_kv=max_seqlen_q)
        res = torch.empty((N1, T1), dtype=torch.float32, device=dout.device)
    else:
        if layout == "BSND":
            B, S1, N1, Dv = dout.shape
        else:
            B, N1, S1, Dv = dout.shape
        q = torch.empty(tuple(dout.shape), dtype=dout.dtype, device="meta")
        plan = get_plan(q, q, q, layout)
        res = torch.empty((B, N1, S1), dtype=torch.float32, device=dout.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dout.device).cuda_stream)
    plan.sfmg(_ptr(dout.contiguous()), _ptr(attn_out.contiguous()), _ptr(cu_seqlens_q), _ptr(res), stream)
    return res
