"""C-ABI checks of the Floyd attention entry points (include/fa_floyd.h) that
need no GPU: the shape rules of page "CANN Floyd注意力梯度算子" (section
约束说明), the workspace size, and the pointer / workspace checks that
fa_floyd_bwd_run and fa_floyd_fwd_run make before any device call."""

import ctypes

import pytest

from flashattention_backward_fa_amd import fa_bwd as fb
from flashattention_backward_fa_amd import floyd as fl

OK = dict(B=1, H=2, N=16, M=128, K=128, D=32)


@pytest.fixture(scope="module")
def lib():
    import os

    if not os.path.exists(fb.LIB_PATH):
        from flashattention_backward_fa_amd import build
        build.build()
    return fb.load_library()


def desc(**kw):
    a = dict(OK, scale_value=0.1, dtype=fb.DTYPE_BF16)
    a.update(kw)
    return fl.make_desc(a["B"], a["H"], a["N"], a["M"], a["K"], a["D"], a["scale_value"], a["dtype"])


def ws_size(lib, d):
    n = ctypes.c_size_t(0)
    return lib.fa_floyd_workspace_size(ctypes.byref(d), ctypes.byref(n)), n.value


def test_workspace_size_formula(lib, monkeypatch):
    monkeypatch.delenv("FA_FLOYD_CHUNK_BYTES", raising=False)
    for kw in (OK, dict(B=2, H=3, N=48, M=256, K=128, D=128)):
        st, n = ws_size(lib, desc(**kw))
        assert st == fb.FA_OK
        N, M, K, D = kw["N"], kw["M"], kw["K"], kw["D"]
        heads = kw["B"] * kw["H"]
        per_head = 12 * N * M * K + 4 * N * M * D + 8 * N * M
        assert heads * per_head <= n <= heads * per_head + 7 * 256
    # a budget of one byte: one head per group
    monkeypatch.setenv("FA_FLOYD_CHUNK_BYTES", "1")
    st, n1 = ws_size(lib, desc(H=4))
    assert st == fb.FA_OK and n1 <= 12 * 16 * 128 * 128 + 4 * 16 * 128 * 32 + 8 * 16 * 128 + 7 * 256


@pytest.mark.parametrize("kw", [dict(N=8), dict(N=24), dict(M=64), dict(M=200), dict(K=96), dict(K=130),
                                dict(D=16), dict(D=96), dict(D=256), dict(B=0), dict(B=2049), dict(H=0),
                                dict(H=257), dict(N=(1 << 20) + 16)])
def test_shape_rules(lib, kw):
    assert ws_size(lib, desc(**kw))[0] == fb.FA_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(dtype=7), dict(scale_value=float("inf")), dict(scale_value=float("nan"))])
def test_invalid_parameters(lib, kw):
    assert ws_size(lib, desc(**kw))[0] == fb.FA_ERR_PARAM_INVALID


def test_abi_version_checked(lib):
    d = desc()
    d.abi_version = 99
    assert ws_size(lib, d)[0] == fb.FA_ERR_PARAM_INVALID


def test_accepts_page_extremes(lib):
    for kw in (dict(N=16, M=128, K=128, D=32), dict(D=64), dict(D=128), dict(B=2048, H=1), dict(H=256)):
        assert ws_size(lib, desc(**kw))[0] == fb.FA_OK, kw
    assert ws_size(lib, desc(N=1 << 20, M=1 << 20, K=1 << 20))[0] == fb.FA_ERR_UNSUPPORTED


def test_run_checks_before_any_device_call(lib):
    """NULL / misaligned pointers and a short workspace are rejected on the
    host (the fake addresses are never dereferenced)."""
    d = desc()
    _, need = ws_size(lib, d)
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    bwd = lambda ptrs, ws, n: lib.fa_floyd_bwd_run(ctypes.byref(d), *ptrs, ws, n, None)
    full = [fake] * 6 + [None] + [fake] * 3 + [fake] * 5
    assert len(full) == 15
    assert bwd(full, fake, need - 1) == fb.FA_ERR_WORKSPACE
    assert bwd(full, None, need) == fb.FA_ERR_WORKSPACE
    for i in [0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12, 13, 14]:
        ptrs = list(full)
        ptrs[i] = None
        assert bwd(ptrs, fake, need) == fb.FA_ERR_NULLPTR, i
        ptrs[i] = odd
        assert bwd(ptrs, fake, need) == fb.FA_ERR_PARAM_INVALID, i
    assert bwd(full, odd, need) == fb.FA_ERR_PARAM_INVALID
    fwd = lambda ptrs, ws, n: lib.fa_floyd_fwd_run(ctypes.byref(d), *ptrs, ws, n, None)
    fptr = [fake] * 5 + [None] + [fake] * 3
    assert fwd(fptr, fake, need - 1) == fb.FA_ERR_WORKSPACE
    for i in [0, 1, 2, 3, 4, 6, 7, 8]:
        ptrs = list(fptr)
        ptrs[i] = None
        assert fwd(ptrs, fake, need) == fb.FA_ERR_NULLPTR, i
    assert lib.fa_floyd_bwd_run(None, *full, fake, need, None) == fb.FA_ERR_NULLPTR
    n = ctypes.c_size_t(0)
    assert lib.fa_floyd_workspace_size(ctypes.byref(d), None) == fb.FA_ERR_NULLPTR
    assert lib.fa_floyd_workspace_size(None, ctypes.byref(n)) == fb.FA_ERR_NULLPTR


def test_binding_shape_checks():
    import torch

    q = torch.zeros((1, 1, 16, 128, 32), dtype=torch.bfloat16)
    k1 = torch.zeros((1, 1, 16, 128, 32), dtype=torch.bfloat16)
    k2 = torch.zeros((1, 1, 128, 128, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fl._shapes(q, k1, k2[:, :, :64])
    with pytest.raises(TypeError):
        fl._check("key1", k1.float(), k1.shape, torch.bfloat16, k1.device)
    with pytest.raises(ValueError):
        fl._mask(torch.zeros((1, 16, 128)), 1, 16, 128, q.device)
