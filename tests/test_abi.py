"""C-ABI checks that need no GPU: the library loads, exports every function
the headers under include/ declare, and fa_bwd_create enforces the constraints of page
"CANN ops-transformer FlashAttnGrad 算子详解", section 四 4.6, with the error
classes of the header.  fa_bwd_run's pointer and workspace checks return
before any device call, so they are exercised here too."""

import ctypes
import math
import os
import re

import pytest

from flashattention_backward_fa_amd import fa_bwd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fb.LIB_PATH):
        from flashattention_backward_fa_amd import build
        build.build()
    return fb.load_library()


def declared_functions():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f), encoding="utf-8").read() for f in sorted(os.listdir(inc))
                   if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|void)\s+(fa_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(fb.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strerror(lib):
    assert lib.fa_bwd_abi_version() == fb.ABI_VERSION == 3
    for st in range(0, 7):
        assert len(fb.strerror(st)) > 0
    assert fb.strerror(99) == "unknown status"


def create(lib, **kw):
    base = dict(layout="BSND", B=2, N1=8, N2=2, S1=256, S2=256, D=128, Dv=128, num_cus=256)
    base.update(kw)
    d = fb.make_desc(**base)
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws))
    if st == fb.FA_OK:
        lib.fa_bwd_destroy(h)
    else:
        assert not h.value
    return st, ws.value


def test_valid_problem_and_workspace_size(lib):
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # dS tiles: 2 bytes per (row, key) of each 128-row group by a band of
    # 32-key slices (all slices of the key sequence without a two-sided window)
    ds = lambda B, N1, S1, S2: B * N1 * ((S1 + 127) // 128) * 128 * ((S2 + 31) // 32) * 32 * 2  # noqa: E731
    # Enough key tiles x heads for every CU: sfmg and dS (dK/dV written by the
    # key-tile kernel, dQ by the GEMM over the stored dS).
    st, ws = create(lib, B=64, N1=8, N2=8, S1=256, S2=256)
    assert st == fb.FA_OK
    assert ws == rnd(64 * 8 * 256 * 4) + rnd(ds(64, 8, 256, 256))
    # A small GQA problem is split over query heads (4) and query ranges (4):
    # 16 fp32 partial sums of dK and of dV per key.
    st, ws = create(lib)
    assert st == fb.FA_OK
    lse, k_elems = 2 * 8 * 256, 2 * 256 * 2 * 128
    assert ws == rnd(lse * 4) + 2 * rnd(16 * k_elems * 4) + rnd(ds(2, 8, 256, 256))
    # ragged lengths round up to whole tiles
    st, ws = create(lib, B=64, N1=8, N2=8, S1=200, S2=300)
    assert st == fb.FA_OK and ws == rnd(64 * 8 * 200 * 4) + rnd(ds(64, 8, 200, 300))
    # a two-sided window bounds the band: ceil((128 + 100 + 20) / 32) + 1 = 9 slices
    st, ws = create(lib, B=4, N1=8, N2=8, S1=4096, S2=4096, mask_mode=2, win_left=100, win_right=20)
    assert st == fb.FA_OK and ws == rnd(4 * 8 * 4096 * 4) + rnd(4 * 32 * 8 * 9 * 8192)
    # causal with a left bound is a two-sided window too: ceil((128 + 1024) / 32) + 1 = 37
    st, ws = create(lib, B=1, N1=8, N2=8, S1=8192, S2=8192, mask_mode=1, win_left=1024)
    assert st == fb.FA_OK and ws == rnd(8 * 8192 * 4) + rnd(64 * 8 * 37 * 8192)
    # past 4 GiB of dS the run takes a chunk of KV heads at a time, in a
    # workspace of one chunk: 8 GiB of dS, 256 MiB per KV head -> 16 heads
    st, ws = create(lib, B=1, N1=32, N2=32, S1=16384, S2=8192)
    assert st == fb.FA_OK and ws == rnd(32 * 16384 * 4) + rnd(ds(1, 16, 16384, 8192))
    st, ws = create(lib, B=1, N1=32, N2=32, S1=8192, S2=8192)   # exactly 4 GiB: one pass
    assert st == fb.FA_OK and ws == rnd(32 * 8192 * 4) + rnd(ds(1, 32, 8192, 8192))
    # GQA: a chunk is whole KV heads (4 query heads each): 8 GiB -> 4 of 8 KV
    # heads; the job split is sized for the 4 heads of one launch (64 tiles x
    # 4 heads x 2 query-head slots = 512 jobs), so 2 partial sums of dK and dV
    st, ws = create(lib, B=1, N1=32, N2=8, S1=16384, S2=8192)
    kv = rnd(8192 * 8 * 128 * 4)
    assert st == fb.FA_OK and ws == rnd(32 * 16384 * 4) + 2 * 2 * kv + rnd(ds(1, 16, 16384, 8192))
    # one KV head past the cap (64 GiB of dS for its 8 query heads): the plan
    # recomputes S and dP for dQ and the workspace holds sfmg only
    st, ws = create(lib, B=1, N1=8, N2=1, S1=65536, S2=65536)
    assert st == fb.FA_OK and ws == rnd(8 * 65536 * 4)
    # the fp32 debugging form needs sfmg only
    st, ws = create(lib, flags=fb.FLAG_FP32_OUT)
    assert st == fb.FA_OK
    assert ws == rnd(lse * 4)
    # fp16 elements (the page's second binary) plan exactly like bf16
    assert create(lib, dtype=fb.DTYPE_FP16) == create(lib, dtype=fb.DTYPE_BF16)
    assert create(lib, dtype=fb.DTYPE_FP16, flags=fb.FLAG_FP32_OUT)[0] == fb.FA_OK


def dq_path(lib, **kw):
    base = dict(layout="BSND", B=2, N1=8, N2=2, S1=256, S2=256, D=128, Dv=128)
    base.update(kw)
    d = fb.make_desc(**base)
    h, ws, out = ctypes.c_void_p(), ctypes.c_size_t(), ctypes.c_int(-1)
    assert lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws)) == fb.FA_OK
    try:
        assert lib.fa_bwd_plan_dq_path(h, ctypes.byref(out)) == fb.FA_OK
    finally:
        lib.fa_bwd_destroy(h)
    return fb.DQ_PATHS[out.value]


def test_plan_dq_path(lib):
    assert dq_path(lib) == "stored_ds"
    assert dq_path(lib, layout="BNSD", mask_mode=1) == "stored_ds"
    assert dq_path(lib, flags=fb.FLAG_DETERMINISTIC) == "stored_ds"
    assert dq_path(lib, layout="TND", S1=256, S2=256, T1=1024, T2=1024) == "stored_ds"
    assert dq_path(lib, B=1, N1=32, N2=32, S1=16384, S2=8192) == "stored_ds"  # chunked
    assert dq_path(lib, B=1, N1=8, N2=1, S1=65536, S2=65536) == "recompute"  # one KV head past 4 GiB
    assert dq_path(lib, flags=fb.FLAG_FP32_OUT) == "fp32_form"
    # short key sequences: one launch per (sequence, KV head)
    assert dq_path(lib, S1=128, S2=128, D=64, Dv=64, B=1, N1=2, N2=2) == "fused"
    assert dq_path(lib, layout="TND", S1=64, S2=64, T1=256, T2=256) == "fused"
    assert dq_path(lib, S1=2048, S2=128, N1=2, N2=2) == "fused"             # 64 (head, block) items
    assert dq_path(lib, S1=2049, S2=128, N1=2, N2=2) == "stored_ds"         # 65
    assert dq_path(lib, S1=128, S2=129) == "stored_ds"                       # two key tiles
    assert dq_path(lib, S1=128, S2=128, D=192, Dv=128) == "stored_ds"        # not instantiated
    # explicit modes
    assert dq_path(lib, dq_mode="recompute") == "recompute"
    assert dq_path(lib, layout="TND", S1=64, S2=64, T1=256, T2=256, dq_mode="recompute") == "recompute"
    assert dq_path(lib, B=1, N1=8, N2=1, S1=65536, S2=65536, dq_mode="stored_ds") == "stored_ds"
    assert dq_path(lib, dq_mode="atomic") == "atomic"
    assert dq_path(lib, S1=128, S2=128, dq_mode="fused") == "fused"
    assert dq_path(lib, S1=256, S2=256, dq_mode="stored_ds") == "stored_ds"
    out = ctypes.c_int()
    assert lib.fa_bwd_plan_dq_path(None, ctypes.byref(out)) == fb.FA_ERR_NULLPTR


def test_dq_mode_rules(lib):
    """dq_mode, num_cus and the determinism flag are checked in fa_bwd_create."""
    assert create(lib, dq_mode=5)[0] == fb.FA_ERR_PARAM_INVALID                 # FP32_FORM is reported only
    assert create(lib, dq_mode=-1)[0] == fb.FA_ERR_PARAM_INVALID
    assert create(lib, dq_mode="atomic", flags=fb.FLAG_DETERMINISTIC)[0] == fb.FA_ERR_PARAM_INVALID
    assert create(lib, dq_mode="recompute", flags=fb.FLAG_FP32_OUT)[0] == fb.FA_ERR_PARAM_INVALID
    assert create(lib, dq_mode="atomic", dtype=fb.DTYPE_FP16)[0] == fb.FA_ERR_UNSUPPORTED
    assert create(lib, dq_mode="fused", S1=256, S2=256)[0] == fb.FA_ERR_UNSUPPORTED      # keys past one tile
    assert create(lib, dq_mode="fused", S1=4096, S2=128, N1=2, N2=2)[0] == fb.FA_ERR_UNSUPPORTED  # 128 items
    assert create(lib, dq_mode="fused", S1=128, S2=128, D=192, Dv=128)[0] == fb.FA_ERR_UNSUPPORTED
    assert create(lib, num_cus=-1)[0] == fb.FA_ERR_PARAM_INVALID
    for m in ("stored_ds", "recompute", "fused"):
        assert create(lib, dq_mode=m, flags=fb.FLAG_DETERMINISTIC, S1=128, S2=128)[0] == fb.FA_OK
    # the fused kernel needs no workspace at all
    assert create(lib, dq_mode="fused", S1=128, S2=128) == (fb.FA_OK, 0)


def test_atomic_mode_rejects_seqused_before_any_launch(lib):
    plan = fb.Plan(fb.make_desc("BSND", 1, 2, 2, 256, 256, 64, 64, dq_mode="atomic"))
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the check fails first
    args = [fake] * 6 + [None, None] + [fake, None] + [fake] * 3
    assert lib.fa_bwd_run(plan.handle, *args, fake, plan.workspace_bytes, None) == fb.FA_ERR_UNSUPPORTED
    args = [fake] * 6 + [None, None] + [None, fake] + [fake] * 3
    assert lib.fa_bwd_run(plan.handle, *args, fake, plan.workspace_bytes, None) == fb.FA_ERR_UNSUPPORTED


def test_job_split_follows_num_cus(lib):
    """The split targets two jobs per CU: more CUs, more partial sums."""
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    kw = dict(B=1, N1=32, N2=8, S1=4096, S2=4096, mask_mode=1)
    lse, kv = rnd(32 * 4096 * 4), rnd(4096 * 8 * 128 * 4)
    ds = rnd(32 * 32 * 128 * 8192)
    # 256 CUs: 32 tiles x 8 KV heads x 2 query-head slots = 512 jobs, 2 partials
    assert create(lib, num_cus=256, **kw) == (fb.FA_OK, lse + 2 * 2 * kv + ds)
    # 128 CUs: 32 x 8 = 256 jobs already, no split and no partials
    assert create(lib, num_cus=128, **kw) == (fb.FA_OK, lse + ds)
    # 1024 CUs: 4 query-head slots x 2 query splits = 8 partials
    assert create(lib, num_cus=1024, **kw) == (fb.FA_OK, lse + 2 * 8 * kv + ds)


def test_workspace_bound_chunks_kv_heads(lib):
    """max_workspace_bytes bounds the workspace: the dS chunk (whole KV heads)
    shrinks to fit, then the split partials; below one KV head's dS the plan
    recomputes S and dP for dQ (AUTO) or refuses (stored_ds forced)."""
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # B=2, N1=8, N2=2 (G=4), S=256: 4 groups x 8 slices x 8 KB per query head
    kw = dict(num_cus=256, S1=256, S2=256)
    per_q = 4 * 8 * 8192
    sf = rnd(2 * 8 * 256 * 4)
    kv = rnd(2 * 256 * 2 * 128 * 4)              # one fp32 copy of k (or v)
    # unbounded: both KV heads, 2 key tiles x 2 heads x 2 batches = 8 jobs -> 4 x 4 = 16 partials
    st, ws = create(lib, **kw)
    assert st == fb.FA_OK and ws == sf + 2 * 16 * kv + rnd(8 * per_q)
    assert dq_path(lib, **kw) == "stored_ds"
    # room for exactly one KV head's dS and nothing else: chunk of 1, no split
    st, ws = create(lib, max_workspace_bytes=sf + 4 * per_q, **kw)
    assert st == fb.FA_OK and ws == sf + 4 * per_q
    # room for both KV heads' dS: the chunk is filled first, the split gets the rest
    st, ws = create(lib, max_workspace_bytes=sf + 4 * per_q + 2 * 2 * kv, **kw)
    assert st == fb.FA_OK and ws == sf + 8 * per_q
    # both KV heads and two partial sums of dK and of dV (four do not fit)
    st, ws = create(lib, max_workspace_bytes=sf + 8 * per_q + 2 * 2 * kv, **kw)
    assert st == fb.FA_OK and ws == sf + 8 * per_q + 2 * 2 * kv
    # not one KV head: AUTO recomputes, with as many partials as fit
    st, ws = create(lib, max_workspace_bytes=sf + 4 * per_q - 1, **kw)
    assert st == fb.FA_OK and ws <= sf + 4 * per_q - 1
    assert dq_path(lib, max_workspace_bytes=sf + 4 * per_q - 1, **kw) == "recompute"
    assert create(lib, max_workspace_bytes=sf, **kw) == (fb.FA_OK, sf)   # sfmg only: no split
    assert create(lib, max_workspace_bytes=sf + 4 * per_q - 1, dq_mode="stored_ds", **kw)[0] == fb.FA_ERR_WORKSPACE
    assert create(lib, max_workspace_bytes=sf - 1, **kw)[0] == fb.FA_ERR_WORKSPACE
    assert create(lib, max_workspace_bytes=sf - 1, dq_mode="recompute", **kw)[0] == fb.FA_ERR_WORKSPACE
    # the atomic mode's fp32 dQ accumulator must fit too
    q_acc = rnd(2 * 256 * 8 * 128 * 4)
    assert create(lib, dq_mode="atomic", max_workspace_bytes=sf + q_acc - 1, **kw)[0] == fb.FA_ERR_WORKSPACE
    assert create(lib, dq_mode="fused", S1=128, S2=128, max_workspace_bytes=1)[0] == fb.FA_OK


def test_tnd_workspace_band(lib):
    """TND stores dS by 128-row group at index cu_q[b] / 128 + b + R, fewer
    than T1 / 128 + B + 1 groups, each with a band of 32-key slices."""
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    st, ws = create(lib, layout="TND", B=4, N1=8, N2=8, S1=1024, S2=1024, T1=4096, T2=4096)
    assert st == fb.FA_OK
    # sfmg, then 2 query-range partial sums of dK and dV (8 key tiles x 4
    # sequences x 8 heads x 2 splits reach 512 jobs), then dS: 37 groups x 8
    # heads x 32 slices (no window: every slice of the longest sequence)
    k_elems = 4096 * 8 * 128
    assert ws == rnd(8 * 4096 * 4) + 2 * rnd(2 * k_elems * 4) + rnd(37 * 8 * 32 * 8192)
    # the varlen workload's shape: 8 sequences, T = 16437, causal window 1024:
    # (128 + 8 + 1) groups x 16 heads x 37 slices, 0.66 GB instead of the
    # 4 GiB of a grid laid out by the longest sequence
    st, ws = create(lib, layout="TND", B=8, N1=16, N2=16, S1=3594, S2=3594, T1=16437, T2=16437,
                    mask_mode=1, win_left=1024)
    assert st == fb.FA_OK
    assert ws == rnd(16 * 16437 * 4) + rnd(137 * 16 * 37 * 8192)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), fb.FA_ERR_SHAPE),
    (dict(B=65536), fb.FA_ERR_SHAPE),
    (dict(N1=6, N2=4), fb.FA_ERR_SHAPE),            # N1 % N2
    (dict(N2=0), fb.FA_ERR_SHAPE),
    (dict(D=128, Dv=192), fb.FA_ERR_SHAPE),          # Dv <= D
    (dict(D=256, Dv=128), fb.FA_ERR_SHAPE),          # D <= 192
    (dict(S1=0), fb.FA_ERR_SHAPE),
    (dict(S1=2**29), fb.FA_ERR_SHAPE),               # index sums must fit 32 bits
    (dict(S2=2**29, N1=1, N2=1, D=64, Dv=64), fb.FA_ERR_SHAPE),
    (dict(mask_mode=0, win_left=5), fb.FA_ERR_SHAPE),  # dense needs no window
    (dict(mask_mode=1, win_right=3), fb.FA_ERR_SHAPE),
    (dict(mask_mode=2, win_left=-2), fb.FA_ERR_SHAPE),
    (dict(mask_mode=3), fb.FA_ERR_PARAM_INVALID),
    (dict(layout=3), fb.FA_ERR_PARAM_INVALID),
    (dict(dtype=2), fb.FA_ERR_PARAM_INVALID),
    (dict(flags=0x10), fb.FA_ERR_PARAM_INVALID),
    (dict(softmax_scale=float("nan")), fb.FA_ERR_PARAM_INVALID),
    (dict(D=96, Dv=96), fb.FA_ERR_UNSUPPORTED),      # head dim not instantiated
])
def test_create_rejects(lib, kw, code):
    assert create(lib, **kw)[0] == code


@pytest.mark.parametrize("kw", [
    dict(mask_mode=1), dict(mask_mode=1, win_left=1024, win_right=0), dict(mask_mode=2, win_left=3, win_right=7),
    dict(mask_mode="causal"), dict(mask_mode=fb.MaskMode.WINDOW, win_left=-1, win_right=-1),
    dict(D=192, Dv=128), dict(D=64, Dv=64), dict(N1=32, N2=8), dict(softmax_scale=0.25),
    dict(flags=fb.FLAG_DETERMINISTIC), dict(flags=fb.FLAG_FP32_OUT),
    dict(flags=fb.FLAG_FP32_OUT | fb.FLAG_DETERMINISTIC, D=192, Dv=128),
])
def test_create_accepts(lib, kw):
    assert create(lib, **kw)[0] == fb.FA_OK


def test_wide_windows_are_clamped_to_the_sequences(lib, monkeypatch, capfd):
    """A left bound past S2 (a right bound past S1) masks nothing that the
    sequence ends do not; the plan clamps it to that width, so a bound of
    2^31 - 1 cannot wrap the kernels' 32-bit sums i + (s2 - s1) + bound."""
    monkeypatch.setenv("FA_BWD_LOG", "1")
    big = 2**31 - 1
    assert create(lib, mask_mode=2, win_left=big, win_right=big, S1=200, S2=300)[0] == fb.FA_OK
    assert create(lib, mask_mode=1, win_left=big, S1=200, S2=300)[0] == fb.FA_OK
    assert create(lib, mask_mode=2, win_left=299, win_right=199, S1=200, S2=300)[0] == fb.FA_OK
    windows = re.findall(r"window=\((-?\d+),(-?\d+)\)", capfd.readouterr().err)
    assert windows == [("300", "200"), ("300", "0"), ("299", "199")]


def test_launch_order_fields_of_the_plan(lib, monkeypatch, capfd):
    """The stored-dS and recompute chains order the dK/dV grid for the
    dispatcher (engine reversal over rounds of one workgroup per CU) and take
    varlen grids sequence by sequence; the fused and atomic forms use neither."""
    monkeypatch.setenv("FA_BWD_LOG", "1")
    assert create(lib, mask_mode=1, num_cus=200)[0] == fb.FA_OK                      # dense, stored dS
    assert tnd_create(lib, [300, 500], [300, 500], mask_mode=1, num_cus=256) == fb.FA_OK  # varlen
    assert create(lib, S1=128, S2=128, mask_mode=1)[0] == fb.FA_OK                    # fused
    assert create(lib, mask_mode=1, dq_mode="atomic")[0] == fb.FA_OK                  # atomic
    logs = re.findall(r"variant=(\d+) .*dq_groups=(\d+) round_wgs=(\d+) seq_major=(\d+)", capfd.readouterr().err)
    assert [(int(v), int(r), int(m)) for v, _, r, m in logs] == [(4, 200, 0), (4, 256, 1), (5, 0, 0), (1, 0, 0)]


def test_abi_version_mismatch(lib):
    d = fb.make_desc("BSND", 1, 2, 2, 64, 64, 64, 64)
    d.abi_version = 7
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws)) == fb.FA_ERR_PARAM_INVALID


def test_null_pointers(lib):
    d = fb.make_desc("BSND", 1, 2, 2, 64, 64, 64, 64)
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.fa_bwd_create(None, ctypes.byref(h), ctypes.byref(ws)) == fb.FA_ERR_NULLPTR
    assert lib.fa_bwd_create(ctypes.byref(d), None, ctypes.byref(ws)) == fb.FA_ERR_NULLPTR
    assert lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), None) == fb.FA_ERR_NULLPTR
    assert lib.fa_bwd_destroy(None) == fb.FA_OK


def tnd_create(lib, lens_q, lens_kv, S1=-1, S2=-1, host=True, T1=None, T2=None, **kw):
    cq = [0]
    for x in lens_q:
        cq.append(cq[-1] + x)
    ck = [0]
    for x in lens_kv:
        ck.append(ck[-1] + x)
    aq = (ctypes.c_int32 * len(cq))(*cq)
    ak = (ctypes.c_int32 * len(ck))(*ck)
    d = fb.make_desc("TND", len(lens_q), 4, 2, S1, S2, 128, 128, cq[-1] if T1 is None else T1,
                     ck[-1] if T2 is None else T2, host_cu_q=aq if host else None, host_cu_kv=ak if host else None,
                     **kw)
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    st = lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws))
    if st == fb.FA_OK:
        lib.fa_bwd_destroy(h)
    return st


def test_tnd_rules(lib):
    assert tnd_create(lib, [5, 0, 9], [3, 4, 9]) == fb.FA_OK
    assert tnd_create(lib, [5, 0, 9], [3, 4, 9], S1=9, S2=9) == fb.FA_OK
    assert tnd_create(lib, [5, 0, 9], [3, 4, 9], S1=8, S2=9) == fb.FA_ERR_SHAPE   # max_seqlen too small
    assert tnd_create(lib, [5, 9], [3, 9], T1=15) == fb.FA_ERR_SHAPE              # cu[B] != T
    assert tnd_create(lib, [5, 9], [3, 9], host=False) == fb.FA_ERR_SHAPE         # no lengths at all
    assert tnd_create(lib, [5, 9], [3, 9], host=False, S1=9, S2=9) == fb.FA_OK
    # host cu_seqlens are refused for dense layouts
    aq = (ctypes.c_int32 * 2)(0, 4)
    d = fb.make_desc("BSND", 1, 2, 2, 4, 4, 64, 64, host_cu_q=aq, host_cu_kv=aq)
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws)) == fb.FA_ERR_SHAPE


def test_misaligned_pointers_rejected_before_any_device_call(lib):
    """Element tensors move in 16-byte pieces, float32 / int32 arrays in words:
    a misaligned pointer is FA_ERR_PARAM_INVALID from every run entry point,
    before anything is launched (the fake addresses are never dereferenced)."""
    plan = fb.Plan(fb.make_desc("BSND", 1, 2, 2, 64, 64, 64, 64, dq_mode="stored_ds"))
    fake, half = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)
    lse_odd = ctypes.c_void_p(0x1002)
    ws = plan.workspace_bytes
    none4 = [None] * 4  # cu_q cu_kv seqused_q seqused_kv
    for i in (0, 1, 2, 3, 4):  # q k v dout attn_out
        args = [fake] * 6
        args[i] = half
        assert lib.fa_bwd_run(plan.handle, *args, *none4, fake, fake, fake, fake, ws, None) == fb.FA_ERR_PARAM_INVALID
    for i in range(3):  # dq dk dv
        outs = [fake] * 3
        outs[i] = half
        assert lib.fa_bwd_run(plan.handle, *([fake] * 6), *none4, *outs, fake, ws, None) == fb.FA_ERR_PARAM_INVALID
        assert lib.fa_bwd_run_noalloc(plan.handle, *([fake] * 6), *none4, *outs, None) == fb.FA_ERR_PARAM_INVALID
    assert lib.fa_bwd_run(plan.handle, *([fake] * 5), lse_odd, *none4, fake, fake, fake, fake, ws,
                          None) == fb.FA_ERR_PARAM_INVALID
    assert lib.fa_fwd_run(plan.handle, half, fake, fake, None, None, None, None, fake, fake,
                          None) == fb.FA_ERR_PARAM_INVALID
    assert lib.fa_fwd_run(plan.handle, fake, fake, fake, None, None, None, None, fake, lse_odd,
                          None) == fb.FA_ERR_PARAM_INVALID
    assert lib.fa_bwd_sfmg(plan.handle, half, fake, None, fake, None) == fb.FA_ERR_PARAM_INVALID


def test_tnd_decreasing_cu_rejected(lib):
    aq = (ctypes.c_int32 * 3)(0, 6, 4)
    d = fb.make_desc("TND", 2, 2, 2, -1, -1, 64, 64, 4, 4, host_cu_q=aq, host_cu_kv=aq)
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.fa_bwd_create(ctypes.byref(d), ctypes.byref(h), ctypes.byref(ws)) == fb.FA_ERR_SHAPE


def test_run_checks_before_any_device_call(lib):
    plan = fb.Plan(fb.make_desc("BSND", 1, 2, 2, 64, 64, 64, 64, dq_mode="stored_ds"))
    assert plan.workspace_bytes > 0
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every check below fails first
    # q k v dout attn_out lse | cu_q cu_kv | seqused_q seqused_kv | dq dk dv
    args = [fake] * 6 + [None, None] + [None, None] + [fake] * 3
    st = lib.fa_bwd_run(plan.handle, *args, None, plan.workspace_bytes, None)
    assert st == fb.FA_ERR_WORKSPACE
    st = lib.fa_bwd_run(plan.handle, *args, fake, plan.workspace_bytes - 1, None)
    assert st == fb.FA_ERR_WORKSPACE
    st = lib.fa_bwd_run(plan.handle, *([fake] * 6), fake, fake, None, None, *([fake] * 3), fake,
                        plan.workspace_bytes, None)
    assert st == fb.FA_ERR_SHAPE   # cu_seqlens given for a dense layout
    st = lib.fa_bwd_run(plan.handle, None, *args[1:], fake, plan.workspace_bytes, None)
    assert st == fb.FA_ERR_NULLPTR
    assert lib.fa_bwd_run(None, *args, fake, plan.workspace_bytes, None) == fb.FA_ERR_NULLPTR
    st = lib.fa_fwd_run(plan.handle, fake, fake, fake, fake, None, None, None, fake, fake, None)
    assert st == fb.FA_ERR_SHAPE   # cu_seqlens given for a dense layout
    st = lib.fa_fwd_run(plan.handle, None, fake, fake, None, None, None, None, fake, fake, None)
    assert st == fb.FA_ERR_NULLPTR
    assert lib.fa_bwd_sfmg(plan.handle, None, fake, None, fake, None) == fb.FA_ERR_NULLPTR


def test_noalloc_refuses_plans_past_the_scratch(lib):
    """fa_bwd_run_noalloc checks the plan against the library's device scratch
    (FA_BWD_SCRATCH_BYTES) before anything touches a device."""
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every check below fails first
    args = [fake] * 6 + [None, None] + [None, None] + [fake] * 3
    big = fb.Plan(fb.make_desc("BSND", 1, 32, 8, 4096, 4096, 128, 128, mask_mode=1))
    assert big.workspace_bytes > fb.SCRATCH_BYTES
    assert lib.fa_bwd_run_noalloc(big.handle, *args, None) == fb.FA_ERR_WORKSPACE
    assert lib.fa_bwd_run_noalloc(None, *args, None) == fb.FA_ERR_NULLPTR
    # bounded by the scratch size, the same problem plans within it
    fit = fb.Plan(fb.make_desc("BSND", 1, 32, 8, 4096, 4096, 128, 128, mask_mode=1,
                               max_workspace_bytes=fb.SCRATCH_BYTES))
    assert 0 < fit.workspace_bytes <= fb.SCRATCH_BYTES
    st = lib.fa_bwd_run_noalloc(fit.handle, None, *args[1:], None)
    assert st == fb.FA_ERR_NULLPTR


def test_mask_mode_names():
    assert fb.mask_mode_value("Causal") == 1
    assert fb.mask_mode_value("window") == 2
    assert fb.mask_mode_value(fb.MaskMode.NONE) == 0
    with pytest.raises(ValueError):
        fb.mask_mode_value("diagonal")


def test_default_scale_is_reported_in_plan(lib):
    # scale 0 -> 1/sqrt(D) is a host decision; a plan must accept it
    assert create(lib, softmax_scale=0.0, D=192, Dv=128)[0] == fb.FA_OK
    assert math.isclose(1 / math.sqrt(192), 0.07216878364870322)


def test_binding_rejects_mixed_or_unknown_element_types():
    """q, k, v, dout and attn_out share one element type, bf16 or fp16; the
    binding checks this before any library call."""
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 8, 2, 64), dtype=torch.float16)
    kb = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    lse = torch.zeros((1, 2, 8), dtype=torch.float32)
    with pytest.raises(TypeError):
        fb.flash_attn_grad(q, kb, q, q, q, lse)
    q32 = q.float()
    with pytest.raises(TypeError):
        fb.flash_attn_grad(q32, q32, q32, q32, q32, lse)
