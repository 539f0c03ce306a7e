"""GPU parity of Floyd attention (page "CANN Floyd注意力梯度算子", section
功能说明 for the formulas, 约束说明 for the shapes, 调用示例 for the all-ones
example) through the C ABI of include/fa_floyd.h, against the fp64 oracle
(oracle/floyd.py) on the same seeded inputs.

The backward's inputs attention_in, softmax_max and softmax_sum come from the
oracle's forward (Y rounded to the element type, the statistics to float32),
never from the library.  Tolerances are those of the ordinary attention
backward: bf16 relative Frobenius 1e-2 and max |err| 2e-2 * max |ref|; fp16
2^3 tighter (1.25e-3, 2.5e-3), from the 8 against 11 significant bits of the
16-bit P and dS operands."""

import math
import os

import numpy as np
import pytest

from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import errors, f64, say
import oracle
import oracle.floyd as OF

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk1", "dv1", "dk2", "dv2")
INPUTS = ("query", "key1", "value1", "key2", "value2")
TOL = {"bf16": (1e-2, 2e-2), "fp16": (1.25e-3, 2.5e-3)}


def torch_dtype(kind):
    import torch

    return torch.float16 if kind == "fp16" else torch.bfloat16


def oracle_side(cfg, x, kind):
    """Oracle forward (for the backward's inputs) and backward, fp64."""
    q, k1, v1, k2, v2, dy = (f64(x[n]) for n in INPUTS + ("dy",))
    scale = OF.default_scale(cfg["D"])
    Y, mx, sm = OF.forward(q, k1, v1, k2, v2, scale, x["mask"])
    Yst = oracle.f16_round(Y) if kind == "fp16" else oracle.bf16_round(Y)
    mx32, sm32 = mx.astype(np.float32), sm.astype(np.float32)
    ref = OF.backward(q, k1, v1, k2, v2, dy, Yst, mx32.astype(np.float64), sm32.astype(np.float64), scale,
                      x["mask"])
    return Yst, mx32, sm32, ref


def gpu_backward(x, Yst, mx32, sm32, kind):
    import torch
    import flashattention_backward_fa_amd.floyd as fl

    dev = torch.device("cuda", 0)
    dt = torch_dtype(kind)
    t = [x[n].to(dev) for n in INPUTS + ("dy",)]
    y = torch.from_numpy(np.ascontiguousarray(Yst)).to(dt).to(dev)
    smax, ssum = torch.from_numpy(mx32).to(dev), torch.from_numpy(sm32).to(dev)
    mask = None if x["mask"] is None else torch.from_numpy(x["mask"]).to(dev)
    out = fl.floyd_attn_grad(*t[:5], t[5], mask, smax, ssum, y)
    torch.cuda.synchronize()
    for o in out:
        assert o.dtype == dt
    return [f64(o.cpu()) for o in out]


def check(got, ref, kind):
    rt, mt = TOL[kind]
    bad = []
    for g, r, name in zip(got, ref, NAMES):
        rel, mx = errors(g, r)
        say(f"    {name}: rel_fro={rel:.3e} max_abs_ratio={mx:.3e}")
        if not (rel <= rt and mx <= mt):
            bad.append(f"{name}: {rel:.3e} / {mx:.3e}")
    assert not bad, "; ".join(bad)


@pytest.mark.parametrize("name", ["floyd_small", "floyd_masked", "floyd_n48"])
def test_floyd_backward_parity(name):
    cfg = W.FLOYD_CONFIGS[name]
    say(f"[floyd] {name}: {cfg}")
    x = W.floyd_inputs(cfg)
    Yst, mx32, sm32, ref = oracle_side(cfg, x, "bf16")
    say(f"[floyd] {name}: launching")
    got = gpu_backward(x, Yst, mx32, sm32, "bf16")
    check(got, ref, "bf16")


def test_floyd_backward_fp16():
    cfg = W.FLOYD_CONFIGS["floyd_masked"]
    say("[floyd fp16] floyd_masked")
    x = W.floyd_inputs(cfg, dtype=torch_dtype("fp16"))
    Yst, mx32, sm32, ref = oracle_side(cfg, x, "fp16")
    got = gpu_backward(x, Yst, mx32, sm32, "fp16")
    check(got, ref, "fp16")


def test_floyd_masked_positions_get_exact_zeros():
    """A masked (n, k) position gets dK1 = dV1 = 0 exactly, and a wholly
    masked row n gets dQ = 0 for every m."""
    cfg = W.FLOYD_CONFIGS["floyd_masked"]
    x = W.floyd_inputs(cfg)
    Yst, mx32, sm32, _ = oracle_side(cfg, x, "bf16")
    dq, dk1, dv1, _, _ = gpu_backward(x, Yst, mx32, sm32, "bf16")
    m = x["mask"][:, 0, :, 0, :].astype(bool)            # [B, N, K]
    sel = np.broadcast_to(m[:, None, :, :], dk1.shape[:-1])
    assert not np.any(dk1[sel]) and not np.any(dv1[sel])
    for (b, n) in cfg["masked_rows"]:
        assert not np.any(dq[b, :, n])


@pytest.mark.parametrize("name", ["floyd_small", "floyd_masked", "floyd_n48"])
def test_floyd_forward_parity(name):
    """fa_floyd_fwd_run against the oracle forward: Y at the element type's
    tolerance, max within 1e-3, sum within 1e-3 relative, 8 equal copies,
    -inf / 0 on wholly masked rows."""
    import torch
    import flashattention_backward_fa_amd.floyd as fl

    cfg = W.FLOYD_CONFIGS[name]
    x = W.floyd_inputs(cfg)
    Y, mx, sm = OF.forward(*(f64(x[n]) for n in INPUTS), OF.default_scale(cfg["D"]), x["mask"])
    dev = torch.device("cuda", 0)
    mask = None if x["mask"] is None else torch.from_numpy(x["mask"]).to(dev)
    out, smax, ssum = fl.floyd_attn(*(x[n].to(dev) for n in INPUTS), mask)
    torch.cuda.synchronize()
    rel, mxr = errors(f64(out.cpu()), Y)
    say(f"[floyd fwd] {name}: Y rel_fro={rel:.3e} max_abs_ratio={mxr:.3e}")
    assert rel <= 1e-2 and mxr <= 2e-2
    gm, gs = smax.cpu().double().numpy(), ssum.cpu().double().numpy()
    assert np.array_equal(gm, np.repeat(gm[..., :1], 8, -1)) and np.array_equal(gs, np.repeat(gs[..., :1], 8, -1))
    dead = ~np.isfinite(mx)
    assert np.array_equal(dead, ~np.isfinite(gm))
    assert np.all(gs[dead] == 0)
    assert np.abs(gm[~dead] - mx[~dead]).max() <= 1e-3
    assert (np.abs(gs[~dead] - sm[~dead]) / sm[~dead]).max() <= 1e-3


def test_floyd_repeatable_and_chunking_invariant(monkeypatch):
    """Two runs are bitwise equal, and so is a run that takes the heads one
    group at a time (FA_FLOYD_CHUNK_BYTES=1: one (b, h) pair per group, so the
    mask's batch index and every tensor offset move with the group)."""
    cfg = W.FLOYD_CONFIGS["floyd_masked"]
    x = W.floyd_inputs(cfg)
    Yst, mx32, sm32, _ = oracle_side(cfg, x, "bf16")
    a = gpu_backward(x, Yst, mx32, sm32, "bf16")
    b = gpu_backward(x, Yst, mx32, sm32, "bf16")
    monkeypatch.setenv("FA_FLOYD_CHUNK_BYTES", "1")
    c = gpu_backward(x, Yst, mx32, sm32, "bf16")
    for u, v, w, name in zip(a, b, c, NAMES):
        assert np.array_equal(u, v), name
        assert np.array_equal(u, w), name


def test_floyd_page_example_closed_form():
    """The page's example (section 调用示例): B = 1, one head, S1 = S2 = S3 =
    256, D = 128, all inputs 1.0, mask all 0, softmaxMax = softmaxSum = 3.0,
    scaleValue = 1/sqrt(128).  Every output element equals its closed form
    (dV1 = M p, dV2 = N p, dK1 = scale M D p, dK2 = scale N D p,
    dQ = 2 scale K D p, p = exp(scale * 2D - 3) / 3), in bf16."""
    import torch
    import flashattention_backward_fa_amd.floyd as fl

    dev = torch.device("cuda", 0)
    B, H, N, M, K, D = 1, 1, 256, 256, 256, 128
    one = lambda *s: torch.ones(s, dtype=torch.bfloat16, device=dev)
    q, dy, y = one(B, H, N, M, D), one(B, H, N, M, D), one(B, H, N, M, D)
    k1, v1, k2, v2 = one(B, H, N, K, D), one(B, H, N, K, D), one(B, H, K, M, D), one(B, H, K, M, D)
    mask = torch.zeros((B, 1, N, 1, K), dtype=torch.uint8, device=dev)
    stat = torch.full((B, H, N, M, 8), 3.0, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(128)
    got = fl.floyd_attn_grad(q, k1, v1, k2, v2, dy, mask, stat, stat, y, scale_value=scale)
    torch.cuda.synchronize()
    p = math.exp(scale * 2 * D - 3.0) / 3.0
    want = [2 * scale * K * D * p, scale * M * D * p, M * p, scale * N * D * p, N * p]
    for g, w, name in zip(got, want, NAMES):
        a = g.double().cpu().numpy()
        err = np.abs(a - w).max() / w
        say(f"    {name}: closed form {w:.6e}, max rel err {err:.2e}")
        assert err <= 1e-2, name


def test_floyd_benchmark_workload_one_head():
    """The benchmark workload (B = 1, H = 8, N = M = K = 256, D = 128) in the
    launch configuration the benchmark times; the oracle's forward runs on
    every head (the backward's inputs) and its backward on head 5, whose five
    gradients are compared element by element (heads are independent)."""
    cfg = W.FLOYD_CONFIGS["floyd"]
    x = W.floyd_inputs(cfg)
    q, k1, v1, k2, v2, dy = (f64(x[n]) for n in INPUTS + ("dy",))
    scale = OF.default_scale(cfg["D"])
    say("[floyd] benchmark workload: oracle forward")
    Y, mx, sm = OF.forward(q, k1, v1, k2, v2, scale, None)
    Yst = oracle.bf16_round(Y)
    mx32, sm32 = mx.astype(np.float32), sm.astype(np.float32)
    say("[floyd] benchmark workload: backward")
    got = gpu_backward(x, Yst, mx32, sm32, "bf16")
    h = slice(5, 6)
    ref = OF.backward(q[:, h], k1[:, h], v1[:, h], k2[:, h], v2[:, h], dy[:, h], Yst[:, h],
                      mx32[:, h].astype(np.float64), sm32[:, h].astype(np.float64), scale, None)
    check([g[:, h] for g in got], ref, "bf16")
