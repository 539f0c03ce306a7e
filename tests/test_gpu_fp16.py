"""GPU parity of the fp16 element type.  Page "CANN ops-transformer
FlashAttnGrad 算子详解", section 五 5.4, registers the operator twice, for bf16
and for fp16 tensors with the same signature; here the same kernels run with
IEEE fp16 inputs, fp16 P and dS operands and fp16 outputs, against the fp64
oracle in stored mode with Y rounded to fp16.

Tolerance: fp16 keeps 11 significant bits (unit roundoff 2^-11 ~ 4.9e-4)
where bf16 keeps 8 (2^-8 ~ 3.9e-3), so the bf16 bounds (relative Frobenius
1e-2, max |err| 2e-2 * max |ref|) shrink by 2^3 to 1.25e-3 and 2.5e-3.  The
few dS elements that fall below fp16's normal range (2^-14) lose relative
accuracy but sit far below the outputs' scale."""

import numpy as np
import pytest

from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import (case_inputs, empty_rows, errors, f64, gpu_backward, max_lengths, oracle_backward,
                         oracle_inputs, say)
from test_gpu_parity import EDGE_CASES, pick, sample_rows
import oracle

pytestmark = pytest.mark.gpu

REL_FRO_TOL_FP16 = 1.25e-3
MAX_ABS_TOL_FP16 = 2.5e-3


def f16():
    import torch

    return torch.float16


def check(triples, rel_tol=REL_FRO_TOL_FP16, max_tol=MAX_ABS_TOL_FP16):
    bad = []
    for got, ref, name in triples:
        rel, mx = errors(got, ref)
        say(f"    {name}: rel_fro={rel:.3e} max_abs_ratio={mx:.3e}")
        if rel > rel_tol or mx > max_tol:
            bad.append(f"{name}: rel_fro {rel:.3e} (tol {rel_tol}), max_abs_ratio {mx:.3e} (tol {max_tol})")
    assert not bad, "; ".join(bad)


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_fp16_parity_full_output(name):
    import torch

    cfg = EDGE_CASES[name]
    say(f"[fp16] {name}: {cfg}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name), dtype=f16())
    Yst, lst = oracle_inputs(cfg, x, "fp16")
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    say(f"[fp16] {name}: launching")
    dq, dk, dv = gpu_backward(cfg, x, Yst, lst)
    check([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")])
    qe, ke = empty_rows(cfg, x, dq.shape, dk.shape)
    assert not np.any(dq[qe]) and not np.any(dk[ke]) and not np.any(dv[ke])


def test_fp16_outputs_are_fp16_and_repeatable():
    import torch
    import flashattention_backward_fa_amd as fa

    cfg = EDGE_CASES["bsnd_causal_gqa4_ragged"]
    x = case_inputs(cfg, seed=7, dtype=f16())
    Yst, lst = oracle_inputs(cfg, x, "fp16")
    dev = torch.device("cuda", 0)
    t = [x[n].to(dev) for n in ("q", "k", "v", "dout")]
    y = torch.from_numpy(np.ascontiguousarray(Yst)).to(torch.float16).to(dev)
    lse = torch.from_numpy(np.ascontiguousarray(lst, dtype=np.float32)).to(dev)
    kw = dict(mask_mode=cfg["mask_mode"], layout=cfg["layout"])
    a = fa.flash_attn_grad(*t, y, lse, **kw)
    b = fa.flash_attn_grad(*t, y, lse, **kw)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert u.dtype == torch.float16
        assert torch.equal(u, w)


def test_fp16_large_workload_sampled():
    """The GQA causal workload (S = 4096) in fp16, in the launch configuration
    of the benchmark, on rows the oracle evaluates one by one."""
    cfg = W.CONFIGS["gqa_causal"]
    x = W.make_inputs(cfg, dtype=f16())
    say("[fp16] gqa_causal: oracle forward")
    Yst, lst = oracle_inputs(cfg, x, "fp16")
    say("[fp16] gqa_causal: backward")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst)
    q_rows, kv_rows = sample_rows(cfg, x)
    rq, rk, rv = oracle.backward_rows(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), Yst, lst, q_rows,
                                      kv_rows, cfg["layout"], x["cu_q"], x["cu_kv"], cfg["softmax_scale"],
                                      cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    got_q = np.stack([pick(gq, cfg, x, b, n, i, "q") for (b, n, i) in q_rows])
    got_k = np.stack([pick(gk, cfg, x, b, n, j, "kv") for (b, n, j) in kv_rows])
    got_v = np.stack([pick(gv, cfg, x, b, n, j, "kv") for (b, n, j) in kv_rows])
    check([(got_q, np.stack(rq), "dq (sampled rows)"), (got_k, np.stack(rk), "dk (sampled rows)"),
           (got_v, np.stack(rv), "dv (sampled rows)")])


@pytest.mark.parametrize("name", ["tiny", "bnsd_causal_s1_gt_s2", "tnd_mixed"])
def test_fp16_forward_parity(name):
    import torch
    import flashattention_backward_fa_amd as fa
    from test_gpu_forward import CASES

    cfg = CASES[name]
    say(f"[fp16 forward] {name}")
    x = case_inputs(cfg, seed=sorted(CASES).index(name), dtype=f16())
    Y, lse = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), cfg["layout"], x["cu_q"], x["cu_kv"],
                            cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    dev = torch.device("cuda", 0)
    cu_q = cu_kv = None
    if cfg["layout"] == "TND":
        cu_q, cu_kv = torch.from_numpy(x["cu_q"]).to(dev), torch.from_numpy(x["cu_kv"]).to(dev)
    mq, mk = max_lengths(cfg, x)
    out, lse_g = fa.flash_attn(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), cu_q, cu_kv, cfg["softmax_scale"],
                               cfg["mask_mode"], cfg["win_left"], cfg["win_right"], mq, mk, cfg["layout"])
    torch.cuda.synchronize()
    assert out.dtype == torch.float16
    check([(f64(out.cpu()), Y, "attn_out")])
    lse_g = lse_g.cpu().double().numpy()
    empty = ~np.isfinite(lse)
    assert np.array_equal(empty, ~np.isfinite(lse_g))
    assert np.abs(lse_g[~empty] - lse[~empty]).max() <= 1e-3


@pytest.mark.parametrize("name", ["bsnd_causal_gqa4_ragged", "tnd_mixed_lengths", "bsnd_d192_dv64_window"])
def test_fp16_inputs_fp32_debug_form(name):
    """fp16 inputs through the fp32 debugging form: fp32 outputs at the fp32
    form's bound (relative Frobenius 1e-4, max |err| 1e-3 * max |ref|)."""
    cfg = EDGE_CASES[name]
    say(f"[fp16 -> fp32] {name}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name), dtype=f16())
    Yst, lst = oracle_inputs(cfg, x, "fp16")
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    dq, dk, dv = gpu_backward(cfg, x, Yst, lst, fp32_out=True)
    check([(dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")], rel_tol=1e-4, max_tol=1e-3)


@pytest.mark.parametrize("name", ["bsnd_causal_gqa4_ragged", "tnd_mixed_lengths", "bnsd_batch3_causal"])
def test_fp16_sfmg_preprocess(name):
    """The standalone preprocess (fa_bwd_sfmg) on fp16 dout / attn_out:
    rowsum(dY * Y) in fp32, to 1e-5 of the sum of absolute products."""
    import torch
    import flashattention_backward_fa_amd as fa

    cfg = EDGE_CASES[name]
    x = case_inputs(cfg, seed=3, dtype=f16())
    Yst, _ = oracle_inputs(cfg, x, "fp16")
    dev = torch.device("cuda", 0)
    cu = torch.from_numpy(x["cu_q"]).to(dev) if cfg["layout"] == "TND" else None
    mq, _ = max_lengths(cfg, x)
    y = torch.from_numpy(np.ascontiguousarray(Yst)).to(torch.float16).to(dev)
    got = fa.sfmg(x["dout"].to(dev), y, cfg["layout"], cu, max_seqlen_q=mq).cpu().double().numpy()
    ref = oracle.sfmg(f64(x["dout"]), Yst, cfg["layout"], x["cu_q"])
    bound = 1e-5 * oracle.sfmg(np.abs(f64(x["dout"])), np.abs(Yst), cfg["layout"], x["cu_q"]) + 1e-30
    assert np.all(np.abs(got - ref) <= bound)
