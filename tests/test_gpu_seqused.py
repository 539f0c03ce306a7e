"""GPU parity with seqused_q / seqused_kv (page "CANN ops-transformer
FlashAttnGrad 算子详解", section 二 2.1 names these optional inputs only).
Reading: of sequence b only the first seqused[b] query rows / keys take part
(clamped to the sequence's length), masks align on the used lengths, and the
gradients of the padding rows are zero.  The oracle follows the same reading
(pinned against the unpadded problem on the CPU); here the library's outputs
are compared with it element by element, at the tolerance of the element type,
and the padding rows must be exact zeros."""

import numpy as np
import pytest

from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import assert_all_close, case_inputs, errors, f64, gpu_backward, max_lengths, say
import oracle

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, seqused_q, seqused_kv)
    "bsnd_gqa_causal": (W.custom("BSND", B=3, N1=8, N2=2, S1=300, S2=300, D=128, Dv=128, mask_mode=1),
                        [300, 131, 0], [250, 300, 77]),
    "bnsd_dense_clamped": (W.custom("BNSD", B=2, N1=2, N2=2, S1=200, S2=333, D=64, Dv=64, softmax_scale=0.2),
                           [500, 64], [1, 333]),
    "tnd_window": (W.custom("TND", N1=4, N2=2, D=128, Dv=128, mask_mode=2, win_left=40, win_right=7,
                            lengths=[200, 129, 64], lengths_kv=[180, 300, 64]), [150, 129, 1], [180, 10, 64]),
    "bsnd_d192_causal_left": (W.custom("BSND", B=2, N1=2, N2=1, S1=260, S2=140, D=192, Dv=128, mask_mode=1,
                                       win_left=50), [259, 33], [140, 90]),
    "kv_only": (W.custom("BSND", B=2, N1=4, N2=4, S1=129, S2=257, D=128, Dv=64, mask_mode=1), None, [200, 128]),
    # short keys: the plan takes the fused one-launch kernel
    "fused_d64": (W.custom("BSND", B=3, N1=4, N2=2, S1=100, S2=128, D=64, Dv=64, mask_mode=1),
                  [100, 37, 0], [128, 90, 5]),
}


def seq_lengths(cfg, x):
    if cfg["layout"] == "TND":
        return list(np.diff(x["cu_q"])), list(np.diff(x["cu_kv"]))
    return [cfg["S1"]] * cfg["B"], [cfg["S2"]] * cfg["B"]


def padding_masks(cfg, x, q_shape, k_shape, uq, ukv):
    """Boolean arrays over the row axes of q and k: True on padding rows."""
    lq, lk = seq_lengths(cfg, x)
    uq = lq if uq is None else uq
    ukv = lk if ukv is None else ukv
    qp = np.zeros(q_shape[:-1], dtype=bool)
    kp = np.zeros(k_shape[:-1], dtype=bool)
    for b in range(len(lq)):
        u1, u2 = min(max(uq[b], 0), lq[b]), min(max(ukv[b], 0), lk[b])
        if cfg["layout"] == "TND":
            qp[x["cu_q"][b] + u1:x["cu_q"][b + 1]] = True
            kp[x["cu_kv"][b] + u2:x["cu_kv"][b + 1]] = True
        elif cfg["layout"] == "BSND":
            qp[b, u1:] = True
            kp[b, u2:] = True
        else:
            qp[b, :, u1:] = True
            kp[b, :, u2:] = True
    return qp, kp


def run_case(name, dtype=None, store="bf16", tol=None, **extra):
    import torch

    if name.startswith("fused"):
        extra.setdefault("dq_mode", "fused")

    cfg, uq, ukv = CASES[name]
    x = case_inputs(cfg, seed=sorted(CASES).index(name), dtype=dtype)
    args = (cfg["layout"], x["cu_q"], x["cu_kv"], cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"],
            cfg["win_right"])
    used = dict(seqused_q=None if uq is None else np.array(uq), seqused_kv=None if ukv is None else np.array(ukv))
    q, k, v, dy = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"])
    Y, lse = oracle.forward(q, k, v, *args, **used)
    Yst, lst = oracle.store(Y, lse, store)
    rq, rk, rv = oracle.backward(q, k, v, dy, Yst, lst, *args, **used)
    dev = torch.device("cuda", 0)
    tens = {n: (None if u is None else torch.tensor(u, dtype=torch.int32, device=dev)) for n, u in used.items()}
    say(f"[seqused] {name}: launching")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, **tens, **extra)
    if tol is None:
        assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    else:
        for got, ref, nm in ((gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")):
            rel, mx = errors(got, ref)
            say(f"    {nm}: rel_fro={rel:.3e} max_abs_ratio={mx:.3e}")
            assert rel <= tol[0] and mx <= tol[1], nm
    qp, kp = padding_masks(cfg, x, gq.shape, gk.shape, uq, ukv)
    assert not np.any(gq[qp]) and not np.any(gk[kp]) and not np.any(gv[kp])


@pytest.mark.parametrize("name", sorted(CASES))
def test_seqused_parity(name):
    run_case(name)


@pytest.mark.parametrize("name", ["bsnd_gqa_causal", "fused_d64"])
def test_seqused_fp16(name):
    import torch

    run_case(name, dtype=torch.float16, store="fp16", tol=(1.25e-3, 2.5e-3))


def test_seqused_fp32_debug_form():
    run_case("tnd_window", tol=(1e-4, 1e-3), fp32_out=True)


@pytest.mark.parametrize("name", ["bsnd_gqa_causal", "tnd_window"])
def test_seqused_forward(name):
    """fa_fwd_run with seqused: used rows match the oracle forward, padding rows
    get attn_out = 0 and softmax_lse = -inf."""
    import torch
    import flashattention_backward_fa_amd as fa

    cfg, uq, ukv = CASES[name]
    x = case_inputs(cfg, seed=11)
    dev = torch.device("cuda", 0)
    used = dict(seqused_q=np.array(uq), seqused_kv=np.array(ukv))
    Y, lse = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), cfg["layout"], x["cu_q"], x["cu_kv"],
                            cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"], cfg["win_right"], **used)
    cu_q = cu_kv = None
    if cfg["layout"] == "TND":
        cu_q, cu_kv = torch.from_numpy(x["cu_q"]).to(dev), torch.from_numpy(x["cu_kv"]).to(dev)
    mq, mk = max_lengths(cfg, x)
    out, lse_g = fa.flash_attn(x["q"].to(dev), x["k"].to(dev), x["v"].to(dev), cu_q, cu_kv, cfg["softmax_scale"],
                               cfg["mask_mode"], cfg["win_left"], cfg["win_right"], mq, mk, cfg["layout"],
                               seqused_q=torch.tensor(uq, dtype=torch.int32, device=dev),
                               seqused_kv=torch.tensor(ukv, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert_all_close([(f64(out.cpu()), Y, "attn_out")])
    lse_g = lse_g.cpu().double().numpy()
    empty = ~np.isfinite(lse)
    assert np.array_equal(empty, ~np.isfinite(lse_g))
    assert np.abs(lse_g[~empty] - lse[~empty]).max() <= 1e-3
