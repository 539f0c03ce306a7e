"""GPU forward (fa_fwd_run through the binding) against the fp64 oracle
forward: attn_out within the bf16 tolerance, softmax_lse to 1e-3 absolute,
and -inf exactly on rows that see no key."""

import numpy as np
import pytest

from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import assert_all_close, case_inputs, f64, max_lengths, say
import oracle

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": W.CONFIGS["tiny"],
    "bsnd_causal_gqa4_ragged": W.custom("BSND", B=1, N1=8, N2=2, S1=300, S2=300, D=128, Dv=128, mask_mode=1),
    "bnsd_causal_s1_gt_s2": W.custom("BNSD", B=2, N1=2, N2=2, S1=260, S2=100, D=128, Dv=128, mask_mode=1),
    "bsnd_window_d192_dv128": W.custom("BSND", B=1, N1=2, N2=1, S1=200, S2=230, D=192, Dv=128, mask_mode=2,
                                       win_left=40, win_right=9),
    "tnd_mixed": W.custom("TND", N1=4, N2=2, D=64, Dv=64, mask_mode=1, win_left=50,
                          lengths=[1, 0, 130, 257, 64], lengths_kv=[1, 5, 130, 200, 0]),
    "mha_causal": W.CONFIGS["mha_causal"],
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_parity(name):
    import torch
    import flashattention_backward_fa_amd as fa

    cfg = CASES[name]
    say(f"[forward] {name}")
    x = case_inputs(cfg, seed=sorted(CASES).index(name))
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
    out = f64(out.cpu())
    lse_g = lse_g.cpu().double().numpy()
    assert_all_close([(out, Y, "attn_out")])
    empty = ~np.isfinite(lse)
    assert np.array_equal(empty, ~np.isfinite(lse_g))
    assert np.all(lse_g[empty] == -np.inf)
    assert np.abs(lse_g[~empty] - lse[~empty]).max() <= 1e-3
