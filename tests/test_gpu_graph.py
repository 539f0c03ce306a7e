"""The backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.
Every launch fa_bwd_run and fa_bwd_run_noalloc make is capturable: kernels
only, no memset nodes, no allocation, no host synchronisation.  Before each
of three replays the inputs change in place and the outputs are overwritten
by eager work; after it the outputs must equal, bit for bit, the eager
backward on the same inputs.  Cases: the stored-dS chain with a split key
tile (fp32 partial sums and their reduce), the fused one-launch kernel, and
the entry point that allocates nothing (its scratch address is fixed when
the graph is captured)."""

import ctypes

import numpy as np
import pytest

from flashattention_backward_fa_amd import fa_bwd as fb
from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import case_inputs, say

pytestmark = pytest.mark.gpu

CASES = {
    "stored_ds_split": (W.custom("BSND", B=1, N1=8, N2=2, S1=300, S2=300, D=128, Dv=128, mask_mode=1),
                        dict(dq_mode="stored_ds", max_workspace_bytes=0), False),
    "fused": (W.custom("BSND", B=2, N1=4, N2=2, S1=128, S2=128, D=64, Dv=64, mask_mode=0),
              dict(dq_mode="fused", max_workspace_bytes=0), False),
    "noalloc": (W.custom("BSND", B=1, N1=8, N2=2, S1=512, S2=512, D=128, Dv=128, mask_mode=1),
                dict(dq_mode="auto", max_workspace_bytes=fb.SCRATCH_BYTES), True),
}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    import torch
    import flashattention_backward_fa_amd as fa

    cfg, mode, noalloc = CASES[name]
    dev = torch.device("cuda", 0)
    x = case_inputs(cfg, seed=11)
    q, k, v, dout = (x[n].to(dev) for n in ("q", "k", "v", "dout"))
    kw = dict(mask_mode=cfg["mask_mode"], win_left=cfg["win_left"], win_right=cfg["win_right"], layout=cfg["layout"])
    out, lse = fa.flash_attn(q, k, v, **kw)
    kw.update(mode)
    base = dout.clone()
    if noalloc:
        lib = fb.load_library()
        plan = fb.get_plan(q, k, v, cfg["layout"], None, None, 0.0, cfg["mask_mode"], cfg["win_left"],
                           cfg["win_right"], -1, -1, dq_mode=mode["dq_mode"],
                           max_workspace_bytes=mode["max_workspace_bytes"])
        assert 0 < plan.workspace_bytes <= fb.SCRATCH_BYTES
        outs = [torch.empty_like(t) for t in (q, k, v)]
        ins = [_ptr(t) for t in (q, k, v, dout, out, lse)] + [None] * 4

        def call():
            s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            st = lib.fa_bwd_run_noalloc(plan.handle, *ins, *[_ptr(t) for t in outs], s)
            assert st == fb.FA_OK, fb.strerror(st)
    else:
        prep = fa.prepare_grad(q, k, v, dout, out, lse, **kw)
        outs = prep.outputs
        plan = prep.plan
        call = prep
    say(f"[graph] {name}: path {plan.dq_path()}")
    call()  # once eagerly, so that nothing is first done inside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        dout.copy_(base * (0.5 + r))
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = fa.flash_attn_grad(q, k, v, dout, out, lse, **kw)
        torch.cuda.synchronize()
        for nm, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(a.float()).all(), f"{name} replay {r}: {nm} not fully written"
            assert torch.equal(a, b), f"{name} replay {r}: {nm} differs from the eager backward"
    del g
