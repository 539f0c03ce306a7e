"""GPU parity of the fp32 debugging form (FA_FLAG_FP32_OUT): float32 dq, dk,
dv with P and dS kept in fp32, against the stored-mode fp64 oracle.

Tolerance: relative Frobenius error <= 1e-4 per output tensor (the stated
bound of the fp32 form), and max |err| <= 1e-3 * max |ref|.  With fp32
products the error comes from fp32 rounding of the dot products and of the
sums over keys or query rows (a few ulp of 2^-24 times the length), far
below both."""

import numpy as np
import pytest

from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import case_inputs, empty_rows, errors, gpu_backward, oracle_backward, oracle_inputs, say
from test_gpu_parity import EDGE_CASES

pytestmark = pytest.mark.gpu

REL_FRO_TOL_FP32 = 1e-4
MAX_ABS_TOL_FP32 = 1e-3

CASES = dict(EDGE_CASES)
CASES["bsnd_causal_gqa4_s1024"] = W.custom("BSND", B=1, N1=8, N2=2, S1=1024, S2=1024, D=128, Dv=128, mask_mode=1)


def check(triples):
    bad = []
    for got, ref, name in triples:
        rel, mx = errors(got, ref)
        say(f"    {name}: rel_fro={rel:.3e} max_abs_ratio={mx:.3e}")
        if rel > REL_FRO_TOL_FP32 or mx > MAX_ABS_TOL_FP32:
            bad.append(f"{name}: rel_fro {rel:.3e}, max_abs_ratio {mx:.3e}")
    assert not bad, "; ".join(bad)


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp32_debug_parity(name):
    cfg = CASES[name]
    say(f"[fp32] {name}: {cfg}")
    seed = sorted(EDGE_CASES).index(name) if name in EDGE_CASES else 99
    x = case_inputs(cfg, seed=seed)
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    say(f"[fp32] {name}: launching")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, fp32_out=True)
    check([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    qe, ke = empty_rows(cfg, x, gq.shape, gk.shape)
    assert not np.any(gq[qe]) and not np.any(gk[ke]) and not np.any(gv[ke])


def test_fp32_debug_is_closer_than_bf16():
    """The fp32 form removes the bf16 roundings of P, dS and the outputs, so
    its error is orders of magnitude below the default path's."""
    cfg = EDGE_CASES["bsnd_causal_gqa4_ragged"]
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index("bsnd_causal_gqa4_ragged"))
    Yst, lst = oracle_inputs(cfg, x)
    ref = oracle_backward(cfg, x, Yst, lst)
    f32 = gpu_backward(cfg, x, Yst, lst, fp32_out=True)
    b16 = gpu_backward(cfg, x, Yst, lst)
    for a, b, r in zip(f32, b16, ref):
        assert errors(a, r)[0] * 20 < errors(b, r)[0]
