"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (bf16 outputs, per tensor, against the stored-mode oracle):
relative Frobenius error <= 1e-2 and max |err| <= 2e-2 * max |ref|.
Every test compares every element of dq, dk and dv: the small edge cases,
and the four large workloads at their full sizes in the launch configuration
the benchmark times (the plan's own dQ mode) and through the recompute mode;
the large workloads also check the sfmg preprocess on every row and, as a
second, independent route, sampled rows that the oracle evaluates one by
one (backward_rows)."""

import math

import numpy as np
import pytest

import oracle
from flashattention_backward_fa_amd import workloads as W

from gpu_helpers import (assert_all_close, case_inputs, empty_rows, f64, gpu_backward, oracle_backward, oracle_inputs, say,
                         max_lengths)

pytestmark = pytest.mark.gpu

EDGE_CASES = {
    "tiny_full": W.CONFIGS["tiny"],
    "bsnd_causal_gqa4_ragged": W.custom("BSND", B=1, N1=8, N2=2, S1=300, S2=300, D=128, Dv=128, mask_mode=1),
    "bsnd_dense_ragged_d64": W.custom("BSND", B=2, N1=2, N2=2, S1=200, S2=333, D=64, Dv=64, softmax_scale=0.2),
    "bnsd_causal_s1_lt_s2_d192": W.custom("BNSD", B=1, N1=2, N2=1, S1=100, S2=260, D=192, Dv=128, mask_mode=1),
    "bnsd_causal_s1_gt_s2_empty_rows": W.custom("BNSD", B=1, N1=2, N2=2, S1=260, S2=100, D=128, Dv=128, mask_mode=1),
    "bsnd_window_37_11": W.custom("BSND", B=1, N1=4, N2=2, S1=250, S2=250, D=128, Dv=128, mask_mode=2,
                                  win_left=37, win_right=11),
    "bsnd_causal_left70": W.custom("BSND", B=1, N1=2, N2=2, S1=333, S2=333, D=128, Dv=128, mask_mode=1,
                                   win_left=70, win_right=0),
    "tnd_mixed_lengths": W.custom("TND", N1=4, N2=2, D=128, Dv=128, mask_mode=1, lengths=[1, 0, 130, 257, 64],
                                  lengths_kv=[1, 5, 130, 200, 0]),
    "tnd_window_dense_heads": W.custom("TND", N1=2, N2=2, D=64, Dv=64, mask_mode=2, win_left=20, win_right=5,
                                       lengths=[77, 128, 3], lengths_kv=[77, 128, 3]),
    "bsnd_gqa8_dv64": W.custom("BSND", B=1, N1=8, N2=1, S1=192, S2=192, D=128, Dv=64, mask_mode=0,
                               softmax_scale=0.05),
    "bsnd_d192_dv64_window": W.custom("BSND", B=1, N1=2, N2=1, S1=160, S2=140, D=192, Dv=64, mask_mode=2,
                                      win_left=-1, win_right=30),
    "bnsd_batch3_causal": W.custom("BNSD", B=3, N1=4, N2=4, S1=129, S2=129, D=64, Dv=64, mask_mode=1),
}


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_parity_full_output(name):
    cfg = EDGE_CASES[name]
    say(f"[parity] {name}: {cfg}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    say(f"[parity] {name}: launching")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    # rows that must vanish (no visible key / no attending query) are exact zeros
    qe, ke = empty_rows(cfg, x, gq.shape, gk.shape)
    assert not np.any(gq[qe]) and not np.any(gk[ke]) and not np.any(gv[ke])
    assert not np.any(rq[qe]) and not np.any(rk[ke])


def test_zero_upstream_gradient_gives_exact_zeros():
    cfg = W.custom("BSND", B=1, N1=4, N2=2, S1=150, S2=150, D=128, Dv=128, mask_mode=1)
    x = case_inputs(cfg, 3)
    x["dout"].zero_()
    Yst, lst = oracle_inputs(cfg, x)
    say("[parity] zero dout")
    for g in gpu_backward(cfg, x, Yst, lst):
        assert not np.any(g)


def test_windows_wider_than_the_sequences_mask_nothing_more():
    """Bounds of 2^31 - 1 act as the sequence widths (the plan clamps them,
    so no 32-bit index sum wraps): bitwise equal to an unbounded left side
    under causal, and the oracle's results under a two-sided window."""
    big = 2**31 - 1
    cfg = W.custom("BSND", B=1, N1=4, N2=2, S1=260, S2=300, D=128, Dv=128, mask_mode=1)
    x = case_inputs(cfg, 5)
    Yst, lst = oracle_inputs(cfg, x)
    say("[parity] causal, left bound 2^31 - 1")
    a = gpu_backward(cfg, x, Yst, lst)
    b = gpu_backward(dict(cfg, win_left=big), x, Yst, lst)
    assert all(np.array_equal(u, w) for u, w in zip(a, b))
    for cfg in (W.custom("BSND", B=1, N1=4, N2=2, S1=260, S2=300, D=128, Dv=128, mask_mode=2, win_left=big,
                         win_right=big),
                W.custom("TND", N1=2, N2=2, D=64, Dv=64, mask_mode=2, win_left=big, win_right=big,
                         lengths=[77, 128, 3], lengths_kv=[90, 40, 3])):
        x = case_inputs(cfg, 6)
        Yst, lst = oracle_inputs(cfg, x)
        rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
        say(f"[parity] window 2^31 - 1 both sides: {cfg['layout']}")
        gq, gk, gv = gpu_backward(cfg, x, Yst, lst)
        assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])


def _metamorphic_inputs():
    cfg = W.custom("BSND", B=1, N1=4, N2=2, S1=200, S2=200, D=128, Dv=128, mask_mode=1)
    x = case_inputs(cfg, 4)
    Yst, lst = oracle_inputs(cfg, x)
    return cfg, x, Yst, lst


def test_doubling_dout_doubles_outputs_bitwise():
    cfg, x, Yst, lst = _metamorphic_inputs()
    say("[meta] dout x2")
    g1 = gpu_backward(cfg, x, Yst, lst)
    x2 = dict(x, dout=x["dout"] * 2)
    g2 = gpu_backward(cfg, x2, Yst, lst)
    assert np.array_equal(2 * g1[1], g2[1]) and np.array_equal(2 * g1[2], g2[2])
    assert np.array_equal(2 * g1[0], g2[0])  # no atomics: dq doubles bitwise too


def test_default_scale_equals_explicit_scale_bitwise():
    cfg, x, Yst, lst = _metamorphic_inputs()
    cfg0 = dict(cfg, softmax_scale=0.0)
    cfg1 = dict(cfg, softmax_scale=1 / math.sqrt(128))
    say("[meta] scale 0 vs 1/sqrt(D)")
    a = gpu_backward(cfg0, x, Yst, lst)
    b = gpu_backward(cfg1, x, Yst, lst)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_layouts_agree_bitwise_on_dk_dv():
    import torch
    cfg, x, Yst, lst = _metamorphic_inputs()
    say("[meta] BSND vs BNSD vs TND")
    g_bsnd = gpu_backward(cfg, x, Yst, lst)
    tr = lambda t: t.transpose(1, 2).contiguous()  # noqa: E731
    xb = dict(x, q=tr(x["q"]), k=tr(x["k"]), v=tr(x["v"]), dout=tr(x["dout"]))
    g_bnsd = gpu_backward(dict(cfg, layout="BNSD"), xb, np.ascontiguousarray(Yst.transpose(0, 2, 1, 3)), lst)
    for a, b in zip(g_bsnd[1:], g_bnsd[1:]):
        assert np.array_equal(a, b.transpose(0, 2, 1, 3))
    cu = np.array([0, 200], dtype=np.int32)
    xt = dict(x, q=x["q"][0], k=x["k"][0], v=x["v"][0], dout=x["dout"][0], cu_q=cu, cu_kv=cu.copy())
    g_tnd = gpu_backward(dict(cfg, layout="TND", lengths=[200]), xt, Yst[0], lst[0])
    for a, b in zip(g_bsnd[1:], g_tnd[1:]):
        assert np.array_equal(a[0], b)
    del torch


# ------------------------------------------------------------------ large workloads

_cache = {}


def big(name, with_ref=True):
    """Inputs, the oracle forward's stored Y / lse and (with_ref) the oracle's
    whole backward of a named workload; one workload is cached at a time."""
    if name not in _cache:
        cfg = W.CONFIGS[name]
        x = W.make_inputs(cfg)
        say(f"[parity] {name}: oracle forward")
        Yst, lst = oracle_inputs(cfg, x)
        _cache.clear()
        _cache[name] = {"cfg": cfg, "x": x, "Yst": Yst, "lst": lst, "ref": None}
    c = _cache[name]
    if with_ref and c["ref"] is None:
        say(f"[parity] {name}: oracle backward (whole tensors)")
        c["ref"] = oracle_backward(c["cfg"], c["x"], c["Yst"], c["lst"])
    return c


def sample_rows(cfg, x, n=40, seed=0):
    rng = np.random.default_rng(seed)
    if cfg["layout"] == "TND":
        lq, lk = np.diff(x["cu_q"]), np.diff(x["cu_kv"])
    else:
        lq, lk = [cfg["S1"]] * cfg["B"], [cfg["S2"]] * cfg["B"]
    B = len(lq)
    q_rows, kv_rows = [], []
    for t in range(n):
        b = int(rng.integers(B))
        picks_q = [0, int(lq[b]) - 1, 63, 64, 127, 128] + [int(rng.integers(lq[b]))]
        picks_k = [0, int(lk[b]) - 1, 127, 128] + [int(rng.integers(lk[b]))]
        q_rows.append((b, int(rng.integers(cfg["N1"])), min(picks_q[t % len(picks_q)], int(lq[b]) - 1)))
        kv_rows.append((b, int(rng.integers(cfg["N2"])), min(picks_k[t % len(picks_k)], int(lk[b]) - 1)))
    return q_rows, kv_rows


def pick(arr, cfg, x, b, n, i, kind):
    L = cfg["layout"]
    if L == "TND":
        cu = x["cu_q"] if kind == "q" else x["cu_kv"]
        return arr[cu[b] + i, n]
    if L == "BSND":
        return arr[b, i, n]
    return arr[b, n, i]


LARGE = ["mha_causal", "gqa_causal", "varlen_window", "wide_qk"]


def test_sfmg_preprocess_large_workloads():
    """The preprocess kernel alone, every row of each large workload."""
    import torch
    import flashattention_backward_fa_amd as fa
    dev = torch.device("cuda", 0)
    for name in LARGE:
        c = big(name, with_ref=False)
        cfg, x, Yst = c["cfg"], c["x"], c["Yst"]
        say(f"[parity] {name}: sfmg preprocess")
        cu = torch.from_numpy(x["cu_q"]).to(dev) if cfg["layout"] == "TND" else None
        mq, _ = max_lengths(cfg, x)
        attn_out = torch.from_numpy(Yst).to(torch.bfloat16).to(dev)
        s_gpu = fa.sfmg(x["dout"].to(dev), attn_out, cfg["layout"], cu, max_seqlen_q=mq).cpu().double().numpy()
        s_ref = oracle.sfmg(f64(x["dout"]), Yst, cfg["layout"], x["cu_q"])
        bound = 1e-5 * oracle.sfmg(np.abs(f64(x["dout"])), np.abs(Yst), cfg["layout"], x["cu_q"]) + 1e-30
        assert np.all(np.abs(s_gpu - s_ref) <= bound)


@pytest.mark.parametrize("Dv,N1,T", [(128, 16, 1000), (128, 32, 77), (64, 32, 1003), (64, 64, 5), (64, 16, 300),
                                      (128, 48, 17)])
def test_sfmg_preprocess_tnd_shapes(Dv, N1, T):
    """The TND preprocess (rows t * N1 + n, sfmg [n][t]) for several head
    counts and both Dv, with T not a multiple of a block's rows and a
    sequence boundary inside a block: every row against the oracle."""
    import torch
    import flashattention_backward_fa_amd as fa
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(700 + Dv + N1 + T)
    dy = torch.from_numpy(rng.standard_normal((T, N1, Dv), dtype=np.float32)).to(torch.bfloat16)
    y = torch.from_numpy(rng.standard_normal((T, N1, Dv), dtype=np.float32)).to(torch.bfloat16)
    cu = np.array([0, T // 3, T], dtype=np.int32)
    say(f"[parity] TND sfmg Dv={Dv} N1={N1} T={T}")
    s_gpu = fa.sfmg(dy.to(dev), y.to(dev), "TND", torch.from_numpy(cu).to(dev),
                    max_seqlen_q=int(np.diff(cu).max())).cpu().double().numpy()
    s_ref = oracle.sfmg(f64(dy), f64(y), "TND", cu)
    bound = 1e-5 * oracle.sfmg(np.abs(f64(dy)), np.abs(f64(y)), "TND", cu) + 1e-30
    assert s_gpu.shape == s_ref.shape and np.all(np.abs(s_gpu - s_ref) <= bound)


@pytest.mark.parametrize("name,dq_mode", [(n, m) for n in LARGE for m in ("auto", "recompute")])
def test_parity_large_workload_full(name, dq_mode):
    """Every element of dq, dk, dv of the full-size workload against the
    oracle's whole backward.  dq_mode "auto": the plan fa_bwd_create picks
    (stored dS on these workloads, as benchmarked); "recompute": the mode that
    keeps no dS, forced here at the benchmark's sizes."""
    import torch  # noqa: F401
    import flashattention_backward_fa_amd as fa
    c = big(name)
    cfg, x, Yst, lst = c["cfg"], c["x"], c["Yst"], c["lst"]
    say(f"[parity] {name}: backward ({dq_mode}) on the GPU")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode=dq_mode)
    if dq_mode == "auto":
        mq, mk = max_lengths(cfg, x)
        plan = fa.fa_bwd.get_plan(x["q"].to("meta"), x["k"].to("meta"), x["v"].to("meta"), cfg["layout"],
                                  *((None, None) if cfg["layout"] != "TND" else
                                    (torch.from_numpy(x["cu_q"]), torch.from_numpy(x["cu_kv"]))),
                                  cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"], cfg["win_right"], mq, mk)
        assert plan.dq_path() == "stored_ds"
    rq, rk, rv = c["ref"]
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    assert np.all(np.isfinite(gq)) and np.all(np.isfinite(gk)) and np.all(np.isfinite(gv))
    # a second route to the same numbers: rows the oracle evaluates one by one
    q_rows, kv_rows = sample_rows(cfg, x)
    sq, sk, sv = oracle.backward_rows(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), Yst, lst, q_rows,
                                      kv_rows, cfg["layout"], x["cu_q"], x["cu_kv"], cfg["softmax_scale"],
                                      cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    for (b, n, i), r in zip(q_rows, sq):
        assert np.allclose(pick(rq, cfg, x, b, n, i, "q"), r, rtol=1e-9, atol=1e-12)
    for (b, n, j), r1, r2 in zip(kv_rows, sk, sv):
        assert np.allclose(pick(rk, cfg, x, b, n, j, "kv"), r1, rtol=1e-9, atol=1e-12)
        assert np.allclose(pick(rv, cfg, x, b, n, j, "kv"), r2, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------------ kernel paths

class _env:
    """Set environment variables read by fa_bwd_create (the job-split tuning
    override) and drop cached plans around the block."""

    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        import os
        from flashattention_backward_fa_amd import fa_bwd as fb
        self.old = {k: os.environ.get(k) for k in self.kv}
        os.environ.update({k: str(v) for k, v in self.kv.items()})
        fb._plans.clear()

    def __exit__(self, *exc):
        import os
        from flashattention_backward_fa_amd import fa_bwd as fb
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        fb._plans.clear()


ATOMIC_CASES = ["bsnd_causal_gqa4_ragged", "tnd_mixed_lengths", "bnsd_causal_s1_lt_s2_d192"]


@pytest.mark.parametrize("name", ATOMIC_CASES)
def test_atomic_dq_mode_parity(name):
    """dq_mode "atomic" (the page's fp32 atomic dQ, section 五 5.2) against the
    oracle: the 8-wavefront kernel at D <= 128, the 4-wavefront one at D = 192."""
    cfg = EDGE_CASES[name]
    say(f"[parity] atomic dQ: {name}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode="atomic")
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])


@pytest.mark.parametrize("split", ["1,1", "2,3", "1,5"])
def test_split_partials_parity(split):
    """dK/dV split over query heads and query ranges, summed by the reduce kernel."""
    cfg = EDGE_CASES["bsnd_causal_gqa4_ragged"]
    say(f"[parity] split {split}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index("bsnd_causal_gqa4_ragged"))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    with _env(FA_BWD_SPLIT=split):
        gq, gk, gv = gpu_backward(cfg, x, Yst, lst)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])


@pytest.mark.parametrize("dq_mode", ["auto", "recompute", "stored_ds", "fused"])
def test_default_path_is_bitwise_repeatable(dq_mode):
    """No atomics in any of these modes: two runs give identical bits (the
    second with the determinism flag, which must not change the plan)."""
    cfg = EDGE_CASES["tnd_mixed_lengths"] if dq_mode != "fused" else EDGE_CASES["tnd_window_dense_heads"]
    x = case_inputs(cfg, seed=1)
    Yst, lst = oracle_inputs(cfg, x)
    say(f"[det] repeat ({dq_mode})")
    a = gpu_backward(cfg, x, Yst, lst, dq_mode=dq_mode)
    b = gpu_backward(cfg, x, Yst, lst, dq_mode=dq_mode, deterministic=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# edge cases whose longest key sequence fits the fused kernel's one tile
FUSED_CASES = sorted(n for n, c in EDGE_CASES.items()
                     if c["D"] in (64, 128) and max(c.get("lengths_kv", c.get("lengths", [c.get("S2", 0)]))) <= 128
                     and (c["layout"] == "TND" or c["S2"] <= 128))


@pytest.mark.parametrize("dq_mode,name", [(m, n) for m in ("recompute", "stored_ds") for n in sorted(EDGE_CASES)]
                         + [("fused", n) for n in FUSED_CASES])
def test_every_mode_parity(dq_mode, name):
    """Each deterministic dQ mode on every edge case it takes, whatever the
    plan would pick, against the oracle, every element: "recompute" (a dQ pass
    recomputing S and dP), "stored_ds" (the dK/dV kernel stores dS and a GEMM
    kernel forms dQ from it) and "fused" (one launch per sequence and KV head)."""
    cfg = EDGE_CASES[name]
    say(f"[parity] {dq_mode}: {name}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode=dq_mode)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    qe, ke = empty_rows(cfg, x, gq.shape, gk.shape)
    assert not np.any(gq[qe]) and not np.any(gk[ke]) and not np.any(gv[ke])


FUSED_EXTRA = {
    "fused_gqa8_s1_256_s2_96": W.custom("BSND", B=1, N1=8, N2=1, S1=256, S2=96, D=128, Dv=128, mask_mode=1),
    "fused_long_queries": W.custom("BNSD", B=2, N1=2, N2=2, S1=1000, S2=128, D=64, Dv=64, mask_mode=0),
    "fused_tnd_window": W.custom("TND", N1=4, N2=1, D=128, Dv=64, mask_mode=2, win_left=17, win_right=3,
                                 lengths=[0, 128, 7, 100, 33], lengths_kv=[5, 128, 0, 90, 33]),
    # D = 64 runs two query groups over alternate items: an odd item count
    # (3 heads x 3 blocks) leaves group 1 idle in the last step
    "fused_d64_gqa3_odd_items": W.custom("BSND", B=2, N1=6, N2=2, S1=80, S2=100, D=64, Dv=64, mask_mode=1),
    # one item in all: group 1 never has work, its dK / dV stay zero
    "fused_d64_single_item": W.custom("BNSD", B=1, N1=1, N2=1, S1=20, S2=128, D=64, Dv=64, mask_mode=2,
                                      win_left=5, win_right=40),
    "fused_d128_single_item": W.custom("BNSD", B=1, N1=1, N2=1, S1=31, S2=77, D=128, Dv=128, mask_mode=0),
}


@pytest.mark.parametrize("name", sorted(FUSED_EXTRA))
def test_fused_kernel_shapes(name):
    """The fused kernel at its limits: GQA 8 (the head loop), many query
    blocks, Dv < D, empty key and query sequences, windows, odd and single
    item counts for the two query groups at D = 64."""
    cfg = FUSED_EXTRA[name]
    say(f"[parity] fused: {name}")
    x = case_inputs(cfg, seed=5)
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode="fused")
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    qe, ke = empty_rows(cfg, x, gq.shape, gk.shape)
    assert not np.any(gq[qe]) and not np.any(gk[ke]) and not np.any(gv[ke])


@pytest.mark.parametrize("dq_mode", ["recompute", "stored_ds"])
@pytest.mark.parametrize("split", ["1,1", "2,3", "1,5"])
def test_both_pairs_split_partials_parity(dq_mode, split):
    """Both pairs with dK/dV split over query heads and query ranges."""
    cfg = EDGE_CASES["bsnd_causal_gqa4_ragged"]
    say(f"[parity] {dq_mode}, split {split}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index("bsnd_causal_gqa4_ragged"))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    with _env(FA_BWD_SPLIT=split):
        gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode=dq_mode)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])


def _min_stored_ds_bound(cfg, x):
    """The smallest max_workspace_bytes a stored-dS plan accepts (bisection on
    fa_bwd_create's answer): it holds sfmg and the dS of one KV head."""
    import torch
    from flashattention_backward_fa_amd import fa_bwd as fb
    mq, mk = max_lengths(cfg, x)
    cu = (None, None) if cfg["layout"] != "TND" else (torch.from_numpy(x["cu_q"]), torch.from_numpy(x["cu_kv"]))
    args = (x["q"].to("meta"), x["k"].to("meta"), x["v"].to("meta"), cfg["layout"], *cu, cfg["softmax_scale"],
            cfg["mask_mode"], cfg["win_left"], cfg["win_right"], mq, mk)

    def ok(bound):
        try:
            fb.get_plan(*args, dq_mode="stored_ds", max_workspace_bytes=bound)
            return True
        except fb.FaBwdError as e:
            assert e.status == fb.FA_ERR_WORKSPACE
            return False

    hi = fb.get_plan(*args, dq_mode="stored_ds").workspace_bytes
    lo = 1
    while lo < hi:
        mid = (lo + hi) // 2
        if ok(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


@pytest.mark.parametrize("name", ["bsnd_causal_gqa4_ragged", "tnd_mixed_lengths", "bnsd_batch3_causal",
                                  "tnd_window_dense_heads", "bsnd_d192_dv64_window"])
def test_stored_ds_one_kv_head_per_pass(name):
    """Stored-dS mode under the smallest workspace bound it accepts: one KV
    head's dS per pass (the dK/dV and dQ launches repeat per head), against
    the oracle."""
    cfg = EDGE_CASES[name]
    say(f"[parity] stored dS, one KV head per pass: {name}")
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index(name))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    bound = _min_stored_ds_bound(cfg, x)
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, dq_mode="stored_ds", max_workspace_bytes=bound)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
    qe, ke = empty_rows(cfg, x, gq.shape, gk.shape)
    assert not np.any(gq[qe]) and not np.any(gk[ke]) and not np.any(gv[ke])


def test_stored_ds_uneven_kv_head_chunks():
    """Three KV heads in chunks of two and one: the bound holds sfmg and 2.5
    KV heads' dS (2 row groups x 2 query heads x 7 slices x 8 KB each)."""
    cfg = W.custom("BSND", B=1, N1=6, N2=3, S1=200, S2=200, D=128, Dv=128, mask_mode=1)
    say("[parity] stored dS, KV-head chunks of 2 and 1")
    x = case_inputs(cfg, seed=11)
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    per_kv = 2 * 2 * 7 * 8192
    sfmg = (6 * 200 * 4 + 255) // 256 * 256
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, max_workspace_bytes=sfmg + per_kv * 5 // 2)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])


def test_workspace_bound_falls_back_to_recompute():
    """A bound below one KV head's dS: the plan recomputes S and dP for dQ,
    with no partial sums when even those do not fit."""
    from flashattention_backward_fa_amd import fa_bwd as fb
    cfg = EDGE_CASES["bsnd_causal_gqa4_ragged"]
    x = case_inputs(cfg, seed=sorted(EDGE_CASES).index("bsnd_causal_gqa4_ragged"))
    Yst, lst = oracle_inputs(cfg, x)
    rq, rk, rv = oracle_backward(cfg, x, Yst, lst)
    sfmg = (8 * 300 * 4 + 255) // 256 * 256
    plan = fb.get_plan(x["q"].to("meta"), x["k"].to("meta"), x["v"].to("meta"), "BSND", None, None, 0.0, 1, -1, -1,
                       max_workspace_bytes=sfmg)
    assert plan.dq_path() == "recompute" and plan.workspace_bytes == sfmg
    say("[parity] workspace bound = sfmg only")
    gq, gk, gv = gpu_backward(cfg, x, Yst, lst, max_workspace_bytes=sfmg)
    assert_all_close([(gq, rq, "dq"), (gk, rk, "dk"), (gv, rv, "dv")])
