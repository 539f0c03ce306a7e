"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: central finite
differences of the oracle's forward, the softmax invariants, the explicit
softmax Jacobian, PyTorch fp64 autograd on a naive attention, pure-Python
loops, closed forms, NumPy's tril/triu, and layout / GQA / varlen / mask
equivalences.  Formulas: page "CANN ops-transformer FlashAttnGrad 算子详解",
section 一 (forward S, P, Y and backward dV, dP, sfmg, dS, dQ, dK); the softmax
Jacobian form p_i (g_i - sum_j p_j g_j) is the one page
"BlockAttentionResidualsGrad" states for its softmax backward step.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(rng, *shape):
    return rng.standard_normal(shape)


def problem(rng, layout="BSND", B=1, N1=2, N2=1, S1=5, S2=7, D=4, Dv=3, lens_q=None, lens_kv=None):
    """Random float64 problem in a layout; TND takes per-sequence lengths."""
    if layout == "TND":
        cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
        cu_kv = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int32)
        T1, T2 = int(cu_q[-1]), int(cu_kv[-1])
        return dict(q=rand(rng, T1, N1, D), k=rand(rng, T2, N2, D), v=rand(rng, T2, N2, Dv),
                    dY=rand(rng, T1, N1, Dv), layout="TND", cu_q=cu_q, cu_kv=cu_kv)
    if layout == "BSND":
        shp = lambda S, N, d: (B, S, N, d)  # noqa: E731
    else:
        shp = lambda S, N, d: (B, N, S, d)  # noqa: E731
    return dict(q=rand(rng, *shp(S1, N1, D)), k=rand(rng, *shp(S2, N2, D)), v=rand(rng, *shp(S2, N2, Dv)),
                dY=rand(rng, *shp(S1, N1, Dv)), layout=layout, cu_q=None, cu_kv=None)


def fwd(p, **kw):
    return oracle.forward(p["q"], p["k"], p["v"], p["layout"], p["cu_q"], p["cu_kv"], **kw)


def bwd(p, Y, lse, **kw):
    return oracle.backward(p["q"], p["k"], p["v"], p["dY"], Y, lse, p["layout"], p["cu_q"], p["cu_kv"], **kw)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 2**-130], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_ties_to_even():
    vals = oracle.bf16_round(np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-9, 3.0]))
    assert list(vals) == [1.0, 1 + 2**-6, 1.0, 3.0]


def test_f16_round_matches_numpy_half_cast():
    """IEEE binary16 rounding against numpy's float64 -> float16 conversion
    (round to nearest even), normal, subnormal and overflowing magnitudes."""
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(2000) * 1e-6,      # subnormal range (below 2**-14)
        rng.standard_normal(2000) * 3e4,       # up to and past the largest finite value
        np.array([0.0, -0.0, 1.0, 65504.0, 65519.0, 65520.0, -65520.0, 2.0**-24, 2.0**-25, 2.0**-14]),
    ])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.f16_round(x), ref)


def test_f16_round_ties_and_limits():
    """Values fixed by the binary16 format: 11 significant bits, ties to even,
    largest finite 65504, spacing 2**-24 below 2**-14."""
    vals = oracle.f16_round(np.array([1 + 2**-11, 1 + 3 * 2**-11, 65504.0, 65519.0, 65520.0, -65520.0,
                                      2.0**-24, 2.0**-25, 3 * 2.0**-25, 2.0**-14 + 2.0**-25]))
    assert list(vals[:4]) == [1.0, 1 + 2**-9, 65504.0, 65504.0]
    assert vals[4] == np.inf and vals[5] == -np.inf
    assert list(vals[6:]) == [2.0**-24, 0.0, 2.0**-23, 2.0**-14]


def test_store_rounds_to_the_element_type():
    Y = np.array([[1 + 2**-9, 1 + 2**-12]])
    assert list(oracle.store(Y, np.zeros(1), "bf16")[0][0]) == [1.0, 1.0]
    assert list(oracle.store(Y, np.zeros(1), "fp16")[0][0]) == [1 + 2**-9, 1.0]


# ------------------------------------------------------------------ masks

@pytest.mark.parametrize("s1,s2", [(6, 6), (4, 9), (9, 4), (1, 1)])
def test_mask_matches_numpy_tril_triu(s1, s2):
    off = s2 - s1
    ones = np.ones((s1, s2), dtype=bool)
    assert np.array_equal(oracle.allowed_matrix(s1, s2, -1, -1), ones)
    assert np.array_equal(oracle.allowed_matrix(s1, s2, -1, 0), np.tril(ones, off))
    for L, R in [(2, 0), (0, 0), (3, 1), (1, 5)]:
        expect = np.tril(ones, off + R) & np.triu(ones, off - L)
        assert np.array_equal(oracle.allowed_matrix(s1, s2, L, R), expect)


def test_mask_bottom_right_example():
    # 3 queries, 5 keys, causal: the last query sees every key, the diagonal
    # sits at key i + 2.
    expect = np.array([[1, 1, 1, 0, 0], [1, 1, 1, 1, 0], [1, 1, 1, 1, 1]], dtype=bool)
    L, R = oracle.mask_bounds(oracle.MASK_CAUSAL)
    assert np.array_equal(oracle.allowed_matrix(3, 5, L, R), expect)


def test_mask_bounds_reading():
    assert oracle.mask_bounds(0) == (-1, -1)
    assert oracle.mask_bounds(1) == (-1, 0)
    assert oracle.mask_bounds(1, 1024, 0) == (1024, 0)
    assert oracle.mask_bounds(2, 1024, 0) == (1024, 0)
    assert oracle.mask_bounds(2, 3, 4) == (3, 4)


def test_scale_rule():
    assert oracle.resolve_scale(0.0, 64) == 1 / 8
    assert oracle.resolve_scale(0.25, 64) == 0.25


# ------------------------------------------------------------------ finite differences

FD_CASES = [
    dict(layout="BSND", mask=(0, -1, -1), scale=0.37),
    dict(layout="BSND", mask=(1, -1, -1), scale=0.0),
    dict(layout="BNSD", mask=(2, 2, 1), scale=0.6),
    dict(layout="BSND", mask=(1, -1, -1), scale=0.5, S1=7, S2=4),     # rows with no key
    dict(layout="TND", mask=(1, 2, 0), scale=0.45, lens_q=[3, 4], lens_kv=[5, 2], N1=4, N2=2),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: f"{c['layout']}-m{c['mask'][0]}")
def test_backward_matches_finite_differences(case):
    rng = np.random.default_rng(7)
    kw = {k: case[k] for k in ("S1", "S2", "lens_q", "lens_kv", "N1", "N2") if k in case}
    p = problem(rng, case["layout"], **kw)
    mode, L, R = case["mask"]
    akw = dict(softmax_scale=case["scale"], mask_mode=mode, win_left=L, win_right=R)

    def loss(q, k, v):
        Y, _ = oracle.forward(q, k, v, p["layout"], p["cu_q"], p["cu_kv"], **akw)
        return float((Y * p["dY"]).sum())

    Y, lse = fwd(p, **akw)
    grads = bwd(p, Y, lse, **akw)
    h = 1e-6
    for gi, name in enumerate(["q", "k", "v"]):
        x = p[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = [p["q"].copy(), p["k"].copy(), p["v"].copy()]
            args[gi][idx] += h
            lp = loss(*args)
            args[gi][idx] -= 2 * h
            lm = loss(*args)
            fd[idx] = (lp - lm) / (2 * h)
        scale_ref = max(np.abs(fd).max(), 1e-3)
        assert np.abs(grads[gi] - fd).max() <= 1e-6 * scale_ref, name


# ------------------------------------------------------------------ invariants

def _heads(rng, S1=9, S2=11, D=5, Dv=4, mask=(1, 3, 0), scale=0.4):
    q, k, v, dY = rand(rng, S1, D), rand(rng, S2, D), rand(rng, S2, Dv), rand(rng, S1, Dv)
    L, R = oracle.mask_bounds(*mask)
    ok = oracle.allowed_matrix(S1, S2, L, R)
    Y, lse = oracle.head_forward(q, k, v, scale, ok)
    return q, k, v, dY, Y, lse, scale, ok


def test_softmax_invariants_exact_mode():
    rng = np.random.default_rng(1)
    q, k, v, dY, Y, lse, scale, ok = _heads(rng)
    r = oracle.head_backward(q, k, v, dY, Y, lse, scale, ok)
    rows = ok.any(axis=1)
    assert np.allclose(r["P"][rows].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(r["dS"].sum(axis=1), 0.0, rtol=0, atol=1e-12)
    assert np.allclose(r["sfmg"], (r["P"] * r["dP"]).sum(axis=1), rtol=0, atol=1e-12)
    assert np.all(r["P"][~ok] == 0)


def test_stored_mode_dS_row_sum_identity():
    rng = np.random.default_rng(2)
    q, k, v, dY, Y, lse, scale, ok = _heads(rng)
    Yst, lst = oracle.store(Y, lse)
    assert lst.dtype == np.float32
    r = oracle.head_backward(q, k, v, dY, Yst, lst.astype(np.float64), scale, ok)
    expect = (dY * (r["P"] @ v)).sum(axis=1) - r["sfmg"] * r["P"].sum(axis=1)
    assert np.allclose(r["dS"].sum(axis=1), expect, rtol=0, atol=1e-12)
    # and the stored-mode sfmg is dY . Y_st, which differs from dY . Y_exact
    assert np.allclose(r["sfmg"], (dY * Yst).sum(axis=1), rtol=0, atol=1e-14)


def test_dS_equals_explicit_softmax_jacobian():
    rng = np.random.default_rng(3)
    q, k, v, dY, Y, lse, scale, ok = _heads(rng, mask=(0, -1, -1))
    r = oracle.head_backward(q, k, v, dY, Y, lse, scale, ok)
    for i in range(q.shape[0]):
        p = r["P"][i]
        J = np.diag(p) - np.outer(p, p)
        assert np.allclose(J @ r["dP"][i], r["dS"][i], rtol=0, atol=1e-12)
        # textbook elementwise form p_j (g_j - sum_l p_l g_l)
        g = r["dP"][i]
        assert np.allclose(p * (g - (p * g).sum()), r["dS"][i], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ library autograd

def _torch_attention(q, k, v, scale, ok, G):
    import torch
    kk = k.repeat_interleave(G, dim=0)
    vv = v.repeat_interleave(G, dim=0)
    S = scale * torch.matmul(q, kk.transpose(1, 2).contiguous())
    S = S.masked_fill(~ok, float("-inf"))
    P = torch.softmax(S, dim=-1)
    P = torch.nan_to_num(P, nan=0.0)
    return torch.matmul(P, vv)


@pytest.mark.parametrize("mask", [(0, -1, -1), (1, -1, -1), (2, 3, 2)])
def test_backward_matches_torch_fp64_autograd(mask):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    B, N1, N2, S1, S2, D, Dv = 2, 4, 2, 13, 10, 8, 6
    p = problem(rng, "BNSD", B=B, N1=N1, N2=N2, S1=S1, S2=S2, D=D, Dv=Dv)
    mode, L, R = mask
    akw = dict(softmax_scale=0.3, mask_mode=mode, win_left=L, win_right=R)
    Y, lse = fwd(p, **akw)
    dq, dk, dv = bwd(p, Y, lse, **akw)
    okm = torch.from_numpy(oracle.allowed_matrix(S1, S2, *oracle.mask_bounds(*mask)))
    for b in range(B):
        q = torch.tensor(p["q"][b], requires_grad=True)
        k = torch.tensor(p["k"][b], requires_grad=True)
        v = torch.tensor(p["v"][b], requires_grad=True)
        out = _torch_attention(q, k, v, 0.3, okm, N1 // N2)
        assert np.allclose(out.detach().numpy(), Y[b], rtol=0, atol=1e-12)
        (out * torch.from_numpy(p["dY"][b])).sum().backward()
        assert np.allclose(q.grad.numpy(), dq[b], rtol=0, atol=1e-11)
        assert np.allclose(k.grad.numpy(), dk[b], rtol=0, atol=1e-11)
        assert np.allclose(v.grad.numpy(), dv[b], rtol=0, atol=1e-11)


# ------------------------------------------------------------------ brute force

def _brute(q, k, v, dY, Y, lse, scale, ok, G):
    """Pure-Python loops over lists; no NumPy arithmetic."""
    N1, S1, D = len(q), len(q[0]), len(q[0][0])
    N2, S2, Dv = len(k), len(k[0]), len(v[0][0])
    dq = [[[0.0] * D for _ in range(S1)] for _ in range(N1)]
    dk = [[[0.0] * D for _ in range(S2)] for _ in range(N2)]
    dv = [[[0.0] * Dv for _ in range(S2)] for _ in range(N2)]
    for n in range(N1):
        m = n // G
        for i in range(S1):
            sf = sum(dY[n][i][e] * Y[n][i][e] for e in range(Dv))
            for j in range(S2):
                if not ok[i][j] or lse[n][i] == -math.inf:
                    continue
                s = scale * sum(q[n][i][d] * k[m][j][d] for d in range(D))
                pij = math.exp(s - lse[n][i])
                dpij = sum(dY[n][i][e] * v[m][j][e] for e in range(Dv))
                dsij = pij * (dpij - sf)
                for e in range(Dv):
                    dv[m][j][e] += pij * dY[n][i][e]
                for d in range(D):
                    dq[n][i][d] += scale * dsij * k[m][j][d]
                    dk[m][j][d] += scale * dsij * q[n][i][d]
    return dq, dk, dv


def test_backward_matches_pure_python_loops_stored_mode():
    rng = np.random.default_rng(5)
    p = problem(rng, "BNSD", B=1, N1=4, N2=2, S1=6, S2=5, D=3, Dv=2)
    for key in ("q", "k", "v", "dY"):
        p[key] = oracle.bf16_round(p[key])
    akw = dict(softmax_scale=0.0, mask_mode=1)
    Y, lse = fwd(p, **akw)
    Yst, lst = oracle.store(Y, lse)
    dq, dk, dv = bwd(p, Yst, lst, **akw)
    ok = oracle.allowed_matrix(6, 5, -1, 0).tolist()
    bq, bk, bv = _brute(p["q"][0].tolist(), p["k"][0].tolist(), p["v"][0].tolist(), p["dY"][0].tolist(),
                        Yst[0].tolist(), lst[0].astype(np.float64).tolist(), 1 / math.sqrt(3), ok, 2)
    assert np.allclose(dq[0], bq, rtol=0, atol=1e-12)
    assert np.allclose(dk[0], bk, rtol=0, atol=1e-12)
    assert np.allclose(dv[0], bv, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ closed forms

def test_single_key_closed_form():
    rng = np.random.default_rng(6)
    p = problem(rng, "BSND", B=1, N1=2, N2=2, S1=5, S2=1, D=4, Dv=3)
    Y, lse = fwd(p)
    dq, dk, dv = bwd(p, Y, lse)
    assert np.allclose(dq, 0, atol=1e-13) and np.allclose(dk, 0, atol=1e-13)
    assert np.allclose(dv[0, 0], p["dY"][0].sum(axis=0), atol=1e-13)


def test_zero_query_uniform_probabilities():
    rng = np.random.default_rng(8)
    p = problem(rng, "BSND", B=1, N1=1, N2=1, S1=6, S2=9, D=4, Dv=3)
    p["q"][:] = 0
    Y, lse = fwd(p)
    assert np.allclose(lse, math.log(9), atol=1e-13)
    _, _, dv = bwd(p, Y, lse)
    for j in range(9):
        assert np.allclose(dv[0, j, 0], p["dY"][0, :, 0].sum(axis=0) / 9, atol=1e-13)


def test_zero_upstream_gradient():
    rng = np.random.default_rng(9)
    p = problem(rng, "BSND", B=2, N1=4, N2=2, S1=5, S2=6, D=4, Dv=4)
    p["dY"][:] = 0
    Y, lse = fwd(p, mask_mode=1)
    for g in bwd(p, Y, lse, mask_mode=1):
        assert not np.any(g)


def test_equal_value_rows_give_zero_dS():
    rng = np.random.default_rng(10)
    p = problem(rng, "BSND", B=1, N1=2, N2=1, S1=5, S2=8, D=4, Dv=3)
    p["v"][:] = p["v"][:, :1]
    Y, lse = fwd(p, mask_mode=2, win_left=2, win_right=1)
    dq, dk, dv = bwd(p, Y, lse, mask_mode=2, win_left=2, win_right=1)
    assert np.allclose(dq, 0, atol=1e-12) and np.allclose(dk, 0, atol=1e-12)
    assert np.abs(dv).max() > 0.1


# ------------------------------------------------------------------ equivalences

def test_gqa_equals_mha_on_repeated_kv():
    rng = np.random.default_rng(12)
    G = 3
    p = problem(rng, "BSND", B=2, N1=6, N2=2, S1=7, S2=9, D=4, Dv=5)
    akw = dict(mask_mode=1, softmax_scale=0.5)
    Y, lse = fwd(p, **akw)
    dq, dk, dv = bwd(p, Y, lse, **akw)
    m = dict(p)
    m["k"] = np.repeat(p["k"], G, axis=2)
    m["v"] = np.repeat(p["v"], G, axis=2)
    Ym, lsem = fwd(m, **akw)
    assert np.allclose(Y, Ym, atol=1e-13) and np.allclose(lse, lsem, atol=1e-13)
    dqm, dkm, dvm = bwd(m, Ym, lsem, **akw)
    assert np.allclose(dq, dqm, atol=1e-12)
    assert np.allclose(dk, dkm.reshape(2, 9, 2, G, 4).sum(axis=3), atol=1e-12)
    assert np.allclose(dv, dvm.reshape(2, 9, 2, G, 5).sum(axis=3), atol=1e-12)


def test_tnd_equals_per_sequence_dense():
    rng = np.random.default_rng(13)
    lens_q, lens_kv = [4, 0, 6, 3], [5, 2, 6, 1]
    p = problem(rng, "TND", N1=4, N2=2, D=4, Dv=3, lens_q=lens_q, lens_kv=lens_kv)
    akw = dict(mask_mode=2, win_left=2, win_right=1, softmax_scale=0.7)
    Y, lse = fwd(p, **akw)
    dq, dk, dv = bwd(p, Y, lse, **akw)
    for b in range(4):
        a, e = p["cu_q"][b], p["cu_q"][b + 1]
        c, f = p["cu_kv"][b], p["cu_kv"][b + 1]
        if e == a:
            continue
        s = dict(q=p["q"][None, a:e], k=p["k"][None, c:f], v=p["v"][None, c:f], dY=p["dY"][None, a:e],
                 layout="BSND", cu_q=None, cu_kv=None)
        if f == c:
            continue
        Ys, ls = fwd(s, **akw)
        assert np.allclose(Ys[0], Y[a:e], atol=1e-13)
        assert np.allclose(ls[0], lse[:, a:e], atol=1e-13)
        gq, gk, gv = bwd(s, Ys, ls, **akw)
        assert np.allclose(gq[0], dq[a:e], atol=1e-12)
        assert np.allclose(gk[0], dk[c:f], atol=1e-12)
        assert np.allclose(gv[0], dv[c:f], atol=1e-12)
    # an empty query sequence leaves its keys with zero gradient
    assert not np.any(dk[5:7]) and not np.any(dv[5:7])


# ------------------------------------------------------------------ seqused (reading)

def test_seqused_at_full_length_changes_nothing():
    rng = np.random.default_rng(21)
    p = problem(rng, "BSND", B=2, N1=4, N2=2, S1=5, S2=7)
    akw = dict(mask_mode=1, softmax_scale=0.6)
    Y, lse = fwd(p, **akw)
    g = bwd(p, Y, lse, **akw)
    used = dict(seqused_q=np.array([5, 5]), seqused_kv=np.array([7, 9]))  # 9 is clamped to 7
    Yu, lu = fwd(p, **akw, **used)
    gu = bwd(p, Y, lse, **akw, **used)
    assert np.array_equal(Y, Yu) and np.array_equal(lse, lu)
    for a, b in zip(g, gu):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("layout", ["BSND", "BNSD", "TND"])
def test_seqused_equals_the_truncated_problem(layout):
    """Used rows of each sequence behave as a problem of the used lengths
    (masks aligned on them); padding rows have Y = 0, lse = -inf and zero
    gradients.  Checked against the unpadded problem, sequence by sequence."""
    rng = np.random.default_rng(22)
    B, S1, S2 = 3, 8, 9
    if layout == "TND":
        lens_q, lens_kv = [8, 3, 6], [9, 5, 9]
        p = problem(rng, "TND", N1=4, N2=2, D=4, Dv=3, lens_q=lens_q, lens_kv=lens_kv)
    else:
        lens_q, lens_kv = [S1] * B, [S2] * B
        p = problem(rng, layout, B=B, N1=4, N2=2, S1=S1, S2=S2, D=4, Dv=3)
    uq, ukv = np.array([5, 0, 20]), np.array([6, 3, 2])
    akw = dict(mask_mode=2, win_left=3, win_right=1, softmax_scale=0.55)
    Y, lse = fwd(p, **akw, seqused_q=uq, seqused_kv=ukv)
    dq, dk, dv = bwd(p, Y, lse, **akw, seqused_q=uq, seqused_kv=ukv)
    parts = [oracle.split_heads(t, layout, c) for t, c in
             ((p["q"], p["cu_q"]), (p["k"], p["cu_kv"]), (p["v"], p["cu_kv"]), (p["dY"], p["cu_q"]),
              (Y, p["cu_q"]), (dq, p["cu_q"]), (dk, p["cu_kv"]), (dv, p["cu_kv"]))]
    lses = oracle.attention._split_lse(lse, layout, p["cu_q"])
    for b in range(B):
        u1, u2 = min(uq[b], lens_q[b]), min(ukv[b], lens_kv[b])
        qb, kb, vb, dyb, yb, dqb, dkb, dvb = (x[b] for x in parts)
        assert not np.any(yb[:, u1:]) and np.all(lses[b][:, u1:] == -np.inf)
        assert not np.any(dqb[:, u1:]) and not np.any(dkb[:, u2:]) and not np.any(dvb[:, u2:])
        t = dict(q=qb[None, :, :u1], k=kb[None, :, :u2], v=vb[None, :, :u2], dY=dyb[None, :, :u1],
                 layout="BNSD", cu_q=None, cu_kv=None)
        if u1 == 0:
            assert not np.any(dkb) and not np.any(dvb)
            continue
        Yt, lt = fwd(t, **akw)
        assert np.allclose(Yt[0], yb[:, :u1], atol=1e-13)
        assert np.allclose(lt[0], lses[b][:, :u1], atol=1e-13)
        gq, gk, gv = bwd(t, Yt, lt, **akw)
        assert np.allclose(gq[0], dqb[:, :u1], atol=1e-12)
        assert np.allclose(gk[0], dkb[:, :u2], atol=1e-12)
        assert np.allclose(gv[0], dvb[:, :u2], atol=1e-12)


def test_seqused_backward_matches_finite_differences():
    """With seqused the backward is still the gradient of the forward, padding
    entries included (their gradient is zero because they do not enter Y)."""
    rng = np.random.default_rng(23)
    p = problem(rng, "BSND", B=2, N1=2, N2=1, S1=4, S2=5, D=3, Dv=2)
    kw = dict(mask_mode=1, softmax_scale=0.7, seqused_q=np.array([3, 4]), seqused_kv=np.array([2, 5]))
    Y, lse = fwd(p, **kw)
    g = bwd(p, Y, lse, **kw)
    h = 1e-6
    for gi, name in enumerate(("q", "k", "v")):
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            for sgn in (1, -1):
                pp = dict(p)
                pp[name] = x.copy()
                pp[name][idx] += sgn * h
                fd[idx] += sgn * float((fwd(pp, **kw)[0] * p["dY"]).sum()) / (2 * h)
        assert np.abs(g[gi] - fd).max() <= 1e-6 * max(np.abs(fd).max(), 1e-3)


def test_wide_window_equals_causal_and_open_window_equals_dense():
    rng = np.random.default_rng(14)
    p = problem(rng, "BSND", B=1, N1=2, N2=2, S1=8, S2=8, D=4, Dv=4)
    Yc, lc = fwd(p, mask_mode=1)
    Yw, lw = fwd(p, mask_mode=2, win_left=8, win_right=0)
    assert np.array_equal(Yc, Yw) and np.array_equal(lc, lw)
    gc = bwd(p, Yc, lc, mask_mode=1)
    gw = bwd(p, Yw, lw, mask_mode=2, win_left=8, win_right=0)
    for a, b in zip(gc, gw):
        assert np.array_equal(a, b)
    Yd, ld = fwd(p, mask_mode=0)
    Yo, lo = fwd(p, mask_mode=2, win_left=-1, win_right=-1)
    assert np.array_equal(Yd, Yo) and np.array_equal(ld, lo)


def test_layouts_agree():
    rng = np.random.default_rng(15)
    p = problem(rng, "BSND", B=1, N1=4, N2=2, S1=6, S2=6, D=4, Dv=3)
    akw = dict(mask_mode=1, softmax_scale=0.0)
    Y, lse = fwd(p, **akw)
    g = bwd(p, Y, lse, **akw)
    tr = lambda x: x.transpose(0, 2, 1, 3).copy()  # noqa: E731
    n = dict(q=tr(p["q"]), k=tr(p["k"]), v=tr(p["v"]), dY=tr(p["dY"]), layout="BNSD", cu_q=None, cu_kv=None)
    Yn, ln = fwd(n, **akw)
    assert np.allclose(tr(Yn), Y, atol=1e-14) and np.allclose(ln, lse, atol=1e-14)
    gn = bwd(n, Yn, ln, **akw)
    for a, b in zip(g, gn):
        assert np.allclose(a, tr(b), atol=1e-13)
    t = dict(q=p["q"][0], k=p["k"][0], v=p["v"][0], dY=p["dY"][0], layout="TND",
             cu_q=np.array([0, 6], np.int32), cu_kv=np.array([0, 6], np.int32))
    Yt, lt = fwd(t, **akw)
    assert np.allclose(Yt, Y[0], atol=1e-14) and np.allclose(lt, lse[0], atol=1e-14)
    gt = bwd(t, Yt, lt, **akw)
    for a, b in zip(g, gt):
        assert np.allclose(a[0], b, atol=1e-13)


def test_linear_in_upstream_gradient():
    rng = np.random.default_rng(16)
    p = problem(rng, "BSND", B=1, N1=2, N2=1, S1=6, S2=7, D=4, Dv=3)
    Y, lse = fwd(p, mask_mode=1)
    Yst, lst = oracle.store(Y, lse)
    g1 = bwd(p, Yst, lst, mask_mode=1)
    p2 = dict(p, dY=2 * p["dY"])
    g2 = bwd(p2, Yst, lst, mask_mode=1)
    for a, b in zip(g1, g2):
        assert np.allclose(2 * a, b, rtol=0, atol=1e-13)


def test_sfmg_definition():
    dY = np.arange(2 * 3 * 2 * 4, dtype=np.float64).reshape(2, 3, 2, 4)
    Y = np.ones_like(dY)
    s = oracle.sfmg(dY, Y, "BSND")
    assert s.shape == (2, 2, 3)
    # row (b=1, s=2, n=1) holds 4 consecutive integers starting at 44
    assert s[1, 1, 2] == 44 + 45 + 46 + 47


def test_backward_rows_match_full_backward():
    rng = np.random.default_rng(17)
    p = problem(rng, "TND", N1=4, N2=2, D=4, Dv=3, lens_q=[9, 0, 12], lens_kv=[7, 3, 12])
    akw = dict(mask_mode=2, win_left=3, win_right=1, softmax_scale=0.0)
    Y, lse = fwd(p, **akw)
    Yst, lst = oracle.store(Y, lse)
    dq, dk, dv = bwd(p, Yst, lst, **akw)
    q_rows = [(0, 1, 3), (2, 3, 11), (0, 0, 0), (2, 0, 5)]
    kv_rows = [(0, 0, 6), (1, 1, 2), (2, 1, 0), (2, 0, 11)]
    rq, rk, rv = oracle.backward_rows(p["q"], p["k"], p["v"], p["dY"], Yst, lst, q_rows, kv_rows,
                                      "TND", p["cu_q"], p["cu_kv"], **akw)
    for (b, n, i), r in zip(q_rows, rq):
        assert np.allclose(dq[p["cu_q"][b] + i, n], r, atol=1e-13)
    for (b, n, j), rk_, rv_ in zip(kv_rows, rk, rv):
        assert np.allclose(dk[p["cu_kv"][b] + j, n], rk_, atol=1e-13)
        assert np.allclose(dv[p["cu_kv"][b] + j, n], rv_, atol=1e-13)


def test_page_example_shapes():
    """The page's BSND GQA call example (section 四 4.8) asserts only that
    dq, dk, dv take the shapes of q, k, v (section 二 2.2)."""
    with open(os.path.join(GOLDEN, "page_example_bsnd_gqa.json")) as f:
        ex = json.load(f)
    B, S1, S2, N1, N2, D, Dv = (ex[k] for k in ("B", "S1", "S2", "N1", "N2", "D", "Dv"))
    rng = np.random.default_rng(ex["seed"])
    p = problem(rng, "BSND", B=B, N1=N1, N2=N2, S1=S1, S2=S2, D=D, Dv=Dv)
    Y, lse = fwd(p, softmax_scale=1 / math.sqrt(D))
    assert lse.shape == (B, N1, S1)
    dq, dk, dv = bwd(p, Y, lse, softmax_scale=1 / math.sqrt(D))
    assert dq.shape == p["q"].shape and dk.shape == p["k"].shape and dv.shape == p["v"].shape
