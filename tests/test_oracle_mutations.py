"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a private copy of the oracle's source (CPU only) and checks that at
least one independent pin (finite differences of the forward, PyTorch fp64
autograd, NumPy tril/triu, GQA-by-repeat, the library's bf16 / fp16 casts,
seqused against the unpadded problem) rejects it."""

import math
import os
import types

import numpy as np
import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTATIONS = {
    "dropped_sfmg": ("dS = P * (dP - sf[:, None])", "dS = P * dP"),
    "sign_flip_dS": ("dS = P * (dP - sf[:, None])", "dS = P * (sf[:, None] - dP)"),
    "dq_without_scale": ("dq = scale * (dS @ k)", "dq = dS @ k"),
    "dk_uses_P": ("dk = scale * (dS.T @ q)", "dk = scale * (P.T @ q)"),
    "dv_uses_Y": ("dv = P.T @ dY", "dv = P.T @ Y"),
    "gqa_interleaved": ("r = head_backward(qb[n1, :u1], kb[n2, :u2], vb[n2, :u2]",
                        "r = head_backward(qb[n1, :u1], kb[n1 % N2, :u2], vb[n1 % N2, :u2]"),
    "lse_log2": ("lse[rows] = m + np.log(", "lse[rows] = m + np.log2("),
    "mask_off_by_one": ("ok &= j <= i + off + right", "ok &= j < i + off + right"),
    "mask_top_left": ("off = s2 - s1\n    i = np.arange(s1)[:, None]", "off = 0\n    i = np.arange(s1)[:, None]"),
    "scale_rule": ("else 1.0 / math.sqrt(D)", "else 1.0 / D"),
    "bf16_bits": ("quantum = np.ldexp(1.0, e - 8)", "quantum = np.ldexp(1.0, e - 7)"),
    "f16_bits": ("quantum = np.ldexp(1.0, e - 11)", "quantum = np.ldexp(1.0, e - 10)"),
    "f16_subnormal_spacing": ("e = np.maximum(e, -13)", "e = np.maximum(e, -14)"),
    "f16_no_overflow": ("np.abs(r) > 65504.0", "np.abs(r) > np.inf"),
    "seqused_kv_ignored": ("u2 = s2 if seqused_kv is None else", "u2 = s2 if True else"),
    "seqused_q_unclamped": ("min(max(int(seqused_q[b]), 0), s1)", "max(int(seqused_q[b]), 0)"),
}


def load_mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation anchor missing: {name}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def fd_pin_fails(mod):
    """Finite differences of the mutant's own forward against its backward,
    GQA causal with S1 != S2 and a non-default scale (and one default-scale
    run)."""
    rng = np.random.default_rng(3)
    B, N1, N2, S1, S2, D, Dv = 1, 4, 2, 4, 6, 3, 2
    q = rng.standard_normal((B, S1, N1, D))
    k = rng.standard_normal((B, S2, N2, D))
    v = rng.standard_normal((B, S2, N2, Dv))
    dY = rng.standard_normal((B, S1, N1, Dv))
    for scale, mode, L, R in [(0.45, 2, 2, 1), (0.0, 1, -1, -1)]:
        kw = dict(softmax_scale=scale, mask_mode=mode, win_left=L, win_right=R)
        Y, lse = mod.forward(q, k, v, "BSND", **kw)
        g = mod.backward(q, k, v, dY, Y, lse, "BSND", **kw)
        h = 1e-6
        for gi, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = [q.copy(), k.copy(), v.copy()]
                args[gi][idx] += h
                lp = float((mod.forward(*args, "BSND", **kw)[0] * dY).sum())
                args[gi][idx] -= 2 * h
                lm = float((mod.forward(*args, "BSND", **kw)[0] * dY).sum())
                fd[idx] = (lp - lm) / (2 * h)
            if np.abs(g[gi] - fd).max() > 1e-6 * max(np.abs(fd).max(), 1e-3):
                return True
    return False


def library_pin_fails(mod):
    """Mask against NumPy tril/triu, scale rule against 1/sqrt(D), and the
    whole backward against PyTorch fp64 autograd with repeat_interleave."""
    ones = np.ones((5, 7), dtype=bool)
    if not np.array_equal(mod.allowed_matrix(5, 7, -1, 0), np.tril(ones, 2)):
        return True
    if not np.array_equal(mod.allowed_matrix(5, 7, 1, 1), np.tril(ones, 3) & np.triu(ones, 1)):
        return True
    if mod.resolve_scale(0.0, 64) != 1 / math.sqrt(64):
        return True
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    N1, N2, S1, S2, D, Dv = 4, 2, 5, 6, 3, 2
    q = rng.standard_normal((1, N1, S1, D))
    k = rng.standard_normal((1, N2, S2, D))
    v = rng.standard_normal((1, N2, S2, Dv))
    dY = rng.standard_normal((1, N1, S1, Dv))
    Y, lse = mod.forward(q, k, v, "BNSD", softmax_scale=0.4, mask_mode=1)
    g = mod.backward(q, k, v, dY, Y, lse, "BNSD", softmax_scale=0.4, mask_mode=1)
    tq, tk, tv = (torch.tensor(a[0], requires_grad=True) for a in (q, k, v))
    S = 0.4 * torch.matmul(tq, tk.repeat_interleave(2, 0).transpose(1, 2).contiguous())
    okm = torch.from_numpy(np.tril(np.ones((S1, S2), dtype=bool), S2 - S1))
    out = torch.matmul(torch.softmax(S.masked_fill(~okm, float("-inf")), -1), tv.repeat_interleave(2, 0))
    (out * torch.from_numpy(dY[0])).sum().backward()
    for a, b in zip(g, (tq.grad, tk.grad, tv.grad)):
        if not np.allclose(a[0], b.numpy(), rtol=0, atol=1e-10):
            return True
    return not np.allclose(Y[0], out.detach().numpy(), rtol=0, atol=1e-12)


def rounding_pin_fails(mod):
    """The stored-mode roundings against the library casts: torch's float ->
    bfloat16 and numpy's float64 -> float16 (both round to nearest even)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000), rng.standard_normal(500) * 1e-6, rng.standard_normal(500) * 3e4])
    ref16 = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    if not np.array_equal(mod.bf16_round(x.astype(np.float32).astype(np.float64)), ref16):
        return True
    with np.errstate(over="ignore"):
        refh = x.astype(np.float16).astype(np.float64)
    return not np.array_equal(mod.f16_round(x), refh)


def seqused_pin_fails(mod):
    """seqused against the unpadded problem of the used lengths (the mutant's
    own plain path), with zero gradients on the padding, and an over-long
    seqused clamped to the sequence."""
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 6, 2, 3))
    k = rng.standard_normal((2, 7, 1, 3))
    v = rng.standard_normal((2, 7, 1, 2))
    dY = rng.standard_normal((2, 6, 2, 2))
    uq, ukv = np.array([4, 9]), np.array([5, 3])
    kw = dict(softmax_scale=0.5, mask_mode=1)
    try:
        Y, lse = mod.forward(q, k, v, "BSND", **kw, seqused_q=uq, seqused_kv=ukv)
        g = mod.backward(q, k, v, dY, Y, lse, "BSND", **kw, seqused_q=uq, seqused_kv=ukv)
    except Exception:
        return True
    for b, (u1, u2) in enumerate(((4, 5), (6, 3))):
        sl = (slice(b, b + 1),)
        Yt, lt = mod.forward(q[sl][:, :u1], k[sl][:, :u2], v[sl][:, :u2], "BSND", **kw)
        gt = mod.backward(q[sl][:, :u1], k[sl][:, :u2], v[sl][:, :u2], dY[sl][:, :u1], Yt, lt, "BSND", **kw)
        for full, part, u in zip(g, gt, (u1, u2, u2)):
            if not np.allclose(full[b, :u], part[0], atol=1e-12) or np.any(full[b, u:]):
                return True
    return False


def test_unmutated_oracle_passes_every_pin():
    src = open(SRC, encoding="utf-8").read()
    mod = types.ModuleType("oracle_plain")
    exec(compile(src, "<plain>", "exec"), mod.__dict__)
    assert not fd_pin_fails(mod)
    assert not library_pin_fails(mod)
    assert not rounding_pin_fails(mod)
    assert not seqused_pin_fails(mod)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = load_mutant(name)
    caught = library_pin_fails(mod) or fd_pin_fails(mod) or rounding_pin_fails(mod) or seqused_pin_fails(mod)
    assert caught, f"pins missed mutation {name}"
