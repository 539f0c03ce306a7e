"""Pins of the Floyd attention oracle (page "CANN Floyd注意力梯度算子", section
功能说明 for the formulas, section 调用示例 for the all-ones example).  Each
function takes an oracle module (the real one or a copy with a planted
mistake) and returns True when the pin rejects it.  Nothing here imports the
HIP library."""

import math

import numpy as np


def rand_problem(B, H, N, M, K, D, seed, masked_rows=(), masked_keys=0.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, M, D))
    k1 = rng.standard_normal((B, H, N, K, D))
    v1 = rng.standard_normal((B, H, N, K, D))
    k2 = rng.standard_normal((B, H, K, M, D))
    v2 = rng.standard_normal((B, H, K, M, D))
    dy = rng.standard_normal((B, H, N, M, D))
    mask = None
    if masked_rows or masked_keys:
        mask = rng.random((B, 1, N, 1, K)) < masked_keys
        for (b, n) in masked_rows:
            mask[b, 0, n, 0, :] = True
    return q, k1, v1, k2, v2, dy, mask


def brute_force(q, k1, v1, k2, v2, dy, scale, mask=None):
    """Pure-Python loops over every (b, h, n, m, k): forward statistics, Y and
    the five gradients from the per-element formulas, no array products.
    Returns (Y, max, sum, dQ, dK1, dV1, dK2, dV2); the gradients use Y and the
    statistics of this same forward."""
    B, H, N, M, D = q.shape
    K = k1.shape[3]
    dot = lambda a, b: sum(float(a[i]) * float(b[i]) for i in range(D))
    Y = np.zeros(q.shape)
    MX = np.full((B, H, N, M), -math.inf)
    SM = np.zeros((B, H, N, M))
    dQ, dK1, dV1 = np.zeros(q.shape), np.zeros(k1.shape), np.zeros(v1.shape)
    dK2, dV2 = np.zeros(k2.shape), np.zeros(v2.shape)
    for b in range(B):
        for h in range(H):
            for n in range(N):
                keys = [k for k in range(K) if mask is None or not mask[b][0][n][0][k]]
                for m in range(M):
                    if not keys:
                        continue
                    s = {k: scale * (dot(q[b, h, n, m], k1[b, h, n, k]) + dot(q[b, h, n, m], k2[b, h, k, m]))
                         for k in keys}
                    mx = max(s.values())
                    ex = {k: math.exp(s[k] - mx) for k in keys}
                    sm = sum(ex.values())
                    MX[b, h, n, m], SM[b, h, n, m] = mx, sm
                    p = {k: ex[k] / sm for k in keys}
                    for d in range(D):
                        Y[b, h, n, m, d] = sum(p[k] * (v1[b, h, n, k, d] + v2[b, h, k, m, d]) for k in keys)
                    g = dy[b, h, n, m]
                    sf = dot(g, Y[b, h, n, m])
                    for k in keys:
                        dsk = p[k] * (dot(g, v1[b, h, n, k]) + dot(g, v2[b, h, k, m]) - sf)
                        for d in range(D):
                            dV1[b, h, n, k, d] += p[k] * g[d]
                            dV2[b, h, k, m, d] += p[k] * g[d]
                            dK1[b, h, n, k, d] += scale * dsk * q[b, h, n, m, d]
                            dK2[b, h, k, m, d] += scale * dsk * q[b, h, n, m, d]
                            dQ[b, h, n, m, d] += scale * dsk * (k1[b, h, n, k, d] + k2[b, h, k, m, d])
    return Y, MX, SM, dQ, dK1, dV1, dK2, dV2


def _close(a, b, tol=1e-10):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    if not np.array_equal(fin, np.isfinite(a)) or not np.array_equal(a[~fin], b[~fin]):
        return False
    return bool(np.all(np.abs(a[fin] - b[fin]) <= tol * (1.0 + np.abs(b[fin]))))


def brute_force_pin_fails(mod):
    """Forward and backward against the loops, with N != M != K, two heads, a
    key mask and one fully masked row of n."""
    for seed, rows, frac in [(1, (), 0.0), (2, ((0, 1),), 0.3), (3, ((1, 0),), 0.5)]:
        q, k1, v1, k2, v2, dy, mask = rand_problem(2, 2, 3, 4, 5, 3, seed, rows, frac)
        scale = 0.37
        try:
            y, mx, sm = mod.forward(q, k1, v1, k2, v2, scale, mask)
            bf = brute_force(q, k1, v1, k2, v2, dy, scale, mask)
            if not (_close(y, bf[0]) and _close(mx[..., 0], bf[1]) and _close(sm[..., 0], bf[2])):
                return True
            if not (np.array_equal(mx[..., 0:1].repeat(8, -1), mx) and np.array_equal(sm[..., 0:1].repeat(8, -1), sm)):
                return True
            g = mod.backward(q, k1, v1, k2, v2, dy, y, mx, sm, scale, mask)
        except (ValueError, AssertionError, IndexError):
            return True
        if not all(_close(a, b) for a, b in zip(g, bf[3:])):
            return True
    return False


def fd_pin_fails(mod):
    """Central differences of the module's own forward (loss sum(Y * dY))
    against its backward, with a key mask."""
    q, k1, v1, k2, v2, dy, mask = rand_problem(1, 2, 2, 3, 4, 2, 7, (), 0.25)
    scale = 0.6
    try:
        y, mx, sm = mod.forward(q, k1, v1, k2, v2, scale, mask)
        g = mod.backward(q, k1, v1, k2, v2, dy, y, mx, sm, scale, mask)
    except (ValueError, AssertionError, IndexError):
        return True
    h = 1e-6
    xs = [q, k1, v1, k2, v2]
    order = [0, 1, 2, 3, 4]  # dQ, dK1, dV1, dK2, dV2
    for gi, xi in enumerate(order):
        fd = np.zeros_like(xs[xi])
        for idx in np.ndindex(xs[xi].shape):
            args = [x.copy() for x in xs]
            args[xi][idx] += h
            lp = float((mod.forward(*args, scale, mask)[0] * dy).sum())
            args[xi][idx] -= 2 * h
            lm = float((mod.forward(*args, scale, mask)[0] * dy).sum())
            fd[idx] = (lp - lm) / (2 * h)
        if g[gi].shape != fd.shape or np.abs(g[gi] - fd).max() > 1e-6 * max(np.abs(fd).max(), 1e-3):
            return True
    return False


def autograd_pin_fails(mod):
    """The backward against PyTorch fp64 autograd of an einsum forward, in
    which the gradients come from the library's differentiation rules."""
    import torch

    q, k1, v1, k2, v2, dy, mask = rand_problem(1, 2, 3, 4, 5, 4, 11, ((0, 2),), 0.2)
    scale = 0.45
    t = [torch.tensor(x, requires_grad=True) for x in (q, k1, v1, k2, v2)]
    s = scale * (torch.einsum("bhnmd,bhnkd->bhnmk", t[0], t[1]) + torch.einsum("bhnmd,bhkmd->bhnmk", t[0], t[3]))
    mt = torch.tensor(mask)
    s = s.masked_fill(mt, -math.inf)
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)  # fully masked rows: 0
    y = torch.einsum("bhnmk,bhnkd->bhnmd", p, t[2]) + torch.einsum("bhnmk,bhkmd->bhnmd", p, t[4])
    (y * torch.tensor(dy)).sum().backward()
    try:
        yo, mx, sm = mod.forward(q, k1, v1, k2, v2, scale, mask)
        g = mod.backward(q, k1, v1, k2, v2, dy, yo, mx, sm, scale, mask)
    except (ValueError, AssertionError, IndexError):
        return True
    if not _close(yo, y.detach().numpy(), 1e-10):
        return True
    return not all(_close(a, x.grad.numpy(), 1e-9) for a, x in zip(g, t))


def reduction_pin_fails(mod):
    """With K2 = V2 = 0 the problem at each (b, h, n) is ordinary attention of
    queries Q[n, :] over keys K1[n, :] (masked keys removed); with K1 = V1 = 0
    and no mask it is ordinary attention at each (b, h, m) of queries Q[:, m]
    over keys K2[:, m].  Compared with the ordinary-attention oracle (page
    "CANN ops-transformer FlashAttnGrad 算子详解"), which has pins of its own."""
    import oracle

    B, H, N, M, K, D = 1, 2, 3, 4, 5, 3
    scale = 0.5
    q, k1, v1, k2, v2, dy, mask = rand_problem(B, H, N, M, K, D, 21, ((0, 1),), 0.3)
    z2 = np.zeros_like(k2)
    try:
        y, mx, sm = mod.forward(q, k1, v1, z2, z2, scale, mask)
        dq, dk1, dv1, dk2, dv2 = mod.backward(q, k1, v1, z2, z2, dy, y, mx, sm, scale, mask)
    except (ValueError, AssertionError, IndexError):
        return True
    for b in range(B):
        for h in range(H):
            for n in range(N):
                keep = [k for k in range(K) if not mask[b, 0, n, 0, k]]
                if not keep:
                    if np.any(y[b, h, n]) or np.any(dq[b, h, n]) or np.any(dk1[b, h, n]) or np.any(dv1[b, h, n]):
                        return True
                    continue
                qq = q[b, h, n][None, None]
                kk, vv = k1[b, h, n, keep][None, None], v1[b, h, n, keep][None, None]
                gg = dy[b, h, n][None, None]
                Y, lse = oracle.forward(qq, kk, vv, "BNSD", softmax_scale=scale)
                rq, rk, rv = oracle.backward(qq, kk, vv, gg, Y, lse, "BNSD", softmax_scale=scale)
                if not (_close(y[b, h, n], Y[0, 0]) and _close(mx[b, h, n, :, 0] + np.log(sm[b, h, n, :, 0]), lse[0, 0])):
                    return True
                if not (_close(dq[b, h, n], rq[0, 0]) and _close(dk1[b, h, n, keep], rk[0, 0])
                        and _close(dv1[b, h, n, keep], rv[0, 0])):
                    return True
                drop = [k for k in range(K) if k not in keep]
                if np.any(dk1[b, h, n, drop]) or np.any(dv1[b, h, n, drop]):
                    return True
    z1 = np.zeros_like(k1)
    try:
        y, mx, sm = mod.forward(q, z1, z1, k2, v2, scale, None)
        dq, dk1, dv1, dk2, dv2 = mod.backward(q, z1, z1, k2, v2, dy, y, mx, sm, scale, None)
    except (ValueError, AssertionError, IndexError):
        return True
    for b in range(B):
        for h in range(H):
            for m in range(M):
                qq, gg = q[b, h, :, m][None, None], dy[b, h, :, m][None, None]
                kk, vv = k2[b, h, :, m][None, None], v2[b, h, :, m][None, None]
                Y, lse = oracle.forward(qq, kk, vv, "BNSD", softmax_scale=scale)
                rq, rk, rv = oracle.backward(qq, kk, vv, gg, Y, lse, "BNSD", softmax_scale=scale)
                if not (_close(y[b, h, :, m], Y[0, 0]) and _close(dq[b, h, :, m], rq[0, 0])
                        and _close(dk2[b, h, :, m], rk[0, 0]) and _close(dv2[b, h, :, m], rv[0, 0])):
                    return True
    return False


def closed_form_pin_fails(mod):
    """The page's example (section 调用示例): B = 1, one head, S1 = S2 = S3 =
    256, D = 128, every input 1.0, no position masked, softmaxMax =
    softmaxSum = 3.0 and scaleValue = 1/sqrt(128).  The page prints no output;
    by hand, every score is s = scale * 2D, every probability p = exp(s - 3) / 3,
    dP = dY . (V1 + V2) = 2D and sfmg = dY . Y = D, so dS = p * D and
      dV1 = M p,  dV2 = N p,  dK1 = scale M D p,  dK2 = scale N D p,
      dQ = 2 scale K D p   (every element).
    Run at the page's sizes in the page's index order [B, N, S1, S2, D]."""
    B, H, N, M, K, D = 1, 1, 256, 256, 256, 128
    scale = 1.0 / math.sqrt(128)
    one = lambda *s: np.ones(s)
    q, dy, y = one(B, H, N, M, D), one(B, H, N, M, D), one(B, H, N, M, D)
    k1, v1 = one(B, H, N, K, D), one(B, H, N, K, D)
    k2, v2 = one(B, H, K, M, D), one(B, H, K, M, D)
    mask = np.zeros((B, 1, N, 1, K), dtype=np.uint8)
    stat = np.full((B, H, N, M, 8), 3.0)
    try:
        dq, dk1, dv1, dk2, dv2 = mod.backward(q, k1, v1, k2, v2, dy, y, stat, stat, scale, mask)
    except (ValueError, AssertionError, IndexError):
        return True
    s = scale * 2 * D
    p = math.exp(s - 3.0) / 3.0
    want = [(dq, 2 * scale * K * D * p), (dk1, scale * M * D * p), (dv1, M * p), (dk2, scale * N * D * p),
            (dv2, N * p)]
    return not all(np.allclose(g, w, rtol=1e-12, atol=0) for g, w in want)


PINS = {
    "brute_force": brute_force_pin_fails,
    "finite_differences": fd_pin_fails,
    "autograd": autograd_pin_fails,
    "ordinary_attention": reduction_pin_fails,
    "page_example": closed_form_pin_fails,
}
