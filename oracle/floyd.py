"""fp64 CPU oracle for Floyd attention: forward (to make attentionIn,
softmaxMax and softmaxSum) and backward (dQ, dK1, dV1, dK2, dV2).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark may import this module.  It shares no code with the HIP library and
never calls it.

Source: page "CANN Floyd注意力梯度算子" (jsqmd.com), section 功能说明 (the
computation formulas) and section 约束说明 / the parameter table of
aclnnFusedFloydAttentionGradGetWorkspaceSize (shapes and dtypes):

  Q, dY, Y   [B, H, N, M, D]
  K1, V1     [B, H, N, K, D]     (share the N axis with Q)
  K2, V2     [B, H, K, M, D]     (share the M axis with Q)
  mask       [B, 1, N, 1, K]     1 = the position takes no part, 0 = it does
  max, sum   [B, H, N, M, 8]     fp32 intermediates of the forward

  forward   S = Mask(scale * (Q K1^T + Q K2^T)) ; P = softmax(S) ; Y = P V1 + P V2
  backward  dV1 = P^T dY ; dV2 = P^T dY ; dQ = scale * (dS K1 + dS K2) ;
            dK1 = scale * dS^T Q ; dK2 = scale * dS^T Q

The page describes the operator as ordinary attention whose QK and PV products
become batch matmuls with a sequence axis as the batch axis.  Written out per
element (the plainest reading that the shapes admit):

  S[n, m, k] = scale * (Q[n, m] . K1[n, k] + Q[n, m] . K2[k, m])
  Y[n, m]    = sum_k P[n, m, k] (V1[n, k] + V2[k, m])

so the K1 / V1 products are batched over n (reducing over m for dK1 / dV1) and
the K2 / V2 products are batched over m (reducing over n for dK2 / dV2).

Readings taken where the page is silent:
  * the 1/sqrt(d) of the backward formulas is the operator's scaleValue (the
    page's example passes 1/sqrt(128) for D = 128);
  * softmaxMax is the row maximum of the scaled, masked scores and softmaxSum
    the sum of exp(S - max) over the row; the 8 trailing entries are copies of
    one value and the backward reads the first; P = exp(S - max) / sum;
  * sfmg = rowsum(dY (.) Y) with Y the attentionIn handed to the backward and
    dS = P (.) (dP - sfmg), dP = dY V1^T + dY V2^T (the softmax derivative,
    as in the ordinary attention backward);
  * a row with every key masked has max = -inf, sum = 0, P = 0 and Y = 0, and
    contributes nothing to any gradient.

Parity status: pinned by tests/test_floyd_oracle.py through the pins of
tests/floyd_pins.py: pure-Python brute force over every (n, m, k), central
finite differences of the forward, PyTorch fp64 autograd of an einsum forward,
reduction to the ordinary attention oracle when one K/V pair is zero, and the
closed form of the page's all-ones example (section 调用示例).
"""

import math

import numpy as np

N_COPIES = 8


def _swap(x):
    return np.swapaxes(x, -1, -2)


def _by_m(x):
    """[B, H, a, M, c] -> [B, H, M, a, c]: the M axis becomes a batch axis."""
    return np.moveaxis(x, 3, 2)


def _from_m(x):
    """Inverse of _by_m."""
    return np.moveaxis(x, 2, 3)


def _mask_bool(mask, B, N, K):
    if mask is None:
        return None
    m = np.asarray(mask).astype(bool)
    assert m.shape == (B, 1, N, 1, K), m.shape
    return m


def scores(q, k1, k2, scale, mask=None):
    """S[b,h,n,m,k] = scale * (Q[n,m].K1[n,k] + Q[n,m].K2[k,m]), masked
    positions set to -inf (section 功能说明, forward formula)."""
    B, H, N, M, D = q.shape
    K = k1.shape[3]
    t1 = q @ _swap(k1)                            # batched over (b, h, n)
    t2 = _from_m(_by_m(q) @ _swap(_by_m(k2)))     # batched over (b, h, m)
    s = scale * (t1 + t2)
    mb = _mask_bool(mask, B, N, K)
    if mb is not None:
        s = np.where(mb, -np.inf, s)
    return s


def forward(q, k1, v1, k2, v2, scale, mask=None):
    """Returns Y [B,H,N,M,D] and softmax max / sum [B,H,N,M,8] (fp64)."""
    s = scores(q, k1, k2, scale, mask)
    mx = s.max(axis=-1)
    live = np.isfinite(mx)
    e = np.where(live[..., None], np.exp(s - np.where(live, mx, 0.0)[..., None]), 0.0)
    sm = e.sum(axis=-1)
    p = np.where(live[..., None], e / np.where(live, sm, 1.0)[..., None], 0.0)
    y = p @ v1 + _from_m(_by_m(p) @ _by_m(v2))
    mx = np.where(live, mx, -np.inf)
    rep = lambda a: np.repeat(a[..., None], N_COPIES, axis=-1)
    return y, rep(mx), rep(sm)


def probabilities(q, k1, k2, scale, softmax_max, softmax_sum, mask=None):
    """P = exp(S - max) / sum from the stored statistics (first of the 8
    copies); rows with max = -inf or sum = 0 give P = 0."""
    s = scores(q, k1, k2, scale, mask)
    mx = np.asarray(softmax_max, dtype=np.float64)[..., 0]
    sm = np.asarray(softmax_sum, dtype=np.float64)[..., 0]
    live = np.isfinite(mx) & (sm > 0)
    safe_mx = np.where(live, mx, 0.0)
    safe_sm = np.where(live, sm, 1.0)
    with np.errstate(over="ignore"):
        p = np.exp(s - safe_mx[..., None]) / safe_sm[..., None]
    return np.where(live[..., None], p, 0.0)


def backward(q, k1, v1, k2, v2, dy, y, softmax_max, softmax_sum, scale, mask=None):
    """(dQ, dK1, dV1, dK2, dV2) in fp64 (section 功能说明, backward formulas)."""
    p = probabilities(q, k1, k2, scale, softmax_max, softmax_sum, mask)
    dp = dy @ _swap(v1) + _from_m(_by_m(dy) @ _swap(_by_m(v2)))
    sfmg = (dy * y).sum(axis=-1)
    ds = p * (dp - sfmg[..., None])
    dv1 = _swap(p) @ dy
    dv2 = _from_m(_swap(_by_m(p)) @ _by_m(dy))
    dk1 = scale * (_swap(ds) @ q)
    dk2 = scale * _from_m(_swap(_by_m(ds)) @ _by_m(q))
    dq = scale * (ds @ k1 + _from_m(_by_m(ds) @ _by_m(k2)))
    return dq, dk1, dv1, dk2, dv2


def flops(B, H, N, M, K, D, mask=None):
    """Algorithmic FLOP of one backward: each unmasked (n, m, k) triple costs
    2*D for each of the ten products Q.K1, Q.K2, dY.V1, dY.V2, dV1, dV2, dK1,
    dK2 and the two terms of dQ, i.e. 20 * D."""
    if mask is None:
        live = B * N * K
    else:
        live = int((~np.asarray(mask).astype(bool)).sum())
    return 20.0 * D * H * M * live


def default_scale(D):
    """1/sqrt(D), the value the page's example passes for scaleValue."""
    return 1.0 / math.sqrt(D)

