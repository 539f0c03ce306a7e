"""fp64 CPU oracle: attention forward (to make Y and softmax_lse) and the
FlashAttention backward (dQ, dK, dV), as plain NumPy definitions.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library and never calls it.

Source of every formula: page "CANN ops-transformer FlashAttnGrad 算子详解"
(discosf.com), section 一 "算子功能与数学原理":

  forward   S = scale * Q K^T ;  P_ij = exp(S_ij - softmax_lse_i) ;  Y = P V
  scale     softmax_scale if it is non-zero, else 1/sqrt(D), D the Q/K head dim
  backward  dV = P^T dY ;  dP = dY V^T ;  sfmg = rowsum(dY (.) Y) ;
            dS = P (.) (dP - sfmg) ;  dQ = scale * dS K ;  dK = scale * dS^T Q
  GQA       N1 query heads share N2 key/value heads, N1 a multiple of N2

and section 四 4.6 (constraints): layouts BSND / BNSD / TND, softmax_lse of
shape (B, N1, S1) for BSND/BNSD and (N1, T1) for TND, TND sequences delimited
by cu_seqlens, dense attention iff mask_mode = 0 with no window.

Readings taken where the page is silent (the enum table and the parameter
table were lost in extraction):
  * mask_mode 0 = none, 1 = causal, 2 = sliding window; the diagonal is aligned
    bottom-right (key j is visible to query i iff j <= i + s2 - s1 [+ win_right]);
  * window bounds are inclusive, -1 means unbounded on that side; causal mode
    keeps win_left as an optional left bound;
  * query head n1 uses key/value head n1 // (N1 / N2) (contiguous groups, the
    loop order B, N2, G, S1, S2 named by the page's BN2GS1S2 template);
  * lse is the natural-log log-sum-exp of the scaled, masked scores; a query
    row with no visible key has lse = -inf and contributes nothing;
  * sfmg uses the attn_out tensor handed to the backward (the stored Y).

Parity status: every function here is pinned by tests/test_oracle.py
(finite differences, softmax invariants, the explicit softmax Jacobian,
pure-Python brute force, closed forms, library routines and equivalences).
"""

import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_WINDOW = 2


def resolve_scale(softmax_scale, D):
    """Scale rule of section 一: a non-zero softmax_scale is used as is; zero
    selects 1/sqrt(D) with D the Query/Key head dim."""
    return float(softmax_scale) if softmax_scale != 0 else 1.0 / math.sqrt(D)


def mask_bounds(mask_mode, win_left=-1, win_right=-1):
    """(left, right) band half-widths for a mask_mode (section 四 4.3/4.6);
    -1 means unbounded.  Causal keeps win_left as an optional left bound and
    closes the right side at the diagonal."""
    if mask_mode == MASK_NONE:
        return -1, -1
    if mask_mode == MASK_CAUSAL:
        return int(win_left), 0
    if mask_mode == MASK_WINDOW:
        return int(win_left), int(win_right)
    raise ValueError(f"unknown mask_mode {mask_mode}")


def allowed_matrix(s1, s2, left, right):
    """Boolean [s1, s2]: True where query i may attend key j.  Bottom-right
    aligned diagonal i + (s2 - s1); band [diag - left, diag + right]."""
    off = s2 - s1
    i = np.arange(s1)[:, None]
    j = np.arange(s2)[None, :]
    ok = np.ones((s1, s2), dtype=bool)
    if left >= 0:
        ok &= j >= i + off - left
    if right >= 0:
        ok &= j <= i + off + right
    return ok


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value (ties to even),
    returned as float64.  bfloat16 keeps 8 significant bits and float32's
    exponent range; below 2**-126 the spacing is fixed at 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    return np.round(x / quantum) * quantum


def f16_round(x):
    """Round float64 values to the nearest IEEE binary16 (fp16) value (ties to
    even), returned as float64.  binary16 keeps 11 significant bits, normal
    numbers down to 2**-14 and a fixed spacing of 2**-24 below; its largest
    finite value is 65504, and magnitudes from 65520 up round to infinity."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -13)
    quantum = np.ldexp(1.0, e - 11)
    r = np.round(x / quantum) * quantum
    return np.where(np.abs(r) > 65504.0, np.copysign(np.inf, x), r)


ROUND = {"bf16": bf16_round, "fp16": f16_round}


# ---------------------------------------------------------------- layouts

def _seq_bounds(layout, B, S, cu):
    if layout == "TND":
        cu = np.asarray(cu, dtype=np.int64)
        return [(int(cu[b]), int(cu[b + 1])) for b in range(len(cu) - 1)]
    return [(0, S)] * B


def split_heads(x, layout, cu=None):
    """Layout tensor -> list over sequences of float64 arrays [N, s, d].
    BSND is [B, S, N, d]; BNSD is [B, N, S, d]; TND is [T, N, d] cut by cu."""
    x = np.asarray(x, dtype=np.float64)
    if layout == "BSND":
        return [x[b].transpose(1, 0, 2) for b in range(x.shape[0])]
    if layout == "BNSD":
        return [x[b] for b in range(x.shape[0])]
    if layout == "TND":
        return [x[a:e].transpose(1, 0, 2) for a, e in _seq_bounds("TND", 0, 0, cu)]
    raise ValueError(layout)


def merge_heads(parts, layout, shape):
    """Inverse of split_heads into a new float64 array of `shape`."""
    out = np.zeros(shape, dtype=np.float64)
    if layout == "BSND":
        for b, p in enumerate(parts):
            out[b] = p.transpose(1, 0, 2)
    elif layout == "BNSD":
        for b, p in enumerate(parts):
            out[b] = p
    elif layout == "TND":
        t = 0
        for p in parts:
            s = p.shape[1]
            out[t:t + s] = p.transpose(1, 0, 2)
            t += s
    else:
        raise ValueError(layout)
    return out


def _split_lse(lse, layout, cu):
    """softmax_lse is (B, N1, S1) for BSND/BNSD and (N1, T1) for TND."""
    lse = np.asarray(lse, dtype=np.float64)
    if layout == "TND":
        return [lse[:, a:e] for a, e in _seq_bounds("TND", 0, 0, cu)]
    return [lse[b] for b in range(lse.shape[0])]


def _merge_lse(parts, layout, shape):
    out = np.zeros(shape, dtype=np.float64)
    if layout == "TND":
        t = 0
        for p in parts:
            out[:, t:t + p.shape[1]] = p
            t += p.shape[1]
    else:
        for b, p in enumerate(parts):
            out[b] = p
    return out


# ---------------------------------------------------------------- one head

def head_forward(q, k, v, scale, allowed):
    """Forward of one (sequence, query head): q [s1, D], k [s2, D], v [s2, Dv].
    Returns Y [s1, Dv] and lse [s1] (natural log; -inf for an empty row)."""
    S = scale * (q @ k.T)
    S = np.where(allowed, S, -np.inf)
    s1 = q.shape[0]
    lse = np.full(s1, -np.inf)
    Y = np.zeros((s1, v.shape[1]))
    rows = allowed.any(axis=1)
    if rows.any():
        Sr = S[rows]
        m = Sr.max(axis=1)
        lse[rows] = m + np.log(np.exp(Sr - m[:, None]).sum(axis=1))
        P = np.exp(Sr - lse[rows][:, None])
        Y[rows] = P @ v
    return Y, lse


def head_backward(q, k, v, dY, Y, lse, scale, allowed):
    """Backward of one (sequence, query head), every step of section 一 kept
    separate.  Returns a dict with P, dP, sfmg, dS, dq, dk, dv."""
    S = scale * (q @ k.T)
    live = allowed & np.isfinite(lse)[:, None]
    P = np.zeros_like(S)
    P[live] = np.exp((S - np.where(np.isfinite(lse), lse, 0.0)[:, None])[live])
    dv = P.T @ dY
    dP = dY @ v.T
    sf = (dY * Y).sum(axis=1)
    dS = P * (dP - sf[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return {"P": P, "dP": dP, "sfmg": sf, "dS": dS, "dq": dq, "dk": dk, "dv": dv}


# ---------------------------------------------------------------- whole problem

def _problem(q, k, layout, cu_q, cu_kv):
    qs = split_heads(q, layout, cu_q)
    ks = split_heads(k, layout, cu_kv)
    if len(qs) != len(ks):
        raise ValueError("q and k hold different numbers of sequences")
    N1, N2 = qs[0].shape[0], ks[0].shape[0]
    if N1 % N2:
        raise ValueError("N1 must be a multiple of N2")
    return qs, ks, N1, N2, N1 // N2


def _lse_shape(q, layout):
    q = np.asarray(q)
    if layout == "TND":
        return (q.shape[1], q.shape[0])
    if layout == "BSND":
        return (q.shape[0], q.shape[2], q.shape[1])
    return (q.shape[0], q.shape[1], q.shape[2])


def used_lengths(b, s1, s2, seqused_q=None, seqused_kv=None):
    """Rows and keys of sequence b that take part (reading: the page only names
    seqused_q / seqused_kv; the first seqused[b] rows of a sequence take part,
    clamped to [0, its length], and the rest are padding)."""
    u1 = s1 if seqused_q is None else min(max(int(seqused_q[b]), 0), s1)
    u2 = s2 if seqused_kv is None else min(max(int(seqused_kv[b]), 0), s2)
    return u1, u2


def forward(q, k, v, layout="BSND", cu_q=None, cu_kv=None, softmax_scale=0.0,
            mask_mode=0, win_left=-1, win_right=-1, seqused_q=None, seqused_kv=None):
    """Y (layout of q with Dv) and lse (float64) for the whole problem.  Rows
    past seqused_q get Y = 0 and lse = -inf; keys past seqused_kv are not
    attended; the diagonal aligns on the used lengths."""
    qs, ks, N1, N2, G = _problem(q, k, layout, cu_q, cu_kv)
    vs = split_heads(v, layout, cu_kv)
    scale = resolve_scale(softmax_scale, qs[0].shape[2])
    left, right = mask_bounds(mask_mode, win_left, win_right)
    Ys, lses = [], []
    for b, (qb, kb, vb) in enumerate(zip(qs, ks, vs)):
        s1, s2 = qb.shape[1], kb.shape[1]
        u1, u2 = used_lengths(b, s1, s2, seqused_q, seqused_kv)
        ok = allowed_matrix(u1, u2, left, right)
        Yb = np.zeros((N1, s1, vb.shape[2]))
        lb = np.full((N1, s1), -np.inf)
        for n1 in range(N1):
            Yb[n1, :u1], lb[n1, :u1] = head_forward(qb[n1, :u1], kb[n1 // G, :u2], vb[n1 // G, :u2], scale, ok)
        Ys.append(Yb)
        lses.append(lb)
    qa = np.asarray(q)
    yshape = qa.shape[:-1] + (np.asarray(v).shape[-1],)
    return merge_heads(Ys, layout, yshape), _merge_lse(lses, layout, _lse_shape(q, layout))


def store(Y, lse, dtype="bf16"):
    """What a forward hands to the backward: Y rounded to the element type
    ("bf16" or "fp16", kept as float64 values) and lse rounded to float32."""
    return ROUND[dtype](Y), np.asarray(lse, dtype=np.float64).astype(np.float32)


def sfmg(dY, Y, layout="BSND", cu_q=None):
    """sfmg = rowsum(dY (.) Y) per (query row, head), in softmax_lse's layout."""
    dYs = split_heads(dY, layout, cu_q)
    Ys = split_heads(Y, layout, cu_q)
    parts = [(a * b).sum(axis=2) for a, b in zip(dYs, Ys)]
    return _merge_lse(parts, layout, _lse_shape(dY, layout))


def backward(q, k, v, dY, Y, lse, layout="BSND", cu_q=None, cu_kv=None,
             softmax_scale=0.0, mask_mode=0, win_left=-1, win_right=-1, seqused_q=None,
             seqused_kv=None):
    """dq, dk, dv (float64, shapes of q, k, v).  dK/dV of key/value head n2
    sum the contributions of its G query heads.  With seqused_q / seqused_kv
    only the used rows and keys take part (see used_lengths); the gradients of
    the rest are zero."""
    qs, ks, N1, N2, G = _problem(q, k, layout, cu_q, cu_kv)
    vs = split_heads(v, layout, cu_kv)
    dYs = split_heads(dY, layout, cu_q)
    Yst = split_heads(Y, layout, cu_q)
    lses = _split_lse(lse, layout, cu_q)
    scale = resolve_scale(softmax_scale, qs[0].shape[2])
    left, right = mask_bounds(mask_mode, win_left, win_right)
    dqs, dks, dvs = [], [], []
    for b, (qb, kb, vb, dyb, yb, lb) in enumerate(zip(qs, ks, vs, dYs, Yst, lses)):
        s1, s2 = qb.shape[1], kb.shape[1]
        u1, u2 = used_lengths(b, s1, s2, seqused_q, seqused_kv)
        ok = allowed_matrix(u1, u2, left, right)
        dqb = np.zeros_like(qb)
        dkb = np.zeros_like(kb)
        dvb = np.zeros_like(vb)
        for n1 in range(N1):
            n2 = n1 // G
            r = head_backward(qb[n1, :u1], kb[n2, :u2], vb[n2, :u2], dyb[n1, :u1], yb[n1, :u1], lb[n1, :u1],
                              scale, ok)
            dqb[n1, :u1] = r["dq"]
            dkb[n2, :u2] += r["dk"]
            dvb[n2, :u2] += r["dv"]
        dqs.append(dqb)
        dks.append(dkb)
        dvs.append(dvb)
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    return (merge_heads(dqs, layout, q.shape), merge_heads(dks, layout, k.shape),
            merge_heads(dvs, layout, v.shape))


def backward_rows(q, k, v, dY, Y, lse, q_rows, kv_rows, layout="BSND", cu_q=None,
                  cu_kv=None, softmax_scale=0.0, mask_mode=0, win_left=-1, win_right=-1):
    """The same backward, evaluated only at chosen rows, for problems too large
    to run whole.  q_rows: list of (b, n1, i) -> dq row; kv_rows: list of
    (b, n2, j) -> (dk row, dv row).  Each row uses the full row (or column) of
    P, dP and sfmg it depends on, straight from the definitions."""
    qs, ks, N1, N2, G = _problem(q, k, layout, cu_q, cu_kv)
    vs = split_heads(v, layout, cu_kv)
    dYs = split_heads(dY, layout, cu_q)
    Yst = split_heads(Y, layout, cu_q)
    lses = _split_lse(lse, layout, cu_q)
    scale = resolve_scale(softmax_scale, qs[0].shape[2])
    left, right = mask_bounds(mask_mode, win_left, win_right)

    def visible(s1, s2, i, j):
        off = s2 - s1
        i = np.asarray(i)[:, None]
        j = np.asarray(j)[None, :]
        ok = np.ones((i.shape[0], j.shape[1]), dtype=bool)
        if left >= 0:
            ok &= j >= i + off - left
        if right >= 0:
            ok &= j <= i + off + right
        return ok

    dq_out = []
    for (b, n1, i) in q_rows:
        qb, kb, vb = qs[b][n1], ks[b][n1 // G], vs[b][n1 // G]
        s1, s2 = qb.shape[0], kb.shape[0]
        li = lses[b][n1, i]
        ok = visible(s1, s2, [i], np.arange(s2))[0] & np.isfinite(li)
        Srow = scale * (kb @ qb[i])
        P = np.where(ok, np.exp(Srow - (li if np.isfinite(li) else 0.0)), 0.0)
        dP = vb @ dYs[b][n1, i]
        sf = float(dYs[b][n1, i] @ Yst[b][n1, i])
        dS = P * (dP - sf)
        dq_out.append(scale * (dS @ kb))

    dk_out, dv_out = [], []
    for (b, n2, j) in kv_rows:
        kb, vb = ks[b][n2], vs[b][n2]
        s2 = kb.shape[0]
        dk = np.zeros(kb.shape[1])
        dv = np.zeros(vb.shape[1])
        for n1 in range(n2 * G, (n2 + 1) * G):
            qb, dyb, yb, lb = qs[b][n1], dYs[b][n1], Yst[b][n1], lses[b][n1]
            s1 = qb.shape[0]
            ok = visible(s1, s2, np.arange(s1), [j])[:, 0] & np.isfinite(lb)
            Scol = scale * (qb @ kb[j])
            P = np.where(ok, np.exp(Scol - np.where(np.isfinite(lb), lb, 0.0)), 0.0)
            dP = dyb @ vb[j]
            sf = (dyb * yb).sum(axis=1)
            dS = P * (dP - sf)
            dv += P @ dyb
            dk += scale * (dS @ qb)
        dk_out.append(dk)
        dv_out.append(dv)
    return dq_out, dk_out, dv_out
