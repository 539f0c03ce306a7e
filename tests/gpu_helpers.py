"""Shared helpers of the GPU parity tests: inputs from the seeded generator,
expected values from the fp64 oracle, the device result from the C ABI
(through the binding), and the tolerance of the comparison."""

import sys

import numpy as np

import oracle
from flashattention_backward_fa_amd import workloads as W

# bf16 outputs against the stored-mode fp64 oracle, per output tensor
REL_FRO_TOL = 1e-2
MAX_ABS_TOL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.double().numpy()


def oracle_inputs(cfg, x, dtype="bf16"):
    """Stored-mode Y (values of the element type) and lse (fp32) from the
    oracle forward."""
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    Y, lse = oracle.forward(q, k, v, cfg["layout"], x["cu_q"], x["cu_kv"], cfg["softmax_scale"],
                            cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    return oracle.store(Y, lse, dtype)


def oracle_backward(cfg, x, Yst, lst):
    return oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["dout"]), Yst, lst, cfg["layout"],
                           x["cu_q"], x["cu_kv"], cfg["softmax_scale"], cfg["mask_mode"], cfg["win_left"],
                           cfg["win_right"])


def max_lengths(cfg, x):
    if cfg["layout"] != "TND":
        return -1, -1
    cq, ck = x["cu_q"], x["cu_kv"]
    return int(np.diff(cq).max()), int(np.diff(ck).max())


def gpu_backward(cfg, x, Yst, lst, **extra):
    import torch
    import flashattention_backward_fa_amd as fa

    dev = torch.device("cuda", 0)
    t = {k: x[k].to(dev) for k in ("q", "k", "v", "dout")}
    attn_out = torch.from_numpy(np.ascontiguousarray(Yst)).to(x["q"].dtype).to(dev)
    lse = torch.from_numpy(np.ascontiguousarray(lst, dtype=np.float32)).to(dev)
    cu_q = cu_kv = None
    if cfg["layout"] == "TND":
        cu_q = torch.from_numpy(x["cu_q"]).to(dev)
        cu_kv = torch.from_numpy(x["cu_kv"]).to(dev)
    mq, mk = max_lengths(cfg, x)
    kw = dict(cu_seqlens_q=cu_q, cu_seqlens_kv=cu_kv, softmax_scale=cfg["softmax_scale"],
              mask_mode=cfg["mask_mode"], win_left=cfg["win_left"], win_right=cfg["win_right"],
              max_seqlen_q=mq, max_seqlen_kv=mk, layout=cfg["layout"])
    kw.update(extra)
    dq, dk, dv = fa.flash_attn_grad(t["q"], t["k"], t["v"], t["dout"], attn_out, lse, **kw)
    torch.cuda.synchronize()
    return f64(dq.cpu()), f64(dk.cpu()), f64(dv.cpu())


def empty_rows(cfg, x, q_shape, k_shape):
    """Boolean arrays over the row axes of q and k: True for query rows that
    see no key and key rows that no query sees (their gradients must be
    exactly zero)."""
    L, R = oracle.mask_bounds(cfg["mask_mode"], cfg["win_left"], cfg["win_right"])
    lay = cfg["layout"]
    qe = np.zeros(q_shape[:-1], dtype=bool)
    ke = np.zeros(k_shape[:-1], dtype=bool)
    if lay == "TND":
        cq, ck = x["cu_q"], x["cu_kv"]
        for b in range(len(cq) - 1):
            ok = oracle.allowed_matrix(int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b]), L, R)
            qe[cq[b]:cq[b + 1], :] = ~ok.any(axis=1)[:, None]
            ke[ck[b]:ck[b + 1], :] = ~ok.any(axis=0)[:, None]
        return qe, ke
    ok = oracle.allowed_matrix(cfg["S1"], cfg["S2"], L, R)
    if lay == "BSND":
        qe[:] = ~ok.any(axis=1)[None, :, None]
        ke[:] = ~ok.any(axis=0)[None, :, None]
    else:
        qe[:] = ~ok.any(axis=1)[None, None, :]
        ke[:] = ~ok.any(axis=0)[None, None, :]
    return qe, ke


def errors(got, ref):
    err = got - ref
    nref = np.linalg.norm(ref)
    mref = np.abs(ref).max() if ref.size else 0.0
    rel = np.linalg.norm(err) / nref if nref > 0 else (0.0 if not np.any(err) else np.inf)
    mx = np.abs(err).max() / mref if mref > 0 else (0.0 if not np.any(err) else np.inf)
    return rel, mx


def assert_all_close(triples):
    """Report every tensor's errors, then fail on the first one out of tolerance."""
    bad = []
    for got, ref, name in triples:
        rel, mx = errors(got, ref)
        say(f"    {name}: rel_fro={rel:.3e} max_abs_ratio={mx:.3e}")
        if rel > REL_FRO_TOL or mx > MAX_ABS_TOL:
            bad.append(f"{name}: rel_fro {rel:.3e} (tol {REL_FRO_TOL}), max_abs_ratio {mx:.3e} (tol {MAX_ABS_TOL})")
    assert not bad, "; ".join(bad)


def case_inputs(cfg, seed=0, dtype=None):
    """Named workloads use their own seed; edge cases use 1000 + seed.
    dtype: torch element type of q, k, v, dout (default bfloat16)."""
    if cfg.get("index", 0) == 0:
        return W.make_inputs_custom(cfg, 1000 + seed, dtype=dtype)
    return W.make_inputs(cfg, dtype=dtype)
