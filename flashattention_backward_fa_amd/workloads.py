"""Seeded synthetic inputs for the five benchmark/parity workloads.

This module only draws random numbers and rounds them to bfloat16 (or, on
request, IEEE fp16); it holds
none of the backward's arithmetic, so both the fp64 oracle (tests) and the
HIP path (tests, bench) take their inputs from here.

Recipe: numpy.random.default_rng(seed), draws in the order q, k, v, dout, each
standard normal float32 in the layout's logical shape, dout multiplied by
`dy_std`, then rounded to bfloat16 (round to nearest even, via torch; fp16
likewise when a caller asks for it).  The
forward output attn_out and softmax_lse are NOT made here: tests take them
from the oracle's forward, the benchmark from the library's own forward.
"""

import math

import numpy as np

# Workload table.  Lengths of the packed varlen workload: the first seed of
# default_rng(seed).integers(256, 4097, 8) whose total lies in [15360, 16896]
# ("about 16k tokens"), i.e. seed 3 -> total 16437.
VARLEN_LENGTHS = [3372, 584, 945, 1165, 952, 3333, 3594, 2492]

CONFIGS = {
    "tiny": dict(index=1, B=1, N1=2, N2=2, S1=128, S2=128, D=64, Dv=64, layout="BSND",
                 mask_mode=0, win_left=-1, win_right=-1, softmax_scale=1.0 / 8, dy_std=1.0),
    "mha_causal": dict(index=2, B=2, N1=16, N2=16, S1=2048, S2=2048, D=128, Dv=128, layout="BSND",
                       mask_mode=1, win_left=-1, win_right=-1, softmax_scale=1.0 / math.sqrt(128), dy_std=0.1),
    "gqa_causal": dict(index=3, B=1, N1=32, N2=8, S1=4096, S2=4096, D=128, Dv=128, layout="BSND",
                       mask_mode=1, win_left=-1, win_right=-1, softmax_scale=1.0 / math.sqrt(128), dy_std=0.1),
    "varlen_window": dict(index=4, lengths=VARLEN_LENGTHS, N1=16, N2=16, D=128, Dv=128, layout="TND",
                          mask_mode=1, win_left=1024, win_right=0, softmax_scale=1.0 / math.sqrt(128),
                          dy_std=1.0),
    "wide_qk": dict(index=5, B=1, N1=16, N2=16, S1=8192, S2=8192, D=192, Dv=128, layout="BNSD",
                    mask_mode=1, win_left=-1, win_right=-1, softmax_scale=1.0 / math.sqrt(192), dy_std=0.1),
}

BENCH_WORKLOAD = "gqa_causal"


def seed_of(cfg):
    return 100 + cfg["index"]


def cu_seqlens(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def shapes(cfg):
    """Logical shapes of q, k, v, dout for a workload dict."""
    L, N1, N2, D, Dv = cfg["layout"], cfg["N1"], cfg["N2"], cfg["D"], cfg["Dv"]
    if L == "TND":
        T = int(sum(cfg["lengths"]))
        return (T, N1, D), (T, N2, D), (T, N2, Dv), (T, N1, Dv)
    B, S1, S2 = cfg["B"], cfg["S1"], cfg["S2"]
    if L == "BSND":
        return (B, S1, N1, D), (B, S2, N2, D), (B, S2, N2, Dv), (B, S1, N1, Dv)
    return (B, N1, S1, D), (B, N2, S2, D), (B, N2, S2, Dv), (B, N1, S1, Dv)


def make_inputs(cfg, seed=None, dtype=None):
    """q, k, v, dout as CPU torch tensors of `dtype` (default torch.bfloat16;
    torch.float16 for the fp16 path), plus cu_seqlens (numpy int32, TND only,
    else None)."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    rng = np.random.default_rng(seed_of(cfg) if seed is None else seed)
    out = {}
    for name, shp in zip(("q", "k", "v", "dout"), shapes(cfg)):
        x = rng.standard_normal(shp, dtype=np.float32)
        if name == "dout":
            x *= np.float32(cfg["dy_std"])
        out[name] = torch.from_numpy(x).to(dtype)
    if cfg["layout"] == "TND":
        cu = cu_seqlens(cfg["lengths"])
        out["cu_q"], out["cu_kv"] = cu, cu.copy()
    else:
        out["cu_q"], out["cu_kv"] = None, None
    return out


def custom(layout="BSND", B=1, N1=2, N2=2, S1=128, S2=128, D=64, Dv=64, mask_mode=0, win_left=-1,
           win_right=-1, softmax_scale=0.0, dy_std=1.0, lengths=None, lengths_kv=None, index=0):
    """A workload dict of any shape (for edge-case tests)."""
    c = dict(index=index, B=B, N1=N1, N2=N2, S1=S1, S2=S2, D=D, Dv=Dv, layout=layout, mask_mode=mask_mode,
             win_left=win_left, win_right=win_right, softmax_scale=softmax_scale, dy_std=dy_std)
    if layout == "TND":
        c["lengths"] = list(lengths)
        c["lengths_kv"] = list(lengths_kv if lengths_kv is not None else lengths)
    return c


def make_inputs_custom(cfg, seed, dtype=None):
    """Like make_inputs, but TND may have different query and key lengths."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    rng = np.random.default_rng(seed)
    L, N1, N2, D, Dv = cfg["layout"], cfg["N1"], cfg["N2"], cfg["D"], cfg["Dv"]
    if L == "TND":
        T1, T2 = int(sum(cfg["lengths"])), int(sum(cfg["lengths_kv"]))
        shp = [(T1, N1, D), (T2, N2, D), (T2, N2, Dv), (T1, N1, Dv)]
    else:
        shp = list(shapes(cfg))
    out = {}
    for name, s in zip(("q", "k", "v", "dout"), shp):
        x = rng.standard_normal(s, dtype=np.float32)
        if name == "dout":
            x *= np.float32(cfg["dy_std"])
        out[name] = torch.from_numpy(x).to(dtype)
    if L == "TND":
        out["cu_q"], out["cu_kv"] = cu_seqlens(cfg["lengths"]), cu_seqlens(cfg["lengths_kv"])
    else:
        out["cu_q"], out["cu_kv"] = None, None
    return out


# Floyd attention (page "CANN Floyd注意力梯度算子").  The benchmark workload
# takes the page's example sizes (S1 = S2 = S3 = 256, D = 128) with 8 heads;
# the page quotes no workload of its own.  mask_p is the probability that a
# (n, k) position is masked; masked_rows lists (b, n) rows masked whole.
FLOYD_CONFIGS = {
    "floyd": dict(index=11, B=1, H=8, N=256, M=256, K=256, D=128, mask_p=0.0, masked_rows=(), dy_std=1.0),
    "floyd_small": dict(index=12, B=1, H=2, N=16, M=128, K=128, D=32, mask_p=0.0, masked_rows=(), dy_std=1.0),
    "floyd_masked": dict(index=13, B=2, H=1, N=32, M=128, K=256, D=64, mask_p=0.2, masked_rows=((0, 5),),
                         dy_std=1.0),
    "floyd_n48": dict(index=14, B=1, H=2, N=48, M=128, K=128, D=128, mask_p=0.1, masked_rows=(), dy_std=0.5),
}


def floyd_inputs(cfg, seed=None, dtype=None):
    """query, key1, value1, key2, value2, dy as CPU torch tensors of `dtype`
    (default bfloat16) in the page's shapes, and the mask as a numpy uint8
    array [B, 1, N, 1, K] (None when the workload masks nothing).  Recipe:
    default_rng(seed); standard normal float32 draws in the order query, key1,
    value1, key2, value2, dy (dy times dy_std), rounded to the element type;
    then the mask as uniform draws < mask_p, with the listed rows set whole."""
    import torch

    dtype = torch.bfloat16 if dtype is None else dtype
    rng = np.random.default_rng(seed_of(cfg) if seed is None else seed)
    B, H, N, M, K, D = (cfg[k] for k in ("B", "H", "N", "M", "K", "D"))
    shp = {"query": (B, H, N, M, D), "key1": (B, H, N, K, D), "value1": (B, H, N, K, D),
           "key2": (B, H, K, M, D), "value2": (B, H, K, M, D), "dy": (B, H, N, M, D)}
    out = {}
    for name, s in shp.items():
        x = rng.standard_normal(s, dtype=np.float32)
        if name == "dy":
            x *= np.float32(cfg["dy_std"])
        out[name] = torch.from_numpy(x).to(dtype)
    mask = None
    if cfg["mask_p"] > 0 or cfg["masked_rows"]:
        mask = (rng.random((B, 1, N, 1, K)) < cfg["mask_p"]).astype(np.uint8)
        for (b, n) in cfg["masked_rows"]:
            mask[b, 0, n, 0, :] = 1
    out["mask"] = mask
    return out
