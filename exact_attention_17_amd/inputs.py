"""Seeded synthetic inputs for the attention forward pass.

This module draws random tensors and holds the named workload shapes.  It
contains none of the attention arithmetic: the tests give the same tensors to
the fp64 oracle and to the HIP library.

Recipe.  The pages generate Q, K and V with torch.randn in the layout
[batch, seq_len, n_heads, d_head], K and V drawn like Q ("Flash Attention 2
Chapter2", the input-shape walk-through).  Here every tensor is drawn in fp32
on the CPU from a torch.Generator seeded per workload, then rounded to the
16-bit type (round-to-nearest-even).  For the packed variable-length
workload the sequence lengths are drawn first, then Q, K and V.
"""
import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}

# Named workloads: shapes of the five configurations the library is measured on.
WORKLOADS = {
    # tiny: one batch, two heads, 128 x 128, d 64
    "tiny": dict(batch=1, heads=2, seqlen_q=128, seqlen_k=128, d_head=64, dtype="bf16", seed=1),
    # slice: 64 queries against 4096 keys/values, d 128 (the worked slice of the Chapter2 page)
    "slice": dict(batch=1, heads=1, seqlen_q=64, seqlen_k=4096, d_head=128, dtype="bf16", seed=2),
    # full: B16 N4096 H16 d128, the headline throughput shape
    "full": dict(batch=16, heads=16, seqlen_q=4096, seqlen_k=4096, d_head=128, dtype="bf16", seed=3),
    # small_head: B64 N512 H16 d32 fp16 (bandwidth / occupancy regime)
    "small_head": dict(batch=64, heads=16, seqlen_q=512, seqlen_k=512, d_head=32, dtype="fp16", seed=4),
    # varlen: 8 packed sequences, lengths uniform in [512, 8192], H16 d128
    "varlen": dict(n_seq=8, len_lo=512, len_hi=8192, heads=16, d_head=128, dtype="bf16", seed=5),
    # causal: the full shape under the causal mask (page "GPU 内核与 FlashAttention", 14.4)
    "causal": dict(batch=16, heads=16, seqlen_q=4096, seqlen_k=4096, d_head=128, dtype="bf16", seed=6,
                   causal=True),
    # gqa: the full shape with 2 K/V heads shared by groups of 8 query heads (same page, 14.2)
    "gqa": dict(batch=16, heads=16, heads_kv=2, seqlen_q=4096, seqlen_k=4096, d_head=128, dtype="bf16",
                seed=7),
}


def dense_qkv(batch, seqlen_q, seqlen_k, heads, d_head, dtype="bf16", seed=0, std=1.0, device="cpu",
              heads_kv=None):
    """Q [B, Nq, H, D], K and V [B, Nk, Hkv, D] (Hkv = heads_kv, default H), N(0, std^2)
    rounded to `dtype`."""
    g = torch.Generator().manual_seed(int(seed))
    dt = DTYPES[dtype]
    hkv = heads if heads_kv is None else heads_kv
    q = (torch.randn((batch, seqlen_q, heads, d_head), generator=g, dtype=torch.float32) * std).to(dt)
    k = (torch.randn((batch, seqlen_k, hkv, d_head), generator=g, dtype=torch.float32) * std).to(dt)
    v = torch.randn((batch, seqlen_k, hkv, d_head), generator=g, dtype=torch.float32).to(dt)
    return q.to(device), k.to(device), v.to(device)


def varlen_lengths(n_seq, len_lo, len_hi, seed):
    """Sequence lengths uniform in [len_lo, len_hi], drawn first from the workload's generator."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randint(int(len_lo), int(len_hi) + 1, (int(n_seq),), generator=g), g


def varlen_qkv(n_seq=None, len_lo=None, len_hi=None, heads=16, d_head=128, dtype="bf16", seed=0,
               lengths=None, device="cpu", heads_kv=None):
    """Packed Q [total, H, D], K and V [total, Hkv, D] (Hkv = heads_kv, default H) and int32
    cu_seqlens [n_seq + 1] (prefix offsets).

    Either draw the lengths (n_seq, len_lo, len_hi) or pass explicit `lengths`.
    Returns (q, k, v, cu_seqlens, max_seqlen).
    """
    if lengths is None:
        lens, g = varlen_lengths(n_seq, len_lo, len_hi, seed)
    else:
        lens = torch.as_tensor(lengths, dtype=torch.int64)
        g = torch.Generator().manual_seed(int(seed))
    cu = torch.zeros(lens.numel() + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    total = int(cu[-1])
    dt = DTYPES[dtype]
    hkv = heads if heads_kv is None else heads_kv
    q = torch.randn((total, heads, d_head), generator=g, dtype=torch.float32).to(dt)
    k = torch.randn((total, hkv, d_head), generator=g, dtype=torch.float32).to(dt)
    v = torch.randn((total, hkv, d_head), generator=g, dtype=torch.float32).to(dt)
    max_len = int(lens.max()) if lens.numel() else 0
    return q.to(device), k.to(device), v.to(device), cu.to(device), max_len


def workload(name, device="cpu"):
    """Inputs of a named workload.

    Dense: dict(q, k, v, scale, cu_seqlens=None, ...shape).  Varlen adds cu_seqlens,
    max_seqlen and lengths.  scale is 1/sqrt(d_head).  Every workload also carries causal
    (bool) and heads_kv (K/V heads).
    """
    w = dict(WORKLOADS[name])
    d = w["d_head"]
    if name == "varlen":
        q, k, v, cu, max_len = varlen_qkv(w["n_seq"], w["len_lo"], w["len_hi"], w["heads"], d,
                                          w["dtype"], w["seed"], device=device)
        lens = (cu[1:] - cu[:-1]).cpu().tolist()
        return dict(q=q, k=k, v=v, cu_seqlens=cu, max_seqlen=max_len, lengths=lens,
                    batch=w["n_seq"], seqlen_q=max_len, seqlen_k=max_len, heads=w["heads"],
                    heads_kv=w["heads"], d_head=d, dtype=w["dtype"], scale=d ** -0.5,
                    seed=w["seed"], causal=False)
    hkv = w.get("heads_kv", w["heads"])
    q, k, v = dense_qkv(w["batch"], w["seqlen_q"], w["seqlen_k"], w["heads"], d, w["dtype"],
                        w["seed"], device=device, heads_kv=hkv)
    return dict(q=q, k=k, v=v, cu_seqlens=None, max_seqlen=None, batch=w["batch"],
                seqlen_q=w["seqlen_q"], seqlen_k=w["seqlen_k"], heads=w["heads"], heads_kv=hkv,
                d_head=d, dtype=w["dtype"], scale=d ** -0.5, seed=w["seed"],
                causal=bool(w.get("causal", False)))


def to_f64(t):
    """Exact fp64 numpy copy of a 16-bit tensor (every bf16/fp16 value is a double)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
