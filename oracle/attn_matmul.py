"""Exact attention in fp64 on the CPU from whole-matrix products (torch CPU ops).

TEST INFRASTRUCTURE ONLY: a second checker for the GPU path, used where the
per-row C oracle (attn_oracle.c) would take minutes -- comparing every element
of the full-size workloads.  Only tests/ may import it.  It shares no code with
the HIP library or with attn_oracle.c; the two oracles are checked against the
same closed-form pins and against each other.

What it computes is the definition of page "GPU 内核与 FlashAttention"
(hs-black), section 10 (S = Q K^T times the logit scale, P = row softmax of S,
O = P V), section 11.1 (the row maximum is subtracted before exponentiating)
and section 13.2 (LSE = m + ln l), with the two options of section 14: the
causal mask of 14.4 (key j hidden from query i when j > i, indices from the
start of the sequence) and the grouped K/V heads of 14.2 (query head h reads
K/V head h // (H / Hkv)).  The packed layout with prefix offsets and an LSE of
[batch, heads, max_seqlen] is that of page "Flash Attention实现深度解析",
section 3.1.

Each step is one library operation on a whole (sequence, head) at once, in the
definition's order, with no blocking or reordering of the sums beyond what the
matrix product does inside itself:
    S = scale * (Q_h @ K_h^T)            fp64 matrix product
    S[i, j] = -inf where masked           causal only
    m = max_j S[i, j]
    E = exp(S - m)
    l = sum_j E[i, j]
    O_h = (E @ V_h) / l                   fp64 matrix product
    LSE = m + ln l
"""
import numpy as np
import torch


def _per_sequence(q, k, v, cu_seqlens, max_seqlen):
    """Yield (b, qs [Lq, H, D], ks [Lk, Hkv, D], vs, o_slice) over the sequences, and return
    the output arrays: dense [B, Nq, H, D] / LSE [B, H, Nq]; packed [total, H, D] /
    LSE [B, H, max_seqlen] with NaN past each sequence's end."""
    if cu_seqlens is None:
        if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
            raise ValueError("dense q, k, v must be [B, N, H, D] with k and v alike")
        batch, nq, heads, d = q.shape
        if k.shape[0] != batch or k.shape[3] != d or heads % k.shape[2]:
            raise ValueError("q and k disagree on batch or d, or k's heads do not divide q's")
        o = np.zeros(q.shape, dtype=np.float64)
        lse = np.full((batch, heads, nq), np.nan, dtype=np.float64)
        seqs = [(b, q[b], k[b], v[b], o[b]) for b in range(batch)]
        return o, lse, seqs
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if q.ndim != 3 or k.ndim != 3 or k.shape != v.shape or q.shape[0] != k.shape[0] or \
            q.shape[2] != k.shape[2] or q.shape[1] % k.shape[1]:
        raise ValueError("packed q must be [total, H, D] and k, v [total, Hkv, D] with Hkv | H")
    batch = cu.shape[0] - 1
    if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != q.shape[0]:
        raise ValueError("cu_seqlens must start at 0, not decrease, and end at total")
    lmax = int(np.max(np.diff(cu))) if batch > 0 else 0
    if max_seqlen is None:
        max_seqlen = lmax
    if max_seqlen < lmax:
        raise ValueError("max_seqlen smaller than the longest sequence")
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.full((batch, q.shape[1], max_seqlen), np.nan, dtype=np.float64)
    seqs = []
    for b in range(batch):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        seqs.append((b, q[sl], k[sl], v[sl], o[sl]))
    return o, lse, seqs


def attention(q, k, v, scale, cu_seqlens=None, max_seqlen=None, causal=False, head_chunk=4):
    """Exact attention in fp64; same layouts and results as oracle.attention().

    Dense: q [B, Nq, H, D], k/v [B, Nk, Hkv, D] -> (O [B, Nq, H, D], LSE [B, H, Nq]).
    Packed: q [total, H, D], k/v [total, Hkv, D], cu_seqlens [B+1] -> (O [total, H, D],
    LSE [B, H, max_seqlen], NaN past each sequence's end).  head_chunk query heads are
    formed at a time (memory: head_chunk x Lq x Lk doubles)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o, lse, seqs = _per_sequence(q, k, v, cu_seqlens, max_seqlen)
    heads, hkv = q.shape[-2], k.shape[-2]
    group = heads // hkv
    for b, qs, ks, vs, os_ in seqs:
        lq, lk = qs.shape[0], ks.shape[0]
        if lq == 0:
            continue
        Q = torch.from_numpy(np.ascontiguousarray(qs.transpose(1, 0, 2)))  # [H, Lq, D]
        K = torch.from_numpy(np.ascontiguousarray(ks.transpose(1, 0, 2)))  # [Hkv, Lk, D]
        V = torch.from_numpy(np.ascontiguousarray(vs.transpose(1, 0, 2)))
        hidden = torch.ones((lq, lk), dtype=torch.bool).triu(1) if causal else None  # j > i
        for h0 in range(0, heads, head_chunk):
            h1 = min(heads, h0 + head_chunk)
            kv_of = torch.tensor([h // group for h in range(h0, h1)], dtype=torch.long)
            Kh, Vh = K.index_select(0, kv_of), V.index_select(0, kv_of)
            S = torch.matmul(Q[h0:h1], Kh.transpose(1, 2)) * scale
            if hidden is not None:
                S.masked_fill_(hidden, -np.inf)
            m = S.amax(dim=-1, keepdim=True)
            E = torch.exp(S - m)
            del S
            l = E.sum(dim=-1, keepdim=True)
            O = torch.matmul(E, Vh) / l
            os_[:, h0:h1, :] = O.permute(1, 0, 2).numpy()
            lse[b, h0:h1, :lq] = (m + torch.log(l)).squeeze(-1).numpy()
    return o, lse


class MatmulOracle:
    """The pins' oracle interface (attention only) over this module, or over a module
    built from altered source text (the planted-mistake tests)."""

    def __init__(self, module=None):
        import sys
        self._m = module or sys.modules[__name__]

    def attention(self, *a, **kw):
        return self._m.attention(*a, **kw)


def source_text():
    with open(__file__, encoding="utf-8") as f:
        return f.read()


def module_from_source(text, name="attn_matmul_variant"):
    """A module executed from source text (an altered copy of this file)."""
    import types
    mod = types.ModuleType(name)
    exec(compile(text, name + ".py", "exec"), mod.__dict__)
    return mod
