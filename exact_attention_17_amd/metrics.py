"""Work and byte accounting for the attention forward pass.

FLOPs: the two products S = Q K^T and O = P V each cost 2 * Nq * Nk * d
multiply-adds per (batch, head), 4 * B * H * Nq * Nk * d in total; softmax
arithmetic is not counted (page "GPU 内核与 FlashAttention", section 10,
counts the two matrix products; the worked slice of "Flash Attention 2
Chapter2" adds a few operations per score on top, see slice_page_flops).

Under the causal mask only the (query, key) pairs with key <= query are work: the
FLOP count is 4 * d * (visible pairs) per (batch, head), about half the dense count
(page "GPU 内核与 FlashAttention", section 14.4).

Bytes: the algorithmic HBM traffic of a fused kernel reads Q, K and V once and
writes O once (16-bit each) plus the fp32 log-sum-exp row.  With grouped K/V heads
(section 14.2) K and V have heads_kv heads.
"""


def causal_pairs(seqlen_q, seqlen_k):
    """(i, j) pairs with j <= i, i < seqlen_q, j < seqlen_k (top-left aligned mask)."""
    n = min(seqlen_q, seqlen_k)
    return n * (n + 1) // 2 + max(seqlen_q - seqlen_k, 0) * seqlen_k


def fwd_flops(batch, heads, seqlen_q, seqlen_k, d_head, causal=False):
    pairs = causal_pairs(seqlen_q, seqlen_k) if causal else seqlen_q * seqlen_k
    return 4 * batch * heads * pairs * d_head


def varlen_fwd_flops(lengths, heads, d_head, causal=False):
    return sum(fwd_flops(1, heads, L, L, d_head, causal) for L in lengths)


def fwd_bytes(batch, heads, seqlen_q, seqlen_k, d_head, elt_bytes=2, with_lse=True, heads_kv=None):
    hkv = heads if heads_kv is None else heads_kv
    qo = 2 * batch * seqlen_q * heads * d_head * elt_bytes
    kv = 2 * batch * seqlen_k * hkv * d_head * elt_bytes
    lse = 4 * batch * heads * seqlen_q if with_lse else 0
    return qo + kv + lse


def varlen_fwd_bytes(lengths, heads, d_head, elt_bytes=2, with_lse=True, heads_kv=None):
    return sum(fwd_bytes(1, heads, L, L, d_head, elt_bytes, with_lse, heads_kv) for L in lengths)


def slice_page_flops(seqlen_q, seqlen_k, d_head, ops_per_score=6):
    """FLOPs of one (batch, head) slice counted the way the Chapter2 page's worked example
    reaches its total: the two products plus a few softmax operations per score
    (max, subtract, exp, sum, scale, normalise: about 6)."""
    return 4 * seqlen_q * seqlen_k * d_head + ops_per_score * seqlen_q * seqlen_k


def standard_attention_hbm_elements(n, d):
    """HBM element accesses of the unfused three-kernel attention (page "GPU 内核与
    FlashAttention", section 10): 4 N^2 + 4 N d."""
    return 4 * n * n + 4 * n * d


def intensity(flops, nbytes):
    return flops / nbytes
