"""Work and byte accounting for the attention forward pass.

FLOPs: the two products S = Q K^T and O = P V each cost 2 * Nq * Nk * d
multiply-adds per (batch, head), 4 * B * H * Nq * Nk * d in total; softmax
arithmetic is not counted (page "GPU 内核与 FlashAttention", section 10,
counts the two matrix products; the worked slice of "Flash Attention 2
Chapter2" adds a few operations per score on top, see slice_page_flops).

Bytes: the algorithmic HBM traffic of a fused kernel reads Q, K and V once and
writes O once (16-bit each) plus the fp32 log-sum-exp row.
"""


def fwd_flops(batch, heads, seqlen_q, seqlen_k, d_head):
    return 4 * batch * heads * seqlen_q * seqlen_k * d_head


def varlen_fwd_flops(lengths, heads, d_head):
    return sum(4 * heads * L * L * d_head for L in lengths)


def fwd_bytes(batch, heads, seqlen_q, seqlen_k, d_head, elt_bytes=2, with_lse=True):
    qo = 2 * batch * seqlen_q * heads * d_head * elt_bytes
    kv = 2 * batch * seqlen_k * heads * d_head * elt_bytes
    lse = 4 * batch * heads * seqlen_q if with_lse else 0
    return qo + kv + lse


def varlen_fwd_bytes(lengths, heads, d_head, elt_bytes=2, with_lse=True):
    return sum(fwd_bytes(1, heads, L, L, d_head, elt_bytes, with_lse) for L in lengths)


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
