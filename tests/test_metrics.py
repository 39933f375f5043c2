"""Work accounting against brute force (CPU only)."""
import itertools

from exact_attention_17_amd import metrics


def test_causal_pairs_brute_force():
    for nq, nk in itertools.product((1, 2, 5, 17, 64), (1, 3, 5, 16, 70)):
        want = sum(1 for i in range(nq) for j in range(nk) if j <= i)
        assert metrics.causal_pairs(nq, nk) == want, (nq, nk)


def test_causal_flops_about_half():
    dense = metrics.fwd_flops(16, 16, 4096, 4096, 128)
    causal = metrics.fwd_flops(16, 16, 4096, 4096, 128, causal=True)
    assert causal == dense // 2 + 4 * 16 * 16 * 128 * 4096 // 2


def test_grouped_heads_bytes():
    # K and V shrink with the number of K/V heads; Q, O and LSE do not
    full = metrics.fwd_bytes(2, 8, 100, 300, 64)
    grouped = metrics.fwd_bytes(2, 8, 100, 300, 64, heads_kv=2)
    assert full - grouped == 2 * 2 * 300 * (8 - 2) * 64 * 2
