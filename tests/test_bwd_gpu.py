"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's gradients.

The forward output O and LSE come from the library's own forward pass (as in training);
dO is seeded N(0,1) rounded to the 16-bit type.  The oracle recomputes everything in fp64
from the same 16-bit Q, K, V and dO.

Bar (derived from the 16-bit roundings of P, dS, O and the outputs): for each of dQ, dK,
dV, max-abs error <= 2e-2 x max|reference| + 1e-4 and mean-abs error <= 1e-2 x
mean|reference| + 1e-5.  The absolute terms cover gradients whose exact value is 0 (one
key, identical keys): there the GPU result is the rounding of D = <dO, O> computed from the
16-bit O, of order |dO| |O| 2^-8 / sqrt(d) per query row.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_17_amd import fa, inputs

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 2e-2, 1e-2
ABS_MAX, ABS_MEAN = 1e-4, 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()
    yield
    torch.cuda.synchronize()


def dout_like(q, seed):
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)


def run_bwd(q, k, v, do, scale, causal=False, cu=None, max_seqlen=None, atomic_dq=False):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    cud = cu.to(dev) if cu is not None else None
    o, lse = fa.fa_fwd_ext(qd, kd, vd, scale=scale, causal=causal, cu_seqlens=cud, max_seqlen=max_seqlen)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, scale=scale, causal=causal, cu_seqlens=cud,
                           max_seqlen=max_seqlen, atomic_dq=atomic_dq)
    torch.cuda.synchronize()
    return [t.cpu().to(torch.float64).numpy() for t in (dq, dk, dv)]


def compare(got, want, what):
    bad = []
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        err = np.abs(g - w)
        ref_max, ref_mean = np.abs(w).max(), np.abs(w).mean()
        say("%s %s: max err %.3g (ref max %.3g, ratio %.2e)  mean err %.3g (ref mean %.3g, ratio %.2e)"
            % (what, name, err.max(), ref_max, err.max() / max(ref_max, 1e-30), err.mean(), ref_mean,
               err.mean() / max(ref_mean, 1e-30)))
        if not (np.all(np.isfinite(g)) and err.max() <= REL_MAX * ref_max + ABS_MAX
                and err.mean() <= REL_MEAN * ref_mean + ABS_MEAN):
            bad.append(name)
    assert not bad, (what, bad)


def check_dense(b, nq, nk, h, hkv, d, dtype, causal, seed, modes=(False, True)):
    q, k, v = inputs.dense_qkv(b, nq, nk, h, d, dtype, seed=seed, heads_kv=hkv)
    do = dout_like(q, seed + 1000)
    scale = d ** -0.5
    want = oracle.attention_bwd(*(inputs.to_f64(t) for t in (q, k, v, do)), scale, causal=causal)
    for atomic in modes:
        what = "bwd B%d nq%d nk%d H%d Hkv%d d%d %s causal=%d atomic_dq=%d" % (b, nq, nk, h, hkv, d, dtype, causal,
                                                                          atomic)
        say("case " + what)
        got = run_bwd(q, k, v, do, scale, causal=causal, atomic_dq=atomic)
        compare(got, want, what)


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (32, "bf16"), (128, "fp16"), (64, "fp16"),
                                     (32, "fp16")])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_square(d, dtype, causal):
    check_dense(2, 256, 256, 2, 2, d, dtype, causal, seed=d + causal)


@pytest.mark.parametrize("nq,nk", [(1, 1), (63, 63), (65, 130), (300, 100), (100, 300), (129, 257), (2, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged(nq, nk, causal):
    check_dense(1, nq, nk, 3, 3, 128, "bf16", causal, seed=nq + 7 * nk)


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_grouped_heads(hkv, causal):
    check_dense(2, 200, 200, 4, hkv, 64, "bf16", causal, seed=50 + hkv)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen(causal):
    lengths = [1, 130, 0, 64, 300, 77]
    q, k, v, cu, max_len = inputs.varlen_qkv(heads=4, d_head=128, dtype="bf16", seed=61, lengths=lengths,
                                             heads_kv=2)
    do = dout_like(q, 62)
    scale = 128 ** -0.5
    want = oracle.attention_bwd(*(inputs.to_f64(t) for t in (q, k, v, do)), scale, cu_seqlens=cu.numpy(),
                                max_seqlen=max_len, causal=causal)
    for atomic in (False, True):
        what = "bwd varlen %s causal=%d atomic_dq=%d" % (lengths, causal, atomic)
        say("case " + what)
        got = run_bwd(q, k, v, do, scale, causal=causal, cu=cu, max_seqlen=max_len, atomic_dq=atomic)
        compare(got, want, what)


def test_bwd_separate_dq_pass_is_deterministic():
    q, k, v = inputs.dense_qkv(1, 700, 700, 4, 128, "bf16", seed=81, heads_kv=2)
    do = dout_like(q, 82)
    a = run_bwd(q, k, v, do, 128 ** -0.5, causal=True)
    b = run_bwd(q, k, v, do, 128 ** -0.5, causal=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_longer_sequence():
    check_dense(1, 1024, 1024, 2, 2, 128, "bf16", True, seed=71)
    check_dense(1, 1024, 1024, 2, 1, 128, "bf16", False, seed=72)


# ------------------------------------------------------------------------------ full size
def _one_per_block(rng, n, block=32):
    """One row in each block of 32 rows (the rows a wavefront owns in both backward kernels),
    at a seeded offset, and the last row."""
    rows = [min(n - 1, b0 + int(rng.integers(block))) for b0 in range(0, n, block)]
    return sorted(set(rows + [n - 1]))


@pytest.mark.parametrize("name", ["full", "causal", "gqa", "varlen"])
def test_bwd_full_size_every_wavefront(name):
    """The named workload at full size, as the benchmark runs it, with dQ, dK and dV prefilled
    with NaN: every element must be written and finite, and in every sequence one row of every
    32-row block of every head (so of every wavefront of every workgroup of the dQ pass and of
    the dK/dV kernel) is compared with the oracle's selected-rows backward."""
    w = inputs.workload(name)
    dev = torch.device("cuda:0")
    say("case bwd full size %s" % name)
    qd, kd, vd = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    cu = w["cu_seqlens"]
    cud = cu.to(dev) if cu is not None else None
    o, lse = fa.fa_fwd_ext(qd, kd, vd, scale=w["scale"], causal=w["causal"], cu_seqlens=cud,
                           max_seqlen=w["max_seqlen"])
    do = dout_like(w["q"], w["seed"] + 1000)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    fa.fa_bwd(qd, kd, vd, o, lse, do.to(dev), dq, dk, dv, scale=w["scale"], causal=w["causal"], cu_seqlens=cud,
              max_seqlen=w["max_seqlen"])
    torch.cuda.synchronize()
    for key, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), (name, key, "unwritten or non-finite elements")
    rng = np.random.default_rng(len(name) + 7)
    heads, hkv = w["heads"], w["heads_kv"]
    errs = {"dQ": [], "dK": [], "dV": []}
    refs = {"dQ": [], "dK": [], "dV": []}
    for b in range(w["batch"]):
        if cu is None:
            n = w["seqlen_q"]
            take = lambda t: t[b]  # noqa: E731
        else:
            s0, s1 = int(cu[b]), int(cu[b + 1])
            n = s1 - s0
            take = lambda t, s0=s0, s1=s1: t[s0:s1]  # noqa: E731
        qrows = [(h, i) for h in range(heads) for i in _one_per_block(rng, n)]
        krows = [(hk, j) for hk in range(hkv) for j in _one_per_block(rng, n)]
        qb, kb, vb, db = (inputs.to_f64(take(t)[None]) for t in (w["q"], w["k"], w["v"], do))
        rq, rk, rv = oracle.attention_bwd_rows(qb, kb, vb, db, w["scale"], [(0, h, i) for h, i in qrows],
                                               [(0, hk, j) for hk, j in krows], causal=w["causal"])
        gq = take(dq)[[i for _, i in qrows], [h for h, _ in qrows]].cpu().to(torch.float64).numpy()
        gk = take(dk)[[j for _, j in krows], [hk for hk, _ in krows]].cpu().to(torch.float64).numpy()
        gv = take(dv)[[j for _, j in krows], [hk for hk, _ in krows]].cpu().to(torch.float64).numpy()
        for key, g, r in (("dQ", gq, rq), ("dK", gk, rk), ("dV", gv, rv)):
            errs[key].append(np.abs(g - r).ravel())
            refs[key].append(np.abs(r).ravel())
        say("  %s sequence %d of %d compared" % (name, b + 1, w["batch"]))
    bad = []
    for key in ("dQ", "dK", "dV"):
        err, ref = np.concatenate(errs[key]), np.concatenate(refs[key])
        say("%s %s (%d compared values): max err %.3g (ref max %.3g)  mean err %.3g (ref mean %.3g)"
            % (name, key, err.size, err.max(), ref.max(), err.mean(), ref.mean()))
        if not (err.max() <= REL_MAX * ref.max() + ABS_MAX and err.mean() <= REL_MEAN * ref.mean() + ABS_MEAN):
            bad.append(key)
    assert not bad, (name, bad)
