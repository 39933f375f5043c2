"""The forward under HIP graph capture: fa_fwd_ext_noalloc (no allocation, split scratch in the
library's static device array) and fa_fwd_ext with a caller workspace, captured once with
torch.cuda.graph and replayed several times, with other eager calls of the library (which
overwrite the shared scratch) and synchronisations between the replays.  Every replay must
equal the eager call on the same inputs bit for bit, also after the captured input buffers are
overwritten with new values; the eager results themselves are held to the oracle's bar
(O max-abs <= 2e-2, mean-abs <= 2e-3, LSE max-abs <= 1e-3)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_17_amd import fa, inputs

pytestmark = pytest.mark.gpu


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


def _nan_like(q, batch, heads, nq):
    o = torch.full_like(q, float("nan"))
    lse = torch.full((batch, heads, nq), float("nan"), dtype=torch.float32, device=q.device)
    return o, lse


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype != torch.float32 else \
        torch.equal(a.view(torch.int32), b.view(torch.int32))


def _oracle_check(q, k, v, scale, causal, o, lse):
    o_r, lse_r = oracle.attention(inputs.to_f64(q.cpu()), inputs.to_f64(k.cpu()), inputs.to_f64(v.cpu()), scale,
                                  causal=causal)
    err = np.abs(inputs.to_f64(o.cpu()) - o_r)
    lerr = np.abs(lse.cpu().double().numpy() - lse_r)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3, (err.max(), err.mean(), lerr.max())


# (batch, nq, nk, heads, heads_kv, d, dtype, causal, num_splits): one call without splits,
# one whose split partials live in the scratch, one with the automatic split count
CASES = [
    (2, 300, 300, 4, 4, 64, "bf16", False, 1),
    (1, 64, 2048, 2, 2, 128, "bf16", False, 8),
    (2, 200, 777, 4, 2, 32, "fp16", True, 0),
]


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_q%d_k%d_h%d_hkv%d_d%d_%s_causal%d_s%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], int(c[7]), c[8]))
def test_graph_replays_equal_eager(case, entry):
    batch, nq, nk, heads, hkv, d, dtype, causal, splits = case
    dev = torch.device("cuda:0")
    say("case graph %s %r" % (entry, case))
    seed = 11 * batch + nq + nk + d
    q, k, v = inputs.dense_qkv(batch, nq, nk, heads, d, dtype, seed=seed, heads_kv=hkv)
    q2, _, _ = inputs.dense_qkv(batch, nq, nk, heads, d, dtype, seed=seed + 1, heads_kv=hkv)
    qd, kd, vd, q2d = q.to(dev), k.to(dev), v.to(dev), q2.to(dev)
    scale = d ** -0.5
    ws = None
    if entry == "workspace":
        n = splits if splits > 0 else fa.FA_MAX_SPLITS
        nbytes = min(fa.fa_fwd_workspace_bytes(batch, nq, heads, d, n), 64 << 20) // 16 * 16
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def call(qq, o, lse):
        if entry == "noalloc":
            fa.fa_fwd_ext_noalloc(qq, kd, vd, o, lse, scale=scale, causal=causal, num_splits=splits)
        else:
            fa.fa_fwd_ext(qq, kd, vd, o, lse, scale=scale, causal=causal, num_splits=splits, workspace=ws)

    # eager results on both inputs (this also does the library's first-call set-up)
    o_e, lse_e = _nan_like(qd, batch, heads, nq)
    call(qd, o_e, lse_e)
    o_e2, lse_e2 = _nan_like(qd, batch, heads, nq)
    call(q2d, o_e2, lse_e2)
    torch.cuda.synchronize()
    _oracle_check(q, k, v, scale, causal, o_e, lse_e)
    _oracle_check(q2, k, v, scale, causal, o_e2, lse_e2)

    # capture with static buffers
    q_s = qd.clone()
    o_s, lse_s = _nan_like(qd, batch, heads, nq)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up on the capturing stream, as torch recommends
        call(q_s, o_s, lse_s)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(q_s, o_s, lse_s)
    torch.cuda.synchronize()

    # an unrelated eager call of the same entry that writes the shared scratch / workspace
    qo, ko, vo = inputs.dense_qkv(1, 64, 4096, 2, 128, "bf16", seed=seed + 2)
    qo, ko, vo = qo.to(dev), ko.to(dev), vo.to(dev)
    wso = torch.empty(fa.fa_fwd_workspace_bytes(1, 64, 2, 128, 16), dtype=torch.uint8, device=dev)

    def disturb():
        oo, lo = _nan_like(qo, 1, 2, 64)
        if entry == "noalloc":
            fa.fa_fwd_ext_noalloc(qo, ko, vo, oo, lo, num_splits=16)
        else:
            fa.fa_fwd_ext(qo, ko, vo, oo, lo, num_splits=16, workspace=wso)
            if ws is not None:
                ws.fill_(0xFF)  # garbage in the captured workspace between replays

    for r in range(3):
        disturb()
        o_s.fill_(float("nan"))
        lse_s.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(o_s, o_e) and _same(lse_s, lse_e), "replay %d differs from the eager call" % r
    # new values in the captured input buffer: the replays read them
    q_s.copy_(q2d)
    for r in range(2):
        disturb()
        o_s.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(o_s, o_e2) and _same(lse_s, lse_e2), "replay %d on new inputs differs" % r
    say("graph %s %r: 5 replays equal the eager calls" % (entry, case))
