"""fa_fwd_ext_noalloc (split scratch in the library's static device array) against
fa_fwd_ext with a caller workspace, through the C ABI: same inputs, same split count, two
calls in a row (the second on a smaller input), bitwise-equal outputs, both within the
oracle bar (O max-abs <= 2e-2, mean-abs <= 2e-3, LSE max-abs <= 1e-3)."""
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


def _pair(q, k, v, scale, causal, splits):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    batch, nq, heads, d = q.shape
    outs = []
    for which in ("workspace", "noalloc"):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((batch, heads, nq), float("nan"), dtype=torch.float32, device=dev)
        if which == "workspace":
            n = splits if splits > 0 else fa.fa_fwd_choose_splits(batch, nq, k.shape[1], heads, d,
                                                                   fa.FA_BF16, causal)
            ws = torch.empty(max(fa.fa_fwd_workspace_bytes(batch, nq, heads, d, n), 16), dtype=torch.uint8,
                             device=dev)
            fa.fa_fwd_ext(qd, kd, vd, o, lse, scale=scale, causal=causal, num_splits=splits, workspace=ws)
        else:
            fa.fa_fwd_ext_noalloc(qd, kd, vd, o, lse, scale=scale, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "static scratch and workspace results differ"
    o_r, lse_r = oracle.attention(inputs.to_f64(q), inputs.to_f64(k), inputs.to_f64(v), scale, causal=causal)
    err = np.abs(inputs.to_f64(o2) - o_r)
    lerr = np.abs(l2.double().numpy() - lse_r)
    say("noalloc splits %d q%s: O max %.3g mean %.3g LSE max %.3g" % (splits, tuple(q.shape), err.max(),
                                                                      err.mean(), lerr.max()))
    assert np.all(np.isfinite(err)) and err.max() <= 2e-2 and err.mean() <= 2e-3 and lerr.max() <= 1e-3


def test_noalloc_matches_workspace_twice_second_smaller():
    w = inputs.workload("slice")  # 64 queries x 4096 keys, d 128
    say("case noalloc slice 16 splits")
    _pair(w["q"], w["k"], w["v"], w["scale"], False, 16)
    q, k, v = inputs.dense_qkv(1, 40, 1000, 2, 128, "bf16", seed=101)
    say("case noalloc smaller causal 4 splits")
    _pair(q, k, v, 128 ** -0.5, True, 4)


def test_noalloc_automatic_split_count():
    q, k, v = inputs.dense_qkv(2, 64, 8192, 4, 128, "bf16", seed=102)
    say("case noalloc automatic splits")
    _pair(q, k, v, 128 ** -0.5, False, 0)


def test_noalloc_rejects_scratch_beyond_its_size():
    dev = torch.device("cuda:0")
    q, k, v = inputs.dense_qkv(8, 512, 512, 16, 128, "bf16", seed=103)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((8, 16, 512), dtype=torch.float32, device=dev)
    need = fa.fa_fwd_workspace_bytes(8, 512, 16, 128, 64)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_ext_noalloc(qd, kd, vd, o, lse, num_splits=64)
    assert e.value.status == fa.FA_ERR_INVALID_ARG and str(need) in str(e.value)
