"""Every compiled tile configuration (the autotuner's whole space) on the extended forward's
option combinations, against the fp64 oracle: for each (dtype, d_head) and each configuration,
three ragged shapes -- causal with grouped K/V heads (dense), causal packed sequences of mixed
lengths, and a few queries over many keys -- each with a split count that rotates over 1, 2, 3
and 5 from one configuration to the next (so every configuration runs unsplit and split).
O and LSE start as NaN; every valid element must be written and within the bar (O max-abs
<= 2e-2, mean-abs <= 2e-3, LSE max-abs <= 1e-3), and LSE padding rows of packed sequences
must stay NaN."""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_17_amd import fa, inputs

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-3
SPLITS = (1, 2, 3, 5)


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


def _shapes(d, dtype):
    """(name, q, k, v, cu, max_len, causal, valid-LSE mask or None, oracle O, oracle LSE)."""
    seed = d + (7 if dtype == "fp16" else 0)
    out = []
    q, k, v = inputs.dense_qkv(2, 345, 345, 4, d, dtype, seed=seed, heads_kv=2)
    o_r, l_r = oracle.attention(inputs.to_f64(q), inputs.to_f64(k), inputs.to_f64(v), d ** -0.5, causal=True)
    out.append(("causal gqa B2 N345 H4 Hkv2", q, k, v, None, None, True, None, o_r, l_r))
    lengths = [37, 300, 1, 129, 511]
    q, k, v, cu, max_len = inputs.varlen_qkv(heads=4, d_head=d, dtype=dtype, seed=seed + 1, lengths=lengths,
                                             heads_kv=1)
    o_r, l_r = oracle.attention(inputs.to_f64(q), inputs.to_f64(k), inputs.to_f64(v), d ** -0.5,
                                cu_seqlens=cu.numpy(), max_seqlen=max_len, causal=True)
    valid = np.zeros((len(lengths), 4, max_len), dtype=bool)
    for b, n in enumerate(lengths):
        valid[b, :, :n] = True
    out.append(("causal packed %s H4 Hkv1" % lengths, q, k, v, cu, max_len, True, valid, o_r, l_r))
    q, k, v = inputs.dense_qkv(1, 77, 903, 2, d, dtype, seed=seed + 2)
    o_r, l_r = oracle.attention(inputs.to_f64(q), inputs.to_f64(k), inputs.to_f64(v), d ** -0.5)
    out.append(("Nq77 Nk903 H2", q, k, v, None, None, False, None, o_r, l_r))
    return out


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 128), ("bf16", 64), ("fp16", 64), ("bf16", 32),
                                     ("fp16", 32)])
def test_every_config_on_causal_grouped_packed_and_split_calls(dtype, d):
    dev = torch.device("cuda:0")
    code = fa.FA_FP16 if dtype == "fp16" else fa.FA_BF16
    shapes = _shapes(d, dtype)
    dev_in = [(qq.to(dev), kk.to(dev), vv.to(dev), cu.to(dev) if cu is not None else None)
              for (_, qq, kk, vv, cu, _, _, _, _, _) in shapes]
    configs = fa.fa_fwd_list_configs(d, code)
    assert len(configs) >= 30, len(configs)
    worst = [0.0, 0.0, 0.0]
    try:
        for ci, c in enumerate(configs):
            fa.fa_fwd_set_config(d, code, c)
            for si, ((name, q, k, v, cu, max_len, causal, valid, o_r, l_r), (qd, kd, vd, cud)) in enumerate(
                    zip(shapes, dev_in)):
                splits = SPLITS[(ci + si) % len(SPLITS)]
                batch = cu.numel() - 1 if cu is not None else q.shape[0]
                nq = max_len if cu is not None else q.shape[1]
                ws = None
                if splits > 1:
                    ws = torch.empty(fa.fa_fwd_workspace_bytes(batch, nq, q.shape[-2], d, splits), dtype=torch.uint8,
                                     device=dev)
                o = torch.full_like(qd, float("nan"))
                lse = torch.full((batch, q.shape[-2], nq), float("nan"), dtype=torch.float32, device=dev)
                what = "%s d%d %r splits %d: %s" % (dtype, d, c, splits, name)
                say("case " + what)
                fa.fa_fwd_ext(qd, kd, vd, o=o, lse=lse, causal=causal, cu_seqlens=cud, max_seqlen=max_len,
                              num_splits=splits, workspace=ws)
                torch.cuda.synchronize()
                o_g = inputs.to_f64(o.cpu())
                l_g = lse.cpu().double().numpy()
                if valid is not None:
                    assert np.all(np.isnan(l_g[~valid])), what + ": LSE padding rows were written"
                    l_g, l_ref = l_g[valid], l_r[valid]
                else:
                    l_ref = l_r
                assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(l_g)), what + ": unwritten or non-finite"
                err = np.abs(o_g - o_r)
                lerr = np.abs(l_g - l_ref)
                worst = [max(worst[0], err.max()), max(worst[1], err.mean()), max(worst[2], lerr.max())]
                assert err.max() <= O_MAX and err.mean() <= O_MEAN and lerr.max() <= LSE_MAX, \
                    (what, err.max(), err.mean(), lerr.max())
    finally:
        fa.fa_fwd_set_config(d, code, None)
    say("%s d%d: %d configurations x 3 shapes, worst O max %.3g mean %.3g LSE max %.3g"
        % (dtype, d, len(configs), worst[0], worst[1], worst[2]))
