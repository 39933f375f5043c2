"""The C ABI on the CPU: the library loads, exports every symbol include/fa_fwd.h
declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import os
import re
import subprocess

import pytest

from exact_attention_17_amd import fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")

A = 0x100000  # a 16-byte aligned fake device address; validation never dereferences it


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_what_binding_lists():
    assert header_functions() == sorted(fa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fa.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(header_functions()) <= exported


def test_version_and_empty_error():
    assert "fa_fwd" in fa.fa_version()


def call(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, seqlen_q=128, seqlen_k=128, n_heads=2, d_head=64,
                scale=0.125, cu_seqlens=None, dtype=fa.FA_BF16, stream=None)
    args.update(over)
    return fa.fa_fwd_raw(**args)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(batch=0), fa.FA_ERR_INVALID_ARG),
    (dict(n_heads=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_q=0), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_k=-3), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=-1), fa.FA_ERR_INVALID_ARG),
    (dict(d_head=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d_head=256), fa.FA_ERR_UNSUPPORTED),
    (dict(q=A + 8), fa.FA_ERR_MISALIGNED),
    (dict(o=A + 2), fa.FA_ERR_MISALIGNED),
    (dict(lse=A + 2), fa.FA_ERR_MISALIGNED),
    (dict(cu_seqlens=A, seqlen_q=100, seqlen_k=200), fa.FA_ERR_INVALID_ARG),
    (dict(seqlen_q=1 << 20, seqlen_k=1 << 20, n_heads=64, d_head=128), fa.FA_ERR_UNSUPPORTED),
])
def test_bad_arguments_rejected_on_host(over, status):
    assert call(**over) == status
    assert fa.fa_last_error() != ""


def test_lse_alignment_4_is_enough_for_checks():
    # A misaligned lse is the only fault here; a 4-byte aligned one passes that check and
    # the call then fails on the (absent) null-pointer q instead.
    assert call(q=None, lse=A + 4) == fa.FA_ERR_INVALID_ARG


def test_config_registry_host_only():
    for dtype in (fa.FA_BF16, fa.FA_FP16):
        for d in (32, 64, 128):
            cfgs = fa.fa_fwd_list_configs(d, dtype)
            assert len(cfgs) == fa.fa_fwd_num_configs(d, dtype) >= 1
            for c in cfgs:
                assert c.stages in (1, 2, 3, 4)
                assert c.schedule in (0, 1, 2, 4, 5)
                if c.schedule in (4, 5):
                    assert c.bc == 32
                if c.schedule == 5:
                    assert c.br == 384 and c.waves == 12 and c.stages == 3
                tile = c.bc * d * 2
                if c.schedule == 1:
                    assert c.br == 64 * c.waves and c.stages == 2
                    assert fa.fa_fwd_config_lds_bytes(d, c) == 5 * tile
                else:
                    if c.schedule == 2:
                        assert c.waves == 8 and c.stages == 3
                    assert c.br == 32 * c.waves
                    assert fa.fa_fwd_config_lds_bytes(d, c) == c.stages * 2 * tile
                assert fa.fa_fwd_config_lds_bytes(d, c) <= 160 * 1024
    with pytest.raises(fa.FaError):
        fa.fa_fwd_num_configs(48, fa.FA_BF16)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_num_configs(64, 7)


def test_default_and_forced_config():
    c = fa.fa_fwd_get_config(16, 4096, 4096, 16, 128, fa.FA_BF16)
    assert c.as_tuple() == (256, 64, 8, 3, 2)
    small = fa.fa_fwd_get_config(1, 64, 4096, 1, 128, fa.FA_BF16)
    assert small.br == 64
    with pytest.raises(fa.FaError):
        fa.fa_fwd_set_config(128, fa.FA_BF16, (96, 64, 3, 2))  # not compiled
    fa.fa_fwd_set_config(128, fa.FA_BF16, (128, 32, 4, 2))
    try:
        assert fa.fa_fwd_get_config(16, 4096, 4096, 16, 128, fa.FA_BF16).as_tuple() == (128, 32, 4, 2, 0)
        # forcing one (d, dtype) leaves the others alone
        assert fa.fa_fwd_get_config(16, 4096, 4096, 16, 64, fa.FA_BF16).as_tuple() == (128, 64, 4, 2, 0)
    finally:
        fa.fa_fwd_set_config(128, fa.FA_BF16, None)
    assert fa.fa_fwd_get_config(16, 4096, 4096, 16, 128, fa.FA_BF16).as_tuple() == (256, 64, 8, 3, 2)


def test_causal_default_config():
    # the causal default at d_head 128 is the three-per-SIMD schedule on 32-key tiles
    c = fa.fa_fwd_get_config_ext(16, 4096, 4096, 16, 128, fa.FA_BF16, causal=True)
    assert c.as_tuple() == (128, 32, 4, 2, 4)
    assert fa.fa_fwd_get_config_ext(16, 4096, 4096, 16, 128, fa.FA_BF16).as_tuple() == \
        fa.fa_fwd_get_config(16, 4096, 4096, 16, 128, fa.FA_BF16).as_tuple()
    # causal must be 0 or 1
    st = fa.lib().fa_fwd_get_config_ext(1, 64, 64, 1, 128, fa.FA_BF16, 0, 2, ctypes.byref(fa.TileConfig()))
    assert st == fa.FA_ERR_INVALID_ARG


def test_autotune_rejects_bad_args_on_host():
    L = fa.lib()
    st = L.fa_fwd_autotune(A, A, A, A, A, 1, 128, 128, 2, 64, ctypes.c_float(0.125), None, 0, None, 0,
                           None, None)
    assert st == fa.FA_ERR_INVALID_ARG  # reps must be >= 1
    st = L.fa_fwd_autotune(None, A, A, A, A, 1, 128, 128, 2, 64, ctypes.c_float(0.125), None, 0, None, 3,
                           None, None)
    assert st == fa.FA_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


def call_ext(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, seqlen_q=128, seqlen_k=128, n_heads=4, n_heads_kv=2,
                d_head=64, scale=0.125, causal=1, cu_seqlens=None, dtype=fa.FA_BF16, num_splits=4,
                workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(over)
    L = fa.lib()
    return L.fa_fwd_ext(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"],
                        args["seqlen_q"], args["seqlen_k"], args["n_heads"], args["n_heads_kv"],
                        args["d_head"], ctypes.c_float(args["scale"]), args["causal"], args["cu_seqlens"],
                        args["dtype"], args["num_splits"], args["workspace"], args["workspace_bytes"],
                        args["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(n_heads_kv=0), fa.FA_ERR_INVALID_ARG),
    (dict(n_heads_kv=3), fa.FA_ERR_INVALID_ARG),          # does not divide 4
    (dict(n_heads_kv=8), fa.FA_ERR_INVALID_ARG),          # more K/V heads than query heads
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=fa.FA_MAX_SPLITS + 1), fa.FA_ERR_INVALID_ARG),
    (dict(workspace=None), fa.FA_ERR_INVALID_ARG),        # 4 splits need a workspace
    (dict(workspace=A + 8), fa.FA_ERR_MISALIGNED),
    (dict(workspace_bytes=4 * 128 * 4 * 65 * 4 - 1), fa.FA_ERR_INVALID_ARG),  # one byte short
    (dict(d_head=80), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(cu_seqlens=A, seqlen_q=64, seqlen_k=128), fa.FA_ERR_INVALID_ARG),
])
def test_ext_bad_arguments_rejected_on_host(over, status):
    assert call_ext(**over) == status
    assert fa.fa_last_error() != ""


def test_workspace_bytes():
    # splits x batch x heads x seqlen_q x (d + 1) x 4
    assert fa.fa_fwd_workspace_bytes(1, 128, 4, 64, 4) == 4 * 128 * 4 * 65 * 4
    assert fa.fa_fwd_workspace_bytes(2, 64, 1, 128, 32) == 32 * 2 * 64 * 129 * 4
    assert fa.fa_fwd_workspace_bytes(3, 10, 2, 32, 1) == 0
    for bad in ((0, 128, 4, 64, 4), (1, 128, 4, 64, 0), (1, 128, 4, 64, fa.FA_MAX_SPLITS + 1)):
        with pytest.raises(fa.FaError):
            fa.fa_fwd_workspace_bytes(*bad)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_workspace_bytes(1, 128, 4, 48, 4)


def test_choose_splits():
    # 64 queries over 4096 keys, one head: one workgroup alone -> split, at most one split per
    # four 64-key tiles
    assert fa.fa_fwd_choose_splits(1, 64, 4096, 1, 128, fa.FA_BF16) == 16
    # a grid that already covers the CUs is not split
    assert fa.fa_fwd_choose_splits(16, 4096, 4096, 16, 128, fa.FA_BF16) == 1
    # few keys: no split possible
    assert fa.fa_fwd_choose_splits(1, 64, 64, 1, 64, fa.FA_BF16) == 1
    # causal top-left: 64 queries see at most 64 keys
    assert fa.fa_fwd_choose_splits(1, 64, 4096, 1, 128, fa.FA_BF16, causal=True) == 1
    n = fa.fa_fwd_choose_splits(2, 256, 8192, 4, 128, fa.FA_BF16)
    assert 1 < n <= fa.FA_MAX_SPLITS
    with pytest.raises(fa.FaError):
        fa.fa_fwd_choose_splits(0, 64, 4096, 1, 128, fa.FA_BF16)


def test_ext_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 4, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd_ext(q, k, k, causal=True)


def test_bwd_workspace_bytes_and_bad_arguments():
    assert fa.fa_bwd_workspace_bytes(2, 100, 4, 64) == 2 * 100 * 4 * 2 * 4
    assert fa.fa_bwd_workspace_bytes(2, 100, 4, 64, atomic_dq=True) == 2 * 100 * 4 * 66 * 4
    with pytest.raises(fa.FaError):
        fa.fa_bwd_workspace_bytes(2, 100, 4, 80)
    L = fa.lib()
    base = dict(q=A, k=A, v=A, o=A, dout=A, lse=A, dq=A, dk=A, dv=A, batch=1, seqlen_q=128, seqlen_k=128,
                n_heads=4, n_heads_kv=2, d_head=64, scale=0.125, causal=0, cu=None, dtype=fa.FA_BF16, atomic_dq=0,
                ws=A, ws_bytes=1 << 30, stream=None)

    def call_bwd(**over):
        a = dict(base, **over)
        return L.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"], a["batch"],
                        a["seqlen_q"], a["seqlen_k"], a["n_heads"], a["n_heads_kv"], a["d_head"],
                        ctypes.c_float(a["scale"]), a["causal"], a["cu"], a["dtype"], a["atomic_dq"], a["ws"],
                        a["ws_bytes"], a["stream"])
    for over, status in ((dict(o=None), fa.FA_ERR_INVALID_ARG), (dict(dout=None), fa.FA_ERR_INVALID_ARG),
                         (dict(dq=None), fa.FA_ERR_INVALID_ARG), (dict(dk=None), fa.FA_ERR_INVALID_ARG),
                         (dict(dv=None), fa.FA_ERR_INVALID_ARG), (dict(ws=None), fa.FA_ERR_INVALID_ARG),
                         (dict(ws=A + 4), fa.FA_ERR_MISALIGNED), (dict(dk=A + 2), fa.FA_ERR_MISALIGNED),
                         (dict(ws_bytes=128 * 4 * 2 * 4 - 1), fa.FA_ERR_INVALID_ARG),
                         (dict(atomic_dq=1, ws_bytes=128 * 4 * 2 * 4), fa.FA_ERR_INVALID_ARG),
                         (dict(atomic_dq=2), fa.FA_ERR_INVALID_ARG), (dict(n_heads_kv=3), fa.FA_ERR_INVALID_ARG),
                         (dict(causal=5), fa.FA_ERR_INVALID_ARG), (dict(d_head=48), fa.FA_ERR_UNSUPPORTED)):
        assert call_bwd(**over) == status, over
        assert fa.fa_last_error() != ""


def call_noalloc(**over):
    args = dict(q=A, k=A, v=A, o=A, lse=A, batch=8, seqlen_q=512, seqlen_k=512, n_heads=16, n_heads_kv=16,
                d_head=128, scale=0.125, causal=0, cu_seqlens=None, dtype=fa.FA_BF16, num_splits=4, stream=None)
    args.update(over)
    return fa.lib().fa_fwd_ext_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"],
                                       args["seqlen_q"], args["seqlen_k"], args["n_heads"], args["n_heads_kv"],
                                       args["d_head"], ctypes.c_float(args["scale"]), args["causal"],
                                       args["cu_seqlens"], args["dtype"], args["num_splits"], args["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(n_heads_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(num_splits=fa.FA_MAX_SPLITS + 1), fa.FA_ERR_INVALID_ARG),
    (dict(d_head=80), fa.FA_ERR_UNSUPPORTED),
    (dict(o=A + 8), fa.FA_ERR_MISALIGNED),
])
def test_noalloc_bad_arguments_rejected_on_host(over, status):
    assert call_noalloc(**over) == status
    assert fa.fa_last_error() != ""


def test_noalloc_rejects_splits_beyond_its_static_scratch_on_host():
    # 8 x 16 heads x 512 rows x 129 floats x 4 bytes = 33.8 MB per split: even 1 split's
    # worth exceeds 16 MiB, so any count > 1 is refused before the device is touched
    need = fa.fa_fwd_workspace_bytes(8, 512, 16, 128, 4)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(num_splits=4) == fa.FA_ERR_INVALID_ARG
    msg = fa.fa_last_error()
    assert str(need) in msg and str(fa.FA_NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    assert re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(16u << 20\)", text)
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20


def test_tune_cache_save_load_reset_host_only(tmp_path):
    fa.fa_fwd_tune_reset()
    try:
        # d_head dtype varlen causal log2_group log2_seqlen_q log2_batch_heads : br bc waves stages schedule ms
        path = tmp_path / "tune.txt"
        path.write_text("# comment\n"
                        "64 1 0 1 2 10 4 : 128 32 4 2 0 0.25000\n"
                        "64 1 0 0 0 10 4 : 999 32 4 2 0 0.1\n"          # not compiled: skipped
                        "garbage line\n")
        assert fa.fa_fwd_tune_load(str(path)) == 1
        cfg, _, src = fa.fa_fwd_query_config(2, 1000, 1000, 8, 64, fa.FA_FP16, n_heads_kv=2, causal=True)
        assert src == "tuned" and cfg.as_tuple() == (128, 32, 4, 2, 0)
        # same size class (ceil log2 of 600 and 1000 is 10; 2 x 8 heads -> 4), other kind: default
        assert fa.fa_fwd_query_config(2, 600, 600, 8, 64, fa.FA_FP16, n_heads_kv=2, causal=True)[2] == "tuned"
        assert fa.fa_fwd_query_config(2, 1000, 1000, 8, 64, fa.FA_FP16, causal=True)[2] == "default"
        assert fa.fa_fwd_query_config(2, 1000, 1000, 8, 64, fa.FA_BF16, n_heads_kv=2, causal=True)[2] == "default"
        out = tmp_path / "saved.txt"
        fa.fa_fwd_tune_save(str(out))
        lines = [ln for ln in out.read_text().splitlines() if not ln.startswith("#")]
        assert lines == ["64 1 0 1 2 10 4 : 128 32 4 2 0 0.25000"]
        fa.fa_fwd_tune_reset()
        assert fa.fa_fwd_query_config(2, 1000, 1000, 8, 64, fa.FA_FP16, n_heads_kv=2, causal=True)[2] == "default"
        with pytest.raises(fa.FaError):
            fa.fa_fwd_tune_load(str(tmp_path / "missing.txt"))
    finally:
        fa.fa_fwd_tune_reset()


def test_tune_cache_environment_variable(tmp_path):
    path = tmp_path / "env_tune.txt"
    path.write_text("128 0 0 0 0 12 8 : 256 64 8 3 0 1.9\n")
    code = ("from exact_attention_17_amd import fa; "
            "c, n, s = fa.fa_fwd_query_config(16, 4096, 4096, 16, 128, fa.FA_BF16); print(c.as_tuple(), s)")
    env = dict(os.environ, FA_FWD_TUNE_CACHE=str(path))
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "(256, 64, 8, 3, 0) tuned"


def test_autotune_ext_rejects_bad_args_on_host():
    L = fa.lib()
    c = fa.TileConfig()
    ms = ctypes.c_float()

    def tune(**over):
        a = dict(q=A, rounds=5, num_splits=1, workspace=None, workspace_bytes=0, n_heads_kv=2, causal=0)
        a.update(over)
        return L.fa_fwd_autotune_ext(a["q"], A, A, A, A, 1, 128, 128, 4, a["n_heads_kv"], 64,
                                     ctypes.c_float(0.125), a["causal"], None, fa.FA_BF16, a["num_splits"],
                                     a["workspace"], a["workspace_bytes"], None, a["rounds"], ctypes.byref(c),
                                     ctypes.byref(ms))
    assert tune(q=None) == fa.FA_ERR_INVALID_ARG
    assert tune(rounds=0) == fa.FA_ERR_INVALID_ARG
    assert tune(rounds=101) == fa.FA_ERR_INVALID_ARG
    assert tune(n_heads_kv=3) == fa.FA_ERR_INVALID_ARG
    assert tune(causal=2) == fa.FA_ERR_INVALID_ARG
    assert tune(num_splits=4) == fa.FA_ERR_INVALID_ARG       # no workspace for 4 splits
    assert tune(num_splits=4, workspace=A + 8, workspace_bytes=1 << 30) == fa.FA_ERR_MISALIGNED
    assert tune(num_splits=-1) == fa.FA_ERR_INVALID_ARG
