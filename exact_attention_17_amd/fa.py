"""Thin ctypes binding over libfa_fwd.so (include/fa_fwd.h).

Argument marshalling only: every step of the forward pass runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is missing this module raises; there is no fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa_fwd.so")

FA_BF16, FA_FP16 = 0, 1
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_MISALIGNED, FA_ERR_HIP = 0, 1, 2, 3, 4
FA_MAX_SPLITS = 128

# Every exported symbol of include/fa_fwd.h.
EXPORTS = ("fa_fwd", "fa_fwd_ext", "fa_fwd_ext_noalloc", "fa_fwd_workspace_bytes", "fa_fwd_choose_splits", "fa_bwd",
           "fa_bwd_workspace_bytes",
           "fa_fwd_autotune", "fa_fwd_autotune_ext", "fa_fwd_tune_ranking", "fa_fwd_tune_reset", "fa_fwd_tune_save",
           "fa_fwd_tune_load", "fa_fwd_set_config", "fa_fwd_get_config", "fa_fwd_get_config_ext",
           "fa_fwd_query_config", "fa_fwd_num_configs", "fa_fwd_list_configs", "fa_fwd_config_lds_bytes",
           "fa_fwd_config_resources", "fa_last_error", "fa_version")


class FaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("fa_fwd status %d: %s" % (status, msg))
        self.status = status


class TileConfig(ctypes.Structure):
    _fields_ = [("br", ctypes.c_int), ("bc", ctypes.c_int), ("waves", ctypes.c_int),
                ("stages", ctypes.c_int), ("schedule", ctypes.c_int)]

    def as_tuple(self):
        return (self.br, self.bc, self.waves, self.stages, self.schedule)

    def __repr__(self):
        return "TileConfig(br=%d, bc=%d, waves=%d, stages=%d, schedule=%d)" % self.as_tuple()


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int


def lib():
    """Load libfa_fwd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime (same soname as the system one).  Load it first so
        # that libfa_fwd.so binds to that runtime: two HIP runtimes in one process do not
        # share devices, memory or streams.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfa_fwd.so is not built: run `python -m exact_attention_17_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.fa_fwd.restype = _i
        L.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _vp, _i, _vp]
        L.fa_fwd_ext.restype = _i
        L.fa_fwd_ext.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _vp, _i,
                                 _i, _vp, ctypes.c_size_t, _vp]
        L.fa_fwd_ext_noalloc.restype = _i
        L.fa_fwd_ext_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _vp,
                                         _i, _i, _vp]
        L.fa_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.fa_fwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.fa_fwd_choose_splits.restype = _i
        L.fa_fwd_choose_splits.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
        L.fa_bwd.restype = _i
        L.fa_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float,
                             _i, _vp, _i, _i, _vp, ctypes.c_size_t, _vp]
        L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i]
        L.fa_fwd_autotune.restype = _i
        L.fa_fwd_autotune.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.c_float, _vp,
                                      _i, _vp, _i, ctypes.POINTER(TileConfig),
                                      ctypes.POINTER(ctypes.c_float)]
        L.fa_fwd_autotune_ext.restype = _i
        L.fa_fwd_autotune_ext.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _vp,
                                          _i, _i, _vp, ctypes.c_size_t, _vp, _i, ctypes.POINTER(TileConfig),
                                          ctypes.POINTER(ctypes.c_float)]
        L.fa_fwd_tune_ranking.restype = _i
        L.fa_fwd_tune_ranking.argtypes = [ctypes.POINTER(TileConfig), ctypes.POINTER(ctypes.c_float), _i]
        L.fa_fwd_tune_reset.restype = _i
        L.fa_fwd_tune_reset.argtypes = []
        L.fa_fwd_tune_save.restype = _i
        L.fa_fwd_tune_save.argtypes = [ctypes.c_char_p]
        L.fa_fwd_tune_load.restype = _i
        L.fa_fwd_tune_load.argtypes = [ctypes.c_char_p]
        L.fa_fwd_query_config.restype = _i
        L.fa_fwd_query_config.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(TileConfig),
                                          ctypes.POINTER(_i), ctypes.POINTER(_i)]
        L.fa_fwd_set_config.restype = _i
        L.fa_fwd_set_config.argtypes = [_i, _i, ctypes.POINTER(TileConfig)]
        L.fa_fwd_get_config.restype = _i
        L.fa_fwd_get_config.argtypes = [_i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(TileConfig)]
        L.fa_fwd_get_config_ext.restype = _i
        L.fa_fwd_get_config_ext.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, ctypes.POINTER(TileConfig)]
        L.fa_fwd_num_configs.restype = _i
        L.fa_fwd_num_configs.argtypes = [_i, _i]
        L.fa_fwd_list_configs.restype = _i
        L.fa_fwd_list_configs.argtypes = [_i, _i, ctypes.POINTER(TileConfig), _i]
        L.fa_fwd_config_lds_bytes.restype = _i
        L.fa_fwd_config_lds_bytes.argtypes = [_i, ctypes.POINTER(TileConfig)]
        L.fa_fwd_config_resources.restype = _i
        L.fa_fwd_config_resources.argtypes = [_i, _i, ctypes.POINTER(TileConfig),
                                              ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i)]
        L.fa_last_error.restype = ctypes.c_char_p
        L.fa_last_error.argtypes = []
        L.fa_version.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        _lib = L
    return _lib


def fa_last_error():
    return lib().fa_last_error().decode()


def fa_version():
    return lib().fa_version().decode()


def _check(status):
    if status != FA_OK:
        raise FaError(status, fa_last_error())
    return status


def fa_fwd_raw(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, d_head, scale, cu_seqlens,
               dtype, stream):
    """The C call with integer pointers; returns the status code (no exception)."""
    return lib().fa_fwd(q, k, v, o, lse, batch, seqlen_q, seqlen_k, n_heads, d_head, float(scale),
                        cu_seqlens, dtype, stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_FP16
    raise TypeError("q, k, v must be bfloat16 or float16")


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _shape_args(q, k, v, cu_seqlens, max_seqlen, grouped=False):
    """-> (batch, seqlen_q, seqlen_k, n_heads, n_heads_kv, d_head).  The library checks that
    n_heads_kv divides n_heads; without grouped, k and v must have q's head count."""
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
            raise ValueError("dense q, k, v must be [B, N, H, D] with k and v alike")
        batch, nq, heads, d = q.shape
        if k.shape[0] != batch or k.shape[3] != d or (not grouped and k.shape[2] != heads):
            raise ValueError("q and k disagree on batch, heads or d_head")
        return batch, nq, k.shape[1], heads, k.shape[2], d
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or \
            k.shape[2] != q.shape[2] or (not grouped and k.shape[1] != q.shape[1]):
        raise ValueError("varlen q must be [total, H, D] and k, v [total, H (or Hkv), D]")
    if max_seqlen is None:
        raise ValueError("varlen calls need max_seqlen")
    return cu_seqlens.numel() - 1, int(max_seqlen), int(max_seqlen), q.shape[1], k.shape[1], q.shape[2]


def _check_tensors(q, k, v, cu_seqlens):
    import torch
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share one dtype")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise TypeError("cu_seqlens must be an int32 device tensor")


def _outputs(q, o, lse, batch, heads, nq):
    """Allocate o and lse, or check caller-supplied ones against what the kernels write: o a
    contiguous device tensor shaped and typed like q, lse a contiguous float32 device tensor
    [batch, n_heads, seqlen_q] (packed: max_seqlen rows per sequence)."""
    import torch
    if o is None:
        o = torch.empty_like(q)
    elif not o.is_cuda or o.device != q.device or not o.is_contiguous() or o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must be a contiguous device tensor on q's device, shaped and typed like q")
    if lse is None:
        lse = torch.empty((batch, heads, nq), dtype=torch.float32, device=q.device)
    elif not lse.is_cuda or lse.device != q.device or not lse.is_contiguous() or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (batch, heads, nq):
        raise ValueError("lse must be a contiguous float32 device tensor [batch, n_heads, seqlen_q] on q's device")
    return o, lse


def fa_fwd(q, k, v, o=None, lse=None, scale=None, cu_seqlens=None, max_seqlen=None, stream=None):
    """Attention forward on torch device tensors; returns (o, lse).

    Dense: q [B, Nq, H, D], k/v [B, Nk, H, D] -> o like q, lse [B, H, Nq] fp32.
    Varlen: q/k/v [total, H, D], cu_seqlens int32 [B+1] on the device, max_seqlen ->
    o like q, lse [B, H, max_seqlen] (rows past a sequence's end untouched).
    o and lse may be given (preallocated); otherwise they are allocated with torch.
    """
    batch, nq, nk, heads, _, d = _shape_args(q, k, v, cu_seqlens, max_seqlen)
    _check_tensors(q, k, v, cu_seqlens)
    if scale is None:
        scale = d ** -0.5
    o, lse = _outputs(q, o, lse, batch, heads, nq)
    st = lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), batch, nq,
                      nk, heads, d, float(scale), cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                      _dtype_code(q), _stream_handle(stream, q.device))
    _check(st)
    return o, lse


def fa_fwd_ext(q, k, v, o=None, lse=None, scale=None, causal=False, cu_seqlens=None, max_seqlen=None,
               num_splits=1, workspace=None, stream=None):
    """Attention forward with grouped K/V heads, the causal mask and split keys; returns (o, lse).

    k and v may have fewer heads than q (a divisor of them: MQA/GQA).  causal masks key j for
    query i when j > i.  num_splits: 1 = no split, 0 = automatic, n > 1 = n splits.  A split
    call needs a device workspace of fa_fwd_workspace_bytes(...) bytes; when workspace is None
    one is allocated with torch (for num_splits = 0, sized for the automatic count).
    """
    import torch
    batch, nq, nk, heads, heads_kv, d = _shape_args(q, k, v, cu_seqlens, max_seqlen, grouped=True)
    _check_tensors(q, k, v, cu_seqlens)
    if scale is None:
        scale = d ** -0.5
    o, lse = _outputs(q, o, lse, batch, heads, nq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    elif num_splits != 1:
        n = num_splits if num_splits > 1 else fa_fwd_choose_splits(
            batch, nq, nk, heads, d, _dtype_code(q), causal, cu_seqlens is not None)
        if n > 1:
            workspace = torch.empty(fa_fwd_workspace_bytes(batch, nq, heads, d, n), dtype=torch.uint8,
                                    device=q.device)
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().fa_fwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), batch, nq,
                          nk, heads, heads_kv, d, float(scale), int(bool(causal)),
                          cu_seqlens.data_ptr() if cu_seqlens is not None else None, _dtype_code(q),
                          int(num_splits), ws_ptr, ws_bytes, _stream_handle(stream, q.device))
    _check(st)
    return o, lse


FA_NOALLOC_SCRATCH_BYTES = 16 << 20


def fa_fwd_ext_noalloc(q, k, v, o, lse, scale=None, causal=False, cu_seqlens=None, max_seqlen=None,
                       num_splits=0, stream=None):
    """fa_fwd_ext without a workspace: split scratch comes from the library's static device
    array (FA_NOALLOC_SCRATCH_BYTES per GPU).  o and lse must be given (nothing is
    allocated).  Returns (o, lse)."""
    if o is None or lse is None:
        raise ValueError("fa_fwd_ext_noalloc writes into caller-supplied o and lse")
    batch, nq, nk, heads, heads_kv, d = _shape_args(q, k, v, cu_seqlens, max_seqlen, grouped=True)
    _check_tensors(q, k, v, cu_seqlens)
    if scale is None:
        scale = d ** -0.5
    o, lse = _outputs(q, o, lse, batch, heads, nq)
    st = lib().fa_fwd_ext_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), batch,
                                  nq, nk, heads, heads_kv, d, float(scale), int(bool(causal)),
                                  cu_seqlens.data_ptr() if cu_seqlens is not None else None, _dtype_code(q),
                                  int(num_splits), _stream_handle(stream, q.device))
    _check(st)
    return o, lse


def fa_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, scale=None, causal=False, cu_seqlens=None,
           max_seqlen=None, atomic_dq=False, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the forward pass given its output o and lse and dout = dPhi/dO.
    Shapes as in fa_fwd_ext (k and v may have fewer heads); dout like q.  atomic_dq selects dQ
    by atomic adds (the pages' Algorithm 2) instead of the separate dQ pass.  A workspace of
    fa_bwd_workspace_bytes(...) bytes is allocated with torch when none is given."""
    import torch
    batch, nq, nk, heads, heads_kv, d = _shape_args(q, k, v, cu_seqlens, max_seqlen, grouped=True)
    _check_tensors(q, k, v, cu_seqlens)
    for t in (o, dout):
        if not t.is_cuda or not t.is_contiguous() or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("o and dout must be contiguous device tensors shaped and typed like q")
    if not lse.is_cuda or lse.dtype != torch.float32 or tuple(lse.shape) != (batch, heads, nq):
        raise ValueError("lse must be a float32 device tensor [batch, n_heads, seqlen_q]")
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if not g.is_cuda or g.device != q.device or not g.is_contiguous() or g.shape != like.shape or \
                g.dtype != like.dtype:
            raise ValueError("%s must be a contiguous device tensor shaped and typed like its input" % name)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(batch, nq, heads, d, atomic_dq), dtype=torch.uint8,
                                device=q.device)
    st = lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), batch, nq, nk, heads, heads_kv, d, float(scale),
                      int(bool(causal)), cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                      _dtype_code(q), int(bool(atomic_dq)), workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), _stream_handle(stream, q.device))
    _check(st)
    return dq, dk, dv


def fa_bwd_workspace_bytes(batch, seqlen_q, n_heads, d_head, atomic_dq=False):
    """Workspace bytes fa_bwd needs."""
    n = lib().fa_bwd_workspace_bytes(batch, seqlen_q, n_heads, d_head, int(bool(atomic_dq)))
    if n == 0:
        raise FaError(FA_ERR_INVALID_ARG, fa_last_error())
    return n


def fa_fwd_workspace_bytes(batch, seqlen_q, n_heads, d_head, num_splits):
    """Workspace bytes fa_fwd_ext needs for num_splits splits (0 for one)."""
    n = lib().fa_fwd_workspace_bytes(batch, seqlen_q, n_heads, d_head, num_splits)
    if n == 0 and num_splits != 1:
        raise FaError(FA_ERR_INVALID_ARG, fa_last_error())
    return n


def fa_fwd_choose_splits(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, causal=False, varlen=False):
    """The split count fa_fwd_ext's automatic choice starts from."""
    n = lib().fa_fwd_choose_splits(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, int(bool(causal)),
                                   int(bool(varlen)))
    if n < 0:
        raise FaError(-n, fa_last_error())
    return n


def fa_fwd_autotune(q, k, v, o, lse, scale=None, cu_seqlens=None, max_seqlen=None, reps=5, stream=None):
    """Tune an fa_fwd call (reps = interleaved rounds) on these buffers; returns (TileConfig, ms)."""
    return fa_fwd_autotune_ext(q, k, v, o, lse, scale=scale, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen,
                               rounds=reps, stream=stream)


def fa_fwd_autotune_ext(q, k, v, o, lse, scale=None, causal=False, cu_seqlens=None, max_seqlen=None,
                        num_splits=1, workspace=None, rounds=5, stream=None):
    """Tune an fa_fwd_ext call of this kind on these buffers (interleaved median timing of every
    compiled configuration); returns (TileConfig, median ms per launch of the winner)."""
    batch, nq, nk, heads, heads_kv, d = _shape_args(q, k, v, cu_seqlens, max_seqlen, grouped=True)
    _check_tensors(q, k, v, cu_seqlens)
    if scale is None:
        scale = d ** -0.5
    o, lse = _outputs(q, o, lse, batch, heads, nq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda:
            raise ValueError("workspace must be a device tensor")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    chosen = TileConfig()
    ms = ctypes.c_float()
    st = lib().fa_fwd_autotune_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   batch, nq, nk, heads, heads_kv, d, float(scale), int(bool(causal)),
                                   cu_seqlens.data_ptr() if cu_seqlens is not None else None, _dtype_code(q),
                                   int(num_splits), ws_ptr, ws_bytes, _stream_handle(stream, q.device),
                                   int(rounds), ctypes.byref(chosen), ctypes.byref(ms))
    _check(st)
    return chosen, ms.value


def fa_fwd_tune_ranking():
    """The last tuning's candidates, fastest first: [(TileConfig, median ms), ...]."""
    n = lib().fa_fwd_tune_ranking(None, None, 0)
    if n < 0:
        raise FaError(-n, fa_last_error())
    cfgs, ms = (TileConfig * max(n, 1))(), (ctypes.c_float * max(n, 1))()
    lib().fa_fwd_tune_ranking(cfgs, ms, n)
    return [(cfgs[i], ms[i]) for i in range(n)]


def fa_fwd_tune_reset():
    return _check(lib().fa_fwd_tune_reset())


def fa_fwd_tune_save(path):
    return _check(lib().fa_fwd_tune_save(os.fsencode(path)))


def fa_fwd_tune_load(path):
    n = lib().fa_fwd_tune_load(os.fsencode(path))
    if n < 0:
        raise FaError(-n, fa_last_error())
    return n


CONFIG_SOURCES = {0: "default", 1: "tuned", 2: "FA_FWD_CONFIG", 3: "forced"}


def fa_fwd_query_config(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, n_heads_kv=None, varlen=False,
                        causal=False):
    """(TileConfig, automatic split count, source) fa_fwd_ext would use for this call kind."""
    c, n, src = TileConfig(), _i(), _i()
    _check(lib().fa_fwd_query_config(batch, seqlen_q, seqlen_k, n_heads, n_heads if n_heads_kv is None else n_heads_kv,
                                     d_head, dtype, int(bool(varlen)), int(bool(causal)), ctypes.byref(c),
                                     ctypes.byref(n), ctypes.byref(src)))
    return c, n.value, CONFIG_SOURCES[src.value]


def fa_fwd_set_config(d_head, dtype, cfg):
    """Force (br, bc, waves, stages) for (d_head, dtype); cfg None = automatic."""
    if cfg is None:
        return _check(lib().fa_fwd_set_config(d_head, dtype, None))
    c = cfg if isinstance(cfg, TileConfig) else TileConfig(*cfg)
    return _check(lib().fa_fwd_set_config(d_head, dtype, ctypes.byref(c)))


def fa_fwd_get_config(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, varlen=False):
    c = TileConfig()
    _check(lib().fa_fwd_get_config(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, int(bool(varlen)),
                                   ctypes.byref(c)))
    return c


def fa_fwd_get_config_ext(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, varlen=False, causal=False):
    c = TileConfig()
    _check(lib().fa_fwd_get_config_ext(batch, seqlen_q, seqlen_k, n_heads, d_head, dtype, int(bool(varlen)),
                                       int(bool(causal)), ctypes.byref(c)))
    return c


def fa_fwd_num_configs(d_head, dtype):
    n = lib().fa_fwd_num_configs(d_head, dtype)
    if n < 0:
        raise FaError(-n, fa_last_error())
    return n


def fa_fwd_list_configs(d_head, dtype):
    n = fa_fwd_num_configs(d_head, dtype)
    arr = (TileConfig * max(n, 1))()
    lib().fa_fwd_list_configs(d_head, dtype, arr, n)
    return [arr[i] for i in range(n)]


def fa_fwd_config_lds_bytes(d_head, cfg):
    c = cfg if isinstance(cfg, TileConfig) else TileConfig(*cfg)
    n = lib().fa_fwd_config_lds_bytes(d_head, ctypes.byref(c))
    if n < 0:
        raise FaError(-n, fa_last_error())
    return n


def fa_fwd_config_resources(d_head, dtype, cfg):
    """(vgprs, spill_bytes, lds_bytes) of a compiled configuration (needs a GPU)."""
    c = cfg if isinstance(cfg, TileConfig) else TileConfig(*cfg)
    a, b, l_ = _i(), _i(), _i()
    _check(lib().fa_fwd_config_resources(d_head, dtype, ctypes.byref(c), ctypes.byref(a), ctypes.byref(b),
                                         ctypes.byref(l_)))
    return a.value, b.value, l_.value
