"""MI355X-native Kimi Delta Attention (KDA) operator.

Python binding of the C ABI in include/kda.h (libkda.so, built in-tree by
gated_delta_rule_amd.build).  This module only marshals arguments: torch
supplies device memory and the current HIP stream, and every step of the
operator runs in the library's HIP kernels.  If the library is missing the
calls raise; there is no fallback.

    o, S_T = chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None)
    o = decode_step(q, k, v, log_alpha, beta, S)       # S updated in place
    o = recurrent_fwd(q, k, v, log_alpha, beta, S, replay=None, n_replay=None,
                      commit=True)                     # up to 64 tokens per request
    q, k, v, log_alpha, beta = prologue(q_raw, k_raw, v_raw, conv_w, a, b, conv_cache)
    out = epilogue(o, g, w)                            # gated RMSNorm of the output
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["chunk_fwd", "decode_step", "recurrent_fwd", "prologue", "epilogue",
           "chunk_fwd_workspace_bytes",
           "library_path", "load_library", "KDAError", "KDA_BF16", "KDA_F32", "HEAD_DIM"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
KDA_BF16, KDA_F32 = 0, 1
HEAD_DIM = 128
_lib = None


class KDAError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise KDAError(f"{_LIB_PATH} not found: build it with "
                       "`python -m gated_delta_rule_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_bytes.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, ip, i32, i64, i32,
                                  i32, i32, fp, fp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, i32, i32, i32, i32,
                                    fp, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_recurrent_fwd.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, vp, vp, vp, fp, fp, ip,
                                      fp, i32, i32, i32, i32, i32, i32, ctypes.c_int, fp, vp]
    lib.kda_recurrent_fwd.restype = ctypes.c_int
    lib.kda_prologue.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, fp, ip, i32, i64, i32, i32,
                                 vp, vp, vp, fp, fp, vp]
    lib.kda_prologue.restype = ctypes.c_int
    lib.kda_epilogue.argtypes = [fp, fp, fp, i64, i32, i32, fp, vp]
    lib.kda_epilogue.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, ip, i32, i64, i32,
                                          i32, i32, fp, fp, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_workspace_bytes_window.argtypes = [i32, i64, i32, i32, i32, i64]
    lib.kda_chunk_bwd_workspace_bytes_window.restype = sz
    lib.kda_chunk_bwd.argtypes = [vp, vp, vp, ctypes.c_int, fp, fp, fp, ip, i32, i64, i32, i32,
                                  i32, fp, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _status(rc: int, what: str):
    if rc != 0:
        msg = load_library().kda_status_str(rc).decode()
        raise KDAError(f"{what}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _in_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise KDAError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, dtype=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise KDAError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise KDAError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise KDAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KDAError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise KDAError(f"{name} is on {t.device}, expected {device}")


def chunk_fwd_workspace_bytes(n_seqs: int, T: int, H: int, varlen: bool) -> int:
    return int(load_library().kda_chunk_fwd_workspace_bytes(n_seqs, T, H, HEAD_DIM,
                                                            HEAD_DIM, int(varlen)))


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
              output_final_state: bool = True, o=None, S_T=None, workspace=None,
              sequence_parallel: bool = True):
    """Chunkwise KDA prefill (see kda_chunk_fwd in include/kda.h).

    Equal-length batch: q, k, log_alpha [B, T, H, 128]; v [B, T, H, 128];
    beta [B, T, H].  Packed varlen batch: the same tensors with a token axis
    [T_total, H, ...] (a leading axis of 1 is allowed) and cu_seqlens int32
    [N+1] on the device.  S0: [N, H, 128, 128] float32 or None.
    Returns (o float32 like v, S_T [N, H, 128, 128] float32 or None).
    sequence_parallel=False keeps equal-length batches on the sequential
    path (no workspace is passed).
    """
    import torch
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    dt = _in_dtype(q)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
        T = q.numel() // (H * dk)
        if q.dim() == 4 and q.shape[0] != 1:
            raise KDAError("packed varlen input must have a leading batch of 1 or none")
    else:
        if q.dim() != 4:
            raise KDAError("q must be [B, T, H, 128] without cu_seqlens")
        n_seqs, T = q.shape[0], q.shape[1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:-1] != q.shape[:-1] \
            or beta.shape != q.shape[:-1]:
        raise KDAError("q/k/log_alpha/v/beta shapes disagree")
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev)
        if tuple(S0.shape) != (n_seqs, H, dk, dv):
            raise KDAError(f"S0 must be {(n_seqs, H, dk, dv)}, got {tuple(S0.shape)}")
    if o is None:
        o = torch.empty(v.shape, dtype=torch.float32, device=dev)
    else:
        _check(o, "o", torch.float32, dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _check(S_T, "S_T", torch.float32, dev)
    ws_bytes = int(lib.kda_chunk_fwd_workspace_bytes(n_seqs, T, H, dk, dv,
                                                     int(cu_seqlens is not None)))
    if cu_seqlens is None and not sequence_parallel:
        ws_bytes, workspace = 0, None
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(log_alpha), _ptr(beta),
                           _ptr(S0), _ptr(cu_seqlens), n_seqs, T, H, dk, dv, _ptr(o),
                           _ptr(S_T), _ptr(workspace),
                           0 if workspace is None else workspace.numel() * workspace.element_size(),
                           ctypes.c_void_p(stream))
    _status(rc, "kda_chunk_fwd")
    return o, S_T


def chunk_bwd_workspace_bytes(n_seqs, T, H, varlen=False, window_tokens=None):
    """kda_chunk_bwd_workspace_bytes, or with window_tokens (equal lengths)
    kda_chunk_bwd_workspace_bytes_window."""
    lib = load_library()
    if window_tokens is None:
        return int(lib.kda_chunk_bwd_workspace_bytes(n_seqs, T, H, 128, 128, int(varlen)))
    if varlen:
        raise KDAError("window_tokens applies to equal-length batches only")
    return int(lib.kda_chunk_bwd_workspace_bytes_window(n_seqs, T, H, 128, 128, int(window_tokens)))


def chunk_bwd(q, k, v, log_alpha, beta, S0, grad_o, grad_S_T=None, cu_seqlens=None, *,
              want_grad_S0: bool = True, workspace=None, window_tokens=None):
    """Backward pass of chunk_fwd (see kda_chunk_bwd in include/kda.h).

    Inputs as for chunk_fwd; grad_o float32 like o; grad_S_T [N, H, 128, 128]
    float32 or None (zero).  Returns (grad_q, grad_k, grad_v, grad_log_alpha,
    grad_beta, grad_S0), all float32 with the shapes of q, k, v, log_alpha,
    beta and S0 ([N, H, 128, 128], or None when want_grad_S0 is False).
    window_tokens (equal lengths, no workspace given): size the workspace for
    that window length instead of the default one.
    """
    import torch
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(grad_o, "grad_o", torch.float32, dev)
    dt = _in_dtype(q)
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
        T = q.numel() // (H * dk)
        if q.dim() == 4 and q.shape[0] != 1:
            raise KDAError("packed varlen input must have a leading batch of 1 or none")
    else:
        if q.dim() != 4:
            raise KDAError("q must be [B, T, H, 128] without cu_seqlens")
        n_seqs, T = q.shape[0], q.shape[1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:-1] != q.shape[:-1] \
            or beta.shape != q.shape[:-1] or grad_o.shape != v.shape:
        raise KDAError("q/k/log_alpha/v/beta/grad_o shapes disagree")
    st_shape = (n_seqs, H, dk, dv)
    for name, t in (("S0", S0), ("grad_S_T", grad_S_T)):
        if t is not None:
            _check(t, name, torch.float32, dev)
            if tuple(t.shape) != st_shape:
                raise KDAError(f"{name} must be {st_shape}, got {tuple(t.shape)}")
    f32 = dict(dtype=torch.float32, device=dev)
    gq, gk = torch.empty(q.shape, **f32), torch.empty(q.shape, **f32)
    gv, gla = torch.empty(v.shape, **f32), torch.empty(q.shape, **f32)
    gb = torch.empty(beta.shape, **f32)
    gS0 = torch.empty(st_shape, **f32) if want_grad_S0 else None
    if window_tokens is not None and cu_seqlens is None:
        ws_bytes = int(lib.kda_chunk_bwd_workspace_bytes_window(n_seqs, T, H, dk, dv,
                                                                int(window_tokens)))
    else:
        ws_bytes = int(lib.kda_chunk_bwd_workspace_bytes(n_seqs, T, H, dk, dv,
                                                         int(cu_seqlens is not None)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(log_alpha), _ptr(beta), _ptr(S0),
                           _ptr(cu_seqlens), n_seqs, T, H, dk, dv, _ptr(grad_o), _ptr(grad_S_T),
                           _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gla), _ptr(gb), _ptr(gS0),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           ctypes.c_void_p(stream))
    _status(rc, "kda_chunk_bwd")
    return gq, gk, gv, gla, gb, gS0


def decode_step(q, k, v, log_alpha, beta, S, *, o=None):
    """One KDA decode step (see kda_decode_step in include/kda.h).

    q, k, log_alpha [B, H, 128]; v [B, H, 128]; beta [B, H];
    S [B, H, 128, 128] float32, updated in place.  Returns o [B, H, 128] fp32.
    """
    import torch
    lib = load_library()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(S, "S", torch.float32, dev)
    dt = _in_dtype(q)
    if q.dim() != 3:
        raise KDAError("q must be [B, H, 128]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:-1] != q.shape[:-1] \
            or beta.shape != q.shape[:-1] or tuple(S.shape) != (B, H, dk, dv):
        raise KDAError("q/k/v/log_alpha/beta/S shapes disagree")
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(o, "o", torch.float32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(log_alpha), _ptr(beta),
                             _ptr(S), B, H, dk, dv, _ptr(o), ctypes.c_void_p(stream))
    _status(rc, "kda_decode_step")
    return o


def recurrent_fwd(q, k, v, log_alpha, beta, S, *, replay=None, n_replay=None, commit=True,
                  o=None):
    """Multi-token recurrent decode (see kda_recurrent_fwd in include/kda.h).

    q, k, log_alpha [B, T, H, 128]; v [B, T, H, 128]; beta [B, T, H] (T <= 64);
    S [B, H, 128, 128] float32, updated in place.  `replay` = (q, k, v,
    log_alpha, beta) of Tr <= 64 tokens per request applied first without
    outputs, `n_replay` int32 [B] (device) how many of them to apply (None:
    all).  commit=False stores the state right after the replay.  Returns
    o [B, T, H, 128] float32.
    """
    import torch
    lib = load_library()
    dev = S.device
    _check(S, "S", torch.float32, dev)
    if S.dim() != 4:
        raise KDAError("S must be [B, H, 128, 128]")
    B, H, dk, dv = S.shape

    def tokens(group, label):
        tq, tk, tv, tla, tb = group
        for name, t in (("q", tq), ("k", tk), ("v", tv)):
            _check(t, f"{label} {name}", tq.dtype, dev)
        _check(tla, f"{label} log_alpha", torch.float32, dev)
        _check(tb, f"{label} beta", torch.float32, dev)
        if tq.dim() != 4 or tq.shape[0] != B or tq.shape[2] != H or tq.shape[3] != dk:
            raise KDAError(f"{label} q must be [B, T, H, 128] matching S")
        if tk.shape != tq.shape or tla.shape != tq.shape or tv.shape[:-1] != tq.shape[:-1] \
                or tb.shape != tq.shape[:-1]:
            raise KDAError(f"{label} q/k/v/log_alpha/beta shapes disagree")
        return tq.shape[1]

    T = tokens((q, k, v, log_alpha, beta), "new")
    dt = _in_dtype(q)
    Tr, rq, rk, rv, rla, rb = 0, None, None, None, None, None
    if replay is not None:
        rq, rk, rv, rla, rb = replay
        Tr = tokens(replay, "replay")
        if rq.dtype != q.dtype:
            raise KDAError("replay and new tokens must share a dtype")
    if n_replay is not None:
        _check(n_replay, "n_replay", torch.int32, dev)
        if n_replay.numel() != B:
            raise KDAError("n_replay must have one entry per request")
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(o, "o", torch.float32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(log_alpha), _ptr(beta),
                               _ptr(rq), _ptr(rk), _ptr(rv), _ptr(rla), _ptr(rb),
                               _ptr(n_replay), _ptr(S), B, T, Tr, H, dk, dv, int(bool(commit)),
                               _ptr(o), ctypes.c_void_p(stream))
    _status(rc, "kda_recurrent_fwd")
    return o


def prologue(q_raw, k_raw, v_raw, conv_w, a, b, conv_cache=None, cu_seqlens=None):
    """Layer prologue (see kda_prologue in include/kda.h): short convolution
    (width 4, with the optional conv cache updated in place), SiLU, L2 norm of
    q and k, log_alpha = -5 sigmoid(a), beta = sigmoid(b).

    q_raw, k_raw, v_raw [B, T, H, 128] (or packed [T, H, 128] with
    cu_seqlens); conv_w [3, H, 128, 4]; a like q_raw (float32); b [..., H];
    conv_cache [N, 3, 3, H, 128] float32 or None.
    Returns (q, k, v in q_raw's dtype, log_alpha float32, beta float32).
    """
    import torch
    lib = load_library()
    dev = q_raw.device
    for name, t in (("q_raw", q_raw), ("k_raw", k_raw), ("v_raw", v_raw)):
        _check(t, name, q_raw.dtype, dev)
    for name, t in (("conv_w", conv_w), ("a", a), ("b", b)):
        _check(t, name, torch.float32, dev)
    dt = _in_dtype(q_raw)
    H, dk = q_raw.shape[-2], q_raw.shape[-1]
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seqs, T = cu_seqlens.numel() - 1, q_raw.numel() // (H * dk)
    else:
        if q_raw.dim() != 4:
            raise KDAError("q_raw must be [B, T, H, 128] without cu_seqlens")
        n_seqs, T = q_raw.shape[0], q_raw.shape[1]
    if k_raw.shape != q_raw.shape or v_raw.shape != q_raw.shape or a.shape != q_raw.shape \
            or b.shape != q_raw.shape[:-1] or tuple(conv_w.shape) != (3, H, dk, 4):
        raise KDAError("prologue input shapes disagree")
    if conv_cache is not None:
        _check(conv_cache, "conv_cache", torch.float32, dev)
        if tuple(conv_cache.shape) != (n_seqs, 3, 3, H, dk):
            raise KDAError(f"conv_cache must be {(n_seqs, 3, 3, H, dk)}")
    q, k, v = (torch.empty_like(q_raw) for _ in range(3))
    log_alpha = torch.empty(q_raw.shape, dtype=torch.float32, device=dev)
    beta = torch.empty(b.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v_raw), dt, _ptr(conv_w),
                          _ptr(conv_cache), _ptr(a), _ptr(b), _ptr(cu_seqlens), n_seqs, T, H,
                          dk, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                          ctypes.c_void_p(stream))
    _status(rc, "kda_prologue")
    return q, k, v, log_alpha, beta


def epilogue(o, g, w, *, out=None):
    """Layer epilogue (see kda_epilogue in include/kda.h): RMSNorm of each
    head's 128 channels with weight w [128], times sigmoid(g).  o, g float32
    [..., H, 128]; out may be o (in place)."""
    import torch
    lib = load_library()
    dev = o.device
    for name, t in (("o", o), ("g", g), ("w", w)):
        _check(t, name, torch.float32, dev)
    H, dv = o.shape[-2], o.shape[-1]
    if g.shape != o.shape or tuple(w.shape) != (dv,):
        raise KDAError("epilogue shapes disagree")
    if out is None:
        out = torch.empty_like(o)
    else:
        _check(out, "out", torch.float32, dev)
    rows = o.numel() // (H * dv)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_epilogue(_ptr(o), _ptr(g), _ptr(w), rows, H, dv, _ptr(out),
                          ctypes.c_void_p(stream))
    _status(rc, "kda_epilogue")
    return out
