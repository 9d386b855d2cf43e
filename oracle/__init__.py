"""KDA oracle: plain fp64 CPU reference for the Kimi Delta Attention operator.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It is
independent of the HIP library: no shared code, headers, tables or helpers.

The recurrence (token by token, fp64, one (sequence, head) unit at a time) and
its reverse-mode derivative (the backward pass) are written in
``kda_oracle.c``; this module builds it with gcc, loads it with
ctypes and wraps it for numpy arrays.  ``reference.py`` holds small numpy
restatements of the special cases the pages name (DeltaNet, gated DeltaNet,
linear attention, the naive DPLR product, the unrolled product) that pin the
oracle, ``chunkwise.py`` holds the CPU chunkwise derivation, and ``layer.py``
the steps on either side of the recurrence in a layer (short convolution with
its cache, activations, norms, gates).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile kda_oracle.c with gcc (-O2, OpenMP) into libkda_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.kda_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, lp, i64, i64,
                                           i64, i64, i64, i64, lp, i64, dp, dp,
                                           ctypes.c_int]
        lib.kda_oracle_forward.restype = ctypes.c_int
        lib.kda_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64,
                                               i64, i64, dp, ctypes.c_int]
        lib.kda_oracle_decode_step.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, lp, i64, i64,
                                            i64, i64, dp, dp, lp, i64, dp, dp,
                                            dp, dp, dp, dp, ctypes.c_int]
        lib.kda_oracle_backward.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def forward(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
            cols=None, units=None, nthreads=0, want_state=True):
    """Run the fp64 recurrence.

    Shapes (token-major): q, k, log_alpha [T, H, dk] (or [B, T, H, dk] with
    equal-length rows, flattened to B*T tokens); v [.., H, dv]; beta [.., H].
    S0: [N, H, dk, dv] or None (zeros).  cu_seqlens: [N+1] or None (then the
    leading batch axis, if any, gives the sequences).
    cols: optional (c0, c1) value-column range to compute (others stay 0).
    units: optional list of (n, h) pairs to compute (others stay 0).
    Returns (o [same leading shape, H, dv] fp64, S_T [N, H, dk, dv] fp64).
    """
    q = np.asarray(q)
    lead = q.shape[:-2]
    H, dk = q.shape[-2], q.shape[-1]
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is None:
        if len(lead) == 2:
            B, T = lead
        else:
            B, T = 1, lead[0]
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    Ttot = int(cu[-1])
    qf = _f64(q).reshape(Ttot, H, dk)
    kf = _f64(k).reshape(Ttot, H, dk)
    vf = _f64(v).reshape(Ttot, H, dv)
    lf = _f64(log_alpha).reshape(Ttot, H, dk)
    bf = _f64(beta).reshape(Ttot, H)
    s0 = None if S0 is None else _f64(S0).reshape(N, H, dk, dv)
    o = np.zeros((Ttot, H, dv), dtype=np.float64)
    st = np.zeros((N, H, dk, dv), dtype=np.float64) if want_state else None
    c0, c1 = (0, dv) if cols is None else (int(cols[0]), int(cols[1]))
    if units is not None:
        ua = np.ascontiguousarray(np.asarray(units, dtype=np.int64).reshape(-1, 2))
        nu = ua.shape[0]
    else:
        ua, nu = None, 0
    rc = _load().kda_oracle_forward(
        _ptr(qf), _ptr(kf), _ptr(vf), _ptr(lf), _ptr(bf), _ptr(s0),
        _ptr(cu, ctypes.c_int64), N, H, dk, dv, c0, c1,
        _ptr(ua, ctypes.c_int64), nu, _ptr(o), _ptr(st), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with code {rc}")
    return o.reshape(lead + (H, dv)), st


def backward(q, k, v, log_alpha, beta, S0, dO, dS_T=None, cu_seqlens=None, *,
             units=None, nthreads=0):
    """Gradients of L = <dO, o> + <dS_T, S_T> through the fp64 recurrence
    (kda_oracle.c, kda_oracle_backward).  Shapes as forward(); dO like o,
    dS_T like S_T (None = zero).  units: optional (n, h) pairs (other rows of
    the outputs stay 0).  Returns (dq, dk, dv, dlog_alpha, dbeta, dS0) in fp64
    with the input shapes (dS0 [N, H, dk, dv])."""
    q = np.asarray(q)
    lead = q.shape[:-2]
    H, dk = q.shape[-2], q.shape[-1]
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is None:
        B, T = lead if len(lead) == 2 else (1, lead[0])
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    Ttot = int(cu[-1])
    qf, kf = _f64(q).reshape(Ttot, H, dk), _f64(k).reshape(Ttot, H, dk)
    vf, lf = _f64(v).reshape(Ttot, H, dv), _f64(log_alpha).reshape(Ttot, H, dk)
    bf = _f64(beta).reshape(Ttot, H)
    s0 = None if S0 is None else _f64(S0).reshape(N, H, dk, dv)
    dof = _f64(dO).reshape(Ttot, H, dv)
    dst = None if dS_T is None else _f64(dS_T).reshape(N, H, dk, dv)
    dq, dkk = np.zeros((Ttot, H, dk)), np.zeros((Ttot, H, dk))
    dvv, dla = np.zeros((Ttot, H, dv)), np.zeros((Ttot, H, dk))
    db, ds0 = np.zeros((Ttot, H)), np.zeros((N, H, dk, dv))
    if units is not None:
        ua = np.ascontiguousarray(np.asarray(units, dtype=np.int64).reshape(-1, 2))
        nu = ua.shape[0]
    else:
        ua, nu = None, 0
    rc = _load().kda_oracle_backward(
        _ptr(qf), _ptr(kf), _ptr(vf), _ptr(lf), _ptr(bf), _ptr(s0),
        _ptr(cu, ctypes.c_int64), N, H, dk, dv, _ptr(dof), _ptr(dst),
        _ptr(ua, ctypes.c_int64), nu, _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dla),
        _ptr(db), _ptr(ds0), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed with code {rc}")
    return (dq.reshape(lead + (H, dk)), dkk.reshape(lead + (H, dk)),
            dvv.reshape(lead + (H, dv)), dla.reshape(lead + (H, dk)),
            db.reshape(lead + (H,)), ds0)


def decode_step(q, k, v, log_alpha, beta, S, *, nthreads=0):
    """One decode step.  q,k,log_alpha [B,H,dk]; v [B,H,dv]; beta [B,H];
    S [B,H,dk,dv] (not modified).  Returns (o [B,H,dv], S_new) in fp64."""
    q = np.asarray(q)
    B, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    s = _f64(S).reshape(B, H, dk, dv).copy()
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_decode_step(
        _ptr(_f64(q)), _ptr(_f64(k)), _ptr(_f64(v)), _ptr(_f64(log_alpha)),
        _ptr(_f64(beta)), _ptr(s), B, H, dk, dv, _ptr(o), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_step failed with code {rc}")
    return o, s
