"""ctypes front-end of the fp64 CPU oracle (test infrastructure only; see ``la_oracle.c``)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

NONE, HEAD, GATE = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
# LA_ORACLE_SANITIZE=1 selects the build with AddressSanitizer and UndefinedBehaviorSanitizer
# (libla_oracle_san.so; the process must preload gcc's libasan: LD_PRELOAD=$(gcc
# -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0).
SANITIZE = os.environ.get("LA_ORACLE_SANITIZE", "") not in ("", "0")
_LIB = os.path.join(_HERE, "libla_oracle_san.so" if SANITIZE else "libla_oracle.so")
_FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]
_SAN_FLAGS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile la_oracle.c with gcc (no fast-math, no FMA contraction) into libla_oracle.so (with
    LA_ORACLE_SANITIZE=1: libla_oracle_san.so, built with the sanitizers as well)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_FLAGS, *(_SAN_FLAGS if SANITIZE else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.orc_recurrence.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, i32, P, f64, P, P, P, i32]
        lib.orc_cumdecay.argtypes = [i64, i64, i64, i32, i32, i32, P, f64, P, P]
        lib.orc_state_scan.argtypes = [i64, i64, i32, i32, i32, P, P, P]
        lib.orc_state_correct.argtypes = [i64, i64, i64, i32, i32, i32, i32, P, P, P, P]
        lib.orc_recurrence_bwd.argtypes = [i64, i64, i64, i32, i32, i32, P, P, P, i32, P, f64, P, P, P,
                                           P, P, P, P, P, i32]
        for f in (lib.orc_recurrence, lib.orc_cumdecay, lib.orc_state_scan, lib.orc_state_correct,
                  lib.orc_recurrence_bwd):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(q, k, v, mode=NONE, decay=None, s_in=None, nseg=1, gate_norm=16.0, threads=None):
    """Token-by-token recurrence in fp64.

    q, k: [B,H,L,dk]; v: [B,H,L,dv] (any float dtype whose values fit float32 exactly);
    decay: None / [H] log-decay / [B,H,L,dk] gate; s_in: [B,H,dk,dv] or None.
    Returns (o [B,H,L,dv] float64, s_out [B,H,nseg,dk,dv] float64).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L)
    dec = None if mode == NONE else _f32(decay)
    if mode == HEAD:
        assert dec.shape == (H,)
    if mode == GATE:
        assert dec.shape == (B, H, L, dk)
    si = None if s_in is None else _f64(s_in)
    if si is not None:
        assert si.shape == (B, H, dk, dv)
    o = np.zeros((B, H, L, dv), np.float64)
    s_out = np.zeros((B, H, nseg, dk, dv), np.float64)
    rc = _load().orc_recurrence(B, H, L, dk, dv, nseg, _ptr(q), _ptr(k), _ptr(v), mode, _ptr(dec),
                                float(gate_norm), _ptr(si), _ptr(o), _ptr(s_out),
                                threads or default_threads())
    if rc != 0:
        raise ValueError("orc_recurrence rejected its arguments")
    return o, s_out


def recurrence_bwd(q, k, v, d_o, mode=NONE, decay=None, s_in=None, ds_out=None, nseg=1, gate_norm=16.0,
                   threads=None):
    """Derivatives of the recurrence, token by token in fp64 (``orc_recurrence_bwd``).

    d_o: [B,H,L,dv] derivative of the loss with respect to o; ds_out: [B,H,nseg,dk,dv] or None
    (zero) with respect to each segment's final state.  Returns (dq, dk, dv, ddecay, ds_in):
    dq, dk [B,H,L,dk], dv [B,H,L,dv], ddecay None (NONE) / [H] with respect to lambda_h (HEAD) /
    [B,H,L,dk] with respect to the raw gate g (GATE), ds_in [B,H,nseg,dk,dv] with respect to each
    segment's initial state.
    """
    q, k, v, d_o = _f32(q), _f32(k), _f32(v), _f32(d_o)
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:3] == (B, H, L) and d_o.shape == v.shape
    dec = None if mode == NONE else _f32(decay)
    if mode == HEAD:
        assert dec.shape == (H,)
    if mode == GATE:
        assert dec.shape == (B, H, L, dk)
    si = None if s_in is None else _f64(s_in)
    if si is not None:
        assert si.shape == (B, H, dk, dv)
    so = None if ds_out is None else _f64(ds_out)
    if so is not None:
        assert so.shape == (B, H, nseg, dk, dv)
    dq = np.zeros((B, H, L, dk))
    dkk = np.zeros((B, H, L, dk))
    dvv = np.zeros((B, H, L, dv))
    dd = None if mode == NONE else np.zeros((H,) if mode == HEAD else (B, H, L, dk))
    ds_in = np.zeros((B, H, nseg, dk, dv))
    rc = _load().orc_recurrence_bwd(B, H, L, dk, dv, nseg, _ptr(q), _ptr(k), _ptr(v), mode, _ptr(dec),
                                    float(gate_norm), _ptr(si), _ptr(d_o), _ptr(so), _ptr(dq), _ptr(dkk),
                                    _ptr(dvv), _ptr(dd), _ptr(ds_in), threads or default_threads())
    if rc != 0:
        raise ValueError("orc_recurrence_bwd failed (%d)" % rc)
    return dq, dkk, dvv, dd, ds_in


def cumdecay(B, H, L, dk, mode=NONE, decay=None, nseg=1, gate_norm=16.0):
    """Inclusive per-segment cumulative decay [B,H,L,dk] and segment totals [B,H,nseg,dk] (fp64)."""
    dec = None if mode == NONE else _f32(decay)
    cum = np.zeros((B, H, L, dk), np.float64)
    tot = np.zeros((B, H, nseg, dk), np.float64)
    rc = _load().orc_cumdecay(B, H, L, dk, nseg, mode, _ptr(dec), float(gate_norm), _ptr(cum), _ptr(tot))
    if rc != 0:
        raise ValueError("orc_cumdecay rejected its arguments")
    return cum, tot


def state_scan(seg_states, seg_decay):
    """Inclusive scan out[p] = diag(seg_decay[p]) out[p-1] + seg_states[p] over axis 2 (fp64)."""
    x = _f64(seg_states)
    lam = _f64(seg_decay)
    B, H, P, dk, dv = x.shape
    assert lam.shape == (B, H, P, dk)
    out = np.zeros_like(x)
    rc = _load().orc_state_scan(B, H, P, dk, dv, _ptr(x), _ptr(lam), _ptr(out))
    if rc != 0:
        raise ValueError("orc_state_scan rejected its arguments")
    return out


def state_correct(q, cum, s_recv, o, nseg=1, seg_begin=0):
    """o[t] += (q_t * cum_t)^T s_recv[p - seg_begin] for tokens of segments p >= seg_begin.

    Returns the corrected copy of o (fp64)."""
    q = _f32(q)
    B, H, L, dk = q.shape
    c = _f64(cum)
    s = _f64(s_recv)
    out = _f64(o).copy()
    dv = out.shape[-1]
    assert c.shape == (B, H, L, dk) and s.shape == (B, H, nseg - seg_begin, dk, dv)
    rc = _load().orc_state_correct(B, H, L, dk, dv, nseg, seg_begin, _ptr(q), _ptr(c), _ptr(s), _ptr(out))
    if rc != 0:
        raise ValueError("orc_state_correct rejected its arguments")
    return out
