"""fp64 CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never does.
The arithmetic lives in ``oracle.c`` (plain C, fp64, the materialised definition);
this file compiles it with gcc and marshals numpy arrays through ctypes.

Functions:
  fwd(q, k, v, scale, causal)            -> (o, lse)   all rows
  fwd_rows(q, k, v, scale, causal, rows) -> (o, lse)   selected flat rows b*H*N+h*N+i
  bwd(q, k, v, dout, scale, causal)      -> (dq, dk, dv)
  bwd_heads(q, k, v, dout, scale, causal, heads) -> (dq, dk, dv) for heads b*H+h
  fwd_padded(q, k, v, scale, causal, lq, lk, dropout)        -> (o, lse)
  bwd_padded(q, k, v, dout, scale, causal, lq, lk, dropout)  -> (dq, dk, dv)
      q, dout [B, H, Nq, d]; k, v [B, H, Nk, d]; lq, lk per-batch valid lengths
      (None = all valid); causal is aligned to the last query and key;
      dropout = (p8, seed, offset) or None (drop probability p8 / 256, 64-bit
      seed, 32-bit offset; see oracle.c).
  philox4x32_10(counter[4], key[2]) -> 4 words;  dropout_mask(B, H, Nq, Nk, p8, seed, offset)
Inputs are float64 arrays [B, H, N, d] (exactly widened 16-bit values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
        lib.oracle_fwd_rows.argtypes = [dp, dp, dp, L, L, L, L, D, I, lp, L, dp, dp, I]
        lib.oracle_fwd_rows.restype = I
        lib.oracle_fwd.argtypes = [dp, dp, dp, L, L, L, L, D, I, dp, dp, I]
        lib.oracle_fwd.restype = I
        lib.oracle_bwd_heads.argtypes = [dp, dp, dp, dp, L, L, L, L, D, I, lp, L, dp, dp, dp, I]
        lib.oracle_bwd_heads.restype = I
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, L, L, L, L, D, I, dp, dp, dp, I]
        lib.oracle_bwd.restype = I
        U = ctypes.c_uint32
        up = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_fwd_padded.argtypes = [dp, dp, dp, L, L, L, L, L, lp, lp, D, I, ctypes.c_uint, U, U, U,
                                          dp, dp]
        lib.oracle_fwd_padded.restype = I
        lib.oracle_bwd_padded.argtypes = [dp, dp, dp, dp, L, L, L, L, L, lp, lp, D, I, ctypes.c_uint, U, U,
                                          U, dp, dp, dp, I]
        lib.oracle_bwd_padded.restype = I
        lib.oracle_philox4x32_10.argtypes = [up, up, up]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_dropout_mask.argtypes = [L, L, L, ctypes.c_uint, U, U, U,
                                            ctypes.POINTER(ctypes.c_ubyte)]
        lib.oracle_dropout_mask.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _as4(x) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError("expected [B, H, N, d]")
    return a


def fwd_rows(q, k, v, scale: float, causal: bool, rows, threads: int | None = None):
    q, k, v = _as4(q), _as4(k), _as4(v)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty(rows.size, np.float64)
    rc = _load().oracle_fwd_rows(_p(q), _p(k), _p(v), B, H, N, d, float(scale), int(bool(causal)),
                                 rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), rows.size,
                                 _p(o), _p(lse), threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_fwd_rows failed ({rc})")
    return o, lse


def fwd(q, k, v, scale: float, causal: bool, threads: int | None = None):
    q, k, v = _as4(q), _as4(k), _as4(v)
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), np.float64)
    rc = _load().oracle_fwd(_p(q), _p(k), _p(v), B, H, N, d, float(scale), int(bool(causal)),
                            _p(o), _p(lse), threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_fwd failed ({rc})")
    return o, lse


def bwd_heads(q, k, v, dout, scale: float, causal: bool, heads, threads: int | None = None):
    q, k, v, dout = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, H, N, d = q.shape
    heads = np.ascontiguousarray(heads, dtype=np.int64).ravel()
    dq = np.empty((heads.size, N, d), np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = _load().oracle_bwd_heads(_p(q), _p(k), _p(v), _p(dout), B, H, N, d, float(scale),
                                  int(bool(causal)), heads.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                  heads.size, _p(dq), _p(dk), _p(dv), threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_bwd_heads failed ({rc})")
    return dq, dk, dv


def bwd(q, k, v, dout, scale: float, causal: bool, threads: int | None = None):
    q, k, v, dout = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    rc = _load().oracle_bwd(_p(q), _p(k), _p(v), _p(dout), B, H, N, d, float(scale), int(bool(causal)),
                            _p(dq), _p(dk), _p(dv), threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_bwd failed ({rc})")
    return dq, dk, dv


def _lens(x, B):
    if x is None:
        return None, None
    a = np.ascontiguousarray(x, dtype=np.int64).ravel()
    if a.size != B:
        raise ValueError("one length per batch entry")
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_long))


def _dropout(dropout):
    """(p8, seed_lo, seed_hi, offset) from (p8, seed, offset) or None."""
    if dropout is None:
        return 0, 0, 0, 0
    p8, seed, offset = dropout
    if not 0 <= int(p8) <= 255:
        raise ValueError("p8 must be in [0, 255]")
    seed = int(seed) & ((1 << 64) - 1)
    return int(p8), seed & 0xFFFFFFFF, seed >> 32, int(offset) & 0xFFFFFFFF


def philox4x32_10(counter, key):
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    out = (ctypes.c_uint32 * 4)()
    _load().oracle_philox4x32_10(c, k, out)
    return [int(x) for x in out]


def dropout_mask(B, H, Nq, Nk, p8, seed, offset):
    """bool [B, H, Nq, Nk]: pairs kept by dropout (see oracle.c)."""
    p8, slo, shi, off = _dropout((p8, seed, offset))
    keep = np.zeros((B, H, Nq, Nk), np.uint8)
    rc = _load().oracle_dropout_mask(B * H, Nq, Nk, p8, slo, shi, off,
                                     keep.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)))
    if rc:
        raise RuntimeError(f"oracle_dropout_mask failed ({rc})")
    return keep.astype(bool)


def fwd_padded(q, k, v, scale: float, causal: bool, lq=None, lk=None, dropout=None):
    q, k, v = _as4(q), _as4(k), _as4(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape:
        raise ValueError("k, v must be [B, H, Nk, d]")
    lqa, lqp = _lens(lq, B)
    lka, lkp = _lens(lk, B)
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), np.float64)
    rc = _load().oracle_fwd_padded(_p(q), _p(k), _p(v), B, H, Nq, Nk, d, lqp, lkp, float(scale),
                                   int(bool(causal)), *_dropout(dropout), _p(o), _p(lse))
    if rc:
        raise RuntimeError(f"oracle_fwd_padded failed ({rc})")
    return o, lse


def bwd_padded(q, k, v, dout, scale: float, causal: bool, lq=None, lk=None, dropout=None,
               threads: int | None = None):
    q, k, v, dout = _as4(q), _as4(k), _as4(v), _as4(dout)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("k, v must be [B, H, Nk, d] and dout like q")
    lqa, lqp = _lens(lq, B)
    lka, lkp = _lens(lk, B)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(k)
    rc = _load().oracle_bwd_padded(_p(q), _p(k), _p(v), _p(dout), B, H, Nq, Nk, d, lqp, lkp,
                                   float(scale), int(bool(causal)), *_dropout(dropout), _p(dq),
                                   _p(dk), _p(dv), threads or default_threads())
    if rc:
        raise RuntimeError(f"oracle_bwd_padded failed ({rc})")
    return dq, dk, dv
