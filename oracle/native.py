"""ctypes front end of the C float64 oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use it. ``build()`` compiles the C file with gcc and OpenMP
into oracle/libkda_oracle.so.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle (gcc -O2, OpenMP, portable x86-64 code)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", _LIB + ".tmp", _SRC,
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.kda_oracle_prefill.argtypes = [fp, fp, fp, fp, ctypes.c_int, fp, ctypes.c_double, fp, ip,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           dp, dp]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [fp, fp, fp, fp, ctypes.c_int, fp, ctypes.c_double, dp, dp,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_decode.restype = ctypes.c_int
        lib.kda_oracle_gdn2_prefill.argtypes = [fp, fp, fp, fp, fp, fp, ctypes.c_double, fp, ip,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, dp, dp]
        lib.kda_oracle_gdn2_prefill.restype = ctypes.c_int
        lib.kda_oracle_gdn2_decode.argtypes = [fp, fp, fp, fp, fp, fp, ctypes.c_double, dp, dp,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int]
        lib.kda_oracle_gdn2_decode.restype = ctypes.c_int
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        lib.kda_oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.kda_oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().kda_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by the following calls (timing only)."""
    _load().kda_oracle_set_num_threads(int(n))


def _f32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", dtype=torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def _prefill(q, k, v, g, beta, scale, h0, cu_seqlens, scalar_gate):
    qf, kf, vf, gf, bf = (_f32(x) for x in (q, k, v, g, beta))
    B, T, H, Dk = qf.shape
    Dv = vf.shape[-1]
    if gf.shape != ((B, T, H) if scalar_gate else (B, T, H, Dk)):
        raise ValueError(f"g has shape {gf.shape}")
    if cu_seqlens is None:
        cu = (np.arange(B + 1, dtype=np.int64) * T).astype(np.int32)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    h0f = None if h0 is None else _f32(h0)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    ht = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    rc = _load().kda_oracle_prefill(
        _p(qf, ctypes.c_float), _p(kf, ctypes.c_float), _p(vf, ctypes.c_float),
        _p(gf, ctypes.c_float), int(scalar_gate), _p(bf, ctypes.c_float), float(scale),
        None if h0f is None else _p(h0f, ctypes.c_float), _p(cu, ctypes.c_int32), N, H, Dk, Dv,
        _p(o, ctypes.c_double), _p(ht, ctypes.c_double))
    if rc != 0:
        raise MemoryError("kda_oracle_prefill failed")
    return o, ht


def prefill(q, k, v, g, beta, scale: float = 1.0, h0=None,
            cu_seqlens: Optional[Sequence[int]] = None):
    """Recurrence over [B, T, H, D] inputs; returns float64 (o [B,T,H,Dv], ht [N,H,Dk,Dv])."""
    return _prefill(q, k, v, g, beta, scale, h0, cu_seqlens, False)


def gdn_prefill(q, k, v, g, beta, scale: float = 1.0, h0=None,
                cu_seqlens: Optional[Sequence[int]] = None):
    """Gated DeltaNet (scalar gate g [B, T, H]); returns float64 (o, ht) as prefill."""
    return _prefill(q, k, v, g, beta, scale, h0, cu_seqlens, True)


def _decode(q, k, v, g, beta, state, scale, scalar_gate):
    qf, kf, vf, gf, bf = (_f32(x) for x in (q, k, v, g, beta))
    N, H, Dk = qf.shape
    Dv = vf.shape[-1]
    if gf.shape != ((N, H) if scalar_gate else (N, H, Dk)):
        raise ValueError(f"g has shape {gf.shape}")
    try:
        import torch
        if isinstance(state, torch.Tensor):
            state = state.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    S = np.array(state, dtype=np.float64, order="C", copy=True)
    o = np.zeros((N, H, Dv), dtype=np.float64)
    rc = _load().kda_oracle_decode(
        _p(qf, ctypes.c_float), _p(kf, ctypes.c_float), _p(vf, ctypes.c_float),
        _p(gf, ctypes.c_float), int(scalar_gate), _p(bf, ctypes.c_float), float(scale),
        _p(S, ctypes.c_double), _p(o, ctypes.c_double), N, H, Dk, Dv)
    if rc != 0:
        raise MemoryError("kda_oracle_decode failed")
    return o, S


def decode(q, k, v, g, beta, state, scale: float = 1.0):
    """One step; returns float64 (o [N,H,Dv], new state [N,H,Dk,Dv])."""
    return _decode(q, k, v, g, beta, state, scale, False)


def gdn_decode(q, k, v, g, beta, state, scale: float = 1.0):
    """One Gated DeltaNet step (g [N, H]); returns float64 (o, new state)."""
    return _decode(q, k, v, g, beta, state, scale, True)


def gdn2_prefill(q, k, v, g, b, w, scale: float = 1.0, h0=None,
                 cu_seqlens: Optional[Sequence[int]] = None):
    """Gated DeltaNet-2 (erase gate b [B,T,H,Dk], write gate w [B,T,H,Dv]); returns float64
    (o, ht) as prefill."""
    qf, kf, vf, gf, bf, wf = (_f32(x) for x in (q, k, v, g, b, w))
    B, T, H, Dk = qf.shape
    Dv = vf.shape[-1]
    if gf.shape != qf.shape or bf.shape != qf.shape or wf.shape != vf.shape:
        raise ValueError("g and b must match q, w must match v")
    if cu_seqlens is None:
        cu = (np.arange(B + 1, dtype=np.int64) * T).astype(np.int32)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    h0f = None if h0 is None else _f32(h0)
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    ht = np.zeros((N, H, Dk, Dv), dtype=np.float64)
    fp = ctypes.c_float
    rc = _load().kda_oracle_gdn2_prefill(
        _p(qf, fp), _p(kf, fp), _p(vf, fp), _p(gf, fp), _p(bf, fp), _p(wf, fp), float(scale),
        None if h0f is None else _p(h0f, fp), _p(cu, ctypes.c_int32), N, H, Dk, Dv,
        _p(o, ctypes.c_double), _p(ht, ctypes.c_double))
    if rc != 0:
        raise MemoryError("kda_oracle_gdn2_prefill failed")
    return o, ht


def gdn2_decode(q, k, v, g, b, w, state, scale: float = 1.0):
    """One Gated DeltaNet-2 step (b [N,H,Dk], w [N,H,Dv]); returns float64 (o, new state)."""
    qf, kf, vf, gf, bf, wf = (_f32(x) for x in (q, k, v, g, b, w))
    N, H, Dk = qf.shape
    Dv = vf.shape[-1]
    if gf.shape != qf.shape or bf.shape != qf.shape or wf.shape != vf.shape:
        raise ValueError("g and b must match q, w must match v")
    try:
        import torch
        if isinstance(state, torch.Tensor):
            state = state.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    S = np.array(state, dtype=np.float64, order="C", copy=True)
    o = np.zeros((N, H, Dv), dtype=np.float64)
    fp = ctypes.c_float
    rc = _load().kda_oracle_gdn2_decode(
        _p(qf, fp), _p(kf, fp), _p(vf, fp), _p(gf, fp), _p(bf, fp), _p(wf, fp), float(scale),
        _p(S, ctypes.c_double), _p(o, ctypes.c_double), N, H, Dk, Dv)
    if rc != 0:
        raise MemoryError("kda_oracle_gdn2_decode failed")
    return o, S
