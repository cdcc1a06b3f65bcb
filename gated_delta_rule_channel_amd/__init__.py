"""KDA (Kimi Delta Attention) forward recurrence on AMD MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libkda.so`` (declared in
``include/kda.h``). This module only marshals arguments: tensors must already
live on the GPU, every step of the computation runs in the library's HIP
kernels, and there is no CPU fallback -- if the library is missing the calls
raise.

    o, ht = fwd_chunked(q, k, v, g, beta, scale=1.0, initial_state=None,
                        output_final_state=True, cu_seqlens=None)
    o = decode_step(q, k, v, g, beta, state, scale=1.0)     # state updated in place

Gated DeltaNet (one scalar gate per token and head, g [B,T,H] / [N,H]) has
the same calls under the names gdn_fwd_chunked and gdn_decode_step; Gated
DeltaNet-2 (erase gate b per key channel and write gate w per value channel in
place of beta) under gdn2_fwd_chunked(q, k, v, g, b, w, ...) and
gdn2_decode_step(q, k, v, g, b, w, state, ...).

Serving state: decode_multi(q, k, v, g, beta, pool, slots=None, snapshots=None)
runs T tokens per request against a slot-indexed state pool; state_copy(dst,
dst_slots, src, src_slots) copies whole states (fork, rollback).

Input preparation: prepare_inputs(q, k, a, b, scale) -> (q^, k^, g, beta) turns raw
projections into the inputs above (normalised q and k, g = log sigmoid(a),
beta = sigmoid(b)) in one pass; fwd_chunked_raw(q, k, v, a, b, scale, ...) does the same
inside the prefill (bf16, d = 128), so the prepared inputs never reach memory.

fwd_chunked_noalloc(...) is fwd_chunked on the library's built-in per-device scratch
array (no workspace argument, up to NOALLOC_SCRATCH_BYTES of workspace).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_SUCCESS = 0
KDA_ERROR_INVALID_VALUE = 1
KDA_ERROR_NOT_SUPPORTED = 2
KDA_ERROR_WORKSPACE = 3
KDA_ERROR_LAUNCH = 4
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

EXPORTED = ("kda_status_string", "kda_fwd_chunked_workspace_size", "kda_fwd_chunked",
            "kda_decode_step", "kda_gdn_fwd_chunked", "kda_gdn_decode_step",
            "kda_gdn2_fwd_chunked", "kda_gdn2_decode_step", "kda_decode_multi",
            "kda_state_copy", "kda_prepare_inputs", "kda_fwd_chunked_noalloc",
            "kda_fwd_chunked_raw")

NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024     # KDA_NOALLOC_SCRATCH_BYTES of kda.h


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


_lib_handle = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libkda.so (built in-tree by gated_delta_rule_channel_amd.build)."""
    global _lib_handle
    if _lib_handle is not None and path is None:
        return _lib_handle
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m gated_delta_rule_channel_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_fwd_chunked_workspace_size.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(sz)]
    lib.kda_fwd_chunked_workspace_size.restype = i
    for name in ("kda_fwd_chunked", "kda_gdn_fwd_chunked", "kda_fwd_chunked_raw"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, sz, vp]
        fn.restype = i
    lib.kda_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, vp, vp, i, i, i, i, i,
                                            i, i, i, vp]
    lib.kda_fwd_chunked_noalloc.restype = i
    for name in ("kda_decode_step", "kda_gdn_decode_step"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, vp, vp, f, vp, vp, i, i, i, i, i, i, vp]
        fn.restype = i
    lib.kda_gdn2_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, i, i, i, i, i,
                                         i, i, i, vp, sz, vp]
    lib.kda_gdn2_fwd_chunked.restype = i
    lib.kda_gdn2_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, f, vp, vp, i, i, i, i, i, i, vp]
    lib.kda_gdn2_decode_step.restype = i
    lib.kda_decode_multi.argtypes = [vp, vp, vp, vp, vp, f, vp, i, vp, vp, vp, i, i, i, i, i, i,
                                     i, vp]
    lib.kda_decode_multi.restype = i
    lib.kda_state_copy.argtypes = [vp, i, vp, vp, i, vp, i, i, i, i, vp]
    lib.kda_state_copy.restype = i
    lib.kda_prepare_inputs.argtypes = [vp, vp, vp, vp, f, vp, vp, vp, vp, ctypes.c_longlong, i, i,
                                       i, vp]
    lib.kda_prepare_inputs.restype = i
    if path is None:
        _lib_handle = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(B: int, T: int, H: int, Dk: int, Dv: int, num_seqs: int, varlen: bool,
                   dtype_code: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().kda_fwd_chunked_workspace_size(B, T, H, Dk, Dv, num_seqs, int(varlen),
                                                       dtype_code, ctypes.byref(out))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_fwd_chunked_workspace_size")
    return int(out.value)


def _check_gpu(*ts):
    ts = [t for t in ts if t is not None]
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    if len({t.device for t in ts}) > 1:
        raise ValueError("all tensors must be on the same device")


def _check_shape(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_same_dtype(ref, **ts):
    for name, t in ts.items():
        if t.dtype != ref.dtype:
            raise TypeError(f"{name} is {t.dtype}, q is {ref.dtype}: q, k, v and beta (or b, w) "
                            "share one dtype")


def fwd_chunked(q, k, v, g, beta, scale: float = 1.0, initial_state=None,
                output_final_state: bool = True, cu_seqlens=None, workspace=None,
                out=None, final_state=None, out_dtype=None) -> Tuple["object", Optional["object"]]:
    """Chunked prefill. q, k, g: [B,T,H,Dk]; v: [B,T,H,Dv]; beta: [B,T,H];
    initial_state: [N,H,Dk,Dv] float32 or None; cu_seqlens: int32 [N+1] (B == 1) or None.
    out_dtype: torch.float32 (default) or torch.bfloat16.
    Returns (o [B,T,H,Dv], ht [N,H,Dk,Dv] float32 or None)."""
    return _fwd_chunked(False, q, k, v, g, beta, scale, initial_state, output_final_state,
                        cu_seqlens, workspace, out, final_state, out_dtype)


def gdn_fwd_chunked(q, k, v, g, beta, scale: float = 1.0, initial_state=None,
                    output_final_state: bool = True, cu_seqlens=None, workspace=None,
                    out=None, final_state=None, out_dtype=None):
    """Gated DeltaNet chunked prefill: as fwd_chunked with g [B,T,H] float32."""
    return _fwd_chunked(True, q, k, v, g, beta, scale, initial_state, output_final_state,
                        cu_seqlens, workspace, out, final_state, out_dtype)


def gdn2_fwd_chunked(q, k, v, g, b, w, scale: float = 1.0, initial_state=None,
                     output_final_state: bool = True, cu_seqlens=None, workspace=None,
                     out=None, final_state=None, out_dtype=None):
    """Gated DeltaNet-2 chunked prefill: as fwd_chunked with the erase gate b [B,T,H,Dk] and
    the write gate w [B,T,H,Dv] (dtype of q) in place of beta."""
    return _fwd_chunked(False, q, k, v, g, None, scale, initial_state, output_final_state,
                        cu_seqlens, workspace, out, final_state, out_dtype, gates=(b, w))


def _fwd_chunked(scalar_gate, q, k, v, g, beta, scale, initial_state, output_final_state,
                 cu_seqlens, workspace, out, final_state, out_dtype, gates=None):
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, g must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    if gates is None:
        _check_same_dtype(q, k=k, v=v, beta=beta)
        _check_shape("beta", beta, (B, T, H))
        extra = (beta,)
    else:
        eb, ew = gates
        _check_same_dtype(q, k=k, v=v, b=eb, w=ew)
        _check_shape("b", eb, (B, T, H, Dk))
        _check_shape("w", ew, (B, T, H, Dv))
        extra = (eb, ew)
    varlen = cu_seqlens is not None
    N = (cu_seqlens.numel() - 1) if varlen else B
    _check_shape("k", k, (B, T, H, Dk))
    _check_shape("g", g, (B, T, H) if scalar_gate else (B, T, H, Dk))
    _check_shape("v", v, (B, T, H, Dv))
    _check_shape("initial_state", initial_state, (N, H, Dk, Dv))
    _check_shape("out", out, (B, T, H, Dv))
    _check_shape("final_state", final_state, (N, H, Dk, Dv))
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")
    if initial_state is not None and initial_state.dtype != torch.float32:
        raise TypeError("initial_state must be float32")
    if final_state is not None and final_state.dtype != torch.float32:
        raise TypeError("final_state must be float32")
    if varlen and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise TypeError("cu_seqlens must be a 1-D int32 tensor")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    _check_gpu(q, k, v, g, *extra, initial_state, cu_seqlens, workspace, out, final_state)
    nbytes = workspace_size(B, T, H, Dk, Dv, N, varlen, code)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    ocode = _dtype_code(o)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty(
            (N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    name = ("kda_gdn2_fwd_chunked" if gates is not None else
            "kda_gdn_fwd_chunked" if scalar_gate else "kda_fwd_chunked")
    st = getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), *(_ptr(t) for t in extra), float(scale),
        _ptr(initial_state),
        _ptr(ht), _ptr(o), _ptr(cu_seqlens), int(N), int(B), int(T), int(H), int(Dk), int(Dv),
        code, ocode, _ptr(workspace), nbytes, _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, name)
    return o, ht


def fwd_chunked_raw(q, k, v, a, b, scale: float = 1.0, initial_state=None,
                    output_final_state: bool = True, cu_seqlens=None, workspace=None,
                    out=None, final_state=None, out_dtype=None):
    """Chunked prefill from the raw projections (kda_fwd_chunked_raw): q, k, a [B,T,H,128] and
    v [B,T,H,128] bfloat16, b [B,T,H] bfloat16; q and k are normalised (q scaled by `scale`),
    g = log sigmoid(a) and beta = sigmoid(b) inside the kernel. Other arguments and the
    returns as fwd_chunked."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, a must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    _check_same_dtype(q, k=k, v=v, beta=b)
    _check_same_dtype(q, a=a)
    _check_shape("b", b, (B, T, H))
    varlen = cu_seqlens is not None
    N = (cu_seqlens.numel() - 1) if varlen else B
    for name, t, shape in (("k", k, (B, T, H, Dk)), ("a", a, (B, T, H, Dk)),
                           ("v", v, (B, T, H, Dv)), ("initial_state", initial_state, (N, H, Dk, Dv)),
                           ("out", out, (B, T, H, Dv)), ("final_state", final_state, (N, H, Dk, Dv))):
        _check_shape(name, t, shape)
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if varlen and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise TypeError("cu_seqlens must be a 1-D int32 tensor")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    _check_gpu(q, k, v, a, b, initial_state, cu_seqlens, workspace, out, final_state)
    nbytes = workspace_size(B, T, H, Dk, Dv, N, varlen, code)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty(
            (N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    st = load_library().kda_fwd_chunked_raw(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), float(scale), _ptr(initial_state),
        _ptr(ht), _ptr(o), _ptr(cu_seqlens), int(N), int(B), int(T), int(H), int(Dk), int(Dv),
        code, _dtype_code(o), _ptr(workspace), nbytes, _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_fwd_chunked_raw")
    return o, ht


def fwd_chunked_noalloc(q, k, v, g, beta, scale: float = 1.0, initial_state=None,
                        output_final_state: bool = True, cu_seqlens=None, out=None,
                        final_state=None, out_dtype=None):
    """kda_fwd_chunked_noalloc: the chunked prefill on the library's built-in device scratch
    (no workspace). Arguments and returns as fwd_chunked; o and ht are allocated here only
    when not passed. Raises KDAError (KDA_ERROR_WORKSPACE) when the call needs more than
    NOALLOC_SCRATCH_BYTES of workspace."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, g must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    _check_same_dtype(q, k=k, v=v, beta=beta)
    _check_shape("beta", beta, (B, T, H))
    varlen = cu_seqlens is not None
    N = (cu_seqlens.numel() - 1) if varlen else B
    _check_shape("k", k, (B, T, H, Dk))
    _check_shape("g", g, (B, T, H, Dk))
    _check_shape("v", v, (B, T, H, Dv))
    _check_shape("initial_state", initial_state, (N, H, Dk, Dv))
    _check_shape("out", out, (B, T, H, Dv))
    _check_shape("final_state", final_state, (N, H, Dk, Dv))
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if varlen and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1):
        raise TypeError("cu_seqlens must be a 1-D int32 tensor")
    _check_gpu(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=out_dtype, device=q.device)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty(
            (N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    st = load_library().kda_fwd_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
        _ptr(ht), _ptr(o), _ptr(cu_seqlens), int(N), int(B), int(T), int(H), int(Dk), int(Dv),
        code, _dtype_code(o), _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_fwd_chunked_noalloc")
    return o, ht


def decode_step(q, k, v, g, beta, state, scale: float = 1.0, out=None, out_dtype=None):
    """One decode step. q, k, g: [N,H,Dk]; v: [N,H,Dv]; beta: [N,H];
    state: [N,H,Dk,Dv] float32, updated in place. Returns o [N,H,Dv] (float32 by default)."""
    return _decode_step(False, q, k, v, g, beta, state, scale, out, out_dtype)


def gdn_decode_step(q, k, v, g, beta, state, scale: float = 1.0, out=None, out_dtype=None):
    """One Gated DeltaNet decode step: as decode_step with g [N,H] float32."""
    return _decode_step(True, q, k, v, g, beta, state, scale, out, out_dtype)


def gdn2_decode_step(q, k, v, g, b, w, state, scale: float = 1.0, out=None, out_dtype=None):
    """One Gated DeltaNet-2 decode step: as decode_step with b [N,H,Dk] and w [N,H,Dv]."""
    return _decode_step(False, q, k, v, g, None, state, scale, out, out_dtype, gates=(b, w))


def _decode_step(scalar_gate, q, k, v, g, beta, state, scale, out, out_dtype, gates=None):
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, g must be [N,H,Dk] and v [N,H,Dv]")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    code = _dtype_code(q)
    if gates is None:
        _check_same_dtype(q, k=k, v=v, beta=beta)
        _check_shape("beta", beta, (N, H))
        extra = (beta,)
    else:
        eb, ew = gates
        _check_same_dtype(q, k=k, v=v, b=eb, w=ew)
        _check_shape("b", eb, (N, H, Dk))
        _check_shape("w", ew, (N, H, Dv))
        extra = (eb, ew)
    _check_shape("k", k, (N, H, Dk))
    _check_shape("g", g, (N, H) if scalar_gate else (N, H, Dk))
    _check_shape("v", v, (N, H, Dv))
    _check_shape("state", state, (N, H, Dk, Dv))
    _check_shape("out", out, (N, H, Dv))
    if g.dtype != torch.float32 or state.dtype != torch.float32:
        raise TypeError("g and state must be float32")
    _check_gpu(q, k, v, g, *extra, state, out)
    o = out if out is not None else torch.empty((N, H, Dv), dtype=out_dtype, device=q.device)
    name = ("kda_gdn2_decode_step" if gates is not None else
            "kda_gdn_decode_step" if scalar_gate else "kda_decode_step")
    st = getattr(load_library(), name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), *(_ptr(t) for t in extra), float(scale),
        _ptr(state), _ptr(o), int(N), int(H), int(Dk), int(Dv), code, _dtype_code(o),
        _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, name)
    return o


def decode_multi(q, k, v, g, beta, pool, slots=None, snapshots=None, scale: float = 1.0,
                 out=None, out_dtype=None):
    """T decode steps per request against a state pool.

    q, k, g: [N,T,H,Dk]; v: [N,T,H,Dv]; beta: [N,T,H]; pool: [P,H,Dk,Dv] float32, slot
    slots[n] (int32 [N] on the device; None = slot n) updated in place to the state after the
    T tokens; snapshots: [N,T,H,Dk,Dv] float32 or None, receives the state after every
    token. Returns o [N,T,H,Dv] (float32 by default)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if q.dim() != 4 or v.dim() != 4 or pool.dim() != 4:
        raise ValueError("q, k, g must be [N,T,H,Dk], v [N,T,H,Dv], pool [P,H,Dk,Dv]")
    N, T, H, Dk = q.shape
    Dv = v.shape[-1]
    P = pool.shape[0]
    code = _dtype_code(q)
    _check_same_dtype(q, k=k, v=v, beta=beta)
    _check_shape("k", k, (N, T, H, Dk))
    _check_shape("g", g, (N, T, H, Dk))
    _check_shape("v", v, (N, T, H, Dv))
    _check_shape("beta", beta, (N, T, H))
    _check_shape("pool", pool, (P, H, Dk, Dv))
    _check_shape("slots", slots, (N,))
    _check_shape("snapshots", snapshots, (N, T, H, Dk, Dv))
    _check_shape("out", out, (N, T, H, Dv))
    if g.dtype != torch.float32 or pool.dtype != torch.float32:
        raise TypeError("g and pool must be float32")
    if snapshots is not None and snapshots.dtype != torch.float32:
        raise TypeError("snapshots must be float32")
    if slots is not None and slots.dtype != torch.int32:
        raise TypeError("slots must be int32")
    if slots is None and P < N:
        raise ValueError("without slots the pool needs one state per request")
    _check_gpu(q, k, v, g, beta, pool, slots, snapshots, out)
    o = out if out is not None else torch.empty((N, T, H, Dv), dtype=out_dtype, device=q.device)
    st = load_library().kda_decode_multi(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(pool), int(P),
        _ptr(slots), _ptr(snapshots), _ptr(o), int(N), int(T), int(H), int(Dk), int(Dv), code,
        _dtype_code(o), _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_decode_multi")
    return o


def state_copy(dst, dst_slots, src, src_slots):
    """dst[dst_slots[i]] = src[src_slots[i]] for whole states. dst: [Pd,H,Dk,Dv] float32;
    src: [Ps,H,Dk,Dv] float32 (a snapshot array may be passed as [N*T,H,Dk,Dv]); slots:
    int32 [n] on the device."""
    import torch
    if dst.dim() != 4 or src.dim() != 4 or tuple(dst.shape[1:]) != tuple(src.shape[1:]):
        raise ValueError("dst and src must be [P,H,Dk,Dv] with the same H, Dk, Dv")
    if dst.dtype != torch.float32 or src.dtype != torch.float32:
        raise TypeError("states must be float32")
    if dst_slots.dtype != torch.int32 or src_slots.dtype != torch.int32:
        raise TypeError("slots must be int32")
    if dst_slots.dim() != 1 or tuple(src_slots.shape) != tuple(dst_slots.shape):
        raise ValueError("dst_slots and src_slots must be 1-D and of one length")
    _check_gpu(dst, src, dst_slots, src_slots)
    _, H, Dk, Dv = dst.shape
    st = load_library().kda_state_copy(
        _ptr(dst), int(dst.shape[0]), _ptr(dst_slots), _ptr(src), int(src.shape[0]),
        _ptr(src_slots), int(dst_slots.numel()), int(H), int(Dk), int(Dv), _stream(dst.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_state_copy")


def prepare_inputs(q, k, a, b, scale: float = 1.0, out=None):
    """q, k, a: [..., H, Dk] raw projections; b: [..., H]. Returns (scale q / |q|, k / |k|,
    g = log sigmoid(a) float32, beta = sigmoid(b)) with the leading dimensions of q; out may
    pass the four output tensors (q and k themselves for in-place normalisation)."""
    import torch
    if q.dim() < 2:
        raise ValueError("q must be [..., H, Dk]")
    H, Dk = q.shape[-2:]
    lead = tuple(q.shape[:-2])
    code = _dtype_code(q)
    _check_same_dtype(q, k=k, v=a, beta=b)
    _check_shape("k", k, q.shape)
    _check_shape("a", a, q.shape)
    _check_shape("b", b, lead + (H,))
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k),
               torch.empty(q.shape, dtype=torch.float32, device=q.device), torch.empty_like(b))
    qo, ko, go, bo = out
    _check_shape("q_out", qo, q.shape)
    _check_shape("k_out", ko, q.shape)
    _check_shape("g_out", go, q.shape)
    _check_shape("beta_out", bo, lead + (H,))
    if go.dtype != torch.float32 or qo.dtype != q.dtype or ko.dtype != q.dtype or bo.dtype != q.dtype:
        raise TypeError("g_out must be float32 and the other outputs of q's dtype")
    _check_gpu(q, k, a, b, qo, ko, go, bo)
    tokens = 1
    for d in lead:
        tokens *= int(d)
    st = load_library().kda_prepare_inputs(
        _ptr(q), _ptr(k), _ptr(a), _ptr(b), float(scale), _ptr(qo), _ptr(ko), _ptr(go), _ptr(bo),
        int(tokens), int(H), int(Dk), code, _stream(q.device))
    if st != KDA_SUCCESS:
        raise KDAError(st, "kda_prepare_inputs")
    return qo, ko, go, bo
