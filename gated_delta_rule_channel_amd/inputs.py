"""Seeded synthetic inputs for the KDA forward recurrence.

This module only draws random numbers and casts them; it holds none of the
recurrence's arithmetic, so both the fp64 oracle and the HIP path can take
their inputs from it.

Recipe (all draws in float64, then cast to the workload dtype with
round-to-nearest-even; consumers that need float64 upcast the cast values):

* every (workload, tensor, head) triple owns its own PCG64 stream, seeded
  with ``numpy.random.default_rng([workload_id, tensor_id, head])``, so any
  head can be regenerated alone (sampled-head parity checks) and heads can
  be drawn in parallel;
* q, k ~ N(0, 1) per element, each token row L2-normalised in float64;
  q is then multiplied by d_k^-1/2 (the query scale is carried by q, and the
  workloads pass scale = 1);
* v ~ N(0, 1); beta = sigmoid(N(0, 1)) per (token, head);
* log-decay g = log(alpha) = -softplus(N(0, 1)) per (token, head, channel);
  the large workloads multiply it by an independent U(0.5, 2) per element;
* the varlen workload picks, per head, 13 "fast" channels with
  g ~ -U(5, 10) and 13 disjoint "slow" channels with g ~ -U(0, 1e-4)
  (about 10 % of 128 each), per token;
* initial states are 0.1 * N(0, 1) where a workload asks for one;
* Gated DeltaNet inputs (scalar gate) reuse q, k, v, beta and states of the
  same workload and replace g by one log-decay per (token, head),
  -softplus(N(0, 1)) times U(0.5, 2) where the workload scales g, from a
  stream of its own;
* Gated DeltaNet-2 inputs reuse q, k, v, g and states of the workload and draw an
  erase gate b = sigmoid(N(0, 1)) per (token, head, key channel) and a write gate
  w = sigmoid(N(0, 1)) per (token, head, value channel), each from its own stream,
  cast to the workload dtype like beta.

Shapes follow the library: q, k, g are [B, T, H, Dk], v is [B, T, H, Dv],
beta is [B, T, H]; varlen packs sequences along T with B = 1 and int32
cu_seqlens; decode tensors are [N, H, D] with a state [N, H, Dk, Dv].
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np
import torch

# tensor ids of the per-head streams
_Q, _K, _V, _BETA, _G, _GFAC, _CHAN, _STATE, _LEN, _GSC, _EB, _EW = range(1, 13)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    H: int
    Dk: int
    Dv: int
    dtype: str               # "f32" or "bf16" (q, k, v, beta, o); g and states are f32
    B: int = 1
    T: int = 0
    N: int = 0               # decode batch / number of varlen sequences
    g_factor: bool = False   # multiply g by U(0.5, 2)
    stress_channels: bool = False
    h0: bool = False         # random initial state
    varlen: bool = False
    decode: bool = False
    lmin: int = 0
    lmax: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    0: Workload(0, "tiny-oracle B1 T64 H1 d16 f32", H=1, Dk=16, Dv=16, dtype="f32", B=1, T=64),
    1: Workload(1, "small-prefill B2 T1024 H4 d64 f32", H=4, Dk=64, Dv=64, dtype="f32", B=2, T=1024,
                h0=True),
    2: Workload(2, "main-prefill B1 T8192 H64 d128 bf16", H=64, Dk=128, Dv=128, dtype="bf16", B=1,
                T=8192, g_factor=True),
    3: Workload(3, "decode N256 H64 d128 bf16, f32 state", H=64, Dk=128, Dv=128, dtype="bf16", N=256,
                g_factor=True, h0=True, decode=True),
    4: Workload(4, "varlen-long N8 L~U[1024,32768] H64 d128 bf16", H=64, Dk=128, Dv=128,
                dtype="bf16", N=8, g_factor=True, stress_channels=True, varlen=True,
                lmin=1024, lmax=32768),
}


def _rng(wid: int, tensor: int, head: int) -> np.random.Generator:
    return np.random.default_rng([wid, tensor, head])


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _n_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def varlen_lengths(w: Workload) -> np.ndarray:
    """Sequence lengths of the varlen workload, L_i ~ U{lmin..lmax}."""
    rng = _rng(w.wid, _LEN, 0)
    return rng.integers(w.lmin, w.lmax, size=w.N, endpoint=True).astype(np.int64)


def cu_seqlens_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _head_draws(w: Workload, h: int, ntok: int):
    """float64 draws for one head: q, k [ntok, Dk], v [ntok, Dv], beta [ntok], g [ntok, Dk]."""
    q = _unit_rows(_rng(w.wid, _Q, h).standard_normal((ntok, w.Dk))) * (w.Dk ** -0.5)
    k = _unit_rows(_rng(w.wid, _K, h).standard_normal((ntok, w.Dk)))
    v = _rng(w.wid, _V, h).standard_normal((ntok, w.Dv))
    beta = _sigmoid(_rng(w.wid, _BETA, h).standard_normal(ntok))
    g = -_softplus(_rng(w.wid, _G, h).standard_normal((ntok, w.Dk)))
    if w.g_factor:
        g = g * _rng(w.wid, _GFAC, h).uniform(0.5, 2.0, size=(ntok, w.Dk))
    if w.stress_channels:
        rc = _rng(w.wid, _CHAN, h)
        nsel = int(round(0.1 * w.Dk))
        perm = rc.permutation(w.Dk)
        fast, slow = perm[:nsel], perm[nsel:2 * nsel]
        g[:, fast] = -rc.uniform(5.0, 10.0, size=(ntok, nsel))
        g[:, slow] = -rc.uniform(0.0, 1e-4, size=(ntok, nsel))
    return q, k, v, beta, g


def _cast(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


@dataclasses.dataclass
class PrefillInputs:
    q: torch.Tensor          # [B, T, H, Dk] workload dtype (CPU)
    k: torch.Tensor
    v: torch.Tensor          # [B, T, H, Dv]
    g: torch.Tensor          # [B, T, H, Dk] float32
    beta: torch.Tensor       # [B, T, H] workload dtype
    h0: Optional[torch.Tensor]  # [N, H, Dk, Dv] float32 or None
    cu_seqlens: Optional[torch.Tensor]  # int32 [N+1] or None
    heads: list              # global head ids held along dim 2
    scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return (self.cu_seqlens.numel() - 1) if self.cu_seqlens is not None else self.q.shape[0]


def prefill_inputs(w: Workload, heads: Optional[Sequence[int]] = None, T: Optional[int] = None,
                   lengths: Optional[Sequence[int]] = None) -> PrefillInputs:
    """Inputs of a prefill workload, optionally for a subset of heads only.

    ``T`` overrides the sequence length of a fixed-length workload and
    ``lengths`` the sequence lengths of the varlen one (shrunken cases);
    per-head streams are unchanged, so a shrunken case is a prefix of the
    full one's draws only when its token count is unchanged.
    """
    assert not w.decode
    heads = list(range(w.H)) if heads is None else list(heads)
    if w.varlen:
        lens = varlen_lengths(w) if lengths is None else np.asarray(lengths, dtype=np.int64)
        cu = cu_seqlens_from_lengths(lens)
        B, Tt = 1, int(cu[-1])
    else:
        cu = None
        B, Tt = w.B, (w.T if T is None else int(T))
    ntok = B * Tt
    Hs = len(heads)
    dt = w.torch_dtype
    q = torch.empty((ntok, Hs, w.Dk), dtype=dt)
    k = torch.empty((ntok, Hs, w.Dk), dtype=dt)
    v = torch.empty((ntok, Hs, w.Dv), dtype=dt)
    g = torch.empty((ntok, Hs, w.Dk), dtype=torch.float32)
    beta = torch.empty((ntok, Hs), dtype=dt)

    def fill(j_h):
        j, h = j_h
        qq, kk, vv, bb, gg = _head_draws(w, h, ntok)
        q[:, j] = _cast(qq, dt)
        k[:, j] = _cast(kk, dt)
        v[:, j] = _cast(vv, dt)
        beta[:, j] = _cast(bb, dt)
        g[:, j] = _cast(gg, torch.float32)

    with _cf.ThreadPoolExecutor(_n_threads()) as ex:
        list(ex.map(fill, list(enumerate(heads))))

    nseq = (len(cu) - 1) if cu is not None else B
    h0 = None
    if w.h0:
        h0 = torch.empty((nseq, Hs, w.Dk, w.Dv), dtype=torch.float32)
        for j, h in enumerate(heads):
            h0[:, j] = _cast(0.1 * _rng(w.wid, _STATE, h).standard_normal((nseq, w.Dk, w.Dv)),
                             torch.float32)
    return PrefillInputs(
        q=q.view(B, Tt, Hs, w.Dk), k=k.view(B, Tt, Hs, w.Dk), v=v.view(B, Tt, Hs, w.Dv),
        g=g.view(B, Tt, Hs, w.Dk), beta=beta.view(B, Tt, Hs), h0=h0,
        cu_seqlens=None if cu is None else torch.from_numpy(cu), heads=heads)


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor      # [N, H, Dk]
    k: torch.Tensor
    v: torch.Tensor      # [N, H, Dv]
    g: torch.Tensor      # [N, H, Dk] float32
    beta: torch.Tensor   # [N, H]
    state: torch.Tensor  # [N, H, Dk, Dv] float32
    heads: list
    scale: float = 1.0


def decode_inputs(w: Workload, heads: Optional[Sequence[int]] = None,
                  N: Optional[int] = None, with_state: bool = True) -> DecodeInputs:
    """Inputs of the decode workload: one token per request against a random state
    (state None when with_state is false; the token draws are the same either way)."""
    assert w.decode
    heads = list(range(w.H)) if heads is None else list(heads)
    n = w.N if N is None else int(N)
    Hs = len(heads)
    dt = w.torch_dtype
    q = torch.empty((n, Hs, w.Dk), dtype=dt)
    k = torch.empty((n, Hs, w.Dk), dtype=dt)
    v = torch.empty((n, Hs, w.Dv), dtype=dt)
    g = torch.empty((n, Hs, w.Dk), dtype=torch.float32)
    beta = torch.empty((n, Hs), dtype=dt)
    state = torch.empty((n, Hs, w.Dk, w.Dv), dtype=torch.float32) if with_state else None

    def fill(j_h):
        j, h = j_h
        qq, kk, vv, bb, gg = _head_draws(w, h, n)
        q[:, j] = _cast(qq, dt)
        k[:, j] = _cast(kk, dt)
        v[:, j] = _cast(vv, dt)
        beta[:, j] = _cast(bb, dt)
        g[:, j] = _cast(gg, torch.float32)
        if with_state:
            state[:, j] = _cast(0.1 * _rng(w.wid, _STATE, h).standard_normal((n, w.Dk, w.Dv)),
                                torch.float32)

    with _cf.ThreadPoolExecutor(_n_threads()) as ex:
        list(ex.map(fill, list(enumerate(heads))))
    return DecodeInputs(q=q, k=k, v=v, g=g, beta=beta, state=state, heads=heads)


def scalar_gate(w: Workload, heads: Sequence[int], ntok: int) -> torch.Tensor:
    """Gated DeltaNet log-decay, one value per (token, head): float32 [ntok, len(heads)]."""
    out = torch.empty((ntok, len(heads)), dtype=torch.float32)
    for j, h in enumerate(heads):
        rng = _rng(w.wid, _GSC, h)
        gg = -_softplus(rng.standard_normal(ntok))
        if w.g_factor:
            gg = gg * rng.uniform(0.5, 2.0, size=ntok)
        out[:, j] = _cast(gg, torch.float32)
    return out


def gdn_prefill_inputs(w: Workload, heads: Optional[Sequence[int]] = None,
                       T: Optional[int] = None,
                       lengths: Optional[Sequence[int]] = None) -> PrefillInputs:
    """prefill_inputs with g replaced by a scalar gate g [B, T, H] (Gated DeltaNet)."""
    x = prefill_inputs(w, heads=heads, T=T, lengths=lengths)
    B, Tt, Hs = x.beta.shape
    x.g = scalar_gate(w, x.heads, B * Tt).view(B, Tt, Hs)
    return x


def gdn_decode_inputs(w: Workload, heads: Optional[Sequence[int]] = None,
                      N: Optional[int] = None) -> DecodeInputs:
    """decode_inputs with g replaced by a scalar gate g [N, H] (Gated DeltaNet)."""
    x = decode_inputs(w, heads=heads, N=N)
    x.g = scalar_gate(w, x.heads, x.beta.shape[0])
    return x


def erase_write_gates(w: Workload, heads: Sequence[int], ntok: int):
    """Gated DeltaNet-2 gates: b [ntok, len(heads), Dk] and w [ntok, len(heads), Dv] in the
    workload dtype, sigmoid(N(0, 1)) per element."""
    dt = w.torch_dtype
    b = torch.empty((ntok, len(heads), w.Dk), dtype=dt)
    wr = torch.empty((ntok, len(heads), w.Dv), dtype=dt)
    for j, h in enumerate(heads):
        b[:, j] = _cast(_sigmoid(_rng(w.wid, _EB, h).standard_normal((ntok, w.Dk))), dt)
        wr[:, j] = _cast(_sigmoid(_rng(w.wid, _EW, h).standard_normal((ntok, w.Dv))), dt)
    return b, wr


def gdn2_prefill_inputs(w: Workload, heads: Optional[Sequence[int]] = None,
                        T: Optional[int] = None, lengths: Optional[Sequence[int]] = None):
    """prefill_inputs plus the Gated DeltaNet-2 gates; returns (inputs, b [B,T,H,Dk],
    w [B,T,H,Dv]). inputs.beta is left in place and unused by Gated DeltaNet-2."""
    x = prefill_inputs(w, heads=heads, T=T, lengths=lengths)
    B, Tt, Hs = x.beta.shape
    b, wr = erase_write_gates(w, x.heads, B * Tt)
    return x, b.view(B, Tt, Hs, w.Dk), wr.view(B, Tt, Hs, w.Dv)


def gdn2_decode_inputs(w: Workload, heads: Optional[Sequence[int]] = None,
                       N: Optional[int] = None):
    """decode_inputs plus the Gated DeltaNet-2 gates b [N,H,Dk] and w [N,H,Dv]."""
    x = decode_inputs(w, heads=heads, N=N)
    b, wr = erase_write_gates(w, x.heads, x.beta.shape[0])
    return x, b, wr
