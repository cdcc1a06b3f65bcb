"""Float64 CPU oracle of the KDA forward recurrence (numpy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``; the library itself never does.

What it computes is the recurrence itself, token by token, in float64 with
no blocking, chunking or reordering. The state S of one head is d_k x d_v
with one row per key channel (the [..., d_k, d_v] layout used by the
reference PyTorch code quoted on "Kimi Delta Attention (KDA)", brain.bigb.es,
section "KDA: one gate per key channel"). One step at token t, in the order
given as five named operations on "Module 03 - KDA I: The Delta-Rule
Recurrence" (jared-hpc.com), section 2:

  (1) forget   S~ = Diag(exp(g_t)) S          per key channel (rows of S)
  (2) predict  v^ = S~^T k_t
  (3) correct  e  = beta_t (v_t - v^)         beta inside the error, as on the
                                              brain.bigb.es page; the same S_t
                                              as applying beta at the write
  (4) write    S  = S~ + k_t e^T
  (5) read     o_t = S^T (scale * q_t)        read after the write

Implementations keep g_t = log(alpha_t) <= 0 and decay by exp(g_t)
(brain.bigb.es, "KDA: one gate per key channel").

Gated DeltaNet (gdn_forward, gdn_decode) is the same recurrence with one
scalar retention gate alpha_t = exp(g_t) per token and head instead of one
per key channel: decay the whole state, then apply the delta rule to the
decayed state ("Notes on Linear Attention", zhilingong.com, section 6;
"From Fast Weight Programmers to KDA", section "Gated Delta Networks").

Gated DeltaNet-2 (gdn2_forward, gdn2_decode) keeps KDA's per-channel decay and
replaces beta by a per-key-channel erase gate b_t and a per-value-channel write
gate w_t: decay, retrieve the old value through the gated key b_t * k_t, then
write the residual w_t * v_t - v^ at the original key ("From Fast Weight
Programmers to KDA", section "Gated DeltaNet-2", written there for the
transposed state).

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(worked example, read-back, locality, orthogonal-key example, additive
brute force, DeltaNet and Gated DeltaNet reductions, operator order,
stability, chunked mirror, resume/varlen/decode consistency; for the scalar
gate: the matrix form alpha (I - beta k k^T) S + beta k v^T, the pure-decay
closed form at beta = 0, and the per-channel recurrence with an equal gate; for
the erase/write gates: the matrix form, the collapse to KDA at b = beta 1,
w = beta 1, and the additive closed form at b = 0).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def kda_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
             beta: float, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray, dict]:
    """One KDA step for one head. S is [Dk, Dv]; returns (S_t, o_t, intermediates).

    Five steps of "Module 03 - KDA I" (jared-hpc.com) section 2, with the
    beta-scaled error of brain.bigb.es "Kimi Delta Attention (KDA)".
    """
    S_tilde = np.exp(g)[:, None] * S            # (1) forget, per key channel
    v_hat = S_tilde.T @ k                       # (2) predict
    e = beta * (v - v_hat)                      # (3) correct
    S_new = S_tilde + np.outer(k, e)            # (4) rank-one write
    o = S_new.T @ (scale * q)                   # (5) read after write
    return S_new, o, {"S_tilde": S_tilde, "v_hat": v_hat, "e": e}


def _segments(Ttot: int, B: int, T: int, cu_seqlens: Optional[np.ndarray]):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def kda_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
                scale: float = 1.0, h0: Optional[np.ndarray] = None,
                cu_seqlens: Optional[np.ndarray] = None,
                mode: str = "kda") -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token recurrence over [B, T, H, D] inputs (float64 results).

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
    h0: [N, H, Dk, Dv] or None (zeros); cu_seqlens: int [N+1] with B == 1, or
    None (then the N = B rows are the sequences).
    Returns o [B, T, H, Dv] and ht [N, H, Dk, Dv].

    ``mode="additive"`` runs plain linear attention instead (S += k v^T, no
    decay, no beta), the first row of the table in "Notes on Linear
    Attention" (zhilingong.com) section 10; it exists only so that the read
    and its causality can be pinned against a brute-force masked (QK^T)V.
    All heads advance together, one token at a time.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    qf = q.reshape(B * T, H, Dk)
    kf = k.reshape(B * T, H, Dk)
    vf = v.reshape(B * T, H, Dv)
    gf = g.reshape(B * T, H, Dk)
    bf = beta.reshape(B * T, H)
    segs = _segments(B * T, B, T, cu_seqlens)
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(segs), H, Dk, Dv))
    for n, (s, e_) in enumerate(segs):
        S = np.zeros((H, Dk, Dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(s, e_):
            if mode == "additive":
                S = S + kf[t][:, :, None] * vf[t][:, None, :]
            else:
                S = np.exp(gf[t])[:, :, None] * S                       # (1) forget
                v_hat = np.einsum("hkv,hk->hv", S, kf[t])               # (2) predict
                err = bf[t][:, None] * (vf[t] - v_hat)                  # (3) correct
                S = S + kf[t][:, :, None] * err[:, None, :]             # (4) write
            o[t] = np.einsum("hkv,hk->hv", S, scale * qf[t])            # (5) read
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def kda_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
               state: np.ndarray, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One recurrence step per (request, head) against a persistent state.

    q, k, g: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H]; state: [N, H, Dk, Dv].
    Returns (o [N, H, Dv], new state). The decode step is the loop body of
    kda_forward applied once.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S = np.exp(g)[..., :, None] * np.asarray(state, dtype=np.float64)   # (1)
    v_hat = np.einsum("nhkv,nhk->nhv", S, k)                            # (2)
    err = beta[..., None] * (v - v_hat)                                 # (3)
    S = S + k[..., :, None] * err[..., None, :]                         # (4)
    o = np.einsum("nhkv,nhk->nhv", S, scale * q)                        # (5)
    return o, S


def gdn_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
                scale: float = 1.0, h0: Optional[np.ndarray] = None,
                cu_seqlens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gated DeltaNet, token by token (float64 results).

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; g, beta: [B, T, H] (g = log alpha, one
    scalar per token and head); h0, cu_seqlens and the returns as in kda_forward.
    Per token, following zhilingong.com section 6: S_bar = alpha_t S, then the delta
    rule on the decayed state, S = S_bar + k_t (beta_t (v_t - S_bar^T k_t))^T, and the
    read o_t = S^T (scale q_t) of the updated state.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    qf, kf, vf = q.reshape(B * T, H, Dk), k.reshape(B * T, H, Dk), v.reshape(B * T, H, Dv)
    af = np.exp(g.reshape(B * T, H))                                    # alpha_t per head
    bf = beta.reshape(B * T, H)
    segs = _segments(B * T, B, T, cu_seqlens)
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(segs), H, Dk, Dv))
    for n, (s, e_) in enumerate(segs):
        S = np.zeros((H, Dk, Dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(s, e_):
            S_bar = af[t][:, None, None] * S                            # retention gate
            err = bf[t][:, None] * (vf[t] - np.einsum("hkv,hk->hv", S_bar, kf[t]))
            S = S_bar + kf[t][:, :, None] * err[:, None, :]             # delta rule
            o[t] = np.einsum("hkv,hk->hv", S, scale * qf[t])            # read
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def gdn_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
               state: np.ndarray, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One Gated DeltaNet step per (request, head): q, k [N, H, Dk]; v [N, H, Dv];
    g, beta [N, H]; state [N, H, Dk, Dv]. Returns (o [N, H, Dv], new state)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S_bar = np.exp(np.asarray(g, dtype=np.float64))[..., None, None] * np.asarray(
        state, dtype=np.float64)
    err = beta[..., None] * (v - np.einsum("nhkv,nhk->nhv", S_bar, k))
    S = S_bar + k[..., :, None] * err[..., None, :]
    return np.einsum("nhkv,nhk->nhv", S, scale * q), S


def gdn2_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, b: np.ndarray,
                 w: np.ndarray, scale: float = 1.0, h0: Optional[np.ndarray] = None,
                 cu_seqlens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gated DeltaNet-2, token by token (float64 results).

    q, k, g, b: [B, T, H, Dk] (b = erase gate per key channel); v, w: [B, T, H, Dv]
    (w = write gate per value channel); h0, cu_seqlens and the returns as in kda_forward.
    Per token, following jonahsamost.bearblog.dev, "Gated DeltaNet-2" (in the d_k x d_v
    layout): S_bar = Diag(exp g_t) S; v^ = S_bar^T (b_t * k_t); S = S_bar + k_t (w_t * v_t - v^)^T;
    then the read o_t = S^T (scale q_t) of the updated state.
    """
    q, k, v, g, b, w = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, b, w))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    fl = lambda a, d: a.reshape(B * T, H, d)
    qf, kf, gf, bf = fl(q, Dk), fl(k, Dk), fl(g, Dk), fl(b, Dk)
    vf, wf = fl(v, Dv), fl(w, Dv)
    segs = _segments(B * T, B, T, cu_seqlens)
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(segs), H, Dk, Dv))
    for n, (s, e_) in enumerate(segs):
        S = np.zeros((H, Dk, Dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(s, e_):
            S_bar = np.exp(gf[t])[:, :, None] * S                          # decay
            v_hat = np.einsum("hkv,hk->hv", S_bar, bf[t] * kf[t])          # gated-key read
            S = S_bar + kf[t][:, :, None] * (wf[t] * vf[t] - v_hat)[:, None, :]
            o[t] = np.einsum("hkv,hk->hv", S, scale * qf[t])               # read
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def gdn2_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, b: np.ndarray,
                w: np.ndarray, state: np.ndarray,
                scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One Gated DeltaNet-2 step per (request, head): q, k, g, b [N, H, Dk]; v, w [N, H, Dv];
    state [N, H, Dk, Dv]. Returns (o [N, H, Dv], new state)."""
    q, k, v, g, b, w = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, b, w))
    S_bar = np.exp(g)[..., :, None] * np.asarray(state, dtype=np.float64)
    v_hat = np.einsum("nhkv,nhk->nhv", S_bar, b * k)
    S = S_bar + k[..., :, None] * (w * v - v_hat)[..., None, :]
    return np.einsum("nhkv,nhk->nhv", S, scale * q), S


def prepare_inputs(q: np.ndarray, k: np.ndarray, a: np.ndarray, b: np.ndarray,
                   scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Raw projections to the recurrence's inputs, in float64 (one token-head row per last
    axis): q^ = scale q / |q| and k^ = k / |k| (normalised queries and keys, zhilingong.com
    sections 4 and 5.3; a zero row stays zero), g = log sigmoid(a) (so that alpha = exp(g)
    lies in (0, 1)), beta = sigmoid(b) (jonahsamost.bearblog.dev)."""
    q, k, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, a, b))

    def unit(x):
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)

    return scale * unit(q), unit(k), -np.logaddexp(0.0, -a), 1.0 / (1.0 + np.exp(-b))
