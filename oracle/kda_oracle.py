"""Float64 CPU oracle of the KDA forward recurrence (numpy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``; the library itself never does.

What it computes is the recurrence itself, token by token, in float64 with
no blocking, chunking or reordering. The state S of one head is d_k x d_v
with one row per key channel and the read is o = S^T q ("Notes on Linear
Attention", zhilingong.com, sections 3 and 11, where S_t = sum_i k_i v_i^T;
the pages that write the state d_v x d_k use its transpose). One step at
token t is the sequence of five operations of "Module 03 - KDA I: The
Delta-Rule Recurrence" (jared-hpc.com), section 2, written out here per key
channel i (row i of S) and value channel j:

  (1) forget   S~[i][j] = alpha_t[i] S[i][j],          alpha_t = exp(g_t)
  (2) predict  v^[j]    = sum_i k_t[i] S~[i][j]
  (3) correct  e[j]     = beta_t (v_t[j] - v^[j])      beta inside the error
  (4) write    S[i][j]  = S~[i][j] + k_t[i] e[j]
  (5) read     o_t[j]   = sum_i (scale q_t[i]) S[i][j]  after the write

Putting beta inside the error gives the same S_t as applying it at the write
("Kimi Delta Attention (KDA)", brain.bigb.es, section "KDA: one gate per key
channel", which also fixes g_t = log(alpha_t) <= 0 as the stored gate). The
loops run over the key channel; heads and value channels are numpy axes.

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


# ------------------------------------------------------------------------------------------
# the five operations, per key channel. S has shape [..., Dk, Dv] (leading axes: heads, or
# requests and heads) and is updated in place; every vector argument has the matching
# leading axes.
# ------------------------------------------------------------------------------------------
def _forget_and_predict(S: np.ndarray, alpha: np.ndarray, k_read: np.ndarray) -> np.ndarray:
    """(1) row i of S decays by alpha[i]; (2) v^ = sum_i k_read[i] S~[i]. Returns v^."""
    v_hat = np.zeros(S.shape[:-2] + S.shape[-1:])
    for i in range(S.shape[-2]):
        S[..., i, :] *= alpha[..., i, None]
        v_hat += k_read[..., i, None] * S[..., i, :]
    return v_hat


def _write_and_read(S: np.ndarray, k: np.ndarray, e: np.ndarray, q: np.ndarray,
                    scale: float) -> np.ndarray:
    """(4) row i of S moves by k[i] e; (5) o = sum_i (scale q[i]) S[i]. Returns o."""
    o = np.zeros(S.shape[:-2] + S.shape[-1:])
    for i in range(S.shape[-2]):
        S[..., i, :] += k[..., i, None] * e
        o += (scale * q[..., i, None]) * S[..., i, :]
    return o


def _additive_write_and_read(S: np.ndarray, k: np.ndarray, v: np.ndarray, q: np.ndarray,
                             scale: float) -> np.ndarray:
    """Plain linear attention: S[i] += k[i] v (no decay, no error), then the same read."""
    return _write_and_read(S, k, v, q, scale)


def kda_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray,
             beta: float, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray, dict]:
    """One KDA step for one head. S is [Dk, Dv]; returns (S_t, o_t, intermediates).

    The five operations of "Module 03 - KDA I" (jared-hpc.com) section 2, with the
    beta-scaled error of brain.bigb.es "Kimi Delta Attention (KDA)".
    """
    S = np.array(S, dtype=np.float64)
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    v_hat = _forget_and_predict(S, np.exp(g), k)
    S_tilde = S.copy()
    e = float(beta) * (v - v_hat)
    o = _write_and_read(S, k, e, q, scale)
    return S, o, {"S_tilde": S_tilde, "v_hat": v_hat, "e": e}


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
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    qf, kf, gf = q.reshape(B * T, H, Dk), k.reshape(B * T, H, Dk), g.reshape(B * T, H, Dk)
    vf = v.reshape(B * T, H, Dv)
    bf = beta.reshape(B * T, H)
    segs = _segments(B * T, B, T, cu_seqlens)
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(segs), H, Dk, Dv))
    for n, (s, e_) in enumerate(segs):
        S = np.zeros((H, Dk, Dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(s, e_):
            if mode == "additive":
                o[t] = _additive_write_and_read(S, kf[t], vf[t], qf[t], scale)
            else:
                v_hat = _forget_and_predict(S, np.exp(gf[t]), kf[t])
                err = bf[t][:, None] * (vf[t] - v_hat)
                o[t] = _write_and_read(S, kf[t], err, qf[t], scale)
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def kda_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
               state: np.ndarray, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One recurrence step per (request, head) against a persistent state.

    q, k, g: [N, H, Dk]; v: [N, H, Dv]; beta: [N, H]; state: [N, H, Dk, Dv].
    Returns (o [N, H, Dv], new state). The decode step is the loop body of
    kda_forward applied once.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    S = np.array(state, dtype=np.float64)
    v_hat = _forget_and_predict(S, np.exp(g), k)
    err = beta[..., None] * (v - v_hat)
    o = _write_and_read(S, k, err, q, scale)
    return o, S


def gdn_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
                scale: float = 1.0, h0: Optional[np.ndarray] = None,
                cu_seqlens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gated DeltaNet, token by token (float64 results).

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; g, beta: [B, T, H] (g = log alpha, one
    scalar per token and head); h0, cu_seqlens and the returns as in kda_forward.
    Per token, following zhilingong.com section 6: every row of the state decays by the
    one gate alpha_t, then the delta rule acts on the decayed state (predict, beta-scaled
    error, rank-one write) and the updated state is read with scale q_t.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
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
            alpha = np.repeat(af[t][:, None], Dk, axis=1)               # the same for every row
            v_hat = _forget_and_predict(S, alpha, kf[t])
            err = bf[t][:, None] * (vf[t] - v_hat)
            o[t] = _write_and_read(S, kf[t], err, qf[t], scale)
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def gdn_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
               state: np.ndarray, scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One Gated DeltaNet step per (request, head): q, k [N, H, Dk]; v [N, H, Dv];
    g, beta [N, H]; state [N, H, Dk, Dv]. Returns (o [N, H, Dv], new state)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    S = np.array(state, dtype=np.float64)
    alpha = np.repeat(np.exp(g)[..., None], S.shape[-2], axis=-1)
    v_hat = _forget_and_predict(S, alpha, k)
    err = beta[..., None] * (v - v_hat)
    return _write_and_read(S, k, err, q, scale), S


def gdn2_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, b: np.ndarray,
                 w: np.ndarray, scale: float = 1.0, h0: Optional[np.ndarray] = None,
                 cu_seqlens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gated DeltaNet-2, token by token (float64 results).

    q, k, g, b: [B, T, H, Dk] (b = erase gate per key channel); v, w: [B, T, H, Dv]
    (w = write gate per value channel); h0, cu_seqlens and the returns as in kda_forward.
    Per token, following jonahsamost.bearblog.dev, "Gated DeltaNet-2" (in the d_k x d_v
    layout): decay each key channel's row by exp(g_t[i]); read the old value through the
    gated key, v^ = sum_i b_t[i] k_t[i] S~[i]; write the residual w_t * v_t - v^ at the
    original key; then read the updated state with scale q_t.
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
            v_hat = _forget_and_predict(S, np.exp(gf[t]), bf[t] * kf[t])
            o[t] = _write_and_read(S, kf[t], wf[t] * vf[t] - v_hat, qf[t], scale)
        ht[n] = S
    return o.reshape(B, T, H, Dv), ht


def gdn2_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, b: np.ndarray,
                w: np.ndarray, state: np.ndarray,
                scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """One Gated DeltaNet-2 step per (request, head): q, k, g, b [N, H, Dk]; v, w [N, H, Dv];
    state [N, H, Dk, Dv]. Returns (o [N, H, Dv], new state)."""
    q, k, v, g, b, w = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, b, w))
    S = np.array(state, dtype=np.float64)
    v_hat = _forget_and_predict(S, np.exp(g), b * k)
    return _write_and_read(S, k, w * v - v_hat, q, scale), S


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
