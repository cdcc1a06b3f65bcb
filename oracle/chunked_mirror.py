"""Float64 numpy evaluation of the chunkwise (UT / WY) form of KDA.

TEST INFRASTRUCTURE (same import rule as the rest of ``oracle/``). It exists
to pin, on the CPU and in float64, that the chunk algebra reaches the
token-by-token result: "Kimi Delta Attention (KDA)" (brain.bigb.es),
section "Two schedules for the same recurrence", states that the recurrent
and chunkwise schedules give identical states and outputs.

Per chunk of C tokens (rows i, j = 0..L-1, L <= C), with S the state at the
chunk start and G_i the inclusive in-chunk cumulative sum of g (the
log-space prefix sums of the same section):

* provisional errors   Ebar_i = beta_i (v_i - S^T (exp(G_i) * k_i))
* coupling             R[i, j] = beta_i sum_c k_i[c] k_j[c] exp(G_i[c]-G_j[c]), j < i
* true errors          (I + R) E = Ebar  (unit lower-triangular solve by
                       forward substitution, "From Fast Weight Programmers to
                       KDA", jonahsamost.bearblog.dev, section "Parallelizing
                       Linear Transformers with the Delta Rule")
* outputs              O = (scale q * exp(G)) S + Aqk E with
                       Aqk[i, j] = scale sum_c q_i[c] k_j[c] exp(G_i[c]-G_j[c]), j <= i
* next state           S' = Diag(exp(G_end)) S + (k * exp(G_end - G))^T E

Sequences never share a chunk; the last chunk of a sequence may be short.
Pairwise decays are exp of differences of prefix sums, never a ratio of
cumulative products (which is 0/0 when a chunk's decay underflows).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _forward_substitution(R: np.ndarray, rhs: np.ndarray) -> np.ndarray:
    """Solve (I + R) X = rhs for strictly lower-triangular R, row by row."""
    X = np.array(rhs, dtype=np.float64, copy=True)
    for i in range(R.shape[0]):
        if i:
            X[i] -= R[i, :i] @ X[:i]
    return X


def chunked_forward(q, k, v, g, beta, scale: float = 1.0, h0: Optional[np.ndarray] = None,
                    cu_seqlens=None, chunk: int = 64):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    qf, kf, vf = q.reshape(B * T, H, Dk), k.reshape(B * T, H, Dk), v.reshape(B * T, H, Dv)
    gf, bf = g.reshape(B * T, H, Dk), beta.reshape(B * T, H)
    if cu_seqlens is None:
        segs = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        segs = [(int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B * T, H, Dv))
    ht = np.zeros((len(segs), H, Dk, Dv))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            for c0 in range(s0, s1, chunk):
                c1 = min(c0 + chunk, s1)
                Kc, Qc, Vc = kf[c0:c1, h], qf[c0:c1, h] * scale, vf[c0:c1, h]
                bc = bf[c0:c1, h]
                G = np.cumsum(gf[c0:c1, h], axis=0)            # [L, Dk] inclusive
                L = c1 - c0
                diff = G[:, None, :] - G[None, :, :]           # G_i - G_j
                lower = np.tril(np.ones((L, L), dtype=bool))   # j <= i
                dec = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)),
                               0.0)
                R = bc[:, None] * np.einsum("ic,jc,ijc->ij", Kc, Kc, dec)
                R = np.tril(R, -1)
                Aqk = np.einsum("ic,jc,ijc->ij", Qc, Kc, dec)  # includes the diagonal
                Ebar = bc[:, None] * (Vc - (Kc * np.exp(G)) @ S)
                E = _forward_substitution(R, Ebar)
                o[c0:c1, h] = (Qc * np.exp(G)) @ S + Aqk @ E
                Gend = G[-1]
                S = np.exp(Gend)[:, None] * S + (Kc * np.exp(Gend[None, :] - G)).T @ E
            ht[n, h] = S
    return o.reshape(B, T, H, Dv), ht
