"""Pins of the float64 oracles against facts the pages and the mathematics fix.

None of these compare the oracle with itself: each checks a printed value, a
closed form, an invariant, a textbook special case or brute force, chosen so
that a plausible slip (transposed state, decay on the wrong axis, missing
beta, read before write, predict before decay, wrong sign) fails at least one.
"""
import json
import os

import numpy as np
import pytest

from gated_delta_rule_channel_amd import inputs as I
from oracle import chunked_mirror, kda_oracle, native

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.double().numpy()


def _prefill_np(x: I.PrefillInputs):
    return (_np(x.q), _np(x.k), _np(x.v), _np(x.g), _np(x.beta),
            None if x.h0 is None else _np(x.h0),
            None if x.cu_seqlens is None else x.cu_seqlens.numpy())


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.fixture(scope="module", autouse=True)
def _built_native():
    native.build()


# --- P1: the worked example ------------------------------------------------------------------
def test_p1_worked_example_step():
    """Printed one-step example (jared-hpc.com Module 03, section 4), exact in float64."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    S0 = np.array(ex["S_prev"])
    k, v = np.array(ex["k"]), np.array(ex["v"])
    g = np.log(np.array(ex["alpha"]))
    S1, o, mid = kda_oracle.kda_step(S0, q=np.zeros(2), k=k, v=v, g=g, beta=ex["beta"])
    np.testing.assert_array_equal(mid["v_hat"], ex["v_hat"])
    # the page applies beta at the write; here beta sits inside e, so e = beta * (v - v^)
    np.testing.assert_array_equal(mid["e"], ex["beta"] * np.array(ex["error_before_beta"]))
    np.testing.assert_array_equal(np.outer(k, mid["e"]), ex["beta_k_eT"])
    np.testing.assert_array_equal(S1, ex["S_t"])
    # the state is not symmetric, so a transposed orientation cannot pass
    assert not np.array_equal(S1, S1.T)


def test_p1_worked_example_through_both_oracles():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    S0 = np.array(ex["S_prev"])[None, None]
    k = np.array(ex["k"])[None, None, None]
    v = np.array(ex["v"])[None, None, None]
    g = np.log(np.array(ex["alpha"]))[None, None, None]
    beta = np.array([[[ex["beta"]]]])
    q = np.array([[[[0.25, -0.75]]]])  # exact in float32
    for fwd in (kda_oracle.kda_forward, native.prefill):
        o, ht = fwd(q, k, v, g, beta, scale=1.0, h0=S0)
        np.testing.assert_array_equal(ht[0, 0], ex["S_t"])
        # read after write: o = S_t^T q
        np.testing.assert_allclose(o[0, 0, 0], np.array(ex["S_t"]).T @ q[0, 0, 0], rtol=0,
                                   atol=1e-15)
    od, Sd = native.decode(q[0], k[0], v[0], g[0], beta[0], S0)
    np.testing.assert_array_equal(Sd[0, 0], ex["S_t"])


# --- P2, P3: read-back and locality --------------------------------------------------------
@pytest.mark.parametrize("seed", range(5))
def test_p2_readback_interpolates_and_overwrites(seed):
    """Unit k: k^T S_t = (1-beta) k^T S~ + beta v, and = v at beta = 1 even under decay.

    brain.bigb.es "DeltaNet: write the error instead of the value"; zhilingong.com section 5.3
    and section 7.2 (the identity survives per-channel decay).
    """
    rng = np.random.default_rng(100 + seed)
    Dk, Dv = 8, 5
    S0 = rng.standard_normal((Dk, Dv))
    k = rng.standard_normal(Dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(Dv)
    g = -rng.uniform(0, 2, Dk)
    for beta in (0.0, 0.3, 1.0):
        S1, _, mid = kda_oracle.kda_step(S0, np.zeros(Dk), k, v, g, beta)
        lhs = S1.T @ k
        rhs = (1 - beta) * (mid["S_tilde"].T @ k) + beta * v
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
        if beta == 1.0:
            np.testing.assert_allclose(lhs, v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_p3_rank_one_locality(seed):
    """(S_t - S~_t)^T x = 0 for every x orthogonal to k_t (brain.bigb.es, DeltaNet section)."""
    rng = np.random.default_rng(200 + seed)
    Dk, Dv = 9, 4
    S0 = rng.standard_normal((Dk, Dv))
    k = rng.standard_normal(Dk)
    v = rng.standard_normal(Dv)
    g = -rng.uniform(0, 3, Dk)
    S1, _, mid = kda_oracle.kda_step(S0, np.zeros(Dk), k, v, g, 0.7)
    for _ in range(4):
        x = rng.standard_normal(Dk)
        x -= (x @ k) / (k @ k) * k
        np.testing.assert_allclose((S1 - mid["S_tilde"]).T @ x, 0, atol=1e-12)
    # and along k itself the change is not zero
    assert np.linalg.norm((S1 - mid["S_tilde"]).T @ k) > 1e-3


# --- P4: two orthogonal keys with a diagonal gate -------------------------------------------
def test_p4_orthogonal_keys_diagonal_gate():
    """zhilingong.com section 11: keys e1, e2; D = Diag(0.2, 0.99)."""
    v1, v2 = np.array([1.5, -2.0, 0.25]), np.array([-0.5, 3.0, 1.0])
    vb = np.array([0.75, 0.5, -1.25])
    ka, kb = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    # additive: two writes at the same key give v1 + v2 in that row
    q = np.zeros((1, 2, 1, 2))
    k = np.stack([ka, ka])[None, :, None, :]
    v = np.stack([v1, v2])[None, :, None, :]
    z = np.zeros((1, 2, 1, 2))
    _, ht = kda_oracle.kda_forward(q, k, v, z, np.ones((1, 2, 1)), mode="additive")
    np.testing.assert_allclose(ht[0, 0, 0], v1 + v2)
    # delta with beta = 1: the second write replaces the row, the other row is untouched
    S0 = np.zeros((2, 3))
    S0[1] = vb
    S1, _, _ = kda_oracle.kda_step(S0, np.zeros(2), ka, v1, np.zeros(2), 1.0)
    S2, _, _ = kda_oracle.kda_step(S1, np.zeros(2), ka, v2, np.zeros(2), 1.0)
    np.testing.assert_allclose(S2[0], v2, atol=1e-15)
    np.testing.assert_allclose(S2[1], vb, atol=0)
    # KDA gate: row a (key channel 0) decays by 0.2, row b by 0.99, before a write at k_b
    g = np.log(np.array([0.2, 0.99]))
    S3, _, _ = kda_oracle.kda_step(S2, np.zeros(2), kb, v1, g, 1.0)
    np.testing.assert_allclose(S3[0], 0.2 * v2, rtol=1e-15)
    np.testing.assert_allclose(S3[1], v1, atol=1e-15)
    # without the write (beta = 0) the decay acts on rows, not on columns
    S4, _, _ = kda_oracle.kda_step(S2, np.zeros(2), kb, v1, g, 0.0)
    np.testing.assert_allclose(S4, np.diag([0.2, 0.99]) @ S2, rtol=1e-15)


# --- P5: additive mode equals brute-force masked (QK^T)V -----------------------------------
@pytest.mark.parametrize("T", [1, 5, 16])
def test_p5_additive_equals_masked_attention(T):
    """zhilingong.com section 2.1 / brain.bigb.es: causal linear attention is tril(QK^T) V,
    including the diagonal (the read follows the write)."""
    rng = np.random.default_rng(T)
    H, Dk, Dv = 2, 6, 3
    q = rng.standard_normal((1, T, H, Dk))
    k = rng.standard_normal((1, T, H, Dk))
    v = rng.standard_normal((1, T, H, Dv))
    o, _ = kda_oracle.kda_forward(q, k, v, np.zeros_like(q), np.ones((1, T, H)),
                                  mode="additive")
    for h in range(H):
        P = np.zeros((T, T))
        for t in range(T):
            for i in range(t + 1):
                P[t, i] = q[0, t, h] @ k[0, i, h]
        np.testing.assert_allclose(o[0, :, h], P @ v[0, :, h], rtol=1e-12, atol=1e-12)


# --- P6, P7: family reductions ----------------------------------------------------------------
def _random_seq(rng, T, Dk, Dv):
    k = rng.standard_normal((T, Dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((T, Dk))
    v = rng.standard_normal((T, Dv))
    beta = rng.uniform(0, 1, T)
    return q, k, v, beta


def test_p6_alpha_one_is_deltanet():
    """g = 0 gives DeltaNet, S_t = S_{t-1} + beta k^T (v - k S_{t-1}) in row-vector form
    (zhilingong.com section 5.1)."""
    rng = np.random.default_rng(6)
    T, Dk, Dv = 20, 7, 5
    q, k, v, beta = _random_seq(rng, T, Dk, Dv)
    S = np.zeros((Dk, Dv))
    ref = []
    for t in range(T):
        S = S + beta[t] * np.outer(k[t], v[t] - k[t] @ S)
        ref.append(q[t] @ S)
    o, ht = kda_oracle.kda_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                   np.zeros((1, T, 1, Dk)), beta[None, :, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-12, atol=1e-12)


def test_p7_uniform_alpha_is_gated_deltanet():
    """A gate equal on all channels gives scalar Gated DeltaNet,
    S_t = alpha (I - beta k k^T) S_{t-1} + beta k v^T (hitreader.com, Gated DeltaNet)."""
    rng = np.random.default_rng(7)
    T, Dk, Dv = 20, 7, 5
    q, k, v, beta = _random_seq(rng, T, Dk, Dv)
    alpha = rng.uniform(0.3, 1.0, T)
    S = np.zeros((Dk, Dv))
    ref = []
    for t in range(T):
        S = alpha[t] * (np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(
            k[t], v[t])
        ref.append(S.T @ q[t])
    g = np.repeat(np.log(alpha)[:, None], Dk, axis=1)
    o, ht = kda_oracle.kda_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                   g[None, :, None], beta[None, :, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-12, atol=1e-12)


def test_closed_form_kda_step():
    """One step equals the closed form S_t = (I - beta k k^T) D S + beta k v^T
    (jared-hpc.com Module 03 section 3; zhilingong.com section 7)."""
    rng = np.random.default_rng(8)
    Dk, Dv = 6, 4
    S0 = rng.standard_normal((Dk, Dv))
    k = rng.standard_normal(Dk)
    v = rng.standard_normal(Dv)
    g = -rng.uniform(0, 2, Dk)
    b = 0.4
    S1, _, _ = kda_oracle.kda_step(S0, np.zeros(Dk), k, v, g, b)
    ref = (np.eye(Dk) - b * np.outer(k, k)) @ np.diag(np.exp(g)) @ S0 + b * np.outer(k, v)
    np.testing.assert_allclose(S1, ref, rtol=1e-13, atol=1e-13)


# --- P8: operator order is visible to the harness ------------------------------------------
def _swapped_order_forward(q, k, v, g, beta):
    """Planted mistake: predict from the undecayed state (D (I - beta k k^T) instead of
    (I - beta k k^T) D)."""
    B, T, H, Dk = q.shape
    S = np.zeros((H, Dk, v.shape[-1]))
    o = np.zeros(v.shape)
    for t in range(T):
        v_hat = np.einsum("hkv,hk->hv", S, k[0, t])
        err = beta[0, t][:, None] * (v[0, t] - v_hat)
        S = np.exp(g[0, t])[:, :, None] * S + k[0, t][:, :, None] * err[:, None, :]
        o[0, t] = np.einsum("hkv,hk->hv", S, q[0, t])
    return o, S


def test_p8_swapped_order_is_detected():
    """jared-hpc.com Module 03 section 3 and brain.bigb.es (Gated DeltaNet): the two orders
    differ; the fp32 acceptance bound (1e-4 max|o|) must see it on the tiny workload."""
    x = I.prefill_inputs(I.WORKLOADS[0])
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    o_ref, ht_ref = kda_oracle.kda_forward(q, k, v, g, beta)
    o_bad, S_bad = _swapped_order_forward(q, k, v, g, beta)
    assert np.max(np.abs(o_bad - o_ref)) > 100 * 1e-4 * np.max(np.abs(o_ref))
    assert np.max(np.abs(S_bad - ht_ref[0])) > 100 * 1e-4 * np.max(np.abs(ht_ref))


# --- P9: non-expansive transition ------------------------------------------------------------
@pytest.mark.parametrize("wid", [0, 1])
def test_p9_frobenius_bound_every_step(wid):
    """Unit k, beta in [0, 1], alpha <= 1: ||S_t||_F <= ||S_{t-1}||_F + beta ||v||
    (brain.bigb.es: I - beta k k^T has eigenvalue 1 - beta along k and 1 elsewhere)."""
    w = I.WORKLOADS[wid]
    x = I.prefill_inputs(w, heads=[0], T=256 if wid == 1 else None)
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    S = np.zeros((w.Dk, w.Dv)) if h0 is None else h0[0, 0].copy()
    for t in range(q.shape[1]):
        kt = k[0, t, 0]
        prev = np.linalg.norm(S)
        S, _, _ = kda_oracle.kda_step(S, q[0, t, 0], kt, v[0, t, 0], g[0, t, 0], beta[0, t, 0])
        # ||I - beta k k^T||_2 = 1 while beta |k|^2 <= 2, and ||beta k v^T||_F = beta |k| |v|
        bound = prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) * np.linalg.norm(kt)
        assert np.linalg.norm(S) <= bound * (1 + 1e-9)


def test_p9_shrunken_varlen_stress():
    w = I.WORKLOADS[4]
    x = I.prefill_inputs(w, heads=[3], lengths=[300])
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    S = np.zeros((w.Dk, w.Dv))
    for t in range(q.shape[1]):
        kt = k[0, t, 0]
        prev = np.linalg.norm(S)
        S, _, _ = kda_oracle.kda_step(S, q[0, t, 0], kt, v[0, t, 0], g[0, t, 0], beta[0, t, 0])
        # bf16 keys are unit only to bf16 precision: the bound carries |k|
        assert np.linalg.norm(S) <= (prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
                                     * np.linalg.norm(kt)) * (1 + 1e-9)


# --- P10: chunkwise algebra reaches the recurrence ------------------------------------------
def _cases():
    yield "c0", I.prefill_inputs(I.WORKLOADS[0])
    yield "c1", I.prefill_inputs(I.WORKLOADS[1], heads=[0, 3], T=200)
    yield "c4-shrunk", I.prefill_inputs(I.WORKLOADS[4], heads=[5], lengths=[130, 1, 64, 63, 0, 97])


@pytest.mark.parametrize("name,x", list(_cases()), ids=lambda v: v if isinstance(v, str) else "")
def test_p10_chunked_mirror_matches(name, x):
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    o_ref, ht_ref = kda_oracle.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    o_chk, ht_chk = chunked_mirror.chunked_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    assert _rel(o_chk, o_ref) <= 1e-10
    assert _rel(ht_chk, ht_ref) <= 1e-10


# --- native oracle vs numpy oracle, P11 consistency ------------------------------------------
@pytest.mark.parametrize("name,x", list(_cases()), ids=lambda v: v if isinstance(v, str) else "")
def test_native_matches_numpy(name, x):
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    o_ref, ht_ref = kda_oracle.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    o_c, ht_c = native.prefill(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, cu_seqlens=cu)
    assert _rel(o_c, o_ref) <= 1e-12
    assert _rel(ht_c, ht_ref) <= 1e-12


def test_scale_is_linear_in_the_read():
    x = I.prefill_inputs(I.WORKLOADS[0])
    o1, ht1 = native.prefill(x.q, x.k, x.v, x.g, x.beta, scale=1.0)
    o2, ht2 = native.prefill(x.q, x.k, x.v, x.g, x.beta, scale=0.37)
    np.testing.assert_allclose(o2, 0.37 * o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(ht1, ht2)


def test_p11_resume_equals_one_pass():
    """Running [0, T1) then [T1, T) from the carried state equals one pass (the state is the
    per-request carry of jared-hpc.com Module 03 section 5)."""
    x = I.prefill_inputs(I.WORKLOADS[1], heads=[1, 2], T=300)
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    o, ht = kda_oracle.kda_forward(q, k, v, g, beta, h0=h0)
    T1 = 77
    sl = lambda a, s: a[:, s]
    oa, ha = kda_oracle.kda_forward(*(sl(a, slice(0, T1)) for a in (q, k, v, g, beta)), h0=h0)
    ob, hb = kda_oracle.kda_forward(*(sl(a, slice(T1, None)) for a in (q, k, v, g, beta)), h0=ha)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hb, ht, rtol=1e-12, atol=1e-12)


def test_p11_varlen_equals_separate_runs_and_decode_steps():
    x = I.prefill_inputs(I.WORKLOADS[4], heads=[0, 7], lengths=[40, 0, 17, 64])
    q, k, v, g, beta, h0, cu = _prefill_np(x)
    o, ht = native.prefill(x.q, x.k, x.v, x.g, x.beta, cu_seqlens=cu)
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        on, hn = kda_oracle.kda_forward(*(a[:, s:e] for a in (q, k, v, g, beta)))
        np.testing.assert_allclose(o[:, s:e], on, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ht[n], hn[0], rtol=1e-12, atol=1e-12)
        # the same sequence as decode steps against a carried state
        S = np.zeros((1,) + ht.shape[1:])
        for t in range(s, e):
            od, S = kda_oracle.kda_decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
            np.testing.assert_allclose(od[0], o[0, t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S[0], ht[n], rtol=1e-12, atol=1e-12)


def test_native_decode_matches_numpy():
    w = I.WORKLOADS[3]
    x = I.decode_inputs(w, heads=[0, 9, 63], N=5)
    args = [t.double().numpy() for t in (x.q, x.k, x.v, x.g, x.beta, x.state)]
    o_ref, S_ref = kda_oracle.kda_decode(*args)
    o_c, S_c = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state)
    assert _rel(o_c, o_ref) <= 1e-12
    assert _rel(S_c, S_ref) <= 1e-12


# --- Gated DeltaNet (scalar gate) -------------------------------------------------------------
def test_gdn_matrix_form():
    """The scalar-gate oracle (decay, then the delta rule on the decayed state) equals the
    matrix form S_t = alpha_t (I - beta_t k_t k_t^T) S_(t-1) + beta_t k_t v_t^T, the second
    form of zhilingong.com section 6 and the recurrence on jonahsamost.bearblog.dev,
    "Gated Delta Networks" (transposed there: S_t^T in this layout), with o_t = S_t^T q_t."""
    rng = np.random.default_rng(61)
    T, Dk, Dv = 24, 6, 5
    q, k, v, beta = _random_seq(rng, T, Dk, Dv)
    alpha = rng.uniform(0.2, 1.0, T)
    S0 = rng.standard_normal((Dk, Dv))
    S = S0.copy()
    ref = []
    for t in range(T):
        S = alpha[t] * (np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) @ S + beta[t] * np.outer(
            k[t], v[t])
        ref.append(S.T @ q[t])
    o, ht = kda_oracle.gdn_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                   np.log(alpha)[None, :, None], beta[None, :, None],
                                   h0=S0[None, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-12, atol=1e-12)
    # alpha = 1 leaves plain DeltaNet; a per-channel reading of alpha would differ here
    o1, _ = kda_oracle.gdn_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                   np.zeros((1, T, 1)), beta[None, :, None])
    S = np.zeros((Dk, Dv))
    for t in range(T):
        S = S + beta[t] * np.outer(k[t], v[t] - k[t] @ S)
    np.testing.assert_allclose(o1[0, -1, 0], S.T @ q[-1], rtol=1e-12, atol=1e-12)


def test_gdn_beta_zero_is_pure_decay():
    """beta = 0 writes nothing: S_t = (prod alpha) S_0 and o_t = exp(G_t) S_0^T q_t with G_t
    the running sum of g (the retention gate alone, zhilingong.com section 6)."""
    rng = np.random.default_rng(62)
    T, H, Dk, Dv = 30, 2, 4, 3
    q = rng.standard_normal((1, T, H, Dk))
    k = rng.standard_normal((1, T, H, Dk))
    v = rng.standard_normal((1, T, H, Dv))
    g = -rng.uniform(0, 0.3, (1, T, H))
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, ht = kda_oracle.gdn_forward(q, k, v, g, np.zeros((1, T, H)), scale=0.5, h0=S0)
    G = np.cumsum(g[0], axis=0)                                          # [T, H]
    o_cf = 0.5 * np.exp(G)[:, :, None] * np.einsum("thi,hij->thj", q[0], S0[0])
    np.testing.assert_allclose(o[0], o_cf, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ht[0], np.exp(G[-1])[:, None, None] * S0[0], rtol=1e-12)


def test_gdn_equals_per_channel_recurrence_with_equal_gate():
    """Gated DeltaNet is KDA with the gate repeated over the key channels (the scalar gate is
    the special case KDA refines, zhilingong.com section 7); two independently written
    oracles, over several sequences and heads."""
    x = I.gdn_prefill_inputs(I.WORKLOADS[4], heads=[1, 6], lengths=[70, 0, 33, 64])
    q, k, v, _, beta, h0, cu = _prefill_np(x)
    gs = x.g.double().numpy()
    o, ht = kda_oracle.gdn_forward(q, k, v, gs, beta, cu_seqlens=cu)
    gk = np.repeat(gs[..., None], q.shape[-1], axis=-1)
    o2, ht2 = kda_oracle.kda_forward(q, k, v, gk, beta, cu_seqlens=cu)
    assert _rel(o, o2) <= 1e-12
    assert _rel(ht, ht2) <= 1e-12


def test_native_gdn_matches_numpy():
    for x in (I.gdn_prefill_inputs(I.WORKLOADS[1], heads=[0, 3], T=130),
              I.gdn_prefill_inputs(I.WORKLOADS[4], heads=[2], lengths=[65, 0, 1, 40])):
        q, k, v, g, beta, h0, cu = _prefill_np(x)
        o_ref, ht_ref = kda_oracle.gdn_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
        o_c, ht_c = native.gdn_prefill(x.q, x.k, x.v, x.g, x.beta, h0=x.h0, cu_seqlens=cu)
        assert _rel(o_c, o_ref) <= 1e-12
        assert _rel(ht_c, ht_ref) <= 1e-12
    y = I.gdn_decode_inputs(I.WORKLOADS[3], heads=[0, 9], N=4)
    args = [t.double().numpy() for t in (y.q, y.k, y.v, y.g, y.beta, y.state)]
    o_ref, S_ref = kda_oracle.gdn_decode(*args, scale=0.7)
    o_c, S_c = native.gdn_decode(y.q, y.k, y.v, y.g, y.beta, y.state, scale=0.7)
    assert _rel(o_c, o_ref) <= 1e-12
    assert _rel(S_c, S_ref) <= 1e-12


def test_gdn_decode_steps_equal_forward():
    x = I.gdn_prefill_inputs(I.WORKLOADS[1], heads=[1], T=20)
    q, k, v, g, beta, h0, _ = _prefill_np(x)
    o, ht = kda_oracle.gdn_forward(q, k, v, g, beta, h0=h0)
    S = h0
    for t in range(q.shape[1]):
        od, S = kda_oracle.gdn_decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        np.testing.assert_allclose(od, o[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, ht, rtol=1e-12, atol=1e-12)


# --- Gated DeltaNet-2 (erase gate b, write gate w) --------------------------------------------
def test_gdn2_matrix_form():
    """The oracle (decay, read through the gated key, write the residual at k) equals the
    one-line update of jonahsamost.bearblog.dev, "Gated DeltaNet-2",
    S_t = S_(t-1) D_t (I - (b_t * k_t) k_t^T) + (w_t * v_t) k_t^T for the d_v x d_k state,
    taken here in that orientation and transposed back."""
    rng = np.random.default_rng(71)
    T, Dk, Dv = 22, 6, 5
    q, k, v, _ = _random_seq(rng, T, Dk, Dv)
    g = -rng.uniform(0, 1, (T, Dk))
    b = rng.uniform(0, 1, (T, Dk))
    w = rng.uniform(0, 1, (T, Dv))
    S0 = rng.standard_normal((Dk, Dv))
    P = S0.T.copy()                                   # d_v x d_k, the page's orientation
    outs = []
    for t in range(T):
        P = P @ np.diag(np.exp(g[t])) @ (np.eye(Dk) - np.outer(b[t] * k[t], k[t])) \
            + np.outer(w[t] * v[t], k[t])
        outs.append(P @ q[t])
    o, ht = kda_oracle.gdn2_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                    g[None, :, None], b[None, :, None], w[None, :, None],
                                    h0=S0[None, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(outs), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], P.T, rtol=1e-12, atol=1e-12)


def test_gdn2_collapses_to_kda():
    """b = beta 1 and w = beta 1 give KDA (jonahsamost.bearblog.dev, "Gated DeltaNet-2"); two
    independently written oracles, packed sequences with an empty one and h0."""
    w_ = I.WORKLOADS[4]
    x = I.prefill_inputs(w_, heads=[3], lengths=[40, 0, 70])
    q, k, v, g, beta, _, cu = _prefill_np(x)
    rng = np.random.default_rng(72)
    h0 = rng.standard_normal((3, 1, q.shape[-1], v.shape[-1]))
    bb = np.repeat(beta[..., None], q.shape[-1], axis=-1)
    ww = np.repeat(beta[..., None], v.shape[-1], axis=-1)
    o, ht = kda_oracle.gdn2_forward(q, k, v, g, bb, ww, h0=h0, cu_seqlens=cu)
    o2, ht2 = kda_oracle.kda_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    assert _rel(o, o2) <= 1e-12
    assert _rel(ht, ht2) <= 1e-12


def test_gdn2_zero_erase_is_gated_linear_attention():
    """b = 0 erases nothing: S_t = Diag(exp g_t) S_(t-1) + k_t (w_t * v_t)^T, so with S_0 = 0
    o_t = sum_(j <= t) (q_t * exp(G_t - G_j)) . k_j (w_j * v_j), brute force over pairs."""
    rng = np.random.default_rng(73)
    T, Dk, Dv = 18, 4, 3
    q = rng.standard_normal((T, Dk))
    k = rng.standard_normal((T, Dk))
    v = rng.standard_normal((T, Dv))
    g = -rng.uniform(0, 0.5, (T, Dk))
    w = rng.uniform(0, 1, (T, Dv))
    G = np.cumsum(g, axis=0)
    ref = np.zeros((T, Dv))
    for t in range(T):
        for j in range(t + 1):
            ref[t] += np.sum(q[t] * np.exp(G[t] - G[j]) * k[j]) * (w[j] * v[j])
    o, _ = kda_oracle.gdn2_forward(q[None, :, None], k[None, :, None], v[None, :, None],
                                   g[None, :, None], np.zeros((1, T, 1, Dk)), w[None, :, None])
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-11, atol=1e-12)


def test_native_gdn2_matches_numpy():
    for x, b, w in (I.gdn2_prefill_inputs(I.WORKLOADS[1], heads=[0, 3], T=130),
                    I.gdn2_prefill_inputs(I.WORKLOADS[4], heads=[2], lengths=[65, 0, 1, 40])):
        q, k, v, g, _, h0, cu = _prefill_np(x)
        o_ref, ht_ref = kda_oracle.gdn2_forward(q, k, v, g, _np(b), _np(w), h0=h0, cu_seqlens=cu)
        o_c, ht_c = native.gdn2_prefill(x.q, x.k, x.v, x.g, b, w, h0=x.h0, cu_seqlens=cu)
        assert _rel(o_c, o_ref) <= 1e-12
        assert _rel(ht_c, ht_ref) <= 1e-12
    y, b, w = I.gdn2_decode_inputs(I.WORKLOADS[3], heads=[0, 9], N=4)
    args = [t.double().numpy() for t in (y.q, y.k, y.v, y.g, b, w, y.state)]
    o_ref, S_ref = kda_oracle.gdn2_decode(*args, scale=0.7)
    o_c, S_c = native.gdn2_decode(y.q, y.k, y.v, y.g, b, w, y.state, scale=0.7)
    assert _rel(o_c, o_ref) <= 1e-12
    assert _rel(S_c, S_ref) <= 1e-12


def test_gdn2_decode_steps_equal_forward():
    x, b, w = I.gdn2_prefill_inputs(I.WORKLOADS[1], heads=[1], T=20)
    q, k, v, g, _, h0, _ = _prefill_np(x)
    bn, wn = _np(b), _np(w)
    o, ht = kda_oracle.gdn2_forward(q, k, v, g, bn, wn, h0=h0)
    S = h0
    for t in range(q.shape[1]):
        od, S = kda_oracle.gdn2_decode(q[:, t], k[:, t], v[:, t], g[:, t], bn[:, t], wn[:, t], S)
        np.testing.assert_allclose(od, o[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, ht, rtol=1e-12, atol=1e-12)


# --- input preparation ------------------------------------------------------------------------
def test_prepare_inputs_closed_forms():
    """Normalised q and k (zhilingong.com, sections 4 and 5.3): unit k parallel to k, |q^| =
    scale, a zero row stays zero; alpha = exp(g) = sigmoid(a) in (0, 1), log sigmoid(0) =
    -log 2, g -> a for a -> -inf and g -> -exp(-a) for a -> +inf without cancelling to 0;
    beta = sigmoid(b) with beta(0) = 1/2 and beta(x) + beta(-x) = 1."""
    import math
    rng = np.random.default_rng(81)
    q = rng.standard_normal((5, 3, 16)) * 3.0
    k = rng.standard_normal((5, 3, 16)) * 0.2
    q[2, 1] = 0.0
    a = np.array([0.0, -40.0, 30.0, 1.5, -2.25])
    b = np.array([0.0, 3.0, -3.0, 0.7, -0.7])
    qh, kh, g, beta = kda_oracle.prepare_inputs(q, k, np.broadcast_to(a[:, None, None], q.shape),
                                                np.broadcast_to(b[:, None], q.shape[:2]),
                                                scale=0.25)
    np.testing.assert_allclose(np.linalg.norm(kh, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.sum(kh * k, axis=-1), np.linalg.norm(k, axis=-1), rtol=1e-14)
    nq = np.linalg.norm(qh, axis=-1)
    assert nq[2, 1] == 0.0 and np.all(qh[2, 1] == 0.0)
    np.testing.assert_allclose(np.delete(nq.ravel(), 2 * 3 + 1), 0.25, rtol=1e-14)
    gs = g[:, 0, 0]
    assert gs[0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert gs[1] == pytest.approx(-40.0, rel=1e-15)
    assert gs[2] == pytest.approx(-math.exp(-30.0), rel=1e-12) and gs[2] < 0.0
    for i in (3, 4):
        assert gs[i] == pytest.approx(math.log(1.0 / (1.0 + math.exp(-a[i]))), rel=1e-14)
    assert np.all(np.exp(gs) < 1.0) and np.all(np.exp(gs) > 0.0)
    bs = beta[:, 0]
    assert bs[0] == 0.5
    assert bs[1] + bs[2] == pytest.approx(1.0, rel=1e-15)
    assert bs[3] + bs[4] == pytest.approx(1.0, rel=1e-15)
