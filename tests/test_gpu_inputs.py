"""Input preparation on the GPU (kda_prepare_inputs through the C ABI) against the float64
oracle: normalised q and k, g = log sigmoid(a), beta = sigmoid(b).

Bounds: a bfloat16 output is the float32 result rounded to nearest even, which is at most
half an ulp (2^-8 relative) from that float32 value; where the float32 value and the exact
one straddle a rounding boundary the two roundings differ by one ulp, so the check is one
bfloat16 ulp, 2^-7 relative, from the oracle's value. Float32 outputs: within 1e-5
relative (g, through expf and log1pf) and 2e-6 (q, k).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_channel_amd as kda
from oracle import kda_oracle, native
from tests.parity_util import check

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _raw(tokens, H, Dk, dtype, seed):
    rng = np.random.default_rng(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.from_numpy(2.0 * rng.standard_normal((tokens, H, Dk))).to(dt)
    k = torch.from_numpy(0.5 * rng.standard_normal((tokens, H, Dk))).to(dt)
    a = torch.from_numpy(3.0 * rng.standard_normal((tokens, H, Dk))).to(dt)
    a[0, 0, :4] = torch.tensor([30.0, -30.0, 0.0, 12.0]).to(dt)      # both tails
    b = torch.from_numpy(2.0 * rng.standard_normal((tokens, H))).to(dt)
    q[1, 0] = 0.0                                                     # a zero row
    return q, k, a, b


def _close(name, got, ref, rtol):
    got = got.double().numpy() if isinstance(got, torch.Tensor) else got
    err = np.abs(got - ref)
    lim = rtol * np.abs(ref)
    worst = float(np.max(err / np.maximum(lim, 1e-300)))
    print(f"  {name}: worst err / bound {worst:.3f}", flush=True)
    assert np.all(err <= lim), f"{name}: worst err / bound {worst:.3f}"


@pytest.mark.parametrize("Dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prepare_inputs_matches_oracle(Dk, dtype):
    tokens, H = 77, 3
    print(f"[inputs] Dk={Dk} {dtype}", flush=True)
    q, k, a, b = _raw(tokens, H, Dk, dtype, 90 + Dk)
    qh, kh, g, beta = kda.prepare_inputs(*(t.to(DEV) for t in (q, k, a, b)), scale=Dk ** -0.5)
    torch.cuda.synchronize()
    rq, rk, rg, rb = kda_oracle.prepare_inputs(*(t.double().numpy() for t in (q, k, a, b)),
                                               scale=Dk ** -0.5)
    r16 = 2.0 ** -7
    _close("q^", qh.cpu(), rq, r16 if dtype == "bf16" else 2e-6)
    _close("k^", kh.cpu(), rk, r16 if dtype == "bf16" else 2e-6)
    _close("g", g.cpu(), rg, 1e-5)
    _close("beta", beta.cpu(), rb, r16 if dtype == "bf16" else 2e-6)
    assert torch.all(qh[1, 0] == 0)
    assert g.dtype == torch.float32 and bool(torch.all(g < 0))


def test_prepare_inputs_in_place_equals_out_of_place():
    q, k, a, b = (t.to(DEV) for t in _raw(130, 4, 128, "bf16", 7))
    print("[inputs] in place", flush=True)
    ref = kda.prepare_inputs(q, k, a, b, scale=0.3)
    g = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    out = kda.prepare_inputs(q, k, a, b, scale=0.3, out=(q, k, g, b))
    torch.cuda.synchronize()
    for x, y in zip(out, ref):
        assert torch.equal(x, y)


def test_prepared_inputs_feed_the_prefill():
    """Raw projections -> prepare_inputs -> fwd_chunked, against the oracle's own preparation
    and recurrence (B1 T300 H4 d128 bf16)."""
    B, T, H, D = 1, 300, 4, 128
    print("[inputs] prepare + prefill", flush=True)
    q, k, a, b = _raw(B * T, H, D, "bf16", 8)
    v = torch.from_numpy(np.random.default_rng(9).standard_normal((B, T, H, D))).bfloat16()
    qh, kh, g, beta = kda.prepare_inputs(*(t.to(DEV) for t in (q, k, a, b)), scale=D ** -0.5)
    rs = lambda t: t.view(B, T, *t.shape[1:])
    o, ht = kda.fwd_chunked(rs(qh), rs(kh), v.to(DEV), rs(g), rs(beta))
    torch.cuda.synchronize()
    rq, rk, rg, rb = kda_oracle.prepare_inputs(*(t.double().numpy() for t in (q, k, a, b)),
                                               scale=D ** -0.5)
    cast = lambda x: torch.from_numpy(x).to(torch.bfloat16)
    o_ref, ht_ref = native.prefill(rs(cast(rq)), rs(cast(rk)), v, rs(torch.from_numpy(rg).float()),
                                   rs(cast(rb)))
    check("o", o.cpu().numpy(), o_ref, "bf16")
    check("ht", ht.cpu().numpy(), ht_ref, "bf16")


def _raw_v(B, T, H, D, seed):
    q, k, a, b = _raw(B * T, H, D, "bf16", seed)
    v = torch.from_numpy(np.random.default_rng(seed + 1).standard_normal((B * T, H, D))).bfloat16()
    rs = lambda t: t.reshape(B, T, *t.shape[1:]).contiguous()
    return rs(q), rs(k), rs(v), rs(a), rs(b)


def _raw_ref(q, k, v, a, b, scale, h0=None, cu=None):
    """The oracle's float64 preparation, then its recurrence."""
    rq, rk, rg, rb = kda_oracle.prepare_inputs(*(t.double().numpy() for t in (q, k, a, b)),
                                               scale=scale)
    f = lambda x: torch.from_numpy(x).float()
    return native.prefill(f(rq), f(rk), v, f(rg), f(rb), h0=h0, cu_seqlens=cu)


@pytest.mark.parametrize("B,T,H", [(1, 300, 4), (2, 130, 3), (1, 64, 2)])
def test_raw_prefill_matches_oracle(B, T, H):
    """kda_fwd_chunked_raw (preparation inside the prefill) against the oracle's preparation
    and recurrence, with a zero query row and saturated gate logits, ragged last chunks."""
    D = 128
    print(f"[inputs] raw prefill B{B} T{T} H{H}", flush=True)
    q, k, v, a, b = _raw_v(B, T, H, D, 20 + T)
    o, ht = kda.fwd_chunked_raw(*(t.to(DEV) for t in (q, k, v, a, b)), scale=D ** -0.5)
    torch.cuda.synchronize()
    o_ref, ht_ref = _raw_ref(q, k, v, a, b, D ** -0.5)
    check("o", o.cpu().numpy(), o_ref, "bf16")
    check("ht", ht.cpu().numpy(), ht_ref, "bf16")


def test_raw_prefill_packed_with_initial_state():
    """Packed sequences (one empty) and an initial state through the raw entry point."""
    D, H = 128, 3
    lens = [70, 0, 129, 5]
    T = sum(lens)
    print("[inputs] raw prefill packed", flush=True)
    q, k, v, a, b = _raw_v(1, T, H, D, 31)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    h0 = torch.from_numpy(0.1 * np.random.default_rng(32).standard_normal((len(lens), H, D, D))).float()
    o, ht = kda.fwd_chunked_raw(*(t.to(DEV) for t in (q, k, v, a, b)), scale=0.1,
                                initial_state=h0.to(DEV), cu_seqlens=cu.to(DEV))
    torch.cuda.synchronize()
    o_ref, ht_ref = _raw_ref(q, k, v, a, b, 0.1, h0=h0, cu=cu.numpy())
    check("o", o.cpu().numpy(), o_ref, "bf16")
    check("ht", ht.cpu().numpy(), ht_ref, "bf16")
    np.testing.assert_array_equal(ht.cpu().numpy()[1], h0.numpy()[1])



def test_raw_prefill_zero_scale_reads_nothing():
    """scale = 0 zeroes every query after normalisation: o is exactly 0, while the state
    (which never sees q) still matches the oracle."""
    B, T, H, D = 1, 150, 2, 128
    print("[inputs] raw prefill scale 0", flush=True)
    q, k, v, a, b = _raw_v(B, T, H, D, 51)
    o, ht = kda.fwd_chunked_raw(*(t.to(DEV) for t in (q, k, v, a, b)), scale=0.0)
    torch.cuda.synchronize()
    _, ht_ref = _raw_ref(q, k, v, a, b, 1.0)
    assert torch.all(o == 0)
    check("ht", ht.cpu().numpy(), ht_ref, "bf16")
