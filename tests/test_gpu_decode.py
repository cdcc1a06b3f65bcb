"""Decode-step parity on the GPU (through the C ABI) against the float64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_channel_amd as kda
from gated_delta_rule_channel_amd import inputs as I
from oracle import native
from tests.parity_util import check

pytestmark = pytest.mark.gpu


def _run(x: I.DecodeInputs, dtype: str):
    dev = torch.device("cuda:0")
    q, k, v, g, b = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta))
    st = x.state.to(dev)
    o = kda.decode_step(q, k, v, g, b, st, scale=x.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), st.cpu().numpy()


def test_decode_full_workload():
    """The decode workload at full size: 256 requests x 64 heads x 128 x 128 fp32 states."""
    w = I.WORKLOADS[3]
    print(f"[decode] {w.name}", flush=True)
    x = I.decode_inputs(w)
    o_ref, S_ref = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state)
    o, S = _run(x, w.dtype)
    check("o", o, o_ref, w.dtype)
    check("state", S, S_ref, w.dtype)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (64, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_shapes(dk, dv, dtype):
    import dataclasses
    w = dataclasses.replace(I.WORKLOADS[3], Dk=dk, Dv=dv, dtype=dtype, H=3, N=5)
    print(f"[decode] dk={dk} dv={dv} {dtype}", flush=True)
    x = I.decode_inputs(w)
    o_ref, S_ref = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state, scale=0.75)
    x.scale = 0.75
    o, S = _run(x, dtype)
    check("o", o, o_ref, dtype)
    check("state", S, S_ref, dtype)


def test_decode_steps_equal_prefill():
    """T decode steps against a carried state equal one prefill over the same tokens."""
    w = I.WORKLOADS[1]
    x = I.prefill_inputs(w, heads=[0, 1], T=70)
    dev = torch.device("cuda:0")
    o_pf, ht_pf = kda.fwd_chunked(*(t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta)),
                                  initial_state=x.h0.to(dev))
    st = x.h0.to(dev).clone()
    outs = []
    for t in range(x.q.shape[1]):
        sl = lambda a: a[:, t].contiguous().to(dev)
        outs.append(kda.decode_step(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), st))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).cpu().numpy()
    check("o(decode) vs o(prefill)", o_dec, o_pf.cpu().numpy(), "f32")
    check("state(decode) vs ht(prefill)", st.cpu().numpy(), ht_pf.cpu().numpy(), "f32")


def test_decode_bf16_output_is_rounded_fp32_output():
    w = I.WORKLOADS[3]
    x = I.decode_inputs(w, heads=[0, 1, 2], N=7)
    dev = torch.device("cuda:0")
    q, k, v, g, b = (t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta))
    s1, s2 = x.state.to(dev), x.state.to(dev)
    o32 = kda.decode_step(q, k, v, g, b, s1)
    o16 = kda.decode_step(q, k, v, g, b, s2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_gate_closed_is_pure_decay(dtype):
    """beta = 0: S' = diag(exp(g)) S exactly as written, and o = scale q^T S'."""
    import dataclasses
    w = dataclasses.replace(I.WORKLOADS[3], H=4, N=9, dtype=dtype)
    x = I.decode_inputs(w)
    x.beta = torch.zeros_like(x.beta)
    x.scale = 0.5
    print(f"[decode] beta = 0 {dtype}", flush=True)
    o_ref, S_ref = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state, scale=0.5)
    o, S = _run(x, dtype)
    check("o", o, o_ref, dtype)
    check("state", S, S_ref, dtype)
    S_cf = np.exp(x.g.double().numpy())[..., None] * x.state.double().numpy()
    o_cf = 0.5 * np.einsum("nhi,nhij->nhj", x.q.double().numpy(), S_cf)
    check("state (closed form)", S, S_cf, "f32")
    check("o (closed form)", o, o_cf, dtype)


def test_decode_no_decay_unit_beta_stores_pair():
    """g = 0, beta = 1 with unit-norm keys: after the step k^T S' = v for every request."""
    import dataclasses
    w = dataclasses.replace(I.WORKLOADS[3], H=4, N=9, dtype="f32")
    x = I.decode_inputs(w)
    x.g = torch.zeros_like(x.g)
    x.beta = torch.ones_like(x.beta)
    print("[decode] g = 0, beta = 1", flush=True)
    o_ref, S_ref = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state)
    o, S = _run(x, "f32")
    check("o", o, o_ref, "f32")
    check("state", S, S_ref, "f32")
    got = np.einsum("nhi,nhij->nhj", x.k.double().numpy(), S.astype(np.float64))
    check("k^T S' vs v", got, x.v.double().numpy(), "f32")


def test_alternating_state_order_gives_identical_results():
    """Successive decode calls visit the states in opposite orders (for the Infinity Cache);
    two consecutive calls on copies of one state must agree bit for bit, for the single-step
    and the multi-token decode."""
    w = I.WORKLOADS[3]
    x = I.decode_inputs(w, heads=list(range(16)), N=32)
    dev = torch.device("cuda:0")
    a = [t.to(dev) for t in (x.q, x.k, x.v, x.g, x.beta)]
    print("[decode] alternating order", flush=True)
    s1, s2 = x.state.to(dev), x.state.to(dev)
    o1 = kda.decode_step(*a, s1)
    o2 = kda.decode_step(*a, s2)
    m = [t[:, None].expand(-1, 3, *t.shape[1:]).contiguous() for t in a]
    p1, p2 = x.state.to(dev), x.state.to(dev)
    r1 = kda.decode_multi(*m, p1)
    r2 = kda.decode_multi(*m, p2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(r1, r2) and torch.equal(p1, p2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_nan_in_one_state_stays_there(dtype):
    """A NaN in one (request, head)'s inputs and another in one state element corrupt only
    those two states and outputs; every other one matches the oracle."""
    import dataclasses
    w = dataclasses.replace(I.WORKLOADS[3], dtype=dtype, H=4, N=6)
    x = I.decode_inputs(w)
    x.k[2, 1, 3] = float("nan")
    x.state[4, 2, 10, 20] = float("nan")
    print(f"[decode] NaN in two states {dtype}", flush=True)
    o_ref, S_ref = native.decode(x.q, x.k, x.v, x.g, x.beta, x.state)
    o, S = _run(x, dtype)
    ok = np.ones((w.N, w.H), dtype=bool)
    ok[2, 1] = ok[4, 2] = False
    check("o (other states)", o[ok], o_ref[ok], dtype)
    check("state (other states)", S[ok], S_ref[ok], dtype)
    assert not np.all(np.isfinite(o[2, 1])) and not np.all(np.isfinite(S[4, 2]))
